"""The 8-bit V-code tile order shared by the library and the tests'
conversions (workloads.v_codes_to_logical / v_codes_from_logical): feature d,
slot t sits at byte 1024 (d / 64) + 256 (t / 4) + 16 (d % 16) + 4 ((d / 16) % 4)
+ t % 4 of its (page, KV head) tile, as include/pkv.h states.  The kernels'
own writes of this order are checked bit for bit against the oracle's
quantizing append in tests/test_gpu_q8.py."""
import numpy as np
import pytest

import workloads as W


def offset(d, t):
    return 1024 * (d // 64) + 256 * (t // 4) + 16 * (d % 16) + 4 * ((d // 16) % 4) + t % 4


@pytest.mark.parametrize("D", [64, 128])
def test_tile_order_matches_documented_offsets(D):
    P, H = 3, 2
    rng = np.random.default_rng(D)
    logical = rng.integers(0, 256, size=(P, H, D, 16), dtype=np.uint8)
    lib = W.v_codes_from_logical(logical)
    assert lib.shape == (P, H, D // 64, 4, 16, 4, 4)
    flat = lib.reshape(P, H, 16 * D)
    offs = np.array([[offset(d, t) for t in range(16)] for d in range(D)])
    assert sorted(offs.ravel().tolist()) == list(range(16 * D))      # a permutation of the tile's bytes
    assert np.array_equal(flat[:, :, offs], logical)
    assert np.array_equal(W.v_codes_to_logical(lib), logical)


def test_lane_reads_its_operand_bytes():
    # Lane L = 16 c + n's 16-byte load j holds slots 4c..4c+3 of features
    # 16 nb + n for nb = 4 j .. 4 j + 3, in that order.
    D = 128
    d = np.arange(D)[:, None]
    t = np.arange(16)[None, :]
    logical = (16 * d + t).astype(np.int32)            # tag of (feature, slot)
    flat = np.empty(16 * D, dtype=np.int32)
    flat[offset(d, t)] = logical
    for lane in (0, 5, 17, 63):
        c, n = lane // 16, lane % 16
        for j in range(D // 64):
            got = flat[1024 * j + 16 * lane: 1024 * j + 16 * lane + 16].reshape(4, 4)
            want = np.array([[16 * (16 * nb + n) + 4 * c + e for e in range(4)] for nb in range(4 * j, 4 * j + 4)])
            assert np.array_equal(got, want)


def test_torch_conversions_agree_with_numpy():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    logical = rng.integers(0, 256, size=(2, 3, 128, 16), dtype=np.uint8)
    lib_t = W.v_codes_from_logical(torch.from_numpy(logical))
    assert np.array_equal(lib_t.numpy(), W.v_codes_from_logical(logical))
    assert np.array_equal(W.v_codes_to_logical(lib_t).numpy(), logical)
