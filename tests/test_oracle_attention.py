"""Pins the attention oracle to things other than itself: closed forms, a
library routine (torch's float64 scaled_dot_product_attention after an
element-by-element gather), brute force, and the invariants the pages state
(paging and tiling change no result; GQA is MHA with each KV head repeated)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A

BS = 16


def _pools(rng, P, Hkv, D, x, dtype=np.float64):
    k = rng.standard_normal((P, Hkv, D // x, BS, x)).astype(dtype)
    v = rng.standard_normal((P, Hkv, D, BS)).astype(dtype)
    return k, v


def _table(rng, P, lens):
    order = rng.permutation(P)
    rows, i = [], 0
    mb = max(1, max((n + BS - 1) // BS for n in lens))
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        nb = (n + BS - 1) // BS
        bt[b, :nb] = order[i:i + nb]
        i += nb
    return bt


def _dense_by_index(k, v, bt_row, n):
    """Element-by-element gather, written from the layout contract directly."""
    Hkv, D, x = k.shape[1], k.shape[2] * k.shape[4], k.shape[4]
    K = np.zeros((n, Hkv, D))
    V = np.zeros((n, Hkv, D))
    for t in range(n):
        p = bt_row[t // BS]
        for h in range(Hkv):
            for d in range(D):
                K[t, h, d] = k[p, h, d // x, t % BS, d % x]
                V[t, h, d] = v[p, h, d, t % BS]
    return K, V


@pytest.mark.parametrize("Hq,Hkv,D,x,lens", [
    (4, 2, 64, 4, [38, 101]),      # the tiny fp32 workload's shape
    (2, 2, 16, 8, [1, 16, 17]),    # MHA, page-boundary lengths
    (8, 1, 32, 8, [33, 5]),        # MQA
    (6, 3, 16, 4, [20]),           # GQA group 2
])
def test_matches_torch_sdpa_float64(Hq, Hkv, D, x, lens):
    rng = np.random.default_rng(7)
    P = sum((n + BS - 1) // BS for n in lens) + 3
    k, v = _pools(rng, P, Hkv, D, x)
    bt = _table(rng, P, lens)
    q = rng.standard_normal((len(lens), Hq, D))
    scale = 1.0 / math.sqrt(D)
    got = A.decode(q, k, v, bt, lens, Hq, Hkv, BS, scale)
    G = Hq // Hkv
    for b, n in enumerate(lens):
        K, V = _dense_by_index(k, v, bt[b], n)
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq][n][D]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(q[b]).unsqueeze(1)                              # [Hq][1][D]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
        np.testing.assert_allclose(got[b], ref[:, 0, :].numpy(), rtol=0, atol=1e-12)


def test_brute_force_python_loops():
    rng = np.random.default_rng(3)
    Hq, Hkv, D, x, lens = 4, 2, 8, 4, [5, 19]
    P = 6
    k, v = _pools(rng, P, Hkv, D, x)
    bt = _table(rng, P, lens)
    q = rng.standard_normal((2, Hq, D))
    scale = 0.37
    got = A.decode(q, k, v, bt, lens, Hq, Hkv, BS, scale)
    for b, n in enumerate(lens):
        for hq in range(Hq):
            h = hq // (Hq // Hkv)
            scores = []
            for t in range(n):
                p, s = bt[b][t // BS], t % BS
                scores.append(scale * sum(q[b, hq, d] * k[p, h, d // x, s, d % x] for d in range(D)))
            den = sum(math.exp(z) for z in scores)
            for d in range(D):
                num = sum(math.exp(scores[t]) * v[bt[b][t // BS], h, d, t % BS] for t in range(n))
                assert abs(got[b, hq, d] - num / den) < 1e-12


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    k, v = _pools(rng, 3, 2, 16, 4)
    bt = np.array([[2, -1]], dtype=np.int32)
    q = rng.standard_normal((1, 4, 16))
    out = A.decode(q, k, v, bt, [1], 4, 2, BS, 0.25)
    for hq in range(4):
        assert np.array_equal(out[0, hq], v[2, hq // 2, :, 0])


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(2)
    k, v = _pools(rng, 4, 1, 16, 4)
    v[:] = 0.625
    bt = np.array([[3, 0, 1]], dtype=np.int32)
    q = rng.standard_normal((1, 2, 16)) * 3
    out = A.decode(q, k, v, bt, [40], 2, 1, BS, 1.0)
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-15)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    k, v = _pools(rng, 3, 1, 16, 4)
    k[:] = rng.standard_normal(4)[None, None, None, None, :]  # every key identical
    bt = np.array([[1, 2]], dtype=np.int32)
    n = 21
    q = rng.standard_normal((1, 1, 16))
    out = A.decode(q, k, v, bt, [n], 1, 1, BS, 0.5)
    mean = np.mean([v[bt[0][t // BS], 0, :, t % BS] for t in range(n)], axis=0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-14)


def test_one_hot_score_selects_one_value():
    rng = np.random.default_rng(5)
    D = 16
    k, v = _pools(rng, 2, 1, D, 4)
    q = rng.standard_normal((1, 1, D))
    k[:] = 0.0
    j = 13
    kj = 64.0 * q[0, 0] / np.dot(q[0, 0], q[0, 0]) * 4  # score_j = 256 >> score_others = 0
    k[1, 0, :, j % BS, :] = kj.reshape(D // 4, 4)
    bt = np.array([[0, 1]], dtype=np.int32)
    out = A.decode(q, k, v, bt, [BS + j + 1], 1, 1, BS, 1.0)
    np.testing.assert_allclose(out[0, 0], v[1, 0, :, j], rtol=0, atol=1e-40 + 1e-100)


def test_two_tokens_worked_weights():
    # scores 0 and ln 3 -> softmax weights 1/4 and 3/4.
    D = 8
    k = np.zeros((1, 1, D // 4, BS, 4))
    v = np.zeros((1, 1, D, BS))
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    k[0, 0, 0, 1, 0] = math.log(3.0)
    v[0, 0, :, 0] = 4.0
    v[0, 0, :, 1] = 8.0
    out = A.decode(q, k, v, np.array([[0]]), [2], 1, 1, BS, 1.0)
    np.testing.assert_allclose(out[0, 0], 0.25 * 4.0 + 0.75 * 8.0, rtol=1e-15)


def test_linear_in_values_and_power_of_two_scale_exact():
    rng = np.random.default_rng(6)
    k, v1 = _pools(rng, 5, 2, 16, 8)
    v2 = rng.standard_normal(v1.shape)
    bt = _table(rng, 5, [30, 45])
    q = rng.standard_normal((2, 4, 16))
    f = lambda vv, qq, sc: A.decode(qq, k, vv, bt, [30, 45], 4, 2, BS, sc)
    np.testing.assert_allclose(f(v1 + 2 * v2, q, 0.3), f(v1, q, 0.3) + 2 * f(v2, q, 0.3),
                               rtol=0, atol=1e-13)
    assert np.array_equal(f(v1, q * 8.0, 0.3 / 8.0), f(v1, q, 0.3))


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(8)
    Hkv, G, D = 3, 4, 16
    k, v = _pools(rng, 7, Hkv, D, 4)
    bt = _table(rng, 7, [50, 33])
    q = rng.standard_normal((2, Hkv * G, D))
    gqa = A.decode(q, k, v, bt, [50, 33], Hkv * G, Hkv, BS, 0.4)
    k_rep = np.repeat(k, G, axis=1)   # KV head h becomes heads h*G .. h*G+G-1
    v_rep = np.repeat(v, G, axis=1)
    mha = A.decode(q, k_rep, v_rep, bt, [50, 33], Hkv * G, Hkv * G, BS, 0.4)
    assert np.array_equal(gqa, mha)
    # and an interleaved head map would differ
    k_il = np.tile(k, (1, G, 1, 1, 1))
    v_il = np.tile(v, (1, G, 1, 1))
    il = A.decode(q, k_il, v_il, bt, [50, 33], Hkv * G, Hkv * G, BS, 0.4)
    assert not np.allclose(gqa, il)


def test_page_permutation_invariance_and_contiguous_equivalence():
    rng = np.random.default_rng(9)
    P, lens = 12, [40, 70]
    k, v = _pools(rng, P, 2, 16, 4)
    bt = _table(rng, P, lens)
    q = rng.standard_normal((2, 2, 16))
    ref = A.decode(q, k, v, bt, lens, 2, 2, BS, 0.25)
    perm = rng.permutation(P)              # physical page p moves to perm[p]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    assert np.array_equal(A.decode(q, k2, v2, bt2, lens, 2, 2, BS, 0.25), ref)
    # contiguous placement: sequence pages laid out in order 0, 1, 2, ...
    used = [bt[b, :(n + BS - 1) // BS] for b, n in enumerate(lens)]
    flat = np.concatenate(used)
    k3, v3 = k[flat], v[flat]
    bt3 = np.full_like(bt, -1)
    i = 0
    for b, u in enumerate(used):
        bt3[b, :len(u)] = np.arange(i, i + len(u))
        i += len(u)
    assert np.array_equal(A.decode(q, k3, v3, bt3, lens, 2, 2, BS, 0.25), ref)


def test_unused_slots_never_read():
    rng = np.random.default_rng(10)
    k, v = _pools(rng, 4, 1, 16, 4)
    bt = np.array([[2, 0, -1]], dtype=np.int32)
    n = 20
    k[2, :, :, :, :] = k[2]
    k[0, :, :, n - BS:, :] = np.nan
    v[0, :, :, n - BS:] = np.nan
    k[1] = np.nan
    v[1] = np.nan
    k[3] = np.nan
    v[3] = np.nan
    out = A.decode(rng.standard_normal((1, 1, 16)), k, v, bt, [n], 1, 1, BS, 0.25)
    assert np.isfinite(out).all()


def test_partials_combine_to_full_attention():
    rng = np.random.default_rng(11)
    n, D = 97, 16
    K = rng.standard_normal((n, D)) * 2
    V = rng.standard_normal((n, D))
    q = rng.standard_normal(D)
    full = A.attend(q, K, V, 0.7)
    for cuts in ([0, 97], [0, 16, 97], [0, 1, 2, 50, 96, 97], [0, 30, 30, 64, 97]):
        parts = [A.partial(q, K[a:b], V[a:b], 0.7) for a, b in zip(cuts[:-1], cuts[1:])]
        got = A.lse_combine([p[0] for p in parts], [p[1] for p in parts])
        np.testing.assert_allclose(got, full, rtol=0, atol=1e-13)


def test_partial_lse_closed_form():
    # equal scores s0 over n tokens: lse = s0 + ln n, output = mean of V.
    n, D = 10, 4
    q = np.array([1.0, 0, 0, 0])
    K = np.zeros((n, D))
    K[:, 0] = 2.5
    V = np.arange(n * D, dtype=np.float64).reshape(n, D)
    o, lse = A.partial(q, K, V, 2.0)
    assert abs(lse - (5.0 + math.log(n))) < 1e-14
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-15)
    o0, l0 = A.partial(q, K[:0], V[:0], 2.0)
    assert l0 == -math.inf and not o0.any()
    # an empty partial weighs nothing
    np.testing.assert_allclose(A.lse_combine([o, o0 + 1e30], [lse, l0]), o, rtol=1e-15)
    assert not A.lse_combine([o0, o0], [l0, l0]).any()


def test_zero_length_sequence_gives_zeros():
    rng = np.random.default_rng(12)
    k, v = _pools(rng, 2, 1, 16, 4)
    out = A.decode(rng.standard_normal((2, 1, 16)), k, v, np.array([[0], [1]]), [0, 3], 1, 1, BS, 1.0)
    assert not out[0].any() and np.isfinite(out[1]).all() and out[1].any()


def test_append_writes_exactly_the_slot_bits():
    rng = np.random.default_rng(13)
    P, Hkv, D, x = 6, 2, 16, 8
    k = rng.integers(0, 2 ** 16, size=(P, Hkv, D // x, BS, x), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(P, Hkv, D, BS), dtype=np.uint16)
    bt = np.array([[4, 1, -1], [0, -1, -1]], dtype=np.int32)
    pos = np.array([21, 15])
    kn = rng.integers(0, 2 ** 16, size=(2, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 2 ** 16, size=(2, Hkv, D), dtype=np.uint16)
    k2, v2 = A.append(k, v, bt, pos, kn, vn, BS)
    kd = (k2 != k)
    vd = (v2 != v)
    exp_k = np.zeros_like(kd)
    exp_v = np.zeros_like(vd)
    # sequence 0: position 21 -> block 1 (page 1), slot 5; sequence 1: position 15 -> page 0, slot 15
    for b, (p, s) in enumerate([(1, 5), (0, 15)]):
        for h in range(Hkv):
            for d in range(D):
                assert k2[p, h, d // x, s, d % x] == kn[b, h, d]
                assert v2[p, h, d, s] == vn[b, h, d]
                exp_k[p, h, d // x, s, d % x] = kn[b, h, d] != k[p, h, d // x, s, d % x]
                exp_v[p, h, d, s] = vn[b, h, d] != v[p, h, d, s]
    assert np.array_equal(kd, exp_k) and np.array_equal(vd, exp_v)


def test_copy_blocks_then_fork_decode_equals_unshared_cache():
    # Three sequences sharing a 40-token prefix (pages shared through the block
    # table) give the same outputs as three private copies of that prefix.
    rng = np.random.default_rng(21)
    Hkv, G, D, x = 2, 3, 16, 4
    k, v = _pools(rng, 12, Hkv, D, x)
    shared = np.array([[5, 9, 2]] * 3, dtype=np.int32)
    q = rng.standard_normal((3, Hkv * G, D))
    out_shared = A.decode(q, k, v, shared, [40] * 3, Hkv * G, Hkv, BS, 0.3)
    k2, v2 = A.copy_blocks(k, v, [5, 9, 2, 5, 9, 2], [0, 1, 3, 4, 6, 7])
    private = np.array([[5, 9, 2], [0, 1, 3], [4, 6, 7]], dtype=np.int32)
    assert np.array_equal(A.decode(q, k2, v2, private, [40] * 3, Hkv * G, Hkv, BS, 0.3), out_shared)
    assert np.array_equal(k2[0], k[5]) and np.array_equal(v2[7], v[2]) and np.array_equal(k2[8], k[8])
