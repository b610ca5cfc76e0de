"""Pins the 8-bit KV-cache oracle to things other than itself: hand-worked
quantizations (scales that are exact in float32), exact round trips of grid
points, the half-step error bound, invariants (zero maps to zero, power-of-two
scaling), the append's slot contract by index, and decode over the quantized
cache against the already pinned decode run on explicitly dequantized pools."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import kv_quant as Q

BS = 16


def test_hand_worked_vector_with_exact_scale():
    # lo = -3.5, hi = 60.25: s = 63.75 / 255 = 0.25 exactly, z = rint(3.5 / 0.25) = 14
    x = np.array([-3.5, 60.25, 0.0, 1.125, 1.375, -0.125, 10.0], dtype=np.float32)
    u, s, z = Q.quantize_vector(x)
    assert s == np.float32(0.25) and z == np.float32(14)
    # rint(x / s) + z: -14+14, 241+14, 0+14, rint(4.5)=4 (half to even)+14, rint(5.5)=6+14,
    # rint(-0.5)=-0 +14, 40+14
    assert u.tolist() == [0, 255, 14, 18, 20, 14, 54]
    xh = Q.dequantize_vector(u, s, z)
    assert xh.tolist() == [-3.5, 60.25, 0.0, 1.0, 1.5, 0.0, 10.0]


@pytest.mark.parametrize("x,s,z,u", [
    ([0.0, 0.0, 0.0], 1.0, 0.0, [0, 0, 0]),                       # all zero: scale 1
    ([0.0, 255.0, 127.5, 128.5], 1.0, 0.0, [0, 255, 128, 128]),   # half to even
    ([2.0, 4.0, 8.0, 255.0 * 4], 4.0, 0.0, [0, 1, 2, 255]),       # all positive: lo = 0
    ([-255.0 * 2, -2.0, -1.0], 2.0, 255.0, [0, 254, 255]),        # all negative: hi = 0; -1/2 rounds to 0
])
def test_special_ranges(x, s, z, u):
    cu, cs, cz = Q.quantize_vector(np.array(x, dtype=np.float32))
    assert (cs, cz) == (np.float32(s), np.float32(z))
    assert cu.tolist() == u


def test_grid_points_round_trip_exactly():
    # s = 0.125, z = 40: the vector's extremes are s*(0 - z) and s*(255 - z)
    s, z = 0.125, 40
    k = np.array([0, 255, 40, 1, 100, 254, 39, 41, 77], dtype=np.int64)
    x = (s * (k - z)).astype(np.float32)
    u, cs, cz = Q.quantize_vector(x)
    assert cs == np.float32(s) and cz == np.float32(z)
    assert np.array_equal(u.astype(np.int64), k)
    assert np.array_equal(Q.dequantize_vector(u, cs, cz), x.astype(np.float64))


def test_random_vectors_error_bound_and_invariants():
    rng = np.random.default_rng(11)
    for trial in range(300):
        D = (64, 128)[trial % 2]
        x = (rng.standard_normal(D) * rng.uniform(1e-3, 50) + rng.uniform(-20, 20)).astype(np.float32)
        u, s, z = Q.quantize_vector(x)
        assert u.dtype == np.uint8 and 0 <= z <= 255 and s > 0
        xh = Q.dequantize_vector(u, s, z)
        err = np.abs(xh - x.astype(np.float64))
        # half a step, except the top of the range, which float32 rounding of
        # s and x / s may push one code past 255 (clipped: at most one step)
        assert (err <= 0.5 * s * (1 + 1e-5) + 1e-30).mean() > 0.99
        assert err.max() <= 1.0 * s * (1 + 1e-5)
        # 0 maps exactly to the zero point
        u0, _, _ = Q.quantize_vector(np.concatenate([x, [0.0]]).astype(np.float32))
        assert Q.dequantize_vector(u0[-1:], s, z)[0] == 0.0
        # power-of-two scaling: same codes and zero point, scale times 2^k
        u2, s2, z2 = Q.quantize_vector((x * np.float32(8.0)).astype(np.float32))
        assert np.array_equal(u2, u) and z2 == z and s2 == np.float32(s * 8)


def _pools(rng, P, Hkv, D):
    kc = rng.integers(0, 256, size=(P, Hkv, D // 16, BS, 16), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(P, Hkv, D, BS), dtype=np.uint8)
    meta = np.zeros((P, Hkv, 4, BS), dtype=np.float32)
    meta[:, :, 0] = rng.uniform(0.005, 0.05, size=(P, Hkv, BS))
    meta[:, :, 1] = rng.integers(0, 256, size=(P, Hkv, BS))
    meta[:, :, 2] = rng.uniform(0.005, 0.05, size=(P, Hkv, BS))
    meta[:, :, 3] = rng.integers(0, 256, size=(P, Hkv, BS))
    return kc, vc, meta


def test_append_writes_exactly_the_slot():
    rng = np.random.default_rng(12)
    P, Hkv, D = 6, 2, 64
    kc, vc, meta = _pools(rng, P, Hkv, D)
    bt = np.array([[4, 1, -1], [2, 5, 0]], dtype=np.int32)
    pos = [17, 35]                     # (page 1, slot 1) and (page 0, slot 3)
    kn = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    kc2, vc2, m2 = Q.append(kc, vc, meta, bt, pos, kn, vn, BS)
    changed = np.zeros((P, BS), dtype=bool)
    for b, (page, slot) in enumerate([(1, 1), (0, 3)]):
        changed[page, slot] = True
        for h in range(Hkv):
            ku, ks, kz = Q.quantize_vector(kn[b, h])
            vu, vs, vz = Q.quantize_vector(vn[b, h])
            for d in range(D):   # the layout contract, element by element
                assert kc2[page, h, d // 16, slot, d % 16] == ku[d]
                assert vc2[page, h, d, slot] == vu[d]
            assert m2[page, h, :, slot].tolist() == [ks, kz, vs, vz]
    for p in range(P):
        for t in range(BS):
            if not changed[p, t]:
                assert np.array_equal(kc2[p, :, :, t], kc[p, :, :, t])
                assert np.array_equal(vc2[p, :, :, t], vc[p, :, :, t])
                assert np.array_equal(m2[p, :, :, t], meta[p, :, :, t])


def _dequantized_dense_pools(kc, vc, meta, X):
    """K [P][Hkv][D/X][16][X] and V [P][Hkv][D][16] float64 pools, filled
    element by element from the codes and meta by the layout contract."""
    P, Hkv, D = vc.shape[0], vc.shape[1], vc.shape[2]
    K = np.zeros((P, Hkv, D // X, BS, X))
    V = np.zeros((P, Hkv, D, BS))
    for p in range(P):
        for h in range(Hkv):
            for t in range(BS):
                ks, kz, vs, vz = (float(v) for v in meta[p, h, :, t])
                for d in range(D):
                    K[p, h, d // X, t, d % X] = ks * (int(kc[p, h, d // 16, t, d % 16]) - kz)
                    V[p, h, d, t] = vs * (int(vc[p, h, d, t]) - vz)
    return K, V


@pytest.mark.parametrize("Hq,Hkv,D,lens", [(8, 2, 64, [40, 5, 17]), (4, 4, 32, [33]), (8, 1, 16, [16, 70])])
def test_decode_equals_decode_of_dequantized_pools(Hq, Hkv, D, lens):
    rng = np.random.default_rng(13)
    P = sum((n + BS - 1) // BS for n in lens) + 2
    kc, vc, meta = _pools(rng, P, Hkv, D)
    order = rng.permutation(P)
    mb = max((n + BS - 1) // BS for n in lens)
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    i = 0
    for b, n in enumerate(lens):
        nb = (n + BS - 1) // BS
        bt[b, :nb] = order[i:i + nb]
        i += nb
    q = rng.standard_normal((len(lens), Hq, D))
    got = Q.decode(q, kc, vc, meta, bt, lens, Hq, Hkv, BS, 1 / math.sqrt(D))
    K, V = _dequantized_dense_pools(kc, vc, meta, 8)
    ref = A.decode(q, K, V, bt, lens, Hq, Hkv, BS, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_decode_brute_force_tiny():
    rng = np.random.default_rng(14)
    Hq, Hkv, D, n = 2, 1, 16, 20
    kc, vc, meta = _pools(rng, 3, Hkv, D)
    bt = np.array([[2, 0]], dtype=np.int32)
    q = rng.standard_normal((1, Hq, D))
    got = Q.decode(q, kc, vc, meta, bt, [n], Hq, Hkv, BS, 0.3)
    for hq in range(Hq):
        sc, vals = [], []
        for t in range(n):
            p, s = bt[0][t // BS], t % BS
            ks, kz, vs, vz = (float(v) for v in meta[p, 0, :, s])
            k = [ks * (int(kc[p, 0, d // 16, s, d % 16]) - kz) for d in range(D)]
            vals.append([vs * (int(vc[p, 0, d, s]) - vz) for d in range(D)])
            sc.append(0.3 * sum(q[0, hq, d] * k[d] for d in range(D)))
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        for d in range(D):
            assert abs(got[0, hq, d] - sum(wi * v[d] for wi, v in zip(w, vals)) / sum(w)) < 1e-12
