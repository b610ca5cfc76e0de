"""Pins the multi-token (causal, optionally windowed) decode oracle to things
other than itself: one query token reduces to the pinned single-token decode;
all tokens as queries is causal self-attention, checked against torch's
float64 scaled_dot_product_attention with a causal (or banded) mask; keys
outside a query's range do not change its output; brute force."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A

from .test_oracle_attention import _pools, _table

BS = 16


def _case(rng, Hq, Hkv, D, lens, x=8):
    P = sum((n + BS - 1) // BS for n in lens) + 2
    k, v = _pools(rng, P, Hkv, D, x)
    bt = _table(rng, P, lens)
    return k, v, bt


def test_one_query_token_is_decode():
    rng = np.random.default_rng(31)
    Hq, Hkv, D, lens = 8, 2, 32, [40, 17, 1]
    k, v, bt = _case(rng, Hq, Hkv, D, lens)
    q = rng.standard_normal((3, Hq, D))
    ref = A.decode(q, k, v, bt, lens, Hq, Hkv, BS, 0.2)
    got = A.decode_multi(q[:, None], k, v, bt, lens, 1, Hq, Hkv, BS, 0.2)
    assert np.array_equal(got[:, 0], ref)


def _dense(k, v, bt_row, n):
    K, V = A.gather(k, v, bt_row, n, BS)      # [n][Hkv][D], pinned in test_oracle_attention
    return torch.from_numpy(K).permute(1, 0, 2), torch.from_numpy(V).permute(1, 0, 2)


@pytest.mark.parametrize("Hq,Hkv,D,n,window", [(4, 2, 32, 37, 0), (2, 2, 16, 50, 0), (8, 1, 16, 33, 0),
                                              (4, 2, 32, 45, 7), (2, 1, 16, 20, 16), (4, 4, 16, 18, 1)])
def test_all_tokens_as_queries_is_causal_self_attention(Hq, Hkv, D, n, window):
    rng = np.random.default_rng(32)
    k, v, bt = _case(rng, Hq, Hkv, D, [n])
    q = rng.standard_normal((1, n, Hq, D))
    got = A.decode_multi(q, k, v, bt, [n], n, Hq, Hkv, BS, 1 / math.sqrt(D), window)
    K, V = _dense(k, v, bt[0], n)
    G = Hq // Hkv
    Kt, Vt = K.repeat_interleave(G, dim=0), V.repeat_interleave(G, dim=0)      # [Hq][n][D]
    qt = torch.from_numpy(q[0]).permute(1, 0, 2)                               # [Hq][n][D]
    i = torch.arange(n)[:, None]
    t = torch.arange(n)[None, :]
    mask = t <= i
    if window > 0:
        mask &= t > i - window
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=1 / math.sqrt(D))
    np.testing.assert_allclose(got[0], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_keys_outside_the_range_do_not_matter():
    rng = np.random.default_rng(33)
    Hq, Hkv, D, n, T, W = 4, 2, 16, 50, 5, 9
    k, v, bt = _case(rng, Hq, Hkv, D, [n], x=4)
    q = rng.standard_normal((1, T, Hq, D))
    base = A.decode_multi(q, k, v, bt, [n], T, Hq, Hkv, BS, 0.3, W)
    for i in range(T):
        lo, hi = A.query_range(n, T, i, W)
        assert (lo, hi) == (n - T + i + 1 - W, n - T + i + 1)
        k2, v2 = k.copy(), v.copy()
        for t in list(range(0, lo)) + list(range(hi, n)):
            p, s = bt[0][t // BS], t % BS
            k2[p, :, :, s, :] = 1e3 * rng.standard_normal(k2[p, :, :, s, :].shape)
            v2[p, :, :, s] = 1e3
        got = A.decode_multi(q, k2, v2, bt, [n], T, Hq, Hkv, BS, 0.3, W)
        assert np.array_equal(got[0, i], base[0, i])
        # and a key inside the range does change it
        t = hi - 1
        v3 = v.copy()
        v3[bt[0][t // BS], :, :, t % BS] += 1.0
        assert not np.array_equal(A.decode_multi(q, k, v3, bt, [n], T, Hq, Hkv, BS, 0.3, W)[0, i], base[0, i])


def test_brute_force_tiny_window():
    rng = np.random.default_rng(34)
    Hq, Hkv, D, n, T, W = 2, 1, 8, 21, 3, 6
    k, v, bt = _case(rng, Hq, Hkv, D, [n], x=4)
    q = rng.standard_normal((1, T, Hq, D))
    got = A.decode_multi(q, k, v, bt, [n], T, Hq, Hkv, BS, 0.5, W)
    for i in range(T):
        pos = n - T + i
        for hq in range(Hq):
            ts = [t for t in range(n) if pos - W < t <= pos]
            sc = []
            for t in ts:
                p, s = bt[0][t // BS], t % BS
                sc.append(0.5 * sum(q[0, i, hq, d] * k[p, 0, d // 4, s, d % 4] for d in range(D)))
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            for d in range(D):
                num = sum(wi * v[bt[0][t // BS], 0, d, t % BS] for wi, t in zip(w, ts))
                assert abs(got[0, i, hq, d] - num / sum(w)) < 1e-12
