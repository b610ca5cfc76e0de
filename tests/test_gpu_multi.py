"""GPU parity of the multi-token decode (the last q_len cached tokens as causal
queries, optionally with a sliding window) through the C ABI, against the
oracle's decode_multi.  Pages wholly before every query's window are
poisoned with NaN on the GPU side: the kernel must not read them."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA

from . import helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_254_amd as m
    return m


def first_block(n, T, W_):
    if W_ <= 0:
        return 0
    lo = n - T + 1 - W_
    return 0 if lo <= 0 else lo // 16


def run_case(pkv, B, Hq, Hkv, D, dtype, lens, T, window, n_items, mc, seed, zero=(), short=()):
    # every attended token (the q_len query tokens included) is already cached;
    # setup leaves NaN in every slot past each length
    w = W.custom("multi", B, Hq, Hkv, D, dtype, list(lens), seed=seed)
    c = H.setup(w, device="cuda", gen_device="cpu")
    att = np.array(lens, dtype=np.int64)
    for b in zero:
        att[b] = 0
    for b in short:
        att[b] = T - 1                                   # fewer cached tokens than queries: invalid
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn((B, T, Hq, D), generator=g).to(W.torch_dtype(w))
    kh, vh = H.f64(c.k_pages), H.f64(c.v_pages)
    ref = OA.decode_multi(H.f64(q), kh, vh, c.bt_np, [n if n >= T else 0 for n in att], T, Hq, Hkv, 16,
                          w.scale, window)
    # poison the pages no query attends (wholly before every window)
    kp, vp = c.k_pages.clone(), c.v_pages.clone()
    for b in range(B):
        for blk in range(first_block(int(att[b]), T, window)):
            p = int(c.bt_np[b, blk])
            kp[p] = float("nan")
            vp[p] = float("nan")
    lens_d = torch.from_numpy(att.astype(np.int32)).cuda()
    dec = pkv.Decoder(B, Hq * T, Hkv, D, W.torch_dtype(w), c.max_blocks, n_items, mc)
    out = torch.full((B, T, Hq, D), float("nan"), dtype=W.torch_dtype(w), device="cuda")
    dec.attn_multi(q.cuda(), kp, vp, c.bt, lens_d, T, w.scale, out, window)
    torch.cuda.synchronize()
    o = H.f64(out)
    for b in short:
        assert np.isnan(o[b]).all()
    keep = [b for b in range(B) if b not in short]
    mx, mean, rel = H.assert_close(o[keep], ref[keep], dtype, f"multi T={T} W={window}")
    return out, o


CASES = [
    # B, Hq, Hkv, D, dtype, lens (attended, queries included), T, window, n_items, min_chunk
    (3, 16, 4, 128, "bf16", [300, 40, 77], 4, 0, 7, 1),        # 16 columns
    (2, 8, 2, 128, "bf16", [129, 260], 3, 0, 5, 1),            # 12 columns, T crossing a page
    (2, 64, 8, 128, "bf16", [500, 90], 8, 0, 6, 2),            # 64 columns: four head blocks
    (3, 4, 4, 64, "f32", [50, 33, 200], 5, 0, 9, 1),           # MHA, fp32
    (3, 8, 2, 128, "bf16", [300, 40, 230], 4, 20, 7, 1),       # sliding window
    (2, 8, 2, 64, "bf16", [400, 70], 6, 1, 4, 1),              # window 1: each token sees itself
    (2, 32, 8, 128, "bf16", [333, 90], 2, 64, 6, 2),           # window of 64, 8 columns
    (2, 8, 2, 128, "bf16", [30, 50], 3, 100, 3, 1),            # window longer than the sequences
    (3, 8, 2, 128, "bf16", [1700, 45, 19], 4, 0, 260, 1),      # > 96 chunks: combine kernel too
    # 103 one-page chunks per pair, so the combine kernel merges; the 32 query
    # tokens' windows start in different pages, so the first chunks hold
    # empty (lse -inf) rows for the later queries
    (2, 4, 2, 128, "bf16", [3000, 70], 32, 1600, 300, 1),
    # 64 columns (wide kernel) with a bound of 76 chunks per pair: the combine
    # kernel merges the long sequence's pairs (about 20 chunks each) and the
    # decode kernel the short ones (at most 8 chunks), in the same call
    (3, 32, 4, 128, "bf16", [1200, 60, 300], 8, 0, 100, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[6]}_W{c[7]}_G{c[1] // c[2]}_{c[4]}" for c in CASES])
def test_multi_parity(pkv, case):
    B, Hq, Hkv, D, dtype, lens, T, window, n_items, mc = case
    H.log(f"multi {case}")
    run_case(pkv, B, Hq, Hkv, D, dtype, lens, T, window, n_items, mc, seed=101)


def test_multi_empty_and_short_sequences(pkv):
    H.log("multi: empty and too-short sequences")
    _, o = run_case(pkv, 4, 8, 2, 128, "bf16", [80, 60, 90, 3], 4, 0, 6, 1, seed=102, zero=(1,), short=(3,))
    assert (o[1] == 0).all()


def test_one_token_equals_single_token_decode(pkv):
    w = W.custom("multi1", 3, 8, 2, 128, "bf16", [70, 0, 200], seed=103)
    c = H.setup(w, device="cuda", gen_device="cpu")
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    dec = pkv.Decoder(3, 8, 2, 128, torch.bfloat16, c.max_blocks, 7, 1)
    a = torch.empty_like(c.q)
    dec(c.q, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, a)
    b = torch.empty((3, 1, 8, 128), dtype=torch.bfloat16, device="cuda")
    dec.attn_multi(c.q[:, None].contiguous(), c.k_pages, c.v_pages, c.bt, c.seq_lens, 1, w.scale, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b[:, 0])


@pytest.mark.parametrize("T,window", [(4, 0), (4, 1024), (8, 0), (16, 0)])
def test_full_size_sampled_multi(pkv, T, window):
    # The full-size GQA layer with q_len query tokens per sequence (and a
    # sliding window), the library's default launch, checked on sampled
    # sequences against the oracle run on just their pages: 16 columns per
    # KV head (one block per wavefront), 32 (two blocks) and 64 (the wide
    # kernel).
    w = W.get("llama3_8b_gqa")
    c = H.setup(w, device="cuda")
    att = c.attended.astype(np.int64)
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    q = torch.stack([W.make_q(w, t, "cuda") for t in range(T)], dim=1).contiguous()
    rng = np.random.default_rng(12)
    bs = sorted({0, B - 1, int(np.argmax(att)), int(np.argmin(att)), int(rng.integers(B))})
    # host copies of the sampled sequences' pages before any HIP call; the
    # oracle appends the step's token to them itself
    host = {}
    for b in bs:
        nblk = (int(att[b]) + 15) // 16
        pages = torch.from_numpy(c.bt_np[b, :nblk].astype(np.int64)).cuda()
        sub = np.arange(nblk, dtype=np.int32)[None, :]
        kp, vp = OA.append(H.f64(c.k_pages.index_select(0, pages)), H.f64(c.v_pages.index_select(0, pages)), sub,
                           [int(c.cached[b])], H.f64(c.k_new[b:b + 1]), H.f64(c.v_new[b:b + 1]), 16)
        host[b] = (kp, vp, nblk)
    # every attended token must be cached: append the step's token first
    # (the other slots past each length stay NaN)
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    torch.cuda.synchronize()
    dec = pkv.Decoder(B, Hq * T, Hkv, D, W.torch_dtype(w), c.max_blocks)
    out = torch.full((B, T, Hq, D), float("nan"), dtype=W.torch_dtype(w), device="cuda")
    H.log(f"multi full T={T} W={window} (n_items={dec.n_items})")
    dec.attn_multi(q, c.k_pages, c.v_pages, c.bt, c.seq_lens, T, w.scale, out, window)
    torch.cuda.synchronize()
    for b in bs:
        kp, vp, nblk = host[b]
        sub = np.arange(nblk, dtype=np.int32)[None, :]
        ref = OA.decode_multi(H.f64(q[b:b + 1]), kp, vp, sub, [int(att[b])], T, Hq, Hkv, 16, w.scale, window)
        mx, mean, rel = H.assert_close(H.f64(out[b:b + 1]), ref, "bf16", f"multi full b={b}")
        H.log(f"  b={b} ({int(att[b])} tokens): max abs {mx:.2e} rel RMS {rel:.2e}")
