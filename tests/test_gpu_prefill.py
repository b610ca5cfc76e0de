"""GPU parity of wide query tiles (q_len x group above 64 columns per KV head:
a prefill chunk, or a long drafted run) through pkv_paged_decode_multi,
which runs the prefill kernel for them, against the oracle's decode_multi.
Pages wholly before every query's window are poisoned with NaN on the GPU
side: the kernel must not read them."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA

from . import helpers as H
from .test_gpu_multi import first_block

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_254_amd as m
    return m


def run_prefill(pkv, B, Hq, Hkv, D, dtype, lens, T, window, seed, zero=(), short=()):
    w = W.custom("prefill", B, Hq, Hkv, D, dtype, list(lens), seed=seed)
    c = H.setup(w, device="cuda", gen_device="cpu")
    att = np.array(lens, dtype=np.int64)
    for b in zero:
        att[b] = 0
    for b in short:
        att[b] = T - 1                                   # fewer cached tokens than queries: invalid
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn((B, T, Hq, D), generator=g).to(W.torch_dtype(w))
    ref = OA.decode_multi(H.f64(q), H.f64(c.k_pages), H.f64(c.v_pages), c.bt_np,
                          [n if n >= T else 0 for n in att], T, Hq, Hkv, 16, w.scale, window)
    kp, vp = c.k_pages.clone(), c.v_pages.clone()
    for b in range(B):
        for blk in range(first_block(int(att[b]), T, window)):
            p = int(c.bt_np[b, blk])
            kp[p] = float("nan")
            vp[p] = float("nan")
    lens_d = torch.from_numpy(att.astype(np.int32)).cuda()
    out = torch.full((B, T, Hq, D), float("nan"), dtype=W.torch_dtype(w), device="cuda")
    pkv.paged_decode_multi(q.cuda(), kp, vp, c.bt, lens_d, T, w.scale, out, window)
    torch.cuda.synchronize()
    o = H.f64(out)
    for b in short:
        assert np.isnan(o[b]).all()
    for b in zero:
        assert (o[b] == 0).all()
    keep = [b for b in range(B) if b not in short]
    H.assert_close(o[keep], ref[keep], dtype, f"prefill T={T} W={window}")
    return o


CASES = [
    # B, Hq, Hkv, D, dtype, lens (attended, queries included), T, window
    (3, 8, 2, 128, "bf16", [300, 80, 129], 20, 0),       # 80 columns: a full tile and a 16-column one
    (2, 32, 8, 128, "bf16", [500, 200], 40, 0),          # GQA group 4, 160 columns
    (2, 64, 8, 128, "bf16", [700, 130], 100, 0),         # group 8, 800 columns, 13 tiles
    (3, 16, 1, 64, "bf16", [200, 90, 17], 17, 0),        # MQA-like group 16, head_dim 64, len == q_len
    (2, 4, 4, 128, "f32", [150, 90], 70, 0),             # MHA fp32 head_dim 128 (32-column tiles)
    (2, 8, 2, 64, "f32", [100, 260], 40, 0),             # fp32 head_dim 64
    (2, 8, 2, 128, "bf16", [90, 200], 90, 0),            # sequence 0 prefilled whole (causal self-attention)
    (3, 8, 2, 128, "bf16", [600, 300, 100], 64, 50),     # sliding window shorter than the chunk
    (2, 32, 8, 128, "bf16", [900, 400], 128, 256),       # window of 256, 512 columns
    (2, 8, 2, 128, "bf16", [300, 200], 40, 1),           # window 1: each token sees itself
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[6]}_W{c[7]}_G{c[1] // c[2]}_D{c[3]}_{c[4]}" for c in CASES])
def test_prefill_parity(pkv, case):
    B, Hq, Hkv, D, dtype, lens, T, window = case
    H.log(f"prefill {case}")
    run_prefill(pkv, B, Hq, Hkv, D, dtype, lens, T, window, seed=211)


def test_prefill_empty_and_short_sequences(pkv):
    run_prefill(pkv, 4, 16, 4, 128, "bf16", [120, 80, 150, 100], 24, 0, seed=212, zero=(1,), short=(3,))


def test_prefill_longest_first_order(pkv):
    """Without a window the prefill kernel hands the sequences to its
    workgroups longest first (ties by index): equal lengths, a zero length and
    an invalid one among them, in a batch it ranks and in one above the
    ranking's 1024-sequence limit, which keeps the sequence order."""
    run_prefill(pkv, 6, 8, 2, 128, "bf16", [150, 300, 150, 40, 300, 90], 24, 0, seed=214, zero=(3,), short=(5,))
    lens = [17 + (b * 7) % 23 for b in range(1030)]
    run_prefill(pkv, 1030, 8, 2, 64, "bf16", lens, 17, 0, seed=215, zero=(1029,))


def test_prefill_just_above_the_split_kernel(pkv):
    """68 columns: four past the 64 the split kernel takes, so the last tile
    holds 4 live columns and 12 idle lanes per MFMA."""
    run_prefill(pkv, 2, 8, 2, 128, "bf16", [200, 64], 17, 0, seed=213)


@pytest.mark.parametrize("T,window", [(128, 0), (128, 1024), (512, 0), (512, 1024)])
def test_full_size_prefill_gqa(pkv, T, window):
    """The full Llama-3-8B-shaped GQA layer with a prefill chunk of T query
    tokens per sequence (the last T cached tokens), the library's default
    launch, checked on sampled rows of sampled sequences against the oracle
    (host copies of those sequences' pages taken before any HIP call)."""
    w = W.get("llama3_8b_gqa")
    c = H.setup(w, device="cuda")
    att = c.attended.astype(np.int64)
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    g = torch.Generator(device="cuda").manual_seed(900 + T)
    q = torch.randn((B, T, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(T + window)
    bs = sorted({int(np.argmax(att)), int(np.argmin(att)), int(rng.integers(B))})
    host = {}
    for b in bs:
        nblk = (int(att[b]) + 15) // 16
        pages = torch.from_numpy(c.bt_np[b, :nblk].astype(np.int64)).cuda()
        sub = np.arange(nblk, dtype=np.int32)[None, :]
        kp, vp = OA.append(H.f64(c.k_pages.index_select(0, pages)), H.f64(c.v_pages.index_select(0, pages)), sub,
                           [int(c.cached[b])], H.f64(c.k_new[b:b + 1]), H.f64(c.v_new[b:b + 1]), 16)
        host[b] = OA.gather(kp, vp, sub[0], int(att[b]), 16)
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    out = torch.full((B, T, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    H.log(f"prefill full T={T} W={window}")
    pkv.paged_decode_multi(q, c.k_pages, c.v_pages, c.bt, c.seq_lens, T, w.scale, out, window)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    qh = {b: H.f64(q[b]) for b in bs}
    got, ref = [], []
    for b in bs:
        K, V = host[b]
        for i in sorted({0, 1, T // 2, T - 2, T - 1, int(rng.integers(T))}):
            lo, hi = OA.query_range(int(att[b]), T, i, window)
            for hq in sorted({0, w.group - 1, w.group, Hq - 1, int(rng.integers(Hq))}):
                h = hq // w.group
                ref.append(OA.attend(qh[b][i, hq], K[lo:hi, h], V[lo:hi, h], w.scale))
                got.append(H.f64(out[b, i, hq]))
    mx, mean, rel = H.assert_close(np.stack(got), np.stack(ref), "bf16", f"prefill full T={T} W={window}")
    H.log(f"  {len(got)} rows of {len(bs)} sequences: max {mx:.2e} mean {mean:.2e} rel {rel:.2e}")
    del c, q, out
    torch.cuda.empty_cache()


def test_prefill_huge_score_takes_the_exact_redo(pkv):
    """One key late in each sequence is 30 times a query vector, so scores
    jump by hundreds (log2 units) past the running maxima set on the first
    pages: the tile is redone with exact maxima.  Against the oracle."""
    B, Hq, Hkv, D, T = 2, 8, 2, 128, 24
    lens = [300, 160]
    w = W.custom("prefill_huge", B, Hq, Hkv, D, "bf16", lens, seed=214)
    c = H.setup(w, device="cuda", gen_device="cpu")
    g = torch.Generator().manual_seed(215)
    q = torch.randn((B, T, Hq, D), generator=g).to(torch.bfloat16)
    k = c.k_pages.cpu()
    X = k.shape[4]
    for b, n in enumerate(lens):
        t = n - 8                                          # seen by the last 8 query tokens only
        p, s = int(c.bt_np[b, t // 16]), t % 16
        for h in range(Hkv):
            k[p, h, :, s, :] = (30.0 * q[b, T - 1, h * (Hq // Hkv)].float()).to(torch.bfloat16).view(D // X, X)
    c.k_pages = k.cuda()
    att = np.array(lens, dtype=np.int64)
    ref = OA.decode_multi(H.f64(q), H.f64(c.k_pages), H.f64(c.v_pages), c.bt_np, att, T, Hq, Hkv, 16, w.scale, 0)
    out = torch.full((B, T, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pkv.paged_decode_multi(q.cuda(), c.k_pages, c.v_pages, c.bt, torch.from_numpy(att.astype(np.int32)).cuda(), T,
                           w.scale, out, 0)
    torch.cuda.synchronize()
    H.assert_close(H.f64(out), ref, "bf16", "prefill huge score")
