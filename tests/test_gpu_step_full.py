"""GPU parity of the call the benchmark times: the fused append + decode
(pkv_decode_step, Decoder.step, the library's default launch), at full size.

* Every single-layer workload: sampled output rows against the oracle (host
  copies of the sampled sequences' pages taken before any HIP call, then
  OA.append and the plain attention), the sampled sequences' pages bit for
  bit against OA.append, and the whole pools: the appended slots hold the new
  token's bits and every other byte is unchanged.
* The 32-layer Llama-3-8B-shaped step exactly as the benchmark runs it: 32
  layer pools, one block table, one Decoder workspace, the layers in order;
  sampled rows of layers 0, 1, 2, 15 and 31 against the oracle.  A partial
  left in the workspace by the previous layer would show up here.
* One full-size GQA step repeated 20 times on one workspace: bit-identical.
* A workspace reused at a smaller batch and then the full one again
  (continuous batching), each call against the oracle.
"""
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


def _sample_rows(w, attended, rng, n_seq=4):
    B, Hq, G = w.batch, w.n_q_heads, w.group
    bs = sorted({0, B - 1, int(np.argmax(attended)), int(np.argmin(attended))} |
                set(rng.integers(0, B, n_seq).tolist()))
    rows = []
    for b in bs:
        for hq in sorted({0, Hq - 1, G - 1, min(Hq - 1, G), int(rng.integers(Hq))}):
            rows.append((b, hq))
    return rows


def _host_pages(c, seqs):
    """Host copies (bits) of the pages the given sequences use, before any HIP call."""
    out = {}
    for b in seqs:
        nblk = (int(c.attended[b]) + H.BS - 1) // H.BS
        pages = torch.from_numpy(c.bt_np[b, :nblk].astype(np.int64)).to(c.k_pages.device)
        out[b] = (pages, H.bits(c.k_pages.index_select(0, pages)), H.bits(c.v_pages.index_select(0, pages)))
    return out


def _check_sampled_pages(c, host, kp, vp):
    """The sampled sequences' pages after the step equal OA.append applied to
    their host copies (relabelled 0..n-1), bit for bit."""
    for b, (pages, k0, v0) in host.items():
        nblk = pages.numel()
        sub = np.arange(nblk, dtype=np.int32)[None, :]
        ek, ev = OA.append(k0, v0, sub, [int(c.cached[b])], H.bits(c.k_new[b:b + 1]), H.bits(c.v_new[b:b + 1]), H.BS)
        assert np.array_equal(H.bits(kp.index_select(0, pages)), ek), f"K pages of sequence {b}"
        assert np.array_equal(H.bits(vp.index_select(0, pages)), ev), f"V pages of sequence {b}"


def _check_whole_pool(c, k_before, v_before, kp, vp):
    """Appended slots hold the new token's bits; every other element is unchanged."""
    w = c.w
    pos = torch.from_numpy(c.cached.astype(np.int64)).to(kp.device)
    bt = c.bt.long()
    pages = bt[torch.arange(w.batch, device=kp.device), pos // H.BS]
    slots = pos % H.BS
    X = kp.shape[4]
    ek = k_before.clone()
    ev = v_before.clone()
    ek[pages, :, :, slots, :] = c.k_new.view(w.batch, w.n_kv_heads, w.head_dim // X, X)
    ev[pages, :, :, slots] = c.v_new
    it = torch.int16 if kp.element_size() == 2 else torch.int32
    assert torch.equal(kp.view(it), ek.view(it)), "K pool differs from the appended definition"
    assert torch.equal(vp.view(it), ev.view(it)), "V pool differs from the appended definition"


SINGLE = ["llama2_7b_mha", "llama3_8b_gqa", "long_70b_gqa", "long_70b_mqa"]


@pytest.mark.parametrize("name", SINGLE)
def test_full_size_fused_step(pkv, name):
    w = W.get(name)
    H.log(f"step {name}: setup")
    c = H.setup(w, device="cuda", poison=True)
    rng = np.random.default_rng(17)
    rows = _sample_rows(w, c.attended, rng)
    refs = H.oracle_rows(c, rows)
    host = _host_pages(c, sorted({b for b, _ in rows}))
    k_before, v_before = c.k_pages.clone(), c.v_pages.clone()
    dec = pkv.Decoder(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, W.torch_dtype(w), c.max_blocks)
    out = torch.full_like(c.q, float("nan"))
    H.log(f"step {name}: n_items={dec.n_items} min_chunk={dec.min_chunk_pages}")
    dec.step(c.q, c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
    torch.cuda.synchronize()
    got = np.stack([H.f64(out[b, hq]) for b, hq in rows])
    mx, mean, rel = H.assert_close(got, np.stack(refs), w.dtype, f"step {name}")
    H.log(f"step {name}: {len(rows)} rows, max {mx:.2e} mean {mean:.2e} rel {rel:.2e}")
    assert torch.isfinite(out.float()).all()
    _check_sampled_pages(c, host, c.k_pages, c.v_pages)
    _check_whole_pool(c, k_before, v_before, c.k_pages, c.v_pages)
    # the same step again on the same workspace (the append rewrites the same bits)
    out2 = torch.empty_like(out)
    dec.step(c.q, c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    del c, out, out2, dec, k_before, v_before
    torch.cuda.empty_cache()


def test_32_layer_step_on_one_workspace(pkv):
    """The Llama-3-8B-shaped step as the benchmark runs it: per layer the fused
    step on that layer's pools, one block table and one Decoder for all 32."""
    w = W.get("llama3_8b_step")
    checked = {0, 1, 2, 15, w.n_layers - 1}
    H.log("32-layer step: setup of layer 0 (block table)")
    base = H.setup(w, layer=0, device="cuda", poison=True)
    free = torch.isnan(base.v_pages[:, 0, 0, :])        # [P][16]: slots that hold no cached token
    rng = np.random.default_rng(5)
    layers = []
    for layer in range(w.n_layers):
        if layer == 0:
            c = base
        else:
            k, v = W.make_pools(w, layer, "cuda")
            k.masked_fill_(free[:, None, None, :, None], float("nan"))
            v.masked_fill_(free[:, None, None, :], float("nan"))
            q = W.make_q(w, layer, "cuda")
            kn, vn = W.make_new_kv(w, layer, "cuda")
            c = H.Case(w, layer, base.cached, base.attended, base.max_blocks, base.bt_np, base.bt, base.positions,
                       base.seq_lens, q, kn, vn, k, v)
        entry = {"case": c}
        if layer in checked:
            rows = _sample_rows(w, c.attended, rng, n_seq=3)
            entry["rows"] = rows
            entry["refs"] = H.oracle_rows(c, rows)
            entry["host"] = _host_pages(c, sorted({b for b, _ in rows}))
        layers.append(entry)
    H.log("32-layer step: oracle rows taken; running the 32 layers on one workspace")
    dec = pkv.Decoder(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, W.torch_dtype(w), base.max_blocks)
    outs = []
    for e in layers:
        c = e["case"]
        out = torch.full_like(c.q, float("nan"))
        dec.step(c.q, c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
        outs.append(out)
    torch.cuda.synchronize()
    for layer, (e, out) in enumerate(zip(layers, outs)):
        assert torch.isfinite(out.float()).all(), f"layer {layer}"
        if "rows" not in e:
            continue
        got = np.stack([H.f64(out[b, hq]) for b, hq in e["rows"]])
        mx, mean, rel = H.assert_close(got, np.stack(e["refs"]), w.dtype, f"32-layer step, layer {layer}")
        _check_sampled_pages(e["case"], e["host"], e["case"].k_pages, e["case"].v_pages)
        H.log(f"  layer {layer}: {len(e['rows'])} rows, max {mx:.2e} mean {mean:.2e} rel {rel:.2e}")
    del layers, outs, dec, base
    torch.cuda.empty_cache()


def test_gqa_step_repeated_is_bit_identical(pkv):
    w = W.get("llama3_8b_gqa")
    c = H.setup(w, device="cuda", poison=True)
    dec = pkv.Decoder(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, W.torch_dtype(w), c.max_blocks)
    first = torch.empty_like(c.q)
    dec.step(c.q, c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, first)
    out = torch.empty_like(c.q)
    for i in range(1, 20):
        out.fill_(float("nan"))
        dec.step(c.q, c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out, first), f"repeat {i} differs"
    counters, work = dec.counters()
    assert int(counters.abs().sum()) == 0 and int(work) == 0
    H.log(f"gqa step repeated 20 times: bit-identical (n_items={dec.n_items})")
    del c, dec, first, out
    torch.cuda.empty_cache()


def test_workspace_reused_at_smaller_batch(pkv):
    """One Decoder sized for batch 12 runs 12 sequences, then the first 6, then
    all 12 again; pairs span several chunks, so every call merges in-kernel
    through the counters at the workspace's end."""
    cached = [50, 130, 7, 300, 0, 95, 260, 33, 16, 15, 180, 71]
    w = W.custom("shrink", 12, 16, 4, 128, "bf16", cached, pool_pages=sum((n + 16) // 16 for n in cached) + 3,
                 seed=77)
    c = H.setup(w, device="cuda", gen_device="cpu")
    ref = H.oracle_full(c)
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    dec = pkv.Decoder(12, 16, 4, 128, torch.bfloat16, c.max_blocks, 9, 2)
    for B in (12, 6, 12, 3):
        out = torch.full((B, 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        dec(c.q[:B].contiguous(), c.k_pages, c.v_pages, c.bt[:B].contiguous(), c.seq_lens[:B].contiguous(), w.scale,
            out)
        torch.cuda.synchronize()
        H.assert_close(H.f64(out), ref[:B], "bf16", f"batch {B}")
        counters, _ = dec.counters()
        assert int(counters.abs().sum()) == 0, f"counters left non-zero after batch {B}"
    with pytest.raises(ValueError):
        dec(torch.zeros((13, 16, 128), dtype=torch.bfloat16, device="cuda"), c.k_pages, c.v_pages, c.bt, c.seq_lens,
            w.scale, torch.empty((13, 16, 128), dtype=torch.bfloat16, device="cuda"))
