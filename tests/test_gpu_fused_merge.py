"""The in-kernel merge of split partials (the chunk that finishes a pair last
merges the pair's partials): parity with the oracle, run-to-run identity on
one workspace (the arrival counters reset themselves), agreement with the
separate combine kernel, large groups (one counter per 16-head block), and
the mixed launch where pairs that may span more than 96 chunks still go to
the combine kernel while the others are merged in the decode kernel."""
import numpy as np
import pytest

import workloads as W

from . import helpers as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_254_amd as m
    return m


def _case(pkv, name, B, Hq, Hkv, D, dtype, cached, seed):
    """Inputs, the oracle's output (append + decode), then the library's append."""
    pages = sum((c + 1 + 15) // 16 for c in cached)
    w = W.custom(name, B, Hq, Hkv, D, dtype, cached, pool_pages=pages + 6, seed=seed)
    c = H.setup(w, device="cuda", gen_device="cpu")
    ref = H.oracle_full(c)
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    return w, c, ref


def _decode(pkv, w, c, n_items, min_chunk, combine_mode=0, dec=None):
    if dec is None:
        dec = pkv.Decoder(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, W.torch_dtype(w), c.max_blocks,
                          n_items, min_chunk, combine_mode=combine_mode)
    out = torch.full_like(c.q, float("nan"))
    dec(c.q, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
    torch.cuda.synchronize()
    return out, dec


def _counters_zero(dec):
    # the arrival counters and the chunk counter sit at the workspace's end
    arrivals, work = dec.counters()
    return int(arrivals.count_nonzero().item()) == 0 and int(work) == 0


def test_repeated_calls_on_one_workspace(pkv):
    w, c, ref = _case(pkv, "fm_rep", 5, 16, 4, 128, "bf16", [300, 17, 95, 250, 40], 71)
    H.log("fused merge: 5 seqs, 20 chunks, 10 calls on one workspace")
    out0, dec = _decode(pkv, w, c, 20, 2)
    H.assert_close(H.f64(out0), ref, "bf16", "fused merge")
    assert _counters_zero(dec)
    for _ in range(9):
        out, _ = _decode(pkv, w, c, 20, 2, dec=dec)
        assert torch.equal(out, out0)
    assert _counters_zero(dec)
    # the separate combine kernel gives the same result within fp32 rounding
    out1, dec1 = _decode(pkv, w, c, 20, 2, combine_mode=1)
    H.assert_close(H.f64(out1), ref, "bf16", "separate combine")
    d = (out1.float() - out0.float()).abs().max().item()
    assert d <= 2 ** -7 * out0.float().abs().max().item(), d
    assert _counters_zero(dec1)


def test_long_pairs_use_the_combine_kernel_beside_fused_ones(pkv):
    # chunks of one page: pair (0, h) spans 101 chunks (> 96, combine kernel),
    # pair (1, h) spans 3 (merged in the decode kernel), sequence 2 is empty
    w, c, ref = _case(pkv, "fm_mixed", 3, 8, 2, 128, "bf16", [1615, 39, 5], 72)
    c.seq_lens[2] = 0
    H.log("fused merge: mixed long/short pairs, 250 chunks of 1 page")
    for mode in (0, 1):
        out, dec = _decode(pkv, w, c, 250, 1, combine_mode=mode)
        o = H.f64(out)
        H.assert_close(o[:2], ref[:2], "bf16", f"mixed mode {mode}")
        assert (o[2] == 0).all()
        again, _ = _decode(pkv, w, c, 250, 1, dec=dec)
        assert torch.equal(again, out)
        assert _counters_zero(dec)


@pytest.mark.parametrize("name,B,Hq,Hkv,D,dtype,cached,n_items,mc", [
    ("fm_g32", 4, 64, 2, 128, "bf16", [200, 60, 130, 7], 12, 2),    # two head blocks per chunk
    ("fm_g48", 2, 48, 1, 64, "f32", [150, 70], 9, 1),               # three blocks (+1 idle wavefront)
    ("fm_g64", 2, 64, 1, 128, "bf16", [500, 33], 16, 2),            # MQA-like
    ("fm_g1", 3, 4, 4, 64, "f32", [80, 300, 15], 25, 1),            # MHA, f32
])
def test_large_groups_and_mha(pkv, name, B, Hq, Hkv, D, dtype, cached, n_items, mc):
    w, c, ref = _case(pkv, name, B, Hq, Hkv, D, dtype, cached, 73)
    H.log(f"fused merge: {name}")
    out, dec = _decode(pkv, w, c, n_items, mc)
    H.assert_close(H.f64(out), ref, dtype, name)
    again, _ = _decode(pkv, w, c, n_items, mc, dec=dec)
    assert torch.equal(again, out)
    assert _counters_zero(dec)


@pytest.mark.parametrize("name,B,Hq,Hkv,D,dtype,cached,n_items", [
    ("cb_300_bf16", 2, 8, 2, 128, "bf16", [4700, 30], 700),   # 294 one-page chunks per pair of sequence 0
    ("cb_282_f32_64", 2, 4, 1, 64, "f32", [4500, 0], 300),    # head_dim 64: two 32-feature slices per row
    ("cb_300_f32_128", 2, 8, 2, 128, "f32", [4700, 30], 700),  # fp32 rows in four 32-feature slices
])
def test_combine_kernel_rows_of_many_partials(pkv, name, B, Hq, Hkv, D, dtype, cached, n_items):
    # More than 256 partials per row: the combine kernel's loop takes a
    # second round trip.  Fused mode sends these pairs to the combine kernel
    # (more than 96 chunks); mode 1 merges every pair there; the split-only
    # call followed by pkv_lse_combine takes the same kernel.
    w, c, ref = _case(pkv, name, B, Hq, Hkv, D, dtype, cached, 74)
    if cached[1] == 0:
        c.seq_lens[1] = 0
        ref[1] = 0.0
    H.log(f"combine kernel: {name}")
    for mode in (0, 1):
        out, _ = _decode(pkv, w, c, n_items, 1, combine_mode=mode)
        H.assert_close(H.f64(out), ref, dtype, f"{name} mode {mode}")
    dec = pkv.Decoder(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, W.torch_dtype(w), c.max_blocks, n_items, 1)
    out = torch.full_like(c.q, float("nan"))
    dec.split(c.q, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
    dec.combine(c.seq_lens, out, c.max_blocks)
    torch.cuda.synchronize()
    H.assert_close(H.f64(out), ref, dtype, f"{name} split + combine")


@pytest.mark.parametrize("name,B,Hq,Hkv,D,dtype,cached", [
    ("cb_rows_bf16", 6, 64, 8, 128, "bf16", [300, 17, 95, 250, 40, 1000]),   # 384 rows: one workgroup per row
    ("cb_rows_f32_64", 5, 64, 4, 64, "f32", [120, 0, 77, 400, 33]),           # 320 rows, head_dim 64
    ("cb_rows_f32_128", 5, 64, 8, 128, "f32", [200, 9, 77, 500, 33]),         # 320 fp32 rows of 128 features
])
def test_combine_kernel_many_rows(pkv, name, B, Hq, Hkv, D, dtype, cached):
    # Enough output rows that the combine kernel gives each row one workgroup
    # (the split into feature slices is for a few long rows).
    w, c, ref = _case(pkv, name, B, Hq, Hkv, D, dtype, cached, 75)
    H.log(f"combine kernel, many rows: {name}")
    out, dec = _decode(pkv, w, c, 60, 2, combine_mode=1)
    H.assert_close(H.f64(out), ref, dtype, name)
    again, _ = _decode(pkv, w, c, 60, 2, dec=dec)
    assert torch.equal(again, out)
