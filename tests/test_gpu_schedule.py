"""The dynamic schedule (one workgroup per CU, chunks handed out from a
counter in the workspace) against the static schedule and the fp64 oracle.

The chunks are fixed by n_items and min_chunk_pages under both schedules;
only which wavefront computes a chunk differs.  So for the same chunking the
two schedules must give bit-identical outputs, and every call must leave the
workspace's counters at zero for the next one."""
import zlib

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


CASES = [
    # name, B, Hq, Hkv, D, dtype, cached lengths, n_items, min_chunk
    ("dyn_mha_bf16_128", 6, 4, 4, 128, "bf16", [0, 15, 16, 300, 999, 47], 40, 2),
    ("dyn_gqa4_bf16_128", 5, 16, 4, 128, "bf16", [1, 700, 33, 1500, 260], 64, 4),
    ("dyn_gqa2_f32_64", 4, 4, 2, 64, "f32", [17, 0, 400, 129], 13, 1),
    ("dyn_g4_f32_128", 3, 8, 2, 128, "f32", [300, 5, 77], 9, 3),
    ("dyn_g16_bf16_64", 3, 32, 2, 64, "bf16", [50, 333, 2], 11, 2),
    ("dyn_default_split", 4, 8, 2, 128, "bf16", [2000, 31, 4000, 640], 0, 0),
]


def _decoder(pkv, w, c, n_items, min_chunk, schedule):
    return pkv.Decoder(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, W.torch_dtype(w), c.max_blocks, n_items,
                       min_chunk, schedule=schedule)


@pytest.mark.parametrize("name,B,Hq,Hkv,D,dtype,cached,n_items,min_chunk", CASES, ids=[s[0] for s in CASES])
def test_dynamic_equals_static_bitwise(pkv, name, B, Hq, Hkv, D, dtype, cached, n_items, min_chunk):
    P = sum((n + 16) // 16 for n in cached) + 5
    w = W.custom(name, B, Hq, Hkv, D, dtype, cached, pool_pages=P, seed=zlib.crc32(name.encode()) % 1000)
    c = H.setup(w, device="cuda", gen_device="cpu")
    H.log(f"schedule {name}")
    ref = H.oracle_full(c)
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    dyn = _decoder(pkv, w, c, n_items, min_chunk, pkv.PKV_SCHEDULE_DYNAMIC)
    assert dyn.schedule == pkv.PKV_SCHEDULE_DYNAMIC
    st = _decoder(pkv, w, c, dyn.n_items, dyn.min_chunk_pages, pkv.PKV_SCHEDULE_STATIC)
    assert st.schedule == pkv.PKV_SCHEDULE_STATIC
    outs = []
    for dec in (dyn, dyn, st):
        out = torch.full_like(c.q, float("nan"))
        dec(c.q, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
        torch.cuda.synchronize()
        outs.append(out)
    H.assert_close(H.f64(outs[0]), ref, dtype, name)
    assert torch.equal(outs[0], outs[1]), "dynamic schedule not run-to-run identical"
    assert torch.equal(outs[0], outs[2]), "dynamic and static schedules differ on the same chunks"
    arrivals, work = dyn.counters()
    assert int(work.item()) == 0 and int(arrivals.abs().sum().item()) == 0


def test_dynamic_fused_step_equals_static(pkv):
    w = W.custom("dyn_step", 5, 8, 2, 128, "bf16", [0, 15, 16, 31, 900], pool_pages=80, seed=61)
    c = H.setup(w, device="cuda", gen_device="cpu")
    ref = H.oracle_full(c)
    res = []
    for schedule in (pkv.PKV_SCHEDULE_DYNAMIC, pkv.PKV_SCHEDULE_STATIC):
        kp, vp = c.k_pages.clone(), c.v_pages.clone()
        dec = _decoder(pkv, w, c, 9, 2, schedule)
        out = torch.empty_like(c.q)
        dec.step(c.q, c.k_new, c.v_new, kp, vp, c.bt, c.seq_lens, w.scale, out)
        torch.cuda.synchronize()
        res.append((out, H.bits(kp), H.bits(vp)))
    H.assert_close(H.f64(res[0][0]), ref, "bf16", "dyn_step")
    assert torch.equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1]) and np.array_equal(res[0][2], res[1][2])


def test_dynamic_many_chunks_per_wavefront(pkv):
    # One-page chunks, about 88 per wavefront: the next chunk is often not
    # known when the loader needs it (the take is then read at once), and a
    # wavefront's list of pending merges fills up and is flushed mid-stream.
    # Pairs span at most 89 chunks, so all of them merge inside the kernel.
    B, Hkv = 128, 8
    rng = np.random.default_rng(5)
    cached = rng.integers(1300, 1400, B).tolist()
    w = W.custom("dyn_many", B, Hkv, Hkv, 64, "bf16", cached, pool_pages=sum((n + 16) // 16 for n in cached) + 8,
                 seed=62)
    c = H.setup(w, device="cuda", gen_device="cpu")
    ref = H.oracle_full(c)
    total = int(sum((n + 15) // 16 for n in c.attended)) * Hkv
    pkv.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.bt, c.positions)
    dyn = _decoder(pkv, w, c, total, 1, pkv.PKV_SCHEDULE_DYNAMIC)
    out = torch.empty_like(c.q)
    for _ in range(2):      # the second call starts from the counters the first left
        dyn(c.q, c.k_pages, c.v_pages, c.bt, c.seq_lens, w.scale, out)
        torch.cuda.synchronize()
        H.assert_close(H.f64(out), ref, "bf16", "dyn_many")
        arrivals, work = dyn.counters()
        assert int(work.item()) == 0 and int(arrivals.abs().sum().item()) == 0
