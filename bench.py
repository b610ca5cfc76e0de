"""Throughput of one paged decode step on one MI355X.

A step is one pass of the whole device path over one batch: for every layer
of the workload, kv_append of each sequence's new token, the split-KV paged
decode kernel, and the log-sum-exp combine.  The page pool and block tables
are built by the library's host allocator before timing; every input is
resident in HBM when the timed region starts.

value = algorithmic KV bytes read per step / step time, where the algorithmic
bytes are 2 (K and V) x head_dim x element size per attended token per KV head
per layer (the per-token KV formula of the pages' chapter 17 equation M_kv).

Prints one JSON line.  Default workload: the Llama-3-8B-shaped decode step,
32 layers of a GQA cache (32 query / 8 KV heads, head_dim 128, bf16) for 256
sequences with lognormal lengths (median 2000), one new token each.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, published
MALL_BYTES = 256 << 20         # last-level (Infinity) cache
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_254_amd", "csrc", "kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_step")
    ap.add_argument("--n-items", type=int, default=0)
    ap.add_argument("--min-chunk", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0, choices=[0, 1, 2],
                    help="work schedule: 0 the library's default, 1 static, 2 dynamic")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-launch-probe", action="store_true",
                    help="skip the launch-cost probe (its cooperative launches; e.g. under a profiler)")
    ap.add_argument("--kv", choices=["dense", "u8"], default="dense",
                    help="cache format: the workload's dtype, or the 8-bit cache (bf16 q/out)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence: the last q-len cached tokens attend causally (no append)")
    ap.add_argument("--window", type=int, default=0, help="sliding window (with --q-len; 0: none)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (one graph per pool-rotation position)")
    ap.add_argument("--separate-combine", action="store_true",
                    help="merge split partials with the combine kernel instead of inside the decode kernel")
    ap.add_argument("--unfused", action="store_true",
                    help="append, split and combine as three launches instead of the fused step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the copy kernel on 1 GiB three times (reference for HBM byte counters)")
    return ap.parse_args()


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Layer:
    pass


def multi_kv_tokens(att, q_len, window):
    """Tokens whose K/V the multi-token decode must read per sequence and KV
    head: the union of the query tokens' key ranges, from the first query's
    window start (0 without a window) to the end."""
    if window <= 0:
        return att.copy()
    return np.minimum(att, window + q_len - 1)


def multi_keys(att, q_len, window):
    """Attended keys summed over every sequence and query token: query i of
    the last q_len tokens of a sequence of n sees keys [lo, hi) with
    hi = n - q_len + i + 1 and lo = max(0, hi - window) (0 without a window)."""
    total = 0
    for n in att:
        hi = int(n) - q_len + 1 + np.arange(q_len)
        lo = np.maximum(0, hi - window) if window > 0 else np.zeros_like(hi)
        total += int(np.maximum(hi - lo, 0).sum())
    return total


def setup(w, device, kv="dense", q_len=1, window=0):
    import torch
    import paged_kv_cache_254_amd as pkv
    import workloads as W
    cached = W.cached_lens(w)
    att = cached + 1
    P = W.pool_pages(w)
    mb = int(max((att + 15) // 16))
    pool = pkv.PagePool(P, W.free_order(w))
    for b in range(w.batch):
        pool.reserve(b, int(cached[b]))
    grown = sum(pool.reserve(b, int(att[b])) for b in range(w.batch))  # the step's new pages
    bt_np = pool.block_table(range(w.batch), mb)
    common = dict(
        bt=torch.from_numpy(bt_np).to(device),
        positions=torch.from_numpy(cached.astype(np.int32)).to(device),
        seq_lens=torch.from_numpy(att.astype(np.int32)).to(device),
    )
    # bytes of cache the step reads per layer: K and V of every attended token
    # (8-bit cache: the codes plus the slot's 16 bytes of scales and zero points)
    per_token_head = 2 * w.head_dim + 16 if kv == "u8" else w.head_dim * 2 * w.elem_bytes
    read_tokens = multi_kv_tokens(att, q_len, window) if q_len > 1 or window > 0 else att
    kv_bytes_layer = int(read_tokens.sum()) * w.n_kv_heads * per_token_head
    # Rotate pool copies so that between two reads of one copy at least twice
    # the last-level cache's size of other KV streams through it, and small
    # caches stream at least 4x that cache per step: no launch can be served
    # from data the previous launches left in the last-level cache.
    n_copies = max(w.n_layers, 1 + math.ceil(2 * MALL_BYTES / kv_bytes_layer))
    if kv_bytes_layer < 2 * MALL_BYTES:
        n_copies = max(n_copies, math.ceil(4 * MALL_BYTES / kv_bytes_layer))
    layers = []
    for i in range(n_copies):
        L = Layer()
        if kv == "u8":
            L.k_pages, L.v_pages, L.meta = W.make_q8_pools(w, i % max(1, w.n_layers), device)
        else:
            L.k_pages, L.v_pages = W.make_pools(w, i % max(1, w.n_layers), device)
        if q_len > 1 or window > 0:
            # [B][q_len][Hq][D]: the query vectors of the last q_len cached tokens
            L.q = torch.stack([W.make_q(w, i * q_len + t, device) for t in range(q_len)], dim=1).contiguous()
        else:
            L.q = W.make_q(w, i, device)
        L.k_new, L.v_new = W.make_new_kv(w, i, device)
        L.out = torch.empty_like(L.q)
        layers.append(L)
    return dict(common, layers=layers, cached=cached, att=att, bt_np=bt_np, mb=mb, P=P,
                kv_bytes_layer=kv_bytes_layer, grown=grown, n_copies=n_copies)


def _oracle_worker(task):
    """One baseline worker process: loads its sequences' host inputs (not
    timed), then runs the oracle over them, whole sequences in order and again
    from the start, until `budget` seconds of its own compute are used.
    Returns (KV bytes covered, seconds, runs)."""
    files, budget, mode, meta = task
    import time as _t
    import numpy as _np
    from oracle import attention as OA
    from oracle import kv_quant as KQ
    xs = []
    for f in files:
        with _np.load(f) as z:
            xs.append({k: z[k] for k in z.files})
    secs, kv, runs = 0.0, 0, 0
    while secs < budget and xs:
        for x in xs:
            t0 = _t.perf_counter()
            bt = _np.arange(x["k"].shape[0], dtype=_np.int32)[None, :]
            att = [int(x["att"])]
            if mode == "multi":
                OA.decode_multi(x["q"], x["k"], x["v"], bt, att, meta["q_len"], meta["hq"], meta["hkv"], 16,
                                meta["scale"], meta["window"])
            elif mode == "u8":
                k2, v2, m2 = KQ.append(x["k"], x["v"], x["m"], bt, [int(x["cached"])], x["kn"], x["vn"], 16)
                KQ.decode(x["q"], k2, v2, m2, bt, att, meta["hq"], meta["hkv"], 16, meta["scale"])
            else:
                k2, v2 = OA.append(x["k"], x["v"], bt, [int(x["cached"])], x["kn"], x["vn"], 16)
                OA.decode(x["q"], k2, v2, bt, att, meta["hq"], meta["hkv"], 16, meta["scale"])
            secs += _t.perf_counter() - t0
            kv += int(x["bytes"])
            runs += 1
            if secs >= budget:
                break
    return kv, secs, runs


def cpu_baseline(w, S, budget_s, kv="dense", q_len=1, window=0, max_workers=16):
    """The oracle, as it stands, on a bounded sample of layer 0: whole
    sequences (append + decode for every query head; with q_len > 1 or a
    window, the multi-token decode), run in parallel worker processes, one
    single-threaded process per core (process parallelism over sequences).
    Each worker runs its share of the sample, repeatedly, for about budget_s
    seconds of compute; value = KV bytes covered by all workers / the longest
    worker's compute time.  cores = the number of workers."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import shutil
    import tempfile
    import workloads as W
    n_workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    L = S["layers"][0]
    rng = np.random.default_rng(0)
    pick = list(rng.permutation(w.batch))
    multi = q_len > 1 or window > 0
    read = multi_kv_tokens(S["att"], q_len, window) if multi else S["att"]
    mode = "multi" if multi else ("u8" if kv == "u8" else "dense")
    # host inputs of whole sequences (pages relabelled 0..n-1), float32 (exact
    # for bf16) or the 8-bit codes, written to files the workers load; at most
    # 2 GiB of them, at least one sequence per worker where the batch allows
    tmp = tempfile.mkdtemp(prefix="pkv_oracle_")
    files, total, cap = [], 0, 2 << 30
    try:
        for b in pick:
            nblk = (int(S["att"][b]) + 15) // 16
            pages = __import__("torch").from_numpy(S["bt_np"][b, :nblk].astype(np.int64)).to(L.k_pages.device)
            x = {"att": np.int64(S["att"][b]), "cached": np.int64(S["cached"][b]),
                 "bytes": np.int64(int(read[b]) * S["kv_bytes_layer"] // int(read.sum())),
                 "q": L.q[b:b + 1].float().cpu().numpy()}
            if kv == "u8":   # V codes into the oracle's [D][16] order
                x.update(k=L.k_pages.index_select(0, pages).cpu().numpy(),
                         v=W.v_codes_to_logical(L.v_pages.index_select(0, pages).cpu().numpy()),
                         m=L.meta.index_select(0, pages).cpu().numpy(),
                         kn=L.k_new[b:b + 1].float().cpu().numpy(), vn=L.v_new[b:b + 1].float().cpu().numpy())
            else:
                x.update(k=L.k_pages.index_select(0, pages).float().cpu().numpy(),
                         v=L.v_pages.index_select(0, pages).float().cpu().numpy(),
                         kn=L.k_new[b:b + 1].float().cpu().numpy(), vn=L.v_new[b:b + 1].float().cpu().numpy())
            nb = sum(a.nbytes for a in x.values())
            if files and total + nb > cap and len(files) >= n_workers:
                break
            f = os.path.join(tmp, f"seq{b}.npz")
            np.savez(f, **x)
            files.append(f)
            total += nb
        n_workers = min(n_workers, len(files))
        shares = [files[i::n_workers] for i in range(n_workers)]
        meta = {"hq": w.n_q_heads, "hkv": w.n_kv_heads, "scale": w.scale, "q_len": q_len, "window": window}
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"
        try:
            with cf.ProcessPoolExecutor(n_workers, mp_context=mp.get_context("spawn")) as ex:
                res = list(ex.map(_oracle_worker, [(sh, budget_s, mode, meta) for sh in shares]))
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    kv_bytes = sum(r[0] for r in res)
    secs = max(r[1] for r in res)
    runs = sum(r[2] for r in res)
    what = f"{q_len}-token decode" if multi else "append + decode"
    return {"value": kv_bytes / secs / 1e9, "unit": "GB/s", "cores": n_workers, "kind": "oracle",
            "sample": f"{runs} whole-sequence runs over {len(files)} of the {w.batch} sequences of layer 0 "
                      f"({what}, all {w.n_q_heads} query heads) in {n_workers} single-threaded worker processes, "
                      f"{kv_bytes / 2**20:.0f} MiB of KV in {secs:.1f} s (longest worker)",
            "seconds": secs}


def gather_probe(w, S, dec, device, steps, u8=False):
    """The gather probe (the decode kernel's tile stream, no arithmetic) on the
    same pools, block table and chunks, rotating the pool copies as the timed
    steps do: GB/s of algorithmic KV bytes."""
    import torch
    import paged_kv_cache_254_amd as pkv
    sink = torch.empty(max(1, dec.n_items), dtype=torch.int32, device=device)
    layers = S["layers"]
    n = max(len(layers), steps)

    def probe(L):
        if u8:
            pkv.gather_probe_q8(L.k_pages, L.v_pages, L.meta, S["bt"], S["seq_lens"], sink, dec.n_items,
                                dec.min_chunk_pages)
        else:
            pkv.gather_probe(L.k_pages, L.v_pages, S["bt"], S["seq_lens"], sink, dec.n_items, dec.min_chunk_pages)
    for i in range(len(layers)):
        probe(layers[i])
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(n):
        probe(layers[i % len(layers)])
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / n
    return S["kv_bytes_layer"] / (ms / 1e3) / 1e9, ms


def hbm_probe(device):
    import torch
    import paged_kv_cache_254_amd as pkv
    props = torch.cuda.get_device_properties(device)
    n_cu = props.multi_processor_count
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=device)
    buf.fill_(1)
    sink = torch.empty(n_cu * 64, dtype=torch.int32, device=device)
    best = 0.0
    for blocks_per_cu in (4, 8, 16):
        nb = n_cu * blocks_per_cu
        for _ in range(2):
            pkv.hbm_read_probe(buf, sink, nb)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(5):
            pkv.hbm_read_probe(buf, sink, nb)
        e.record()
        torch.cuda.synchronize()
        best = max(best, 5 * buf.numel() / (s.elapsed_time(e) / 1e3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def traffic_for(workload, kv="dense"):
    """HBM bytes per split-kernel launch from committed rocprofv3 counters, if
    they were taken on the current kernel source; otherwise None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}{'_u8' if kv == 'u8' else ''}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sha") != kernel_sha():
        return None
    return d.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this path is single-GPU by design", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_254_amd as pkv
    import workloads as W

    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            pkv.copy_probe(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "launches": 3}))
        return
    w = W.get(args.workload)
    log(f"setup {w.name}")
    u8 = args.kv == "u8"
    if u8 and w.dtype != "bf16":
        print("--kv u8 takes a bf16 workload (its q and out stay bf16)", file=sys.stderr)
        sys.exit(2)
    T, window = args.q_len, args.window
    multi = T > 1 or window > 0
    if multi and (u8 or args.unfused or args.separate_combine or T < 1 or window < 0):
        print("--q-len/--window take the dense cache, with the library's own merge", file=sys.stderr)
        sys.exit(2)
    S = setup(w, device, args.kv, T, window)
    dt = torch.uint8 if u8 else W.torch_dtype(w)
    # More than 64 query columns per KV head (q_len x group): the library runs
    # its prefill kernel, which needs no workspace and no Decoder.
    wide = multi and T * w.group > 64
    # the multi-token decode runs q_len x Hq query columns: the Decoder is built for them
    dec = None if wide else pkv.Decoder(w.batch, w.n_q_heads * T, w.n_kv_heads, w.head_dim, dt, S["mb"],
                                        args.n_items, args.min_chunk, device=device,
                                        combine_mode=1 if args.separate_combine else 0, schedule=args.schedule)
    # One kernel per layer when every pair can be merged inside the decode
    # kernel: a pair spans at most ceil(max_blocks / min_chunk) + 1 chunks, and
    # the library merges pairs of at most 96 chunks there, or 24 in its wide
    # kernel (33 to 64 query columns per KV head), whose larger merges it
    # leaves to the combine kernel.
    wide_decode = not wide and T * w.group > 32
    one_kernel = wide or (not args.separate_combine and
                          -(-S["mb"] // dec.min_chunk_pages) + 1 <= (24 if wide_decode else 96))
    layers = S["layers"]
    n_layers = w.n_layers
    kv_step = S["kv_bytes_layer"] * n_layers
    stream = torch.cuda.current_stream()
    rot = [0]

    def step(ev=None):
        """One step: per layer the library's full call (decode kernel, plus
        the combine kernel where the library needs it).  With ev (3 events
        per layer: before the decode kernel, after it, after the combine) the
        two halves are called separately when the library launches two
        kernels, so each can be timed; the kernels are the same."""
        stream = torch.cuda.current_stream()   # the capture stream while a graph is recorded
        for li in range(n_layers):
            L = layers[rot[0] % len(layers)]
            rot[0] += 1
            if multi:
                # one library call (decode kernel, merge inside it or in the combine kernel)
                if ev is not None:
                    ev[3 * li].record(stream)
                if wide:
                    pkv.paged_decode_multi(L.q, L.k_pages, L.v_pages, S["bt"], S["seq_lens"], T, w.scale, L.out,
                                           window, stream=stream)
                else:
                    dec.attn_multi(L.q, L.k_pages, L.v_pages, S["bt"], S["seq_lens"], T, w.scale, L.out, window,
                                   stream)
                if ev is not None:
                    ev[3 * li + 1].record(stream)
                    ev[3 * li + 2].record(stream)
                continue
            if u8 and args.unfused:
                # the quantizing append kernel, then the decode over the 8-bit cache
                pkv.kv_append_q8(L.k_new, L.v_new, L.k_pages, L.v_pages, L.meta, S["bt"], S["positions"], stream)
                if ev is not None:
                    ev[3 * li].record(stream)
                if ev is None or one_kernel:
                    dec.attn_q8(L.q, L.k_pages, L.v_pages, L.meta, S["bt"], S["seq_lens"], w.scale, L.out, stream)
                    if ev is not None:
                        ev[3 * li + 1].record(stream)
                else:
                    dec.split_q8(L.q, L.k_pages, L.v_pages, L.meta, S["bt"], S["seq_lens"], w.scale, L.out, stream)
                    if ev is not None:
                        ev[3 * li + 1].record(stream)
                    dec.combine(S["seq_lens"], L.out, S["mb"], stream)
                if ev is not None:
                    ev[3 * li + 2].record(stream)
                continue
            if u8:
                if ev is None or one_kernel:
                    # the library's step: quantizing append fused into the decode kernel
                    if ev is not None:
                        ev[3 * li].record(stream)
                    dec.step_q8(L.q, L.k_new, L.v_new, L.k_pages, L.v_pages, L.meta, S["bt"], S["seq_lens"],
                                w.scale, L.out, stream)
                    if ev is not None:
                        ev[3 * li + 1].record(stream)
                        ev[3 * li + 2].record(stream)
                    continue
                # timed halves: the quantizing append, then the decode kernel and the combine
                pkv.kv_append_q8(L.k_new, L.v_new, L.k_pages, L.v_pages, L.meta, S["bt"], S["positions"], stream)
                ev[3 * li].record(stream)
                dec.split_q8(L.q, L.k_pages, L.v_pages, L.meta, S["bt"], S["seq_lens"], w.scale, L.out, stream)
                ev[3 * li + 1].record(stream)
                dec.combine(S["seq_lens"], L.out, S["mb"], stream)
                ev[3 * li + 2].record(stream)
                continue
            if args.unfused:
                pkv.kv_append(L.k_new, L.v_new, L.k_pages, L.v_pages, S["bt"], S["positions"], stream)
            if ev is not None:
                ev[3 * li].record(stream)
            if ev is None or one_kernel:
                if args.unfused:
                    dec(L.q, L.k_pages, L.v_pages, S["bt"], S["seq_lens"], w.scale, L.out, stream)
                else:
                    dec.step(L.q, L.k_new, L.v_new, L.k_pages, L.v_pages, S["bt"], S["seq_lens"], w.scale,
                             L.out, stream)
                if ev is not None:
                    ev[3 * li + 1].record(stream)
                    ev[3 * li + 2].record(stream)
                continue
            if args.unfused:
                dec.split(L.q, L.k_pages, L.v_pages, S["bt"], S["seq_lens"], w.scale, L.out, stream)
            else:
                dec.step_split(L.q, L.k_new, L.v_new, L.k_pages, L.v_pages, S["bt"], S["seq_lens"], w.scale,
                               L.out, stream)
            ev[3 * li + 1].record(stream)
            dec.combine(S["seq_lens"], L.out, S["mb"], stream)
            ev[3 * li + 2].record(stream)

    log(f"warmup {args.warmup} (n_items={dec.n_items if dec else 'prefill'}, copies={len(layers)})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graphs = []
    if args.graph:
        # one captured step per rotation position, so replaying graph i % r
        # walks the pool copies exactly as the eager loop does
        positions = len(layers) // n_layers if len(layers) % n_layers == 0 else len(layers)
        if positions > 64:
            print(f"--graph: {positions} rotation positions is too many graphs for this workload",
                  file=sys.stderr)
            sys.exit(2)
        rot[0] = 0
        for _ in range(positions):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            graphs.append(g)
        for g in graphs:     # replay once before timing
            g.replay()
        torch.cuda.synchronize()
        log(f"captured {len(graphs)} graphs of {n_layers} layer(s)")

    # timed region: whole steps
    t_s, t_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_s.record(stream)
    for i in range(args.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step()
    t_e.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_s.elapsed_time(t_e) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # per-kernel durations, same launches with events between them
    n_launch = args.steps * n_layers
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3 * n_launch)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[3 * n_layers * i: 3 * n_layers * (i + 1)])
    torch.cuda.synchronize()
    split_ms = [evs[3 * k].elapsed_time(evs[3 * k + 1]) for k in range(n_launch)]
    comb_ms = [evs[3 * k + 1].elapsed_time(evs[3 * k + 2]) for k in range(n_launch)]
    # Average launch of the decode kernel.  When a step is exactly one decode
    # launch per layer, the timed region's average is that launch's duration
    # (back to back on one stream, as rocprofv3's kernel trace times it);
    # otherwise the events around each launch isolate it from the other
    # kernels of the step, at the price of the events' own time (~1 %).
    events_avg = float(np.mean(split_ms))
    single_launch = one_kernel and not args.unfused and not graphs
    split_avg = ms_per_step / n_layers if single_launch else events_avg
    timing = ("timed-region average, one decode launch per layer" if single_launch
              else "events around each decode launch")
    achieved = S["kv_bytes_layer"] / (split_avg / 1e3) / 1e9
    value = kv_step / (ms_per_step / 1e3) / 1e9
    # Algorithmic FLOPs per launch: 4 x head_dim per (query token, query head,
    # attended key); with several query tokens each attends its own causal
    # (windowed) range.  Above the ridge (peak FLOP/s / peak bytes/s) the
    # launch is bound by the matrix cores, below it by HBM.
    keys = multi_keys(S["att"], T, window)
    flops_layer = 4 * w.head_dim * w.n_q_heads * keys
    intensity = flops_layer / S["kv_bytes_layer"]
    mfma_bound = intensity > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    tflops = flops_layer / (split_avg / 1e3) / 1e12
    traffic = None if multi else traffic_for(w.name, args.kv)   # counters are taken on the one-token decode

    probe = None if args.no_probe else hbm_probe(device)
    gprobe = None
    if not args.no_probe and not multi:
        gprobe = gather_probe(w, S, dec, device, args.steps * n_layers, u8)
    # Fixed cost per kernel launch on this stream (an empty kernel, one
    # workgroup per CU): ordinary, cooperative, and cooperative with one
    # grid-wide barrier (what folding the combine into the decode kernel
    # would need).
    launch_us = None
    if not args.no_probe and not args.no_launch_probe:
        launch_us = {k: round(pkv.launch_probe(m, stream=stream), 2)
                     for k, m in (("launch", 0), ("cooperative", 1), ("cooperative_grid_barrier", 2))}
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(w, S, args.cpu_seconds, args.kv, T, window)
        cpu.pop("seconds", None)

    rec = {
        "metric": "KV-cache GB/s read and % of MI355X HBM peak for paged GQA decode attention",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("u8 cache, bf16 q/out" if u8 else "bf16") if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "block_size": 16, "layers": n_layers,
            "attended_tokens": int(S["att"].sum()), "kv_bytes_per_step": kv_step,
            "accumulate": "fp32", "n_items": dec and dec.n_items, "min_chunk_pages": dec and dec.min_chunk_pages,
            "schedule": "one workgroup per 4 query tiles, no split" if wide else
                        {1: "static", 2: "dynamic"}.get(dec.schedule, dec.schedule),
            "pool_copies": len(layers),
            "append": ("separate kernel" if args.unfused else
                       "quantizing, fused into the decode kernel" if u8 else "fused into the decode kernel"),
            "merge": "combine kernel" if not one_kernel else "inside the decode kernel",
            "kv_cache": "8-bit codes + per-token scale/zero (2D+16 B per token and head)" if u8 else w.dtype,
            "launch": "hip graph replay" if graphs else "eager",
            **({"q_len": T, "window": window, "append": "none (tokens cached before the step)",
                "merge": "library call (split + merge; timed together)"} if multi else {}),
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.batch * T / (ms_per_step / 1e3), 1),
        "roofline": ({
            "bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
        } if mfma_bound else {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        }) | {
            "kernel": ("prefill_kernel" if wide else
                       "wide_kernel" if (u8 or w.dtype == "bf16") and 32 < T * w.group <= 64 else "split_kernel"),
            "avg_launch_ms": round(split_avg, 5),
            "timing": timing, "avg_launch_ms_events": round(events_avg, 5),
            "algorithmic_bytes_per_launch": S["kv_bytes_layer"], "algorithmic_flops_per_launch": int(flops_layer),
            "flop_per_byte": round(intensity, 2), "kv_gbs": round(achieved, 2), "tflops": round(tflops, 3),
        },
        "split_median_ms": round(float(np.median(split_ms)), 5),
        "split_min_ms": round(float(np.min(split_ms)), 5),
        "split_max_ms": round(float(np.max(split_ms)), 5),
        "combine_avg_ms": None if one_kernel or multi else round(float(np.mean(comb_ms)), 5),
        "hbm_read_probe_gbs": None if probe is None else round(probe, 1),
        "pct_of_read_probe": None if probe is None else round(100 * value / probe, 1),
        "gather_probe_gbs": None if gprobe is None else round(gprobe[0], 1),
        "gather_probe_ms": None if gprobe is None else round(gprobe[1], 5),
        "pct_of_gather_probe": None if gprobe is None else round(100 * achieved / gprobe[0], 1),
        "launch_probe_us": launch_us,
        "cpu_baseline": cpu,
        "kernel_sha": kernel_sha(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
