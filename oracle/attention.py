"""Paged decode attention, written as its plain definition in fp64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages define it:

* Attention of one query over a sequence's keys and values:
  softmax(q K^T / sqrt(d)) V  ("Part 6 - Inference Fundamentals" on evaltude,
  section "Q, K, V - and why they force a cache"; evaltude docs "Transformer
  inference mechanics", section "What Q, K, and V do in causal attention").
  The scale is an explicit argument; the workloads pass 1/sqrt(d).
* Causal masking: a query at position t attends to keys up to t (same docs
  section).  In decode the single new query is the last position, so the mask
  is just "token index < seq_len"; the new token attends to itself.
* Head sharing: MHA gives each query head its own K/V head, MQA shares one,
  GQA shares each K/V head across a group (docs section "MHA versus MQA versus
  GQA").  Groups are contiguous: with N = K * G (CS336 lecture 10 notes,
  "Arithmetic-intensity refresher" notation), query head hq reads K/V head
  hq // G.
* Paging: each sequence's cache lives in fixed-size blocks, 16 tokens by
  default, found through a per-request block table that maps logical positions
  to physical blocks ("Inference Engines" chapter 17, "The Breakthrough";
  CS336 notes, "PagedAttention (vLLM)").  Token t of sequence b is slot t % bs
  of physical page block_table[b][t // bs].
* Split attention: the page on FlashAttention (byteknotlabs "Efficient
  inference", section "FlashAttention: exact attention without the matrix")
  states that attention over a long key sequence can be computed block by
  block, tracking the largest score and the sum of exponentials seen so far,
  and that the per-block results then merge into the exact answer (the
  formula itself did not survive on the page).  ``partial`` and
  ``lse_combine`` write that merge out: a partial over a token range is its
  normalised output plus the natural log of its softmax denominator, and the
  merge weighs each partial by exp(lse - max lse).
* Appending: each decode step writes the new token's K and V into each layer's
  cache (docs section "What the KV cache stores per layer").
* Several query tokens at once (``decode_multi``): the last q_len cached
  tokens each attend causally, optionally within a sliding window (see
  ``query_range``); the speculative-decoding passages of "Inference Engines"
  and the CS336 notes ("Exploit checking is faster than generating") run the
  target model once over all drafted tokens.

Physical layout read here (a caller/library contract; the pages fix only the
block size): K pages ``[P][Hkv][D/X][bs][X]``, V pages ``[P][Hkv][D][bs]``.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def _as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def gather(k_pages, v_pages, block_table_row, n_tokens: int,
           block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Dense K, V of one sequence, shape [n][Hkv][D], in fp64.

    Token t is slot t % bs of page block_table_row[t // bs]: the used pages are
    stacked in logical order, each page's [bs] slots become consecutive tokens,
    and the tail past n_tokens (unused slots of the last page) is dropped."""
    n_kv, chunks, bs, x = k_pages.shape[1], k_pages.shape[2], k_pages.shape[3], k_pages.shape[4]
    assert bs == block_size and v_pages.shape[3] == block_size
    d = chunks * x
    n_blocks = (n_tokens + block_size - 1) // block_size
    pages = np.asarray(block_table_row[:n_blocks], dtype=np.int64)
    if n_blocks and (pages.min() < 0 or pages.max() >= k_pages.shape[0]):
        raise IndexError("block table entry outside the pool")
    kp = np.asarray(k_pages[pages])              # [blk][Hkv][D/X][bs][X]
    vp = np.asarray(v_pages[pages])              # [blk][Hkv][D][bs]
    K = kp.transpose(0, 3, 1, 2, 4).reshape(n_blocks * bs, n_kv, d)[:n_tokens]
    V = vp.transpose(0, 3, 1, 2).reshape(n_blocks * bs, n_kv, d)[:n_tokens]
    return _as_f64(K), _as_f64(V)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query q [D] over K, V [n][D]; zeros if n = 0.

    The maximum score is subtracted before exponentiating; that leaves the
    softmax unchanged and keeps exp() finite."""
    q = _as_f64(q)
    K = _as_f64(K)
    V = _as_f64(V)
    if K.shape[0] == 0:
        return np.zeros(q.shape[0], dtype=np.float64)
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """Attention restricted to the given tokens, and the natural log of its
    softmax denominator: (softmax(s) V, log sum_t exp(s_t)) with s = scale * K q.
    An empty range gives (zeros, -inf)."""
    q = _as_f64(q)
    if K.shape[0] == 0:
        return np.zeros(q.shape[0], dtype=np.float64), -math.inf
    s = scale * (_as_f64(K) @ q)
    m = s.max()
    w = np.exp(s - m)
    return (w @ _as_f64(V)) / w.sum(), float(m + math.log(w.sum()))


def lse_combine(outs: Sequence[np.ndarray], lses: Sequence[float]) -> np.ndarray:
    """Merge partials of disjoint token ranges: weights exp(lse_i - max lse),
    out = sum_i w_i o_i / sum_i w_i.  Ranges with lse = -inf weigh nothing; if
    every range is empty the result is zeros."""
    lses = np.asarray(lses, dtype=np.float64)
    outs = [_as_f64(o) for o in outs]
    if len(outs) == 0 or not np.isfinite(lses).any():
        return np.zeros_like(outs[0]) if outs else np.zeros(0)
    m = lses.max()
    w = np.exp(lses - m)
    acc = np.zeros_like(outs[0])
    for wi, oi in zip(w, outs):
        if wi > 0.0:
            acc = acc + wi * oi
    return acc / w.sum()


def decode(q, k_pages, v_pages, block_table, seq_lens, n_q_heads: int, n_kv_heads: int,
           block_size: int, scale: float) -> np.ndarray:
    """Decode attention for a batch: out[b, hq] = attend(q[b, hq], K_b[:, hq // G],
    V_b[:, hq // G]) over the seq_lens[b] tokens of sequence b.  Returns fp64
    [B][Hq][D]."""
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    group = n_q_heads // n_kv_heads
    q = _as_f64(q)
    B, _, d = q.shape
    out = np.zeros((B, n_q_heads, d), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        K, V = gather(k_pages, v_pages, block_table[b], n, block_size)
        for hq in range(n_q_heads):
            h = hq // group
            out[b, hq] = attend(q[b, hq], K[:, h, :], V[:, h, :], scale)
    return out


def query_range(seq_len: int, q_len: int, i: int, window: int) -> Tuple[int, int]:
    """Keys [lo, hi) that query token i of the last q_len cached tokens attends.

    Query i sits at position seq_len - q_len + i and, causally, sees keys up
    to and including its own position (evaltude docs, "What Q, K, and V do in
    causal attention").  With a sliding window of W > 0 it sees only the last
    W of those (CS336 lecture 10 notes, "Local attention & sparse variants":
    each token attends to the last K)."""
    hi = seq_len - q_len + i + 1
    lo = max(0, hi - window) if window > 0 else 0
    return lo, hi


def decode_multi(q, k_pages, v_pages, block_table, seq_lens, q_len: int, n_q_heads: int,
                 n_kv_heads: int, block_size: int, scale: float, window: int = 0) -> np.ndarray:
    """Attention of the last q_len cached tokens of each sequence (a drafted
    run being verified in one pass, or a prefill chunk), each over the keys
    query_range gives: out[b, i, hq] = attend(q[b, i, hq], K_b[lo:hi, h],
    V_b[lo:hi, h]) with h = hq // G.  q and out are [B][q_len][Hq][D];
    seq_lens count every cached token, the q_len new ones included (the
    drafted tokens' K/V are appended first; "Inference Engines", the
    speculative-decoding paragraph: the target model runs once over the whole
    drafted sequence).  q_len = 1, window = 0 is decode()."""
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    group = n_q_heads // n_kv_heads
    q = _as_f64(q)
    B, T, _, d = q.shape
    assert T == q_len
    out = np.zeros((B, T, n_q_heads, d), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        K, V = gather(k_pages, v_pages, block_table[b], n, block_size)
        for i in range(T):
            lo, hi = query_range(n, T, i, window)
            if hi <= 0:
                continue
            for hq in range(n_q_heads):
                h = hq // group
                out[b, i, hq] = attend(q[b, i, hq], K[lo:hi, h, :], V[lo:hi, h, :], scale)
    return out


def copy_blocks(k_pages, v_pages, src_pages, dst_pages):
    """Copies of the pools where page dst_pages[i] holds page src_pages[i]'s
    contents (every KV head, K and V): the copy half of block-level
    copy-on-write (CS336 lecture 10 notes, "PagedAttention (vLLM)": shared
    blocks are split only when generations diverge)."""
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    for s, d in zip(src_pages, dst_pages):
        k_out[int(d)] = k_pages[int(s)]
        v_out[int(d)] = v_pages[int(s)]
    return k_out, v_out


def append(k_pages, v_pages, block_table, positions, k_new, v_new, block_size: int):
    """Copies of the pools with the step's new K/V written into their slots:
    for each sequence b and KV head h, token positions[b] goes to slot
    positions[b] % bs of page block_table[b][positions[b] // bs].  A pure copy
    of the caller's elements (any dtype, compared bit for bit)."""
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    x = k_pages.shape[4]
    B, n_kv, d = k_new.shape
    for b in range(B):
        pos = int(positions[b])
        page = int(block_table[b][pos // block_size])
        slot = pos % block_size
        for h in range(n_kv):
            for i in range(d):
                k_out[page, h, i // x, slot, i % x] = k_new[b, h, i]
                v_out[page, h, i, slot] = v_new[b, h, i]
    return k_out, v_out
