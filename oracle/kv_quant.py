"""8-bit KV cache: uniform integer quantization of each cached K/V vector, and
paged decode over the dequantized cache (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages define it:

* A cached element may be stored in fewer bytes; the KV byte estimate
  multiplies by "bytes per cached element" and cache quantization changes the
  physical allocation (evaltude docs "Transformer inference mechanics: QKV,
  KV cache, and attention", section "What the KV cache stores per layer").
* Uniform integer quantization maps values to integers with a scale and a
  zero point, and the KV cache is one of the tensors it is applied to;
  per-group scales (groups of 128 elements in the page's example) keep the
  rounding error small (byteknotlabs "Efficient inference: KV cache, GQA,
  FlashAttention, speculative decoding, quantization", section "Quantization:
  fewer bytes per weight"; the formula itself was lost from the page; the
  exercise "Size a deployment" sizes an int8 KV cache).  CS336 lecture 10
  notes, "Quantization & pruning": quantize and dequantize via a scale and a
  zero point.

Readings taken where the pages leave the details open:

* Group = one token's vector of one KV head (head_dim elements; 128 on the
  larger workloads, the page's example group size), separately for K and V.
* 8-bit unsigned codes with a zero point (asymmetric):
    lo = min(min(x), 0), hi = max(max(x), 0)      (0 is always representable)
    s  = (hi - lo) / 255, or 1 when hi == lo (all-zero vector)
    z  = rint(-lo / s)                            (an integer in [0, 255])
    u  = clamp(rint(x / s) + z, 0, 255)
    x^ = s * (u - z)
  rint is round-half-to-even.  s, z and u are decided in float32 (the
  kernel's precision), so both sides produce the same codes bit for bit;
  dequantization and attention are then fp64.
* Storage per (page, KV head), 16 token slots, D features:
    K codes  uint8 [D/16][16][16]  (token t, feature 16c + x at [c][t][x])
    V codes  uint8 [D][16]         (feature d, token t at [d][t])
    meta     float32 [4][16]       (k_scale, k_zero, v_scale, v_zero) per slot
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import attention as A

CODE_MAX = 255


def quantize_vector(x) -> Tuple[np.ndarray, np.float32, np.float32]:
    """(codes uint8[D], scale, zero) of one vector, decided in float32."""
    x = np.asarray(x, dtype=np.float32)
    lo = np.float32(min(np.float32(x.min()), np.float32(0.0)))
    hi = np.float32(max(np.float32(x.max()), np.float32(0.0)))
    s = np.float32((hi - lo) / np.float32(CODE_MAX))
    if s == 0:
        s = np.float32(1.0)
    z = np.float32(np.rint(np.float32(-lo / s)))
    u = np.rint(x / s).astype(np.float32) + z
    codes = np.clip(u, 0, CODE_MAX).astype(np.uint8)
    return codes, s, z


def dequantize_vector(codes, scale, zero) -> np.ndarray:
    """x^ = scale * (codes - zero), in fp64 (exact: a 9-bit integer times a
    float32 scale)."""
    return np.float64(scale) * (np.asarray(codes, dtype=np.float64) - np.float64(zero))


def append(k_codes, v_codes, meta, block_table, positions, k_new, v_new, block_size: int):
    """Copies of the pools with each sequence's new token quantized into slot
    positions[b] % block_size of page block_table[b][positions[b] // block_size],
    for every KV head (K and V quantized separately)."""
    kc = np.array(k_codes, copy=True)
    vc = np.array(v_codes, copy=True)
    mt = np.array(meta, copy=True)
    B, n_kv, D = np.asarray(k_new).shape
    for b in range(B):
        pos = int(positions[b])
        page = int(block_table[b][pos // block_size])
        slot = pos % block_size
        for h in range(n_kv):
            ku, ks, kz = quantize_vector(np.asarray(k_new[b, h], dtype=np.float32))
            vu, vs, vz = quantize_vector(np.asarray(v_new[b, h], dtype=np.float32))
            for d in range(D):
                kc[page, h, d // 16, slot, d % 16] = ku[d]
                vc[page, h, d, slot] = vu[d]
            mt[page, h, :, slot] = (ks, kz, vs, vz)
    return kc, vc, mt


def dequantized_tiles(k_codes, v_codes, meta, page: int, head: int):
    """The [bs][D] keys and values one (page, KV head) holds, dequantized."""
    ku = k_codes[page, head].transpose(1, 0, 2).reshape(k_codes.shape[3], -1)   # [bs][D]
    vu = v_codes[page, head].T                                                  # [bs][D]
    m = meta[page, head]
    K = dequantize_vector(ku, m[0][:, None], m[1][:, None])
    V = dequantize_vector(vu, m[2][:, None], m[3][:, None])
    return K, V


def gather(k_codes, v_codes, meta, block_table_row, n_tokens: int, block_size: int):
    """Dequantized K and V [n_tokens][Hkv][D] of one sequence."""
    n_kv, D = v_codes.shape[1], v_codes.shape[2]
    K = np.zeros((n_tokens, n_kv, D))
    V = np.zeros((n_tokens, n_kv, D))
    for blk in range((n_tokens + block_size - 1) // block_size):
        page = int(block_table_row[blk])
        t0, t1 = blk * block_size, min(n_tokens, (blk + 1) * block_size)
        for h in range(n_kv):
            Kt, Vt = dequantized_tiles(k_codes, v_codes, meta, page, h)
            K[t0:t1, h] = Kt[: t1 - t0]
            V[t0:t1, h] = Vt[: t1 - t0]
    return K, V


def decode(q, k_codes, v_codes, meta, block_table, seq_lens, n_q_heads: int, n_kv_heads: int,
           block_size: int, scale: float) -> np.ndarray:
    """Decode attention over the dequantized cache: out[b, hq] =
    softmax(scale * q K^T) V with K, V the dequantized tokens of sequence b
    and KV head hq // G (zero rows for empty sequences)."""
    q = np.asarray(q, dtype=np.float64)
    G = n_q_heads // n_kv_heads
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        n = int(seq_lens[b])
        if n == 0:
            continue
        K, V = gather(k_codes, v_codes, meta, block_table[b], n, block_size)
        for hq in range(n_q_heads):
            out[b, hq] = A.attend(q[b, hq], K[:, hq // G], V[:, hq // G], scale)
    return out
