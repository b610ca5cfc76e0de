"""KV-cache byte accounting (oracle; test infrastructure only).

The pages give one formula in three notations:

* "Inference Engines" (hoshank.vercel.app, book chapter 17), section
  "The Mathematics", equation M_kv:  M = 2 * L * n_kv * d_h * s * b * p.
* "Efficient inference" (learn.byteknotlabs.com lesson 7-10), "Key ideas":
  KV cache per token = 2 * L * n_kv * d_head * bytes.
* "Transformer inference mechanics" (evaltude docs), section "What the KV cache
  stores per layer": 2 x layers x resident tokens x KV heads x head dimension
  x bytes per cached element.

The factor 2 counts keys and values.  The same chapter 17 section gives the
MHA-to-GQA cache ratio n_h / n_kv, with n_kv = 1 the MQA case.
"""
from __future__ import annotations


def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                   batch: int, bytes_per_elem: int) -> int:
    """M_kv = 2 * L * n_kv * d_h * s * b * p (chapter 17, "The Mathematics")."""
    return 2 * n_layers * n_kv_heads * head_dim * seq_len * batch * bytes_per_elem


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int,
                       bytes_per_elem: int) -> int:
    """Per-token form (byteknotlabs "Key ideas"): M_kv with s = b = 1."""
    return kv_cache_bytes(n_layers, n_kv_heads, head_dim, 1, 1, bytes_per_elem)


def mha_to_gqa_ratio(n_q_heads: int, n_kv_heads: int) -> float:
    """M_kv(MHA) / M_kv(GQA) at equal L, d_h, s, b, p (chapter 17 ratio equation)."""
    mha = kv_cache_bytes(1, n_q_heads, 1, 1, 1, 1)
    gqa = kv_cache_bytes(1, n_kv_heads, 1, 1, 1, 1)
    return mha / gqa


def attended_kv_bytes(seq_lens, n_kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    """Bytes of K and V that one layer's decode step must read: the per-layer,
    per-token figure summed over every attended token of every sequence."""
    per_token = kv_bytes_per_token(1, n_kv_heads, head_dim, bytes_per_elem)
    return int(sum(int(n) for n in seq_lens)) * per_token
