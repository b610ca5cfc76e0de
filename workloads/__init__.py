"""Seeded synthetic inputs for the paged decode-attention path.

This module is the only code shared by the oracle side and the HIP side of the
tests, the benchmark and the smoke check.  It draws random numbers and fixes
shapes; it holds none of the method's arithmetic (no gather, no attention, no
page allocation, no byte accounting).

Workloads (the shapes of the pages' own examples):

* ``tiny_f32``      batch 2, cached lengths {37, 100}, 4 query / 2 KV heads,
                    head_dim 64, fp32, a 32-page pool.
* ``llama2_7b_mha`` batch 16 x 4096 tokens, 32 / 32 heads, head_dim 128, bf16
                    (one layer of the Llama-2-7B fp16 example: 0.5 MiB/token
                    over 32 layers, 32 GiB for 16 such sequences; byteknotlabs
                    "Efficient inference", section "The KV cache").
* ``llama3_8b_gqa`` batch 64, lengths uniform in [512, 8192], 32 / 8 heads.
* ``long_70b_gqa``  batch 1 x 131072 tokens, 64 / 8 heads (the 70B shape of the
                    same page's "Exercises").
* ``long_70b_mqa``  the same with a single KV head (MQA).
* ``llama3_8b_step`` batch 256, lognormal cached lengths (median 2000, sigma 1,
                    clipped to [16, 32768]), 32 / 8 heads, 32 layers.

Every workload appends one new token per sequence in its step and then attends
over the whole cache.  ``cached_lens`` are the lengths before the append and
``attended_lens`` after it.  Where a workload states the length it is "at"
(every ``llama2_7b_mha`` sequence at 4096, ``long_*`` at 131072,
``llama3_8b_gqa`` in [512, 8192]) that stated length is the attended one; for
``tiny_f32`` and ``llama3_8b_step`` the stated lengths are the cached ones.

Physical page layout (the contract between the caller, the library and the
oracle; the pages fix only that a block holds 16 tokens):

* K pool ``[P][Hkv][D / X][16][X]`` with ``X = 16 / sizeof(elem)`` (8 for bf16,
  4 for fp32): each token's key is cut into 16-byte pieces, and the pieces of
  all 16 tokens that cover the same feature range are stored next to each other.
* V pool ``[P][Hkv][D][16]``: the page holds V transposed (feature-major).
* 8-bit pools (``make_q8_pools``): K codes ``[P][Hkv][D / 16][16][16]``, V codes
  ``[P][Hkv][D / 64][4][16][4][4]`` in the library's order (the oracle keeps
  ``[D][16]``; ``v_codes_to_logical`` converts), meta ``[P][Hkv][4][16]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str               # "f32" or "bf16"
    lens: str                # how lengths are drawn (see cached_lens)
    n_layers: int = 1
    block_size: int = BLOCK_SIZE
    pool_pages: Optional[int] = None   # None: ceil(1.25 x pages needed)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 2, 4, 2, 64, "f32", "fixed:37,100:cached",
                         pool_pages=32, seed=1000),
    "llama2_7b_mha": Workload("llama2_7b_mha", 16, 32, 32, 128, "bf16",
                              "fixed:4096:attended", seed=2000),
    "llama3_8b_gqa": Workload("llama3_8b_gqa", 64, 32, 8, 128, "bf16",
                              "uniform:512,8192:attended", seed=3000),
    "long_70b_gqa": Workload("long_70b_gqa", 1, 64, 8, 128, "bf16",
                             "fixed:131072:attended", seed=4000),
    "long_70b_mqa": Workload("long_70b_mqa", 1, 64, 1, 128, "bf16",
                             "fixed:131072:attended", seed=4100),
    "llama3_8b_step": Workload("llama3_8b_step", 256, 32, 8, 128, "bf16",
                               "lognormal:2000,1.0,16,32768:cached",
                               n_layers=32, seed=5000),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def custom(name: str, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
           dtype: str, cached: List[int], pool_pages: Optional[int] = None,
           seed: int = 0, n_layers: int = 1) -> Workload:
    """A small hand-shaped workload for tests (cached lengths given explicitly)."""
    assert len(cached) == batch
    spec = "fixed:" + ",".join(str(int(x)) for x in cached) + ":cached"
    return Workload(name, batch, n_q_heads, n_kv_heads, head_dim, dtype, spec,
                    n_layers=n_layers, pool_pages=pool_pages, seed=seed)


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([w.seed, stream]))


def cached_lens(w: Workload) -> np.ndarray:
    """Lengths held in the cache before the step's append (int64, one per sequence)."""
    kind, args, which = w.lens.split(":")
    if kind == "fixed":
        vals = [int(x) for x in args.split(",")]
        lens = np.array(vals if len(vals) == w.batch else vals * w.batch, dtype=np.int64)
    elif kind == "uniform":
        lo, hi = (int(x) for x in args.split(","))
        lens = _rng(w, 1).integers(lo, hi, size=w.batch, endpoint=True).astype(np.int64)
    elif kind == "lognormal":
        med, sigma, lo, hi = (float(x) for x in args.split(","))
        z = _rng(w, 1).standard_normal(w.batch)
        lens = np.clip(np.rint(np.exp(math.log(med) + sigma * z)), lo, hi).astype(np.int64)
    else:
        raise ValueError(w.lens)
    lens = lens[: w.batch]
    return lens - 1 if which == "attended" else lens


def attended_lens(w: Workload) -> np.ndarray:
    return cached_lens(w) + 1


def pages_needed(w: Workload) -> int:
    bs = w.block_size
    return int(sum((int(n) + bs - 1) // bs for n in attended_lens(w)))


def pool_pages(w: Workload) -> int:
    if w.pool_pages is not None:
        return w.pool_pages
    return int(math.ceil(1.25 * pages_needed(w)))


def free_order(w: Workload, layer: int = 0) -> np.ndarray:
    """Seeded random permutation of the physical page ids (the pool's initial free list)."""
    return _rng(w, 2).permutation(pool_pages(w)).astype(np.int32)


def k_pool_shape(w: Workload, num_pages: Optional[int] = None):
    x = 16 // w.elem_bytes
    P = pool_pages(w) if num_pages is None else num_pages
    return (P, w.n_kv_heads, w.head_dim // x, w.block_size, x)


def v_pool_shape(w: Workload, num_pages: Optional[int] = None):
    P = pool_pages(w) if num_pages is None else num_pages
    return (P, w.n_kv_heads, w.head_dim, w.block_size)


def torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _gen(device, seed: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_q(w: Workload, layer: int = 0, device="cpu"):
    import torch
    g = _gen(device, w.seed * 1000 + 10 * layer + 1)
    return torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=g, device=device,
                       dtype=torch.float32).to(torch_dtype(w))


def make_new_kv(w: Workload, layer: int = 0, device="cpu"):
    import torch
    g = _gen(device, w.seed * 1000 + 10 * layer + 2)
    k = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32).to(torch_dtype(w))
    v = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32).to(torch_dtype(w))
    return k, v


def make_pools(w: Workload, layer: int = 0, device="cpu"):
    """K and V pools filled with N(0,1) in every slot (used or not)."""
    import torch
    g = _gen(device, w.seed * 1000 + 10 * layer + 3)
    dt = torch_dtype(w)
    k = torch.randn(k_pool_shape(w), generator=g, device=device, dtype=dt)
    v = torch.randn(v_pool_shape(w), generator=g, device=device, dtype=dt)
    return k, v


def q8_pool_shapes(w: Workload, num_pages: Optional[int] = None):
    """(k_codes, v_codes, meta) shapes of the 8-bit cache for this workload, in
    the library's layout: v_codes [P][Hkv][D/64][4][16][4][4] (see
    v_codes_to_logical)."""
    P = pool_pages(w) if num_pages is None else num_pages
    D = w.head_dim
    return ((P, w.n_kv_heads, D // 16, 16, 16), (P, w.n_kv_heads, D // 64, 4, 16, 4, 4), (P, w.n_kv_heads, 4, 16))


# The library's 8-bit V-code tile [D/64][4][16][4][4] holds feature
# d = 64 j + 16 i + n, slot t = 4 c + e at [j][c][n][i][e]; the oracle's pools
# keep the plain [D][16] (feature, slot) order.  Both conversions are the same
# swap of the c and i axes (a pure byte permutation); numpy arrays or torch
# tensors.
_V_SWAP = (0, 1, 2, 5, 4, 3, 6)


def v_codes_to_logical(v):
    """Library-order 8-bit V codes [P][Hkv][D/64][4][16][4][4] -> [P][Hkv][D][16]."""
    P, H, J = v.shape[:3]
    t = v.permute(*_V_SWAP) if hasattr(v, "permute") else v.transpose(_V_SWAP)
    return t.reshape(P, H, 64 * J, 16)


def v_codes_from_logical(v):
    """[P][Hkv][D][16] 8-bit V codes -> the library's order [P][Hkv][D/64][4][16][4][4]."""
    P, H, D = v.shape[:3]
    t = v.reshape(P, H, D // 64, 4, 16, 4, 4)
    t = t.permute(*_V_SWAP) if hasattr(t, "permute") else t.transpose(_V_SWAP)
    return t.contiguous() if hasattr(t, "contiguous") else np.ascontiguousarray(t)


def make_q8_pools(w: Workload, layer: int = 0, device="cpu"):
    """8-bit cache pools as random inputs: codes uniform in [0, 255]; per slot
    scales uniform in [0.02, 0.03] (about the scale of an N(0,1) vector over
    255 steps) and integer zero points uniform in [118, 138]."""
    import torch
    g = _gen(device, w.seed * 1000 + 10 * layer + 5)
    ks, vs, ms = q8_pool_shapes(w)
    k = torch.randint(0, 256, ks, generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    v = torch.randint(0, 256, vs, generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    meta = torch.empty(ms, device=device, dtype=torch.float32)
    meta[:, :, 0::2] = torch.rand(ms[:2] + (2, ms[3]), generator=g, device=device) * 0.01 + 0.02
    meta[:, :, 1::2] = torch.randint(118, 139, ms[:2] + (2, ms[3]), generator=g, device=device).float()
    return k, v, meta
