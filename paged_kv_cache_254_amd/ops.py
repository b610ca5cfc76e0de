"""Thin torch-facing wrappers over the libpkv C ABI (argument marshalling only;
every step runs in the library's HIP kernels or host C++)."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _lib
from ._lib import PKV_BF16, PKV_F32, PKV_U8, DecodeOpts, check, lib

BLOCK_SIZE = 16


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.uint8:
        return PKV_U8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr()


def _opts(n_items: int = 0, min_chunk_pages: int = 0, combine_mode: int = 0, schedule: int = 0):
    return ctypes.byref(DecodeOpts(int(n_items), int(min_chunk_pages), int(combine_mode), int(schedule)))


# ----------------------------------------------------------------- host side
def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return int(lib.pkv_kv_bytes_per_token(n_layers, n_kv_heads, head_dim, elem_bytes))


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, seq_len, batch, elem_bytes) -> int:
    return int(lib.pkv_kv_cache_bytes(n_layers, n_kv_heads, head_dim, seq_len, batch, elem_bytes))


class PagePool:
    """The library's host page pool (C++), with a free list in the given order."""

    def __init__(self, num_pages: int, free_order: Optional[Sequence[int]] = None):
        self._h = ctypes.c_void_p()
        if free_order is None:
            check(lib.pkv_pool_create(num_pages, None, ctypes.byref(self._h)), "pkv_pool_create")
        else:
            arr = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            check(lib.pkv_pool_create(num_pages, arr.ctypes.data_as(_lib._pi32), ctypes.byref(self._h)),
                  "pkv_pool_create")
        self.num_pages = num_pages

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value:
            lib.pkv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def num_free(self) -> int:
        return check(lib.pkv_pool_num_free(self._h), "pkv_pool_num_free")

    def reserve(self, seq_id: int, n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
        n = ctypes.c_int32()
        check(lib.pkv_seq_reserve(self._h, seq_id, n_tokens, block_size, ctypes.byref(n)), "pkv_seq_reserve")
        return n.value

    def release(self, seq_id: int) -> None:
        check(lib.pkv_seq_release(self._h, seq_id), "pkv_seq_release")

    def fork(self, parent: int, child: int) -> None:
        check(lib.pkv_seq_fork(self._h, parent, child), "pkv_seq_fork")

    def reserve_for_write(self, seq_id: int, position: int, block_size: int = BLOCK_SIZE):
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        check(lib.pkv_seq_reserve_for_write(self._h, seq_id, position, block_size, ctypes.byref(src),
                                            ctypes.byref(dst)), "pkv_seq_reserve_for_write")
        return None if src.value < 0 else (src.value, dst.value)

    def num_blocks(self, seq_id: int) -> int:
        n = ctypes.c_int32()
        check(lib.pkv_seq_num_blocks(self._h, seq_id, ctypes.byref(n)), "pkv_seq_num_blocks")
        return n.value

    def block_table(self, seq_ids: Sequence[int], max_blocks: int) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        out = np.empty((len(ids), max_blocks), dtype=np.int32)
        check(lib.pkv_build_block_table(self._h, ids.ctypes.data_as(_lib._pi64), len(ids), max_blocks,
                                        out.ctypes.data_as(_lib._pi32)), "pkv_build_block_table")
        return out


def decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_items: int) -> int:
    return check(int(lib.pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, n_items)),
                 "pkv_decode_workspace_bytes")


def decode_resolve(dtype_code: int, head_dim: int, n_q_heads: int, n_kv_heads: int, batch: int,
                   max_blocks: int, n_items: int = 0, min_chunk_pages: int = 0, combine_mode: int = 0,
                   schedule: int = 0):
    """(n_items, min_chunk_pages, workspace_bytes, schedule) the device calls use for these shapes."""
    res = DecodeOpts()
    ws = ctypes.c_int64()
    check(lib.pkv_decode_resolve(dtype_code, head_dim, n_q_heads, n_kv_heads, batch, max_blocks,
                                 _opts(n_items, min_chunk_pages, combine_mode, schedule), ctypes.byref(res),
                                 ctypes.byref(ws)), "pkv_decode_resolve")
    return res.n_items, res.min_chunk_pages, ws.value, res.schedule


def decode_plan(seq_lens: Sequence[int], n_kv_heads: int, max_blocks: int, n_items: int,
                min_chunk_pages: int):
    """(chunk_pages, first_chunk[B][Hkv], last_chunk[B][Hkv]) as the kernels compute them."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = len(lens)
    C = ctypes.c_int32()
    first = np.empty((B, n_kv_heads), dtype=np.int32)
    last = np.empty((B, n_kv_heads), dtype=np.int32)
    check(lib.pkv_decode_plan(lens.ctypes.data_as(_lib._pi32), B, n_kv_heads, BLOCK_SIZE, max_blocks, n_items,
                              min_chunk_pages, ctypes.byref(C), first.ctypes.data_as(_lib._pi32),
                              last.ctypes.data_as(_lib._pi32)), "pkv_decode_plan")
    return C.value, first, last


# --------------------------------------------------------------- device side
def kv_append(k_new, v_new, k_pages, v_pages, block_table, positions, stream=None) -> None:
    if not (k_new.dtype == v_new.dtype == k_pages.dtype == v_pages.dtype):
        raise TypeError("kv_append: k_new, v_new and the pools must share dtype")
    B, n_kv, D = k_new.shape
    check(lib.pkv_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                            _ptr(positions), B, n_kv, D, BLOCK_SIZE, block_table.shape[1], k_pages.shape[0],
                            _dtype_code(k_new), _stream(stream)), "pkv_kv_append")


def copy_blocks(k_pages, v_pages, src_pages, dst_pages, stream=None) -> None:
    """Copy every KV head's K and V tile of page src_pages[i] to dst_pages[i]."""
    import torch
    if src_pages.shape != dst_pages.shape or src_pages.dtype != torch.int32 or dst_pages.dtype != torch.int32:
        raise ValueError("src_pages and dst_pages must be int32 tensors of one shape")
    n = src_pages.numel()
    check(lib.pkv_copy_blocks(_ptr(k_pages), _ptr(v_pages), _ptr(src_pages), _ptr(dst_pages), n,
                              k_pages.shape[1], k_pages.shape[2] * k_pages.shape[4], BLOCK_SIZE, k_pages.shape[0],
                              _dtype_code(k_pages), _stream(stream)), "pkv_copy_blocks")


def kv_append_tokens(k_new, v_new, k_pages, v_pages, block_table, positions, stream=None) -> None:
    """Append q_len tokens per sequence: k_new, v_new [B][q_len][Hkv][D] at
    positions[b] + i (one kv_append launch per token)."""
    import torch
    T = k_new.shape[1]
    for i in range(T):
        kv_append(k_new[:, i].contiguous(), v_new[:, i].contiguous(), k_pages, v_pages, block_table,
                  (positions + i).to(torch.int32), stream)


def q8_pool_shapes(num_pages: int, n_kv_heads: int, head_dim: int):
    """Shapes of the 8-bit cache's (k_codes uint8, v_codes uint8, meta float32)
    in the library's layout (include/pkv.h): v_codes [P][Hkv][D/64][4][16][4][4]
    holds feature d = 64 j + 16 i + n, token t = 4 c + e at [j][c][n][i][e]."""
    return ((num_pages, n_kv_heads, head_dim // 16, BLOCK_SIZE, 16),
            (num_pages, n_kv_heads, head_dim // 64, 4, 16, 4, 4),
            (num_pages, n_kv_heads, 4, BLOCK_SIZE))


def kv_append_q8(k_new, v_new, k_codes, v_codes, meta, block_table, positions, stream=None) -> None:
    """Quantize each sequence's new K/V token into the 8-bit cache at positions[b]."""
    import torch
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8 or meta.dtype != torch.float32:
        raise TypeError("kv_append_q8: k_codes and v_codes uint8, meta float32")
    B, n_kv, D = k_new.shape
    check(lib.pkv_kv_append_q8(_ptr(k_new), _ptr(v_new), _ptr(k_codes), _ptr(v_codes), _ptr(meta),
                               _ptr(block_table), _ptr(positions), B, n_kv, D, BLOCK_SIZE, block_table.shape[1],
                               k_codes.shape[0], _dtype_code(k_new), _stream(stream)), "pkv_kv_append_q8")


class Decoder:
    """Holds the resolved work split and a workspace for one decode shape
    (batch, heads, head_dim, dtype and the block-table width max_blocks).
    The workspace starts zero-filled, as the in-kernel merge's arrival
    counters and the dynamic schedule's chunk counter require; combine_mode 1
    always merges with the combine kernel.  schedule: PKV_SCHEDULE_AUTO (0),
    _STATIC (1) or _DYNAMIC (2); self.schedule holds the resolved one."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype, max_blocks: int,
                 n_items: int = 0, min_chunk_pages: int = 0, device="cuda", combine_mode: int = 0,
                 schedule: int = 0):
        import torch
        code = {torch.bfloat16: PKV_BF16, torch.float32: PKV_F32, torch.uint8: PKV_U8}[dtype]
        self.n_items, self.min_chunk_pages, self.ws_bytes, self.schedule = decode_resolve(
            code, head_dim, n_q_heads, n_kv_heads, batch, max_blocks, n_items, min_chunk_pages, combine_mode,
            schedule)
        self.combine_mode = combine_mode
        self.workspace = torch.zeros(max(256, self.ws_bytes), dtype=torch.uint8, device=device)
        self.shape = (batch, n_q_heads, n_kv_heads, head_dim)
        self.max_blocks = max_blocks

    def _check_batch(self, B: int):
        if B > self.shape[0]:
            raise ValueError(f"batch {B} is larger than the {self.shape[0]} this Decoder's workspace was sized for")

    def _args(self, q, k_pages, v_pages, block_table, seq_lens, scale, out, stream):
        if not (q.dtype == k_pages.dtype == v_pages.dtype == out.dtype) or _dtype_code(q) == PKV_U8:
            raise TypeError("dense decode: q, k_pages, v_pages and out must share dtype bf16 or float32")
        B, Hq, D = q.shape
        self._check_batch(B)
        return (_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), Hq,
                k_pages.shape[1], D, BLOCK_SIZE, float(scale), _ptr(out), _stream(stream), B,
                block_table.shape[1], k_pages.shape[0], _dtype_code(q), _ptr(self.workspace),
                self.workspace.numel(), _opts(self.n_items, self.min_chunk_pages, self.combine_mode, self.schedule))

    def __call__(self, q, k_pages, v_pages, block_table, seq_lens, scale, out, stream=None):
        check(lib.pkv_paged_decode_attn(*self._args(q, k_pages, v_pages, block_table, seq_lens, scale, out,
                                                    stream)), "pkv_paged_decode_attn")
        return out

    def _step_args(self, q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, scale, out, stream):
        if not (q.dtype == k_new.dtype == v_new.dtype == k_pages.dtype == v_pages.dtype == out.dtype) or \
                _dtype_code(q) == PKV_U8:
            raise TypeError("dense decode step: all tensors must share dtype bf16 or float32")
        B, Hq, D = q.shape
        self._check_batch(B)
        return (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                _ptr(seq_lens), Hq, k_pages.shape[1], D, BLOCK_SIZE, float(scale), _ptr(out), _stream(stream),
                B, block_table.shape[1], k_pages.shape[0], _dtype_code(q), _ptr(self.workspace),
                self.workspace.numel(), _opts(self.n_items, self.min_chunk_pages, self.combine_mode, self.schedule))

    def step(self, q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, scale, out, stream=None):
        """Append each sequence's new token at seq_lens - 1 and attend, in one pass."""
        check(lib.pkv_decode_step(*self._step_args(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens,
                                                   scale, out, stream)), "pkv_decode_step")
        return out

    def step_split(self, q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, scale, out, stream=None):
        """The split half of step(); follow with combine()."""
        check(lib.pkv_decode_step_split(*self._step_args(q, k_new, v_new, k_pages, v_pages, block_table,
                                                         seq_lens, scale, out, stream)), "pkv_decode_step_split")

    def split(self, q, k_pages, v_pages, block_table, seq_lens, scale, out, stream=None):
        check(lib.pkv_paged_decode_split(*self._args(q, k_pages, v_pages, block_table, seq_lens, scale, out,
                                                     stream)), "pkv_paged_decode_split")

    def combine(self, seq_lens, out, max_blocks: int, stream=None):
        _, Hq, Hkv, D = self.shape
        B = out.shape[0]
        self._check_batch(B)
        check(lib.pkv_lse_combine(_ptr(self.workspace), self.workspace.numel(), _ptr(seq_lens), B, Hq, Hkv, D,
                                  BLOCK_SIZE, max_blocks, _ptr(out), _dtype_code(out),
                                  _opts(self.n_items, self.min_chunk_pages, self.combine_mode, self.schedule), _stream(stream)),
              "pkv_lse_combine")

    def attn_multi(self, q, k_pages, v_pages, block_table, seq_lens, q_len: int, scale, out, window: int = 0,
                   stream=None):
        """Attention of the last q_len cached tokens of each sequence (causal,
        optional sliding window).  q, out: [B][q_len][Hq][D].  Build the
        Decoder with n_q_heads * q_len query heads (the workspace is sized by
        columns per KV head)."""
        if not (q.dtype == k_pages.dtype == v_pages.dtype == out.dtype) or _dtype_code(q) == PKV_U8:
            raise TypeError("decode_multi: q, k_pages, v_pages and out must share dtype bf16 or float32")
        B, T, Hq, D = q.shape
        self._check_batch(B)
        if T != q_len or self.shape[1] != Hq * q_len:
            raise ValueError("q must be [B][q_len][Hq][D] and the Decoder built for Hq * q_len heads")
        check(lib.pkv_paged_decode_multi(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens),
                                         Hq, k_pages.shape[1], D, BLOCK_SIZE, q_len, window, float(scale), _ptr(out),
                                         _stream(stream), B, block_table.shape[1], k_pages.shape[0], _dtype_code(q),
                                         _ptr(self.workspace), self.workspace.numel(),
                                         _opts(self.n_items, self.min_chunk_pages, self.combine_mode, self.schedule)),
              "pkv_paged_decode_multi")
        return out

    def _q8_args(self, q, k_codes, v_codes, meta, block_table, seq_lens, scale, out, stream):
        import torch
        if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16 or k_codes.dtype != torch.uint8 or \
                v_codes.dtype != torch.uint8 or meta.dtype != torch.float32:
            raise TypeError("8-bit decode: q and out bf16, k_codes and v_codes uint8, meta float32")
        B, Hq, D = q.shape
        self._check_batch(B)
        return (_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(meta), _ptr(block_table), _ptr(seq_lens), Hq,
                k_codes.shape[1], D, BLOCK_SIZE, float(scale), _ptr(out), _stream(stream), B, block_table.shape[1],
                k_codes.shape[0], _ptr(self.workspace), self.workspace.numel(),
                _opts(self.n_items, self.min_chunk_pages, self.combine_mode, self.schedule))

    def attn_q8(self, q, k_codes, v_codes, meta, block_table, seq_lens, scale, out, stream=None):
        """Decode over the 8-bit cache (Decoder built with dtype=torch.uint8; q and out bf16)."""
        check(lib.pkv_paged_decode_attn_q8(*self._q8_args(q, k_codes, v_codes, meta, block_table, seq_lens, scale,
                                                          out, stream)), "pkv_paged_decode_attn_q8")
        return out

    def split_q8(self, q, k_codes, v_codes, meta, block_table, seq_lens, scale, out, stream=None):
        check(lib.pkv_paged_decode_split_q8(*self._q8_args(q, k_codes, v_codes, meta, block_table, seq_lens, scale,
                                                           out, stream)), "pkv_paged_decode_split_q8")

    def step_q8(self, q, k_new, v_new, k_codes, v_codes, meta, block_table, seq_lens, scale, out, stream=None):
        """Quantizing append at seq_lens - 1, then decode over the 8-bit cache."""
        a = self._q8_args(q, k_codes, v_codes, meta, block_table, seq_lens, scale, out, stream)
        check(lib.pkv_decode_step_q8(a[0], _ptr(k_new), _ptr(v_new), *a[1:]), "pkv_decode_step_q8")
        return out

    def counters(self):
        """(arrival counters [B][Hkv][4], chunk counter) int32 copies of the
        counters, which sit at the workspace's end counted backwards."""
        import torch
        B, Hq, Hkv, D = self.shape
        i = self.workspace.view(torch.int32)
        end = i.numel()
        n = B * Hkv * 4
        return i[end - 1 - n: end - 1].flip(0).view(B, Hkv, 4).clone(), i[end - 1].clone()

    def partials(self):
        """Views (partial_o [slots][G][D], partial_lse [slots][G]) into the workspace."""
        import torch
        B, Hq, Hkv, D = self.shape
        G = Hq // Hkv
        slots = self.n_items + B * Hkv
        f = self.workspace[: self.ws_bytes].view(torch.float32)
        return f[: slots * G * D].view(slots, G, D), f[slots * G * D: slots * G * (D + 1)].view(slots, G)


def paged_decode_attn(q, k_pages, v_pages, block_table, seq_lens, scale, out=None, n_items: int = 0,
                      min_chunk_pages: int = 0, stream=None):
    import torch
    if out is None:
        out = torch.empty_like(q)
    dec = Decoder(q.shape[0], q.shape[1], k_pages.shape[1], q.shape[2], q.dtype, block_table.shape[1], n_items,
                  min_chunk_pages, device=q.device)
    return dec(q, k_pages, v_pages, block_table, seq_lens, scale, out, stream)


def hbm_read_probe(buf, sink, n_blocks: int, stream=None) -> None:
    check(lib.pkv_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), n_blocks,
                                 _stream(stream)), "pkv_hbm_read_probe")


def copy_probe(dst, src, stream=None) -> None:
    check(lib.pkv_copy_probe(_ptr(dst), _ptr(src), src.numel() * src.element_size(), _stream(stream)),
          "pkv_copy_probe")


def launch_probe(mode: int, grid: int = 0, iters: int = 200, bar=None, stream=None) -> float:
    """Mean microseconds per launch of an empty kernel (see pkv_launch_probe):
    mode 0 ordinary, 1 cooperative, 2 cooperative with one grid-wide barrier
    in bar (device int32 [3], zeroed; allocated here when None)."""
    import ctypes
    if mode == 2 and bar is None:
        import torch
        bar = torch.zeros(3, dtype=torch.int32, device="cuda")
    us = ctypes.c_float(0.0)
    check(lib.pkv_launch_probe(int(mode), int(grid), int(iters), _ptr(bar) if bar is not None else None,
                               ctypes.byref(us), _stream(stream)), "pkv_launch_probe")
    return float(us.value)


def gather_probe(k_pages, v_pages, block_table, seq_lens, sink, n_items: int = 0, min_chunk_pages: int = 0,
                 stream=None) -> None:
    """The decode kernel's tile stream without arithmetic (see pkv_gather_probe),
    on pools in the library's layout, k_pages [P][Hkv][D/X][16][X]; sink:
    device int32 with at least n_items entries."""
    B = block_table.shape[0]
    Hkv = k_pages.shape[1]
    D = k_pages.shape[2] * k_pages.shape[4]
    check(lib.pkv_gather_probe(_ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), Hkv, D, B,
                               block_table.shape[1], k_pages.shape[0], _dtype_code(k_pages), 0, 0, int(n_items),
                               int(min_chunk_pages), _ptr(sink), sink.numel() * sink.element_size(), _stream(stream)),
          "pkv_gather_probe")


def gather_probe_q8(k_codes, v_codes, meta, block_table, seq_lens, sink, n_items: int = 0,
                    min_chunk_pages: int = 0, stream=None) -> None:
    """The 8-bit decode kernel's tile stream without arithmetic (see
    pkv_gather_probe_q8), on an 8-bit cache in the library's layout:
    k_codes [P][Hkv][16 * D] uint8 (any shape with P and Hkv leading), meta
    [P][Hkv][64] float32; sink: device int32 with at least n_items entries."""
    B = block_table.shape[0]
    P, Hkv = k_codes.shape[0], k_codes.shape[1]
    D = k_codes[0, 0].numel() // 16
    check(lib.pkv_gather_probe_q8(_ptr(k_codes), _ptr(v_codes), _ptr(meta), _ptr(block_table), _ptr(seq_lens), Hkv,
                                  D, B, block_table.shape[1], P, int(n_items), int(min_chunk_pages), _ptr(sink),
                                  sink.numel() * sink.element_size(), _stream(stream)),
          "pkv_gather_probe_q8")


def paged_decode_multi(q, k_pages, v_pages, block_table, seq_lens, q_len: int, scale, out, window: int = 0,
                       workspace=None, n_items: int = 0, min_chunk_pages: int = 0, stream=None):
    """pkv_paged_decode_multi: the last q_len cached tokens of each sequence
    attend causally (optional sliding window).  q, out: [B][q_len][Hq][D].
    Query tiles of more than 64 columns per KV head (q_len x Hq / Hkv) run the
    prefill kernel and need no workspace; smaller ones need one sized for
    Hq * q_len query heads (or use Decoder.attn_multi)."""
    B, T, Hq, D = q.shape
    if T != q_len:
        raise ValueError("q must be [B][q_len][Hq][D]")
    ws, ws_bytes = (0, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    check(lib.pkv_paged_decode_multi(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), Hq,
                                     k_pages.shape[1], D, BLOCK_SIZE, q_len, window, float(scale), _ptr(out),
                                     _stream(stream), B, block_table.shape[1], k_pages.shape[0], _dtype_code(q),
                                     ws or None, ws_bytes, _opts(n_items, min_chunk_pages, 0, 0)),
          "pkv_paged_decode_multi")
    return out
