"""ctypes loader for libpkv.so.  Importing this module fails loudly if the
library has not been built: there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_OUT_OF_PAGES = -3
PKV_ERR_WORKSPACE = -4
PKV_ERR_HIP = -5
PKV_ERR_NOT_FOUND = -6
PKV_ERR_EXISTS = -7
PKV_F32 = 0
PKV_BF16 = 1
PKV_U8 = 2
PKV_SCHEDULE_AUTO = 0
PKV_SCHEDULE_STATIC = 1
PKV_SCHEDULE_DYNAMIC = 2


class PkvError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


class DecodeOpts(ctypes.Structure):
    _fields_ = [("n_items", ctypes.c_int32), ("min_chunk_pages", ctypes.c_int32),
                ("combine_mode", ctypes.c_int32), ("schedule", ctypes.c_int32)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                      " or `python paged_kv_cache_254_amd/build.py`")

# One HIP runtime per process: torch ships its own libamdhip64 (same SONAME as
# the system one libpkv.so links against).  Loading torch first makes the
# dynamic loader satisfy libpkv.so's dependency with torch's already-loaded
# runtime, so device pointers and streams from torch are valid in the library.
try:
    import torch  # noqa: F401
except ImportError:
    pass

lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _u64, _f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                    ctypes.c_void_p, ctypes.c_size_t)
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)

SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_kv_cache_bytes": (_u64, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "pkv_kv_bytes_per_token": (_u64, [_i64, _i64, _i64, _i64]),
    "pkv_pool_create": (ctypes.c_int, [_i32, _pi32, ctypes.POINTER(_vp)]),
    "pkv_pool_destroy": (None, [_vp]),
    "pkv_pool_num_free": (_i32, [_vp]),
    "pkv_seq_reserve": (ctypes.c_int, [_vp, _i64, _i64, _i32, _pi32]),
    "pkv_seq_release": (ctypes.c_int, [_vp, _i64]),
    "pkv_seq_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "pkv_seq_reserve_for_write": (ctypes.c_int, [_vp, _i64, _i64, _i32, _pi32, _pi32]),
    "pkv_seq_num_blocks": (ctypes.c_int, [_vp, _i64, _pi32]),
    "pkv_build_block_table": (ctypes.c_int, [_vp, _pi64, _i32, _i32, _pi32]),
    "pkv_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _vp]),
    "pkv_paged_decode_attn": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                             _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                             ctypes.POINTER(DecodeOpts)]),
    "pkv_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                       _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                       ctypes.POINTER(DecodeOpts)]),
    "pkv_decode_step_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                               _vp, _vp, _i32, _i32, _i32, _i32, ctypes.POINTER(DecodeOpts)]),
    "pkv_decode_step_split": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                             _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                             ctypes.POINTER(DecodeOpts)]),
    "pkv_paged_decode_split": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                              _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                              ctypes.POINTER(DecodeOpts)]),
    "pkv_lse_combine": (ctypes.c_int, [_vp, _sz, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32,
                                       ctypes.POINTER(DecodeOpts), _vp]),
    "pkv_decode_workspace_bytes": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_resolve": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(DecodeOpts),
                                          ctypes.POINTER(DecodeOpts), ctypes.POINTER(ctypes.c_int64)]),
    "pkv_decode_plan": (ctypes.c_int, [_pi32, _i32, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32, _pi32]),
    "pkv_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_decode_multi": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                              _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                              ctypes.POINTER(DecodeOpts)]),
    "pkv_kv_append_q8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _vp]),
    "pkv_paged_decode_attn_q8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                                _vp, _vp, _i32, _i32, _i32, _vp, _sz,
                                                ctypes.POINTER(DecodeOpts)]),
    "pkv_paged_decode_split_q8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                                 _vp, _vp, _i32, _i32, _i32, _vp, _sz,
                                                 ctypes.POINTER(DecodeOpts)]),
    "pkv_decode_step_q8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _f32, _vp, _vp, _i32, _i32, _i32, _vp, _sz,
                                          ctypes.POINTER(DecodeOpts)]),
    "pkv_hbm_read_probe": (ctypes.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "pkv_copy_probe": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "pkv_launch_probe": (ctypes.c_int, [_i32, _i32, _i32, _vp, _vp, _vp]),
    "pkv_gather_probe": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _i32,
                                        _i32, _vp, _sz, _vp]),
    "pkv_gather_probe_q8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                                           _sz, _vp]),
}

for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def check(status: int, fn: str) -> int:
    if status < 0:
        raise PkvError(status, fn, lib.pkv_last_error().decode())
    return status
