"""Paged GQA decode attention for MI355X (gfx950): a HIP library behind a C
ABI (``include/pkv.h``) with this thin Python binding.

Importing the package loads ``libpkv.so``; it raises ImportError if the
library has not been built, and there is no CPU or PyTorch fallback.
"""
from ._lib import (LIB_PATH, PKV_BF16, PKV_F32, PKV_SCHEDULE_AUTO, PKV_SCHEDULE_DYNAMIC,  # noqa: F401
                   PKV_SCHEDULE_STATIC, PKV_U8, PkvError, lib)
from .ops import (BLOCK_SIZE, Decoder, PagePool, copy_blocks, copy_probe, decode_resolve,  # noqa: F401
                  decode_plan, decode_workspace_bytes, gather_probe, gather_probe_q8, hbm_read_probe, kv_append,
                  kv_append_q8, kv_append_tokens, launch_probe, q8_pool_shapes,
                  kv_bytes_per_token, kv_cache_bytes, paged_decode_attn, paged_decode_multi)

__version__ = lib.pkv_version().decode()
