"""MI355X (gfx950) compressed-KV decode attention: LowRAM's decode-step hot path.

The HIP library (liblowram.so, C ABI in include/lowram.h) does all the work;
this package marshals torch tensors into it.
"""
from . import _lib
from ._lib import LowramError
from .api import (DecodeCall, alloc_cache, alloc_reuse, cache_bytes, compress, decode_attn, decode_attn_reuse,
                  decode_kernel, reuse_current, reuse_tile_bytes,
                  dense_decode_attn, dense_workspace, evict, fit_predictor, k_eff, key_basis, make_dims, repack, with_, workspace,
                  workspace_bytes)

__all__ = ["DecodeCall", "LowramError", "alloc_cache", "alloc_reuse", "cache_bytes", "compress", "decode_attn",
           "decode_attn_reuse", "reuse_current", "reuse_tile_bytes",
           "decode_kernel", "dense_decode_attn", "dense_workspace", "evict", "fit_predictor", "k_eff", "key_basis", "make_dims", "repack", "with_",
           "workspace", "workspace_bytes", "_lib"]
