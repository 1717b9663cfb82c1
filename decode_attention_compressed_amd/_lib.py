"""ctypes view of include/lowram.h.  Loads the in-tree liblowram.so and fails
loudly when it is missing: there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblowram.so")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = range(5)
F32, BF16, F16, I8 = range(4)
OP_COMPRESS, OP_DECODE, OP_EVICT, OP_DENSE, OP_REPACK, OP_FIT, OP_BASIS = range(7)
NOALLOC_SCRATCH_BYTES = 32 << 20   # LOWRAM_NOALLOC_SCRATCH_BYTES

DIM_FIELDS = ("batch", "layers", "heads_q", "heads_kv", "head_dim", "rank", "hidden", "n_ctx",
              "chunk", "top_k", "n_tail", "n_res", "act", "coeff", "resid")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in DIM_FIELDS]

    def as_dict(self):
        return {n: getattr(self, n) for n in DIM_FIELDS}


class Model(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("basis", "w1", "b1", "w2", "b2")]


class Cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("coeff", "coeff_scale", "landmark", "res_ptr", "res_idx", "res_val", "res_scale")]


class Predictor(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "b1", "w2", "b2")]


class Reuse(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_void_p), ("slot_chunk", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("clock", ctypes.c_void_p), ("slots", ctypes.c_int32)]


class LowramError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lowram status {status}: {msg}")
        self.status = status
        self.msg = msg


_lib = None

P = ctypes.POINTER
vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64

SIGNATURES = {
    "lowram_workspace_bytes": [P(Dims), i32, P(sz)],
    "lowram_cache_bytes": [P(Dims), P(ctypes.c_uint64), P(ctypes.c_uint64)],
    "lowram_decode_kernel": [P(Dims), P(i32)],
    "lowram_compress": [P(Dims), P(Model), vp, vp, P(Cache), vp, sz, vp],
    "lowram_decode_attn": [P(Dims), i32, P(Model), P(Cache), vp, vp, vp, vp, vp, vp, sz, vp],
    "lowram_decode_select": [P(Dims), i32, P(Model), P(Cache), vp, vp, vp, sz, vp],
    "lowram_decode_attend": [P(Dims), i32, P(Model), P(Cache), vp, vp, vp, vp, sz, vp],
    "lowram_decode_combine": [P(Dims), i32, P(Model), vp, vp, sz, vp],
    "lowram_evict": [P(Dims), P(Model), P(Cache), vp, i32, i32, i32, P(Cache), vp, vp, vp, sz, vp],
    "lowram_repack": [P(Dims), P(Model), P(Cache), vp, vp, i32, P(Cache), vp, sz, vp],
    "lowram_fit_predictor": [P(Dims), P(Model), vp, vp, i32, ctypes.c_float, P(Predictor), vp, vp, sz, vp],
    "lowram_key_basis": [P(Dims), vp, i32, vp, vp, sz, vp],
    "lowram_reuse_tile_bytes": [P(Dims), P(sz)],
    "lowram_decode_attn_noalloc": [P(Dims), i32, P(Model), P(Cache), vp, vp, vp, vp, vp, vp],
    "lowram_decode_attn_reuse": [P(Dims), i32, P(Model), P(Cache), vp, vp, vp, vp, vp, P(Reuse), vp, vp, sz, vp],
    "lowram_dense_decode_attn": [P(Dims), vp, vp, vp, i32, i64, vp, vp, sz, vp],
    "lowram_status_string": [i32],
    "lowram_last_error": [],
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                              "or `python decode_attention_compressed_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("lowram_status_string", "lowram_last_error") else ctypes.c_int
        _lib = L
    return _lib


def check(status: int):
    if status != OK:
        raise LowramError(status, lib().lowram_last_error().decode())
