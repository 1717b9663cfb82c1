"""Torch-facing binding of the lowram C ABI (argument marshalling only).

Every computation runs in the HIP library; torch provides device memory and
the current stream.  Shapes and dtypes are checked here so that mistakes
surface as Python exceptions, and the library re-validates everything.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib as L
from ._lib import LowramError  # noqa: F401  (re-export)

TORCH_DT = {L.F32: torch.float32, L.BF16: torch.bfloat16, L.I8: torch.int8}
NAME_DT = {"f32": L.F32, "bf16": L.BF16, "i8": L.I8, "f16": L.F16}


def make_dims(batch, layers, heads_q, heads_kv, head_dim, rank, hidden, n_ctx, chunk, top_k,
              n_tail, n_res, act="bf16", coeff="bf16", resid="bf16") -> L.Dims:
    d = L.Dims()
    vals = dict(batch=batch, layers=layers, heads_q=heads_q, heads_kv=heads_kv, head_dim=head_dim,
                rank=rank, hidden=hidden, n_ctx=n_ctx, chunk=chunk, top_k=top_k, n_tail=n_tail,
                n_res=n_res, act=NAME_DT.get(act, act), coeff=NAME_DT.get(coeff, coeff),
                resid=NAME_DT.get(resid, resid))
    for k, v in vals.items():
        setattr(d, k, int(v))
    return d


def with_(d: L.Dims, **kw) -> L.Dims:
    vals = d.as_dict()
    vals.update(kw)
    out = L.Dims()
    for k, v in vals.items():
        setattr(out, k, int(v))
    return out


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def n_chunks(d: L.Dims) -> int:
    return d.n_ctx // d.chunk


def k_eff(d: L.Dims) -> int:
    return min(d.top_k, n_chunks(d))


def workspace_bytes(d: L.Dims, op: int) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.lib().lowram_workspace_bytes(ctypes.byref(d), op, ctypes.byref(n)))
    return n.value


def workspace(d: L.Dims, op: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(1, workspace_bytes(d, op)), dtype=torch.uint8, device=device)


DECODE_KERNELS = {0: "none", 1: "chain", 2: "mfma", 3: "valu", 4: "absorb"}


def decode_kernel(d: L.Dims) -> str:
    """Which rebuild-and-attend kernel decode calls with dims d run:
    "chain", "absorb", "mfma", "valu" or "none" (no chunk selected)."""
    p = ctypes.c_int32(-1)
    L.check(L.lib().lowram_decode_kernel(ctypes.byref(d), ctypes.byref(p)))
    return DECODE_KERNELS[p.value]


def cache_bytes(d: L.Dims):
    c, dn = ctypes.c_uint64(0), ctypes.c_uint64(0)
    L.check(L.lib().lowram_cache_bytes(ctypes.byref(d), ctypes.byref(c), ctypes.byref(dn)))
    return c.value, dn.value


def cache_shapes(d: L.Dims) -> dict:
    B, G, H, dh, r, N, C = d.batch, d.layers, d.heads_kv, d.head_dim, d.rank, d.n_ctx, d.chunk
    n_c = N // C
    shapes = {
        "coeff": ((B, N, r), TORCH_DT[d.coeff]),
        "landmark": ((B, n_c, r), torch.float32),
        "res_ptr": ((B, G, H, n_c + 1), torch.int32),
        "res_idx": ((B, G, H, max(d.n_res, 0)), torch.int32),
        "res_val": ((B, G, H, max(d.n_res, 0), dh), TORCH_DT[d.resid]),
    }
    if d.coeff == L.I8:
        shapes["coeff_scale"] = ((B, r), torch.float16)
    if d.resid == L.I8:
        shapes["res_scale"] = ((B, G, H, dh), torch.float16)
    return shapes


def alloc_cache(d: L.Dims, device="cuda") -> dict:
    return {k: torch.zeros(s, dtype=t, device=device) for k, (s, t) in cache_shapes(d).items()}


def cache_struct(d: L.Dims, c: dict) -> L.Cache:
    s = L.Cache()
    for k, (shape, dt) in cache_shapes(d).items():
        setattr(s, k, _ptr(c[k], dt, shape, k).value if c.get(k) is not None else None)
    return s


def model_shapes(d: L.Dims) -> dict:
    B, G, H, dh, r, F = d.batch, d.layers, d.heads_kv, d.head_dim, d.rank, d.hidden
    D = G * H * dh
    return {"basis": (B, D, r), "w1": (B, G, H, F, dh), "b1": (B, G, H, F),
            "w2": (B, G, H, dh, F), "b2": (B, G, H, dh)}


def model_struct(d: L.Dims, m: dict) -> L.Model:
    s = L.Model()
    dt = TORCH_DT[d.act]
    for k, shape in model_shapes(d).items():
        setattr(s, k, _ptr(m[k], dt, shape, k).value)
    return s


# ---------------------------------------------------------------------------
def compress(d: L.Dims, model: dict, k, v, cache: dict, ws=None, stream=None):
    dt = TORCH_DT[d.act]
    kv_shape = (d.batch, d.layers, d.heads_kv, d.n_ctx, d.head_dim)
    ws = workspace(d, L.OP_COMPRESS, k.device) if ws is None else ws
    L.check(L.lib().lowram_compress(ctypes.byref(d), ctypes.byref(model_struct(d, model)),
                                    _ptr(k, dt, kv_shape, "k"), _ptr(v, dt, kv_shape, "v"),
                                    ctypes.byref(cache_struct(d, cache)), _ptr(ws, torch.uint8),
                                    ws.numel(), _stream(stream)))
    return cache


def _decode_common(d, q, k_tail, v_tail):
    dt = TORCH_DT[d.act]
    qp = _ptr(q, dt, (d.batch, d.heads_q, d.head_dim), "q")
    tail_shape = (d.batch, d.layers, d.heads_kv, d.n_tail, d.head_dim)
    kt = _ptr(k_tail, dt, tail_shape, "k_tail") if d.n_tail else None
    vt = _ptr(v_tail, dt, tail_shape, "v_tail") if d.n_tail else None
    return qp, kt, vt


def decode_attn(d: L.Dims, layer: int, model: dict, cache: dict, q, k_tail, v_tail, out=None,
                sel_out=None, ws=None, stream=None):
    qp, kt, vt = _decode_common(d, q, k_tail, v_tail)
    out = torch.empty_like(q) if out is None else out
    ws = workspace(d, L.OP_DECODE, q.device) if ws is None else ws
    sp = _ptr(sel_out, torch.int32, (d.batch, d.heads_kv, k_eff(d)), "sel_out")
    L.check(L.lib().lowram_decode_attn(ctypes.byref(d), layer, ctypes.byref(model_struct(d, model)),
                                       ctypes.byref(cache_struct(d, cache)), qp, kt, vt,
                                       _ptr(out, TORCH_DT[d.act], tuple(q.shape), "out"), sp,
                                       _ptr(ws, torch.uint8), ws.numel(), _stream(stream)))
    return out


def reuse_tile_bytes(d: L.Dims) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.lib().lowram_reuse_tile_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def alloc_reuse(d: L.Dims, slots: int, device="cuda") -> dict:
    """A fresh reuse table: slot_chunk -1 (both halves), stamps and clocks 0."""
    B, G, H = d.batch, d.layers, d.heads_kv
    return {"tiles": torch.empty((B, G, H, slots, reuse_tile_bytes(d)), dtype=torch.uint8, device=device),
            "slot_chunk": torch.full((B, G, H, 2, slots), -1, dtype=torch.int32, device=device),
            "slot_stamp": torch.zeros((B, G, H, 2, slots), dtype=torch.int32, device=device),
            "clock": torch.zeros((B, G, H), dtype=torch.int32, device=device), "slots": slots}


def reuse_current(r: dict):
    """(slot_chunk, slot_stamp) of each head's current half, [B][G][Hkv][slots], on the host."""
    clock = r["clock"].cpu().numpy()
    half = (clock & 1)[..., None, None]
    ch = np.take_along_axis(r["slot_chunk"].cpu().numpy(), half, axis=3)[:, :, :, 0]
    st = np.take_along_axis(r["slot_stamp"].cpu().numpy(), half, axis=3)[:, :, :, 0]
    return ch, st


def reuse_struct(d: L.Dims, r: dict) -> L.Reuse:
    B, G, H, S = d.batch, d.layers, d.heads_kv, r["slots"]
    s = L.Reuse()
    s.tiles = _ptr(r["tiles"], torch.uint8, (B, G, H, S, reuse_tile_bytes(d)), "tiles").value
    s.slot_chunk = _ptr(r["slot_chunk"], torch.int32, (B, G, H, 2, S), "slot_chunk").value
    s.slot_stamp = _ptr(r["slot_stamp"], torch.int32, (B, G, H, 2, S), "slot_stamp").value
    s.clock = _ptr(r["clock"], torch.int32, (B, G, H), "clock").value
    s.slots = S
    return s


def decode_attn_reuse(d: L.Dims, layer: int, model: dict, cache: dict, q, k_tail, v_tail, reuse: dict,
                      out=None, sel_out=None, hits_out=None, ws=None, stream=None):
    qp, kt, vt = _decode_common(d, q, k_tail, v_tail)
    out = torch.empty_like(q) if out is None else out
    ws = workspace(d, L.OP_DECODE, q.device) if ws is None else ws
    sp = _ptr(sel_out, torch.int32, (d.batch, d.heads_kv, k_eff(d)), "sel_out")
    hp = _ptr(hits_out, torch.int32, (d.batch, d.heads_kv), "hits_out")
    L.check(L.lib().lowram_decode_attn_reuse(ctypes.byref(d), layer, ctypes.byref(model_struct(d, model)),
                                             ctypes.byref(cache_struct(d, cache)), qp, kt, vt,
                                             _ptr(out, TORCH_DT[d.act], tuple(q.shape), "out"), sp,
                                             ctypes.byref(reuse_struct(d, reuse)), hp, _ptr(ws, torch.uint8),
                                             ws.numel(), _stream(stream)))
    return out


class DecodeCall:
    """Pre-marshalled arguments of one decode call, for tight loops and timing:
    the three stages can be issued separately on the current stream."""

    def __init__(self, d, layer, model, cache, q, k_tail, v_tail, out, ws, sel_out=None):
        self.d = d
        self.layer = layer
        self.qp, self.kt, self.vt = _decode_common(d, q, k_tail, v_tail)
        self.mp = model_struct(d, model)
        self.cp = cache_struct(d, cache)
        self.op = _ptr(out, TORCH_DT[d.act], tuple(q.shape), "out")
        self.sp = _ptr(sel_out, torch.int32, (d.batch, d.heads_kv, k_eff(d)), "sel_out")
        self.wp = _ptr(ws, torch.uint8)
        self.wn = ws.numel()
        self._keep = (q, k_tail, v_tail, out, ws, sel_out, model, cache)

    def select(self, stream=None):
        L.check(L.lib().lowram_decode_select(ctypes.byref(self.d), self.layer, ctypes.byref(self.mp),
                                             ctypes.byref(self.cp), self.qp, self.sp, self.wp, self.wn,
                                             _stream(stream)))

    def attend(self, stream=None):
        L.check(L.lib().lowram_decode_attend(ctypes.byref(self.d), self.layer, ctypes.byref(self.mp),
                                             ctypes.byref(self.cp), self.qp, self.kt, self.vt, self.wp,
                                             self.wn, _stream(stream)))

    def combine(self, stream=None):
        L.check(L.lib().lowram_decode_combine(ctypes.byref(self.d), self.layer, ctypes.byref(self.mp),
                                              self.op, self.wp, self.wn, _stream(stream)))

    def __call__(self, stream=None):
        L.check(L.lib().lowram_decode_attn(ctypes.byref(self.d), self.layer, ctypes.byref(self.mp),
                                           ctypes.byref(self.cp), self.qp, self.kt, self.vt, self.op,
                                           self.sp, self.wp, self.wn, _stream(stream)))


def evict(d: L.Dims, model: dict, src: dict, obs_q, keep: int, dst=None, keep_out=None, ws=None,
          stream=None, n_res=None):
    """Returns (dst cache, dims of the evicted cache, keep indices).

    The evicted cache holds n_res residual rows per (b, layer, kv head).  By
    default that is the largest number the kept chunks of any head carry: a
    first library call reports the rows per head (dst NULL), the host reads
    them (one stream synchronisation, once per context) and the second call
    fills a cache of that size.  Pass n_res to skip the first call."""
    dt = TORCH_DT[d.act]
    n_obs = 0 if obs_q is None else obs_q.shape[0]
    dev = src["coeff"].device
    ws = workspace(d, L.OP_EVICT, dev) if ws is None else ws
    qp = _ptr(obs_q, dt, (n_obs, d.batch, d.layers, d.heads_q, d.head_dim), "obs_q") if n_obs else None
    keep_out = torch.empty((d.batch, keep), dtype=torch.int32, device=dev) if keep_out is None else keep_out
    kp = _ptr(keep_out, torch.int32, (d.batch, keep), "keep_out")
    if n_res is None:
        live = torch.empty((d.batch, d.layers, d.heads_kv), dtype=torch.int32, device=dev)
        L.check(L.lib().lowram_evict(ctypes.byref(d), ctypes.byref(model_struct(d, model)),
                                     ctypes.byref(cache_struct(d, src)), qp, n_obs, keep, 0, None, kp,
                                     _ptr(live, torch.int32, None, "live"), _ptr(ws, torch.uint8),
                                     ws.numel(), _stream(stream)))
        n_res = int(live.max().item())
    d2 = with_(d, n_ctx=keep * d.chunk, n_res=n_res)
    if dst is None:
        dst = alloc_cache(d2, dev)
        if d.coeff == L.I8:
            dst["coeff_scale"] = src["coeff_scale"]
        if d.resid == L.I8:
            dst["res_scale"] = src["res_scale"]
    L.check(L.lib().lowram_evict(ctypes.byref(d), ctypes.byref(model_struct(d, model)),
                                 ctypes.byref(cache_struct(d, src)), qp, n_obs, keep, n_res,
                                 ctypes.byref(cache_struct(d2, dst)), kp, None,
                                 _ptr(ws, torch.uint8), ws.numel(), _stream(stream)))
    return dst, d2, keep_out


def repack(d: L.Dims, model: dict, src: dict, k_tail, v_tail, n_new_res: int, dst=None, ws=None,
           stream=None):
    """Move the oldest d.chunk tail tokens into the cache as one new chunk.
    Returns (dst cache, its dims: n_ctx + chunk, n_res + n_new_res, n_tail - chunk)."""
    dt = TORCH_DT[d.act]
    d2 = with_(d, n_ctx=d.n_ctx + d.chunk, n_res=d.n_res + n_new_res, n_tail=d.n_tail - d.chunk)
    dev = k_tail.device
    if dst is None:
        dst = alloc_cache(d2, dev)
        if d.coeff == L.I8:
            dst["coeff_scale"] = src["coeff_scale"]
        if d.resid == L.I8:
            dst["res_scale"] = src["res_scale"]
    ws = workspace(d, L.OP_REPACK, dev) if ws is None else ws
    tail_shape = (d.batch, d.layers, d.heads_kv, d.n_tail, d.head_dim)
    L.check(L.lib().lowram_repack(ctypes.byref(d), ctypes.byref(model_struct(d, model)),
                                  ctypes.byref(cache_struct(d, src)),
                                  _ptr(k_tail, dt, tail_shape, "k_tail"),
                                  _ptr(v_tail, dt, tail_shape, "v_tail"), n_new_res,
                                  ctypes.byref(cache_struct(d2, dst)), _ptr(ws, torch.uint8),
                                  ws.numel(), _stream(stream)))
    return dst, d2


def fit_predictor(d: L.Dims, model: dict, k, v, steps: int, lr: float, out=None, with_loss=True,
                  ws=None, stream=None):
    """Fit the value predictor by gradient descent on the context (k, v).
    Returns (weights dict with w1, b1, w2, b2 in act dtype, loss [B][G][Hkv][steps+1]
    float64 or None).  out may be the model dict itself (in-place update)."""
    dt = TORCH_DT[d.act]
    dev = k.device
    shapes = model_shapes(d)
    if out is None:
        out = {n: torch.empty(shapes[n], dtype=dt, device=dev) for n in ("w1", "b1", "w2", "b2")}
    loss = (torch.empty((d.batch, d.layers, d.heads_kv, steps + 1), dtype=torch.float64, device=dev)
            if with_loss else None)
    pr = L.Predictor()
    for n in ("w1", "b1", "w2", "b2"):
        setattr(pr, n, _ptr(out[n], dt, shapes[n], n).value)
    ws = workspace(d, L.OP_FIT, dev) if ws is None else ws
    kv_shape = (d.batch, d.layers, d.heads_kv, d.n_ctx, d.head_dim)
    L.check(L.lib().lowram_fit_predictor(ctypes.byref(d), ctypes.byref(model_struct(d, model)),
                                         _ptr(k, dt, kv_shape, "k"), _ptr(v, dt, kv_shape, "v"),
                                         int(steps), float(lr), ctypes.byref(pr),
                                         _ptr(loss, torch.float64, None, "loss"), _ptr(ws, torch.uint8),
                                         ws.numel(), _stream(stream)))
    return out, loss


def key_basis(d: L.Dims, k, iterations: int = 8, out=None, ws=None, stream=None):
    """The group key basis [B][D][r] (act dtype) from the prefill keys k."""
    dt = TORCH_DT[d.act]
    D = d.layers * d.heads_kv * d.head_dim
    out = torch.empty((d.batch, D, d.rank), dtype=dt, device=k.device) if out is None else out
    ws = workspace(d, L.OP_BASIS, k.device) if ws is None else ws
    kv_shape = (d.batch, d.layers, d.heads_kv, d.n_ctx, d.head_dim)
    L.check(L.lib().lowram_key_basis(ctypes.byref(d), _ptr(k, dt, kv_shape, "k"), int(iterations),
                                     _ptr(out, dt, (d.batch, D, d.rank), "basis"), _ptr(ws, torch.uint8),
                                     ws.numel(), _stream(stream)))
    return out


def dense_workspace(d: L.Dims, n_tokens: int, device="cuda") -> torch.Tensor:
    return workspace(with_(d, n_ctx=n_tokens), L.OP_DENSE, device)


def dense_decode_attn(d: L.Dims, q, k_all, v_all, layer: int, out=None, ws=None, stream=None):
    """Uncompressed decode attention at `layer` over a dense cache k_all / v_all
    of shape [B][G][Hkv][n][dh] (n tokens per sequence)."""
    dt = TORCH_DT[d.act]
    B, G, H, n, dh = k_all.shape
    if (B, H, dh) != (d.batch, d.heads_kv, d.head_dim) or not 0 <= layer < G:
        raise ValueError("dense cache shape does not match dims / layer")
    for name, t in (("k_all", k_all), ("v_all", v_all)):
        _ptr(t, dt, (B, G, H, n, dh), name)
    off = layer * H * n * dh * k_all.element_size()
    out = torch.empty_like(q) if out is None else out
    ws = dense_workspace(d, n, q.device) if ws is None else ws
    L.check(L.lib().lowram_dense_decode_attn(ctypes.byref(d), _ptr(q, dt, (B, d.heads_q, dh), "q"),
                                             ctypes.c_void_p(k_all.data_ptr() + off),
                                             ctypes.c_void_p(v_all.data_ptr() + off), n, G * H * n * dh,
                                             _ptr(out, dt, tuple(q.shape), "out"),
                                             _ptr(ws, torch.uint8), ws.numel(), _stream(stream)))
    return out
