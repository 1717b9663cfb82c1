"""Glue between the seeded generator, the oracle and the HIP library in tests:
numpy stored arrays <-> torch device tensors, and shape -> lowram dims."""
from __future__ import annotations

import os

import numpy as np
import torch

from synth.configs import BF16, F32, I8, Shape

NP_TO_TORCH = {np.float32: torch.float32, np.float16: torch.float16, np.int8: torch.int8,
               np.int32: torch.int32}


def dims_of(s: Shape, top_k: int | None = None, n_ctx: int | None = None, n_res: int | None = None):
    from decode_attention_compressed_amd import make_dims
    return make_dims(s.B, s.G, s.Hq, s.Hkv, s.dh, s.r, s.F, s.N if n_ctx is None else n_ctx, s.C,
                     s.k if top_k is None else top_k, s.T, s.n_res if n_res is None else n_res,
                     s.act, s.coeff, s.resid)


def to_dev(a: np.ndarray, tag: str | None = None, device="cuda") -> torch.Tensor:
    """Stored numpy array -> device tensor.  uint16 arrays hold bf16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 and tag != "f16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> stored numpy array (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(inp: dict, keys=("k", "v", "k_tail", "v_tail", "basis", "w1", "b1", "w2", "b2", "q")) -> dict:
    return {k: to_dev(inp[k]) for k in keys if k in inp}


def model_of(dev: dict) -> dict:
    return {k: dev[k] for k in ("basis", "w1", "b1", "w2", "b2")}


def cache_to_host(cache: dict) -> dict:
    return {k: (to_host(v) if v is not None else None) for k, v in cache.items()}


def f32_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


#: worst |gpu - oracle| / tolerance seen by each test (printed at the end of a run)
MARGINS: dict = {}


def within_tol(gpu: np.ndarray, ref: np.ndarray, atol=2e-3, rtol=1e-2):
    """|gpu - oracle| <= atol + rtol * |oracle| elementwise.  Returns (ok, worst
    ratio |gpu - oracle| / (atol + rtol |oracle|)); ok means the ratio is <= 1.
    The ratio is also recorded under the running test's name."""
    ratio = float(np.max(np.abs(gpu - ref) / (atol + rtol * np.abs(ref))))
    name = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" (")[0]
    MARGINS[name] = max(MARGINS.get(name, 0.0), ratio)
    return ratio <= 1.0, ratio


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """ulps between two bf16 bit arrays of the same sign-magnitude ordering."""
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), u + 0x8000)
    return np.abs(ordered(a) - ordered(b))
