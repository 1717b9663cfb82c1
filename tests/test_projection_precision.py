"""Why the compress projection (C1) runs in float64 (CPU only).

On a llama8b-32k-shaped sample (bf16 keys of 4 layers x 8 kv heads on the
group's bf16 basis, 2048 tokens, r = 512), an fp32 accumulation of the exact
bf16 products in the matrix cores' 32-wide blocks puts some stored bf16
coefficients more than one bf16 ulp from the rounding of the float64 sum (the
stage-isolated parity bar), all of them in trailing ranks.  A rounding-error
bound per coefficient (gamma * sum |k_d u_d|) straddles a bf16 rounding
boundary for nearly every coefficient, so a certified fp32 pass with a float64
recompute of the flagged ones would recompute nearly everything.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
torch = pytest.importorskip("torch")
from synth import gen  # noqa: E402
from synth.configs import LLAMA8B_32K, small  # noqa: E402


def _bf16(x):
    """Round float64 values to bf16 (nearest even) and back."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _from_bits(u):
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_fp32_projection_misses_the_one_ulp_bar_and_certification_flags_most():
    s = small(LLAMA8B_32K, B=1, N=2048)
    inp = gen.make(s, steps=1)
    k = _from_bits(inp["k"][0])                       # [G][Hkv][N][dh]
    kb = k.transpose(2, 0, 1, 3).reshape(s.N, -1)     # [N][D], D index (l, h, d)
    U = _from_bits(inp["basis"][0])                   # [D][r]
    c64 = kb @ U
    c32 = np.zeros(c64.shape, np.float32)
    for k0 in range(0, kb.shape[1], 32):              # exact bf16 products, fp32 block sums
        c32 = (c32 + (kb[:, k0:k0 + 32] @ U[k0:k0 + 32]).astype(np.float32)).astype(np.float32)
    r64, r32 = _bf16(c64), _bf16(c32.astype(np.float64))
    step = np.abs(_bf16(np.abs(c64) * (1 + 2.0 ** -8)) - np.abs(r64))   # one bf16 ulp at each value
    step = np.where(step == 0, np.abs(r64) * 2.0 ** -7, step)
    off = np.abs(r32 - r64) > 1.01 * step
    assert off.mean() > 1e-3                          # measured 0.34%
    ranks = np.nonzero(off)[1]
    assert np.median(ranks) > 128                     # trailing ranks (measured median 293 of 512)
    S = np.abs(kb) @ np.abs(U)
    E = (kb.shape[1] // 32 + 32) * 2.0 ** -24 * S     # 160 roundings along the chain
    lo, hi = _bf16(c32.astype(np.float64) - E), _bf16(c32.astype(np.float64) + E)
    flagged = lo != hi
    assert flagged.mean() > 0.5                       # measured 93%
    assert not np.any(~flagged & (r32 != r64))        # the bound itself is sound here
