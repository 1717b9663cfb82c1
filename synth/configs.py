"""Workload shapes for compressed-KV decode attention.

Each shape is one xKV group of G adjacent layers over B sequences.  The five
named workloads follow the shapes the LowRAM pages evaluate on (Mistral-7B,
Llama-3.1-8B and Qwen3.5-4B class heads; "Качество проверяли..." section of
the rit.work LowRAM page) with synthetic data standing in for RULER and
LongBench.  Fields a workload leaves open inherit from the Llama-8B shape.

This module only describes sizes.  It holds no arithmetic of the method.
"""
from __future__ import annotations

import dataclasses
import math

#: storage dtype tags shared by the generator, the oracle and the binding
F64, F32, BF16, F16, I8 = "f64", "f32", "bf16", "f16", "i8"


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    cfg_id: int          # seeds the generator
    B: int               # sequences
    G: int               # layers per xKV group
    Hq: int              # query heads
    Hkv: int             # KV heads
    dh: int              # head dim
    r: int               # rank of the group basis
    F: int               # predictor hidden width
    N: int               # compressed (prefill) tokens
    C: int               # chunk length
    k: int               # chunks selected per KV head each step
    T: int               # uncompressed tail tokens
    rho: float           # residual fraction
    act: str = BF16      # q, out, K, V, tail, basis, predictor weights
    coeff: str = BF16    # coefficient storage
    resid: str = BF16    # residual storage
    steps: int = 64      # decode steps of the workload
    outlier_frac: float = 0.0   # fraction of tokens with x20 value noise
    evict_keep: float = 1.0     # fraction of chunks kept by eviction
    n_obs: int = 0              # observation queries per (b, layer) for eviction
    key_cols: int = 0           # 0: all D spectrum columns drawn
    key_scale: float = 1.0      # keys drawn with this standard deviation per element
    q_scale: float = 1.0        # queries drawn with this standard deviation per element
    w1_scale: float = 1.0       # factor on the value model's first layer (and so on the predictor's)

    # ----- derived sizes -------------------------------------------------
    @property
    def D(self) -> int:
        return self.G * self.Hkv * self.dh

    @property
    def n_c(self) -> int:
        return self.N // self.C

    @property
    def n_res(self) -> int:
        # residual count per (b, l, h): the top fraction rounded up
        return min(self.N, int(math.ceil(self.rho * self.N - 1e-9)))

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def m_cols(self) -> int:
        """Spectrum columns the key generator draws (0.9**320 < 1e-14)."""
        if self.key_cols:
            return min(self.key_cols, self.D)
        return self.D if self.D < 2048 else 320

    @property
    def keep_chunks(self) -> int:
        return self.n_c if self.evict_keep >= 1.0 else int(math.floor(self.evict_keep * self.n_c))

    @property
    def N_after(self) -> int:
        return self.keep_chunks * self.C

    @property
    def k_eff(self) -> int:
        return min(self.k, self.keep_chunks)

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


TINY = Shape("tiny-fp32", 0, B=1, G=2, Hq=4, Hkv=2, dh=64, r=32, F=128, N=1024, C=64,
             k=4, T=16, rho=0.25, act=F32, coeff=F32, resid=F32, steps=8)
LLAMA8B_32K = Shape("llama8b-32k", 1, B=4, G=4, Hq=32, Hkv=8, dh=128, r=512, F=256,
                    N=32768, C=128, k=32, T=128, rho=0.125)
MISTRAL7B_16K = Shape("mistral7b-16k", 2, B=16, G=4, Hq=32, Hkv=8, dh=128, r=512, F=256,
                      N=16384, C=128, k=16, T=128, rho=0.125)
QWEN4B_64K = Shape("qwen4b-64k", 3, B=4, G=2, Hq=16, Hkv=4, dh=256, r=384, F=512,
                   N=65536, C=256, k=16, T=256, rho=0.10, outlier_frac=0.01)
COMPOSED_128K = Shape("composed-int8-evict-128k", 4, B=2, G=4, Hq=32, Hkv=8, dh=128, r=256,
                      F=256, N=131072, C=128, k=64, T=128, rho=0.0625, coeff=I8, resid=I8,
                      evict_keep=0.25, n_obs=8)

ALL = (TINY, LLAMA8B_32K, MISTRAL7B_16K, QWEN4B_64K, COMPOSED_128K)
BY_NAME = {s.name: s for s in ALL}


def small(s: Shape, **kw) -> Shape:
    """A reduced copy of a workload that a CPU oracle finishes in seconds.

    Keeps head dims, rank, predictor width, chunk length and dtypes (so every
    tile shape of the GPU path is exercised) and shrinks batch and context.
    """
    defaults = dict(B=min(s.B, 2), N=16 * s.C, steps=2)
    if s.evict_keep < 1.0:
        defaults["N"] = 32 * s.C
    defaults.update(kw)
    out = s.replace(**defaults)
    if out.k > out.keep_chunks:
        out = out.replace(k=max(1, out.keep_chunks // 4))
    return out
