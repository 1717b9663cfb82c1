"""Seeded synthetic inputs for compressed-KV decode attention.

The LowRAM pages evaluate on real models (RULER and LongBench runs of
Mistral-7B, Llama-3.1-8B and Qwen3.5-4B, rit.work LowRAM page, quality
section).  Neither the datasets nor the weights are available, so this module
draws inputs with those head shapes and the statistical structure the method
relies on:

* keys of a group of adjacent layers share a low-dimensional subspace
  (zicq.com English summary, "Cross-Layer Low-Rank Key Compression"): the
  concatenated group key K_cat = Z diag(sigma) Q^T with a Haar-random frame Q
  and a geometric spectrum sigma_i = c * 0.9**i, c chosen so that each key
  element has unit variance;
* values are largely predictable from their keys within a head (abstract of
  arXiv 2611.07025): V = MLP_true(K) + 0.1 * Student-t(3) noise, with optional
  x20 outlier tokens;
* queries are i.i.d. N(0, 1).

Shape.key_scale and Shape.q_scale widen the key and query distributions (keys
of norm ~100, queries x16) to drive the softmax into its peaked regime;
Shape.w1_scale scales the value model's first layer (1 / key_scale keeps the
hidden activations and values at their usual scale).

The basis handed to the method is the population principal frame Q[:, :r]
(the leading principal directions of the generated keys), and the predictor
handed to the method is MLP_true itself.

This module is shared by the oracle and the GPU tests.  It produces stored
inputs only; none of the method's steps (projection, prediction, selection,
attention) live here.  The MLP below is the data model that generates the
values, evaluated on the exact keys before storage.
"""
from __future__ import annotations

import concurrent.futures
import contextlib
import os

import numpy as np

from .configs import BF16, F16, F32, F64, Shape

SEED_ROOT = 20261106
STREAM_K, STREAM_FRAME, STREAM_MLP, STREAM_NOISE, STREAM_OUTLIER, STREAM_Q, STREAM_OBS, STREAM_QCORR = range(8)


def _rng(cfg_id: int, b: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg_id, b, stream, *sub]))


# ----------------------------------------------------------------------------
# storage casts (round to nearest even)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to nearest even.  For finite x the 32-bit sum cannot wrap
    (|bits| <= 0x7F7FFFFF plus the sign bit, plus at most 0x8000); NaNs are
    stored as the quiet NaN 0x7FC0."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast generated values to a storage dtype (bf16 as uint16 bit patterns)."""
    if dtype == F64:
        return np.ascontiguousarray(x, dtype=np.float64)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x, dtype=np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(dtype)


def load(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored values to float64."""
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
def haar_frame(rng: np.random.Generator, n: int, p: int) -> np.ndarray:
    """n x p matrix with orthonormal columns, Haar distributed (sign-fixed QR)."""
    a = rng.standard_normal((n, p))
    q, r = np.linalg.qr(a)
    q *= np.sign(np.diag(r))[None, :]
    return q


def spectrum(D: int) -> np.ndarray:
    c = np.sqrt(D * 0.19 / (1.0 - 0.81 ** D))
    return c * 0.9 ** np.arange(D)


@contextlib.contextmanager
def _one_blas_thread(on: bool):
    """BLAS limited to one thread while several Python threads call it."""
    if not on:
        yield
        return
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        yield
        return
    with threadpool_limits(limits=1, user_api="blas"):
        yield


def _mlp_true(x, w1, b1, w2, b2):
    pre = x @ w1.T + b1
    h = pre / (1.0 + np.exp(-pre))
    return h @ w2.T + b2


def make(s: Shape, seed_offset: int = 0, steps: int | None = None, noise_scale: float = 0.1,
         with_dense: bool = False, progress=None, workers: int = 0) -> dict:
    """Draw one workload.  Returns stored arrays keyed by name.  `progress`,
    if given, is called as progress(done, B) after each sequence.  `workers`
    caps the threads that draw concurrently (0: one per CPU, at most 16).

    Layouts (row-major):
      k, v            [B][G][Hkv][N][dh]
      k_tail, v_tail  [B][G][Hkv][T][dh]
      basis           [B][D][r]   (D ordered as (layer, kv head, dim))
      w1 [B][G][Hkv][F][dh]  b1 [B][G][Hkv][F]  w2 [B][G][Hkv][dh][F]  b2 [B][G][Hkv][dh]
      q               [steps][G][B][Hq][dh]
      obs_q           [n_obs][B][G][Hq][dh]       (only when s.n_obs > 0)
      outliers        [B][n_out] int64 token indices with x20 noise
    """
    B, G, Hkv, dh, N, T, D, r, F = s.B, s.G, s.Hkv, s.dh, s.N, s.T, s.D, s.r, s.F
    steps = s.steps if steps is None else steps
    cid = s.cfg_id * 1000 + seed_offset
    act = s.act
    work = np.float64 if act in (F64, F32) else np.float32
    m = s.m_cols
    sig = s.key_scale * spectrum(D)[:m]
    n_out = int(round(s.outlier_frac * N))

    out = {
        "k": np.empty((B, G, Hkv, N, dh), dtype=_np_dtype(act)),
        "v": np.empty((B, G, Hkv, N, dh), dtype=_np_dtype(act)),
        "k_tail": np.empty((B, G, Hkv, T, dh), dtype=_np_dtype(act)),
        "v_tail": np.empty((B, G, Hkv, T, dh), dtype=_np_dtype(act)),
        "basis": np.empty((B, D, r), dtype=_np_dtype(act)),
        "w1": np.empty((B, G, Hkv, F, dh), dtype=_np_dtype(act)),
        "b1": np.empty((B, G, Hkv, F), dtype=_np_dtype(act)),
        "w2": np.empty((B, G, Hkv, dh, F), dtype=_np_dtype(act)),
        "b2": np.empty((B, G, Hkv, dh), dtype=_np_dtype(act)),
        "outliers": np.zeros((B, n_out), dtype=np.int64),
    }
    def keys_of(b: int):
        """Keys, basis and predictor of sequence b; returns the exact keys
        [G][Hkv][N + T][dh] and the stored predictor for the value draws."""
        frame = haar_frame(_rng(cid, b, STREAM_FRAME), D, max(m, r))
        z = _rng(cid, b, STREAM_K).standard_normal((N + T, m)).astype(work)
        kcat = (z * sig.astype(work)[None, :]) @ frame[:, :m].T.astype(work)
        del z
        out["basis"][b] = store(frame[:, :r], act)
        kfull = kcat.reshape(N + T, G, Hkv, dh).transpose(1, 2, 0, 3)
        out["k"][b] = store(kfull[:, :, :N], act)
        out["k_tail"][b] = store(kfull[:, :, N:], act)

        mrng = _rng(cid, b, STREAM_MLP)
        w1 = store(s.w1_scale * mrng.standard_normal((G, Hkv, F, dh)) / np.sqrt(dh), act)
        b1 = store(0.1 * mrng.standard_normal((G, Hkv, F)), act)
        w2 = store(mrng.standard_normal((G, Hkv, dh, F)) / np.sqrt(F), act)
        b2 = store(0.1 * mrng.standard_normal((G, Hkv, dh)), act)
        out["w1"][b], out["b1"][b], out["w2"][b], out["b2"][b] = w1, b1, w2, b2
        if n_out:
            out["outliers"][b] = np.sort(_rng(cid, b, STREAM_OUTLIER).choice(N, size=n_out, replace=False))
        return kfull

    def values_of(b: int, l: int, h: int, kfull) -> None:
        """Values of (sequence b, layer l, kv head h): the value model on the
        exact keys plus heavy-tailed noise from a generator of their own."""
        W1, B1 = load(out["w1"][b, l, h], act).astype(work), load(out["b1"][b, l, h], act).astype(work)
        W2, B2 = load(out["w2"][b, l, h], act).astype(work), load(out["b2"][b, l, h], act).astype(work)
        vals = _mlp_true(kfull[l, h], W1, B1, W2, B2)
        noise = noise_scale * _rng(cid, b, STREAM_NOISE, l, h).standard_t(3, size=(N + T, dh))
        if n_out:
            noise[out["outliers"][b]] *= 20.0
        vals = vals + noise.astype(work)
        out["v"][b, l, h] = store(vals[:N], act)
        out["v_tail"][b, l, h] = store(vals[N:], act)

    # Every array comes from generators seeded by (workload, sequence, stream)
    # and, for the value noise, (layer, kv head), so the draws can run in any
    # order or concurrently with the same result.  The keys of a group of
    # sequences are drawn one sequence at a time (their products use every
    # BLAS thread); the values of the group's (sequence, layer, head) items
    # then run on threads with single-threaded BLAS (numpy releases the GIL in
    # its generators, products and elementwise loops).  Grouping bounds the
    # exact keys held in memory.
    n_thr = max(1, min(workers if workers else (os.cpu_count() or 1), 16))
    if B * N * G * Hkv * dh < (1 << 24):
        n_thr = 1
    with concurrent.futures.ThreadPoolExecutor(max_workers=n_thr) as ex:
        for b0 in range(0, B, n_thr):
            bs = list(range(b0, min(B, b0 + n_thr)))
            keys = {b: keys_of(b) for b in bs}
            items = [(b, l, h) for b in bs for l in range(G) for h in range(Hkv)]
            with _one_blas_thread(n_thr > 1):
                list(ex.map(lambda it: values_of(*it, keys[it[0]]), items))
            del keys
            if progress is not None:
                progress(bs[-1] + 1, B)

    out["q"] = make_queries(s, steps, seed_offset)
    if s.n_obs:
        out["obs_q"] = make_obs_queries(s, seed_offset)
    if with_dense:
        out["k_dense"] = np.concatenate([out["k"], out["k_tail"]], axis=3)
        out["v_dense"] = np.concatenate([out["v"], out["v_tail"]], axis=3)
    return out


def make_queries(s: Shape, steps: int, seed_offset: int = 0) -> np.ndarray:
    cid = s.cfg_id * 1000 + seed_offset
    q = np.empty((steps, s.G, s.B, s.Hq, s.dh), dtype=_np_dtype(s.act))
    for b in range(s.B):
        draws = _rng(cid, b, STREAM_Q).standard_normal((steps, s.G, s.Hq, s.dh))
        q[:, :, b] = store(s.q_scale * draws, s.act)
    return q


def make_correlated_queries(s: Shape, steps: int, rho: float, seed_offset: int = 0) -> np.ndarray:
    """Queries of consecutive decode steps that drift slowly, [steps][G][B][Hq][dh]
    stored: q_0 ~ N(0, 1) and q_s = rho q_{s-1} + sqrt(1 - rho^2) xi_s per (b, l),
    so each step keeps unit variance and successive steps tend to pick the same
    chunks.  (Consecutive tokens' queries are related; i.i.d. queries are the
    other extreme.)"""
    cid = s.cfg_id * 1000 + seed_offset
    q = np.empty((steps, s.G, s.B, s.Hq, s.dh), dtype=_np_dtype(s.act))
    for b in range(s.B):
        xi = _rng(cid, b, STREAM_QCORR).standard_normal((steps, s.G, s.Hq, s.dh))
        cur = xi[0]
        q[0, :, b] = store(cur, s.act)
        for st in range(1, steps):
            cur = rho * cur + np.sqrt(1.0 - rho * rho) * xi[st]
            q[st, :, b] = store(cur, s.act)
    return q


def make_obs_queries(s: Shape, seed_offset: int = 0) -> np.ndarray:
    cid = s.cfg_id * 1000 + seed_offset
    q = np.empty((s.n_obs, s.B, s.G, s.Hq, s.dh), dtype=_np_dtype(s.act))
    for b in range(s.B):
        draws = _rng(cid, b, STREAM_OBS).standard_normal((s.n_obs, s.G, s.Hq, s.dh))
        q[:, b] = store(draws, s.act)
    return q


def _np_dtype(tag: str):
    return {F64: np.float64, F32: np.float32, F16: np.float16, BF16: np.uint16}[tag]
