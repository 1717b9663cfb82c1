"""CPU oracle for LowRAM compressed-KV decode attention (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

What it computes, by source:

* M_KV = 2 L H_kv d_h N s -- zicq.com English summary, "Core Mechanism".
* Values are predicted from keys, V_hat = f(K), and the cache keeps
  delta = V - V_hat only for the tokens the predictor reconstructs worst --
  same section, and the abstract of arXiv 2611.07025 (mlinfo.pages.dev).
* Keys of a group of adjacent layers are stored as low-dimensional per-token
  coefficients on a shared basis ("Cross-Layer Low-Rank Key Compression" on
  the zicq.com English summary; xKV on the rit.work page).
* At decode the context is split into chunks, the chunks suited to the current
  query are picked, only those are rebuilt, and post-prefill tokens stay
  uncompressed (rit.work page, section on generation).
* Attention A = softmax(Q K^T / sqrt(d_h)), O = A V -- OjaKV page, section 3.
* Quantisation and eviction compose with the pipeline (abstract; zicq.com
  "Composition with Quantization and Eviction").

Where the pages leave a step open, the reading taken here is stated in the
docstring of the function that takes it (scorer = group-summed query against
the chunk's mean coefficient; predictor input = reconstructed key; squared L2
error per (layer, head); lowest index wins ties; symmetric per-channel int8
with fp16 scales; eviction by the group-summed score of observation queries;
tail growth by re-packing the oldest C tail tokens as a new chunk against the
existing basis, predictor and int8 scales; test-time fitting of the predictor
as full-batch gradient descent on the mean squared value error; the key basis
as the leading eigenvectors of the group's key Gram matrix).

Stored tensors are passed as numpy arrays in their storage dtype: float64,
float32, float16, int8, or uint16 holding bfloat16 bit patterns.
"""
from __future__ import annotations

import math

import numpy as np

F64, F32, BF16, F16, I8 = "f64", "f32", "bf16", "f16", "i8"


# ============================================================================
# number formats (round to nearest, ties to even)
# ============================================================================
def _round_sig(x: np.ndarray, sig_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 values to `sig_bits` significant bits, RNE.

    The grid spacing at x is 2**(e - sig_bits) with x = m 2**e, 0.5 <= |m| < 1,
    and never below 2**min_exp (gradual underflow).  x / spacing is an exact
    power-of-two scaling, so np.rint applies round-half-even exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    spacing_exp = np.maximum(e - sig_bits, min_exp)
    return np.ldexp(np.rint(np.ldexp(x, -spacing_exp)), spacing_exp)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 (8 significant bits) bit patterns, single rounding."""
    y = _round_sig(x, 8, -133)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)  # exact: y is on the bf16 grid (inf if too large)
    return (y32.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f16(x: np.ndarray) -> np.ndarray:
    """float64 -> float16, single rounding (11 significant bits)."""
    y = _round_sig(x, 11, -24)
    with np.errstate(over="ignore"):
        return y.astype(np.float16)


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64."""
    if dtype == BF16:
        return from_bf16_bits(x)
    return np.asarray(x, dtype=np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> stored representation in `dtype` (not for i8: see quantise)."""
    if dtype == F64:
        return np.asarray(x, dtype=np.float64).copy()
    if dtype == F32:
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == BF16:
        return to_bf16_bits(x)
    if dtype == F16:
        return to_f16(x)
    raise ValueError(dtype)


def quantise(x: np.ndarray, axis: int):
    """Symmetric per-channel int8 with fp16 scales (composition with quantisation,
    zicq.com "Composition with Quantization and Eviction").

    Reading: the channel is every index of the axes other than `axis`;
    s = fp16(max |x| / 127) over `axis`; q = clamp(rne(x / s), -127, 127);
    a channel whose scale is zero stores zeros.  Returns (q int8, s float16).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[axis] == 0:
        amax = np.zeros_like(x.sum(axis=axis, keepdims=True))
    else:
        amax = np.max(np.abs(x), axis=axis, keepdims=True)
    s16 = to_f16(amax / 127.0)
    s = s16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(x / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, np.squeeze(s16, axis=axis)


def dequantise(q: np.ndarray, s: np.ndarray, axis: int) -> np.ndarray:
    return q.astype(np.float64) * np.expand_dims(s.astype(np.float64), axis)


# ============================================================================
# compress side
# ============================================================================
def basis_slice(U: np.ndarray, l: int, h: int, Hkv: int, dh: int) -> np.ndarray:
    """U_{l,h}: rows (l, h, 0..dh-1) of the D x r group basis (D ordered (l, h, d))."""
    r0 = (l * Hkv + h) * dh
    return U[r0:r0 + dh, :]


def project(k_cat: np.ndarray, U: np.ndarray) -> np.ndarray:
    """Per-token group coefficients c_t = U^T k_t^cat (N x r), float64.

    Cross-layer key compression stores low-dimensional coefficients on a basis
    shared by the group (zicq.com English summary, "Cross-Layer Low-Rank Key
    Compression").  Reading: the coefficients are per token and shared by
    every layer and head of the group; the basis rows are sliced per (l, h).
    """
    return k_cat @ U


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def predict(khat: np.ndarray, w1, b1, w2, b2) -> np.ndarray:
    """V_hat = f(K): per-head 2-layer MLP with SiLU (abstract: "lightweight
    per-head predictor"; zicq.com "Core Mechanism": V_hat = f(K)).

    Reading: f(k) = W2 SiLU(W1 k + b1) + b2 applied to the reconstructed key,
    the only key available at decode.
    """
    return silu(khat @ w1.T + b1) @ w2.T + b2


def l2_errors(v: np.ndarray, vhat: np.ndarray) -> np.ndarray:
    """Squared L2 reconstruction error per token (ranking key for residuals)."""
    d = v - vhat
    return np.sum(d * d, axis=-1)


def topk_indices(key: np.ndarray, k: int) -> np.ndarray:
    """The k indices with the largest key, lowest index first among equal keys,
    returned in ascending index order."""
    n = key.shape[0]
    k = max(0, min(k, n))
    order = np.lexsort((np.arange(n), -key))  # primary: key desc, secondary: index asc
    return np.sort(order[:k]).astype(np.int64)


def landmarks(cdeq: np.ndarray, C: int) -> np.ndarray:
    """Chunk landmark = mean coefficient of the chunk's C tokens, rounded to fp32.

    Reading of "picks the fragments suited to the current query" (rit.work,
    generation section): each chunk is summarised by its mean coefficient.
    """
    N, r = cdeq.shape
    return cdeq.reshape(N // C, C, r).mean(axis=1).astype(np.float32)


def compress(inp: dict, s, stored: dict | None = None) -> dict:
    """Compress a prefill: project keys, predict values, keep residuals for the
    worst tokens, summarise chunks.  `inp` holds stored arrays (see synth.gen);
    `s` carries sizes and dtypes.  Returns the stored cache and fp64 side data.

    `stored` (optional) supplies already-stored coefficients ("coeff", and
    "coeff_scale" for int8) that replace step 1's rounding, so the later steps
    can be checked on exactly the bits another implementation stored.

    Steps (per sequence b):
      1. c_t = U^T k_t^cat; store c~ = round(c) (or int8 + fp16 scales per
         coefficient channel).
      2. k_hat_{t,l,h} = U_{l,h} deq(c~_t).
      3. v_hat = f_{l,h}(k_hat).
      4. e_t = ||v_t - v_hat_t||^2 per (l, h).
      5. R_{l,h} = top ceil(rho N) tokens by (e desc, t asc); store
         delta_t = round(v_t - v_hat_t) for t in R, CSR by chunk, sorted by t
         (or int8 + fp16 scales per (l, h, dim) over R).
      6. landmark_j = mean of deq(c~_t) over chunk j, fp32.
    """
    B, G, Hkv, dh, N, C, r = s.B, s.G, s.Hkv, s.dh, s.N, s.C, s.r
    n_c, n_res = N // C, s.n_res
    act, cdt, rdt = s.act, s.coeff, s.resid
    U_all = decode(inp["basis"], act)
    out = {
        "coeff": [], "coeff_scale": [], "landmark": [], "res_ptr": [], "res_idx": [],
        "res_val": [], "res_scale": [], "errors": [], "c_exact": [],
    }
    for b in range(B):
        U = U_all[b]
        k = decode(inp["k"][b], act)                     # [G][Hkv][N][dh]
        v = decode(inp["v"][b], act)
        k_cat = k.transpose(2, 0, 1, 3).reshape(N, -1)   # token-major, (l, h, d)
        c = project(k_cat, U)
        out["c_exact"].append(c)
        if stored is not None:
            cst = np.asarray(stored["coeff"][b])
            out["coeff"].append(cst)
            if cdt == I8:
                cs = np.asarray(stored["coeff_scale"][b])
                out["coeff_scale"].append(cs)
                cdeq = dequantise(cst, cs, axis=0)
            else:
                cdeq = decode(cst, cdt)
        elif cdt == I8:
            cq, cs = quantise(c, axis=0)
            cdeq = dequantise(cq, cs, axis=0)
            out["coeff"].append(cq)
            out["coeff_scale"].append(cs)
        else:
            cst = round_to(c, cdt)
            out["coeff"].append(cst)
            cdeq = decode(cst, cdt)
        out["landmark"].append(landmarks(cdeq, C))
        ptr_b, idx_b, val_b, sc_b, err_b = [], [], [], [], []
        for l in range(G):
            for h in range(Hkv):
                Ulh = basis_slice(U, l, h, Hkv, dh)
                khat = cdeq @ Ulh.T
                w1, b1 = decode(inp["w1"][b, l, h], act), decode(inp["b1"][b, l, h], act)
                w2, b2 = decode(inp["w2"][b, l, h], act), decode(inp["b2"][b, l, h], act)
                vhat = predict(khat, w1, b1, w2, b2)
                e = l2_errors(v[l, h], vhat)
                err_b.append(e)
                R = topk_indices(e, n_res)
                delta = v[l, h][R] - vhat[R]
                if rdt == I8:
                    dq, ds = quantise(delta, axis=0)
                    val_b.append(dq)
                    sc_b.append(ds)
                else:
                    val_b.append(round_to(delta, rdt))
                idx_b.append(R.astype(np.int32))
                ptr_b.append(csr_pointers(R, C, n_c))
        out["res_ptr"].append(np.stack(ptr_b).reshape(G, Hkv, n_c + 1))
        out["res_idx"].append(np.stack(idx_b).reshape(G, Hkv, n_res))
        out["res_val"].append(np.stack(val_b).reshape(G, Hkv, n_res, dh))
        if rdt == I8:
            out["res_scale"].append(np.stack(sc_b).reshape(G, Hkv, dh))
        out["errors"].append(np.stack(err_b).reshape(G, Hkv, N))
    cache = {k2: (np.stack(v2) if v2 else None) for k2, v2 in out.items()}
    return cache


def csr_pointers(R: np.ndarray, C: int, n_c: int) -> np.ndarray:
    """ptr[j] = number of residual tokens with index < j*C (R sorted ascending)."""
    ptr = np.zeros(n_c + 1, dtype=np.int32)
    for j in range(n_c + 1):
        ptr[j] = int(np.sum(R < j * C))
    return ptr


def coeff_deq(cache: dict, b: int, cdt: str) -> np.ndarray:
    if cdt == I8:
        return dequantise(cache["coeff"][b], cache["coeff_scale"][b], axis=0)
    return decode(cache["coeff"][b], cdt)


def resid_deq(cache: dict, b: int, l: int, h: int, rdt: str) -> np.ndarray:
    if rdt == I8:
        return dequantise(cache["res_val"][b, l, h], cache["res_scale"][b, l, h], axis=0)
    return decode(cache["res_val"][b, l, h], rdt)


# ============================================================================
# decode side
# ============================================================================
def kv_head_of(g: int, Hq: int, Hkv: int) -> int:
    """GQA: contiguous groups of Hq/Hkv query heads share a KV head."""
    return (g * Hkv) // Hq


def chunk_scores(landmark: np.ndarray, U: np.ndarray, q: np.ndarray, l: int, h: int,
                 Hq: int, Hkv: int, dh: int) -> np.ndarray:
    """s_j = q~ . landmark_j with q~ = U_{l,h}^T sum_{g in grp(h)} q_g (fp64).

    Reading of the query-driven chunk choice (rit.work, generation section):
    the group-summed query mapped into coefficient space, scored against each
    chunk's mean coefficient.  Each score is an independent row-wise sum, so
    equal landmark rows give equal scores.
    """
    grp = [g for g in range(Hq) if kv_head_of(g, Hq, Hkv) == h]
    qsum = np.sum(q[grp], axis=0)
    qt = basis_slice(U, l, h, Hkv, dh).T @ qsum
    return np.sum(landmark.astype(np.float64) * qt[None, :], axis=1)


def select_chunks(scores: np.ndarray, k: int) -> np.ndarray:
    """top-min(k, n_c) chunks by (score desc, index asc), ascending."""
    return topk_indices(scores, k)


def softmax_attend(qg: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """o = softmax(keys q / sqrt(d_h)) vals, two-pass with the max subtracted
    (OjaKV page, section 3, attention definition)."""
    a = keys @ qg / math.sqrt(qg.shape[-1])
    p = np.exp(a - np.max(a))
    p = p / np.sum(p)
    return p @ vals


def decode_layer(cache: dict, inp: dict, s, l: int, q: np.ndarray, top_k: int,
                 N: int | None = None, return_parts: bool = False):
    """One decode step of attention at layer l of the group for B sequences.

    q: [B][Hq][dh] stored.  Uses the stored cache (coeff, landmarks, residuals),
    the stored basis and predictor, and the stored tail of layer l.
    Returns (out [B][Hq][dh] float64, sel [B][Hkv][k'] int64).

    For each (b, h): score chunks, pick the top k, rebuild the keys
    k_hat = U_{l,h} deq(c~) and values v_hat + [t in R] delta of the picked
    chunks only, append the uncompressed tail, and attend each query head of
    the group over that set.
    """
    B, Hq, Hkv, dh, C = s.B, s.Hq, s.Hkv, s.dh, s.C
    act, cdt, rdt = s.act, s.coeff, s.resid
    N = s.N if N is None else N
    n_c = N // C
    kk = max(0, min(top_k, n_c))
    out = np.zeros((B, Hq, dh))
    sel = np.zeros((B, Hkv, kk), dtype=np.int64)
    parts = {}
    U_all = decode(inp["basis"], act)
    for b in range(B):
        U = U_all[b]
        qb = decode(q[b], act)
        cdeq = coeff_deq(cache, b, cdt) if n_c else np.zeros((0, s.r))
        for h in range(Hkv):
            if n_c and kk:
                sc = chunk_scores(cache["landmark"][b], U, qb, l, h, Hq, Hkv, dh)
                S = select_chunks(sc, kk)
            else:
                S = np.zeros(0, dtype=np.int64)
            sel[b, h] = S
            toks = (S[:, None] * C + np.arange(C)[None, :]).reshape(-1)
            Ulh = basis_slice(U, l, h, Hkv, dh)
            khat = cdeq[toks] @ Ulh.T
            w1, b1 = decode(inp["w1"][b, l, h], act), decode(inp["b1"][b, l, h], act)
            w2, b2 = decode(inp["w2"][b, l, h], act), decode(inp["b2"][b, l, h], act)
            vals = predict(khat, w1, b1, w2, b2) if len(toks) else np.zeros((0, dh))
            # residuals of the picked chunks: CSR slice per chunk
            ptr = cache["res_ptr"][b, l, h]
            R = cache["res_idx"][b, l, h]
            dv = resid_deq(cache, b, l, h, rdt) if R.shape[0] else np.zeros((0, dh))
            pos = {int(t): i for i, t in enumerate(toks)}
            for j in S:
                for e in range(int(ptr[j]), int(ptr[j + 1])):
                    vals[pos[int(R[e])]] += dv[e]
            kt = decode(inp["k_tail"][b, l, h], act)
            vt = decode(inp["v_tail"][b, l, h], act)
            keys = np.concatenate([khat, kt], axis=0)
            allv = np.concatenate([vals, vt], axis=0)
            if keys.shape[0] == 0:
                raise ValueError("nothing to attend: no chunks selected and no tail")
            for g in range(Hq):
                if kv_head_of(g, Hq, Hkv) == h:
                    out[b, g] = softmax_attend(qb[g], keys, allv)
            if return_parts:
                parts[(b, h)] = (keys, allv)
    if return_parts:
        return out, sel, parts
    return out, sel


def dense_decode_layer(q: np.ndarray, k: np.ndarray, v: np.ndarray, Hq: int, Hkv: int) -> np.ndarray:
    """Uncompressed decode attention: q [B][Hq][dh], k/v [B][Hkv][n][dh] float64."""
    B, _, dh = q.shape
    out = np.zeros((B, Hq, dh))
    for b in range(B):
        for g in range(Hq):
            h = kv_head_of(g, Hq, Hkv)
            out[b, g] = softmax_attend(q[b, g], k[b, h], v[b, h])
    return out


# ============================================================================
# eviction (composition with eviction)
# ============================================================================
def eviction_scores(cache: dict, inp: dict, s, obs_q: np.ndarray) -> np.ndarray:
    """acc[b][j] = sum over observation queries w, layers l and KV heads h of the
    chunk score s^{(w)}_{l,h,j} (fp64).

    Reading of "eviction removes low-value tokens" (zicq.com Chinese summary,
    composition section): since coefficients are shared by the whole group, a
    chunk's value is its score summed over the group's layers and heads and
    over a window of observation queries.
    """
    B, G, Hq, Hkv, dh = s.B, s.G, s.Hq, s.Hkv, s.dh
    n_c = cache["landmark"].shape[1]
    acc = np.zeros((B, n_c))
    U_all = decode(inp["basis"], s.act)
    for b in range(B):
        for w in range(obs_q.shape[0]):
            for l in range(G):
                qb = decode(obs_q[w, b, l], s.act)
                for h in range(Hkv):
                    acc[b] += chunk_scores(cache["landmark"][b], U_all[b], qb, l, h, Hq, Hkv, dh)
    return acc


def evict(cache: dict, inp: dict, s, obs_q: np.ndarray, keep: int) -> dict:
    """Keep the top `keep` chunks by (acc desc, j asc) per sequence and compact
    them in ascending chunk order.  Residuals of evicted chunks are dropped;
    kept residual tokens are renumbered to their new positions.  Residual
    arrays keep their capacity; res_ptr[n_c'] gives the live count."""
    B, G, Hkv, C = s.B, s.G, s.Hkv, s.C
    acc = eviction_scores(cache, inp, s, obs_q)
    n_res = cache["res_idx"].shape[-1]
    dh = cache["res_val"].shape[-1]
    new = {k: None for k in cache}
    new["keep"] = np.stack([topk_indices(acc[b], keep) for b in range(B)])
    new["acc"] = acc
    new["coeff"] = np.stack([
        cache["coeff"][b].reshape(-1, C, cache["coeff"].shape[-1])[new["keep"][b]].reshape(-1, cache["coeff"].shape[-1])
        for b in range(B)])
    new["coeff_scale"] = cache.get("coeff_scale")
    new["landmark"] = np.stack([cache["landmark"][b][new["keep"][b]] for b in range(B)])
    new["res_scale"] = cache.get("res_scale")
    ptr = np.zeros((B, G, Hkv, keep + 1), dtype=np.int32)
    idx = np.zeros((B, G, Hkv, n_res), dtype=np.int32)
    val = np.zeros((B, G, Hkv, n_res, dh), dtype=cache["res_val"].dtype)
    for b in range(B):
        for l in range(G):
            for h in range(Hkv):
                op, oi, ov = cache["res_ptr"][b, l, h], cache["res_idx"][b, l, h], cache["res_val"][b, l, h]
                n = 0
                for jn, jo in enumerate(new["keep"][b]):
                    ptr[b, l, h, jn] = n
                    for e in range(int(op[jo]), int(op[jo + 1])):
                        idx[b, l, h, n] = int(oi[e]) - jo * C + jn * C
                        val[b, l, h, n] = ov[e]
                        n += 1
                ptr[b, l, h, keep] = n
    new["res_ptr"], new["res_idx"], new["res_val"] = ptr, idx, val
    return new


# ============================================================================
# tail growth: re-pack the oldest tail chunk into the compressed cache
# ============================================================================
def quantise_with(x: np.ndarray, scale: np.ndarray, axis: int) -> np.ndarray:
    """int8 with given per-channel fp16 scales: q = clamp(rne(x / s), -127, 127),
    zero where s = 0 (the rule of `quantise`, scales kept)."""
    x = np.asarray(x, dtype=np.float64)
    s = np.expand_dims(np.asarray(scale).astype(np.float64), axis)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(x / np.where(s > 0, s, 1.0)), 0.0)
    return np.clip(q, -127, 127).astype(np.int8)


def repack(cache: dict, model: dict, k_new: np.ndarray, v_new: np.ndarray, s, m: int,
           stored_coeff: np.ndarray | None = None) -> dict:
    """Append C post-prefill tokens to the compressed cache as one new chunk.

    The rit.work page (section on generation) keeps tokens generated after the
    prefill uncompressed; the pages do not say what happens as that tail grows.
    Reading taken here: once C tail tokens have accumulated they are compressed
    the way the prefill was, against the existing basis and predictor, and
    appended as chunk n_c:
      1. c_t = U^T k_t^cat for the C tokens; stored rounded to the coefficient
         dtype, or for int8 with the cache's existing per-channel scales
         (clamped; the scales, and so every stored value, stay unchanged);
      2. landmark_{n_c} = mean of the stored (dequantised) c_t, fp32;
      3. per (l, h): e_t = ||v_t - f(U_{l,h} deq(c~_t))||^2 over the C tokens and
         the m tokens with the largest e (lowest index first on ties) keep
         delta = v - v_hat, stored rounded (int8: existing per-dim scales);
         residual sets of earlier chunks are unchanged;
      4. the residual CSR gains one chunk: the new entries follow the live ones
         (res_ptr[n_c] of the old cache), token indices N + t ascending.
    k_new, v_new: [B][G][Hkv][C][dh] stored act dtype.  `stored_coeff` (optional,
    [B][C][r] stored) replaces step 1's rounding so that steps 2-4 can be
    checked on another implementation's stored bits.  Returns the new cache
    (residual capacity old capacity + m).
    """
    B, G, Hkv, dh, C, r = s.B, s.G, s.Hkv, s.dh, s.C, s.r
    act, cdt, rdt = s.act, s.coeff, s.resid
    N = cache["coeff"].shape[1]
    n_c = N // C
    cap = cache["res_idx"].shape[-1]
    U_all = decode(model["basis"], act)
    coeff_new, lm_new = [], []
    ptr = np.zeros((B, G, Hkv, n_c + 2), dtype=np.int32)
    idx = np.zeros((B, G, Hkv, cap + m), dtype=np.int32)
    val = np.zeros((B, G, Hkv, cap + m, dh), dtype=cache["res_val"].dtype)
    errors = np.zeros((B, G, Hkv, C))
    for b in range(B):
        U = U_all[b]
        k = decode(k_new[b], act)
        v = decode(v_new[b], act)
        k_cat = k.transpose(2, 0, 1, 3).reshape(C, -1)
        c = project(k_cat, U)
        if stored_coeff is not None:
            cst = np.asarray(stored_coeff[b])
        elif cdt == I8:
            cst = quantise_with(c, cache["coeff_scale"][b], axis=0)
        else:
            cst = round_to(c, cdt)
        cdeq = dequantise(cst, cache["coeff_scale"][b], axis=0) if cdt == I8 else decode(cst, cdt)
        coeff_new.append(cst)
        lm_new.append(landmarks(cdeq, C))
        for l in range(G):
            for h in range(Hkv):
                Ulh = basis_slice(U, l, h, Hkv, dh)
                khat = cdeq @ Ulh.T
                w1, b1 = decode(model["w1"][b, l, h], act), decode(model["b1"][b, l, h], act)
                w2, b2 = decode(model["w2"][b, l, h], act), decode(model["b2"][b, l, h], act)
                vhat = predict(khat, w1, b1, w2, b2)
                e = l2_errors(v[l, h], vhat)
                errors[b, l, h] = e
                R = topk_indices(e, m)
                delta = v[l, h][R] - vhat[R]
                if rdt == I8:
                    dst = quantise_with(delta, cache["res_scale"][b, l, h], axis=0)
                else:
                    dst = round_to(delta, rdt)
                op = cache["res_ptr"][b, l, h]
                live = int(op[n_c])
                ptr[b, l, h, :n_c + 1] = op
                ptr[b, l, h, n_c + 1] = live + m
                idx[b, l, h, :live] = cache["res_idx"][b, l, h, :live]
                idx[b, l, h, live:live + m] = N + R
                val[b, l, h, :live] = cache["res_val"][b, l, h, :live]
                val[b, l, h, live:live + m] = dst
    new = dict(cache)
    new["coeff"] = np.concatenate([cache["coeff"], np.stack(coeff_new)], axis=1)
    new["landmark"] = np.concatenate([cache["landmark"], np.stack(lm_new)], axis=1)
    new["res_ptr"], new["res_idx"], new["res_val"] = ptr, idx, val
    new["repack_errors"] = errors
    return new


# ============================================================================
# the group key basis at prefill
# ============================================================================
def key_basis(inp: dict, s, N: int | None = None):
    """Principal directions of a group's keys (float64).

    xKV finds a few principal directions of the keys and shares the basis
    across adjacent layers (rit.work page, keys section; zicq.com English
    summary, "Cross-Layer Low-Rank Key Compression").  Reading: for each
    sequence, U = the eigenvectors of K_cat^T K_cat for its r largest
    eigenvalues, K_cat the N x D stored keys of tokens [0, N) concatenated
    over (layer, kv head, dim); descending order, each vector's entry of
    largest magnitude made positive.
    Returns (U [B][D][r] float64, eigenvalues [B][r] descending).
    """
    B, r = s.B, s.r
    N = s.N if N is None else N
    Us, lams = [], []
    for b in range(B):
        k = decode(inp["k"][b][:, :, :N], s.act)
        kcat = k.transpose(2, 0, 1, 3).reshape(N, -1)
        lam, vec = np.linalg.eigh(kcat.T @ kcat)
        order = np.argsort(-lam, kind="stable")[:r]
        U = vec[:, order]
        piv = np.argmax(np.abs(U), axis=0)
        U = U * np.sign(U[piv, np.arange(r)])[None, :]
        Us.append(U)
        lams.append(lam[order])
    return np.stack(Us), np.stack(lams)


def residual_energy(inp: dict, s, U: np.ndarray, N: int | None = None) -> np.ndarray:
    """||K_cat - K_cat U U^T||_F^2 / ||K_cat||_F^2 per sequence (float64), for a
    basis U [B][D][r] given in float64."""
    N = s.N if N is None else N
    out = np.zeros(s.B)
    for b in range(s.B):
        k = decode(inp["k"][b][:, :, :N], s.act)
        kcat = k.transpose(2, 0, 1, 3).reshape(N, -1)
        rec = (kcat @ U[b]) @ U[b].T
        out[b] = np.sum((kcat - rec) ** 2) / np.sum(kcat ** 2)
    return out


# ============================================================================
# test-time fitting of the value predictor
# ============================================================================
def predictor_loss_grad(khat: np.ndarray, v: np.ndarray, w1, b1, w2, b2):
    """L = (1/N) sum_t ||v_t - f(k_hat_t)||^2 over the N tokens of one head and
    its gradient with respect to (W1, b1, W2, b2), by the chain rule (fp64).

    With a = W1 k + b1, SiLU(a) = a s(a), s the logistic function, the
    derivative is SiLU'(a) = s(a) (1 + a (1 - s(a))).
    """
    N = khat.shape[0]
    a = khat @ w1.T + b1
    sg = 1.0 / (1.0 + np.exp(-a))
    hid = a * sg
    r = hid @ w2.T + b2 - v
    loss = float(np.sum(r * r)) / N
    gv = (2.0 / N) * r                       # dL / d v_hat
    gw2 = gv.T @ hid
    gb2 = gv.sum(axis=0)
    ga = (gv @ w2) * (sg * (1.0 + a * (1.0 - sg)))
    gw1 = ga.T @ khat
    gb1 = ga.sum(axis=0)
    return loss, (gw1, gb1, gw2, gb2)


def fit_predictor(inp: dict, s, steps: int, lr: float, init: dict | None = None) -> dict:
    """Fit each head's value predictor to its context at test time.

    The abstract fits a lightweight per-head predictor at test time, either
    from scratch or from a meta-learned initialisation that needs fewer
    steps; the rit.work page (values section) trains it during prefill on the
    context's keys to reproduce their values.  Reading taken here: `steps`
    steps of full-batch gradient descent with step size `lr` on the mean
    squared value error L above, per (b, l, h), starting from `init`'s
    weights (default: the ones in inp), with the reconstructed keys
    k_hat = U_{l,h} deq(c~) as inputs -- the keys the predictor sees at decode
    -- where c~ are the coefficients compress stores (same rounding; int8
    scales over the N tokens).  The weights are kept in float64 across the
    steps and rounded to the act dtype once at the end.
    Returns {"w1", "b1", "w2", "b2"} (stored act dtype) and "loss"
    [B][G][Hkv][steps + 1]: L before each step and after the last one.
    """
    B, G, Hkv, dh, N = s.B, s.G, s.Hkv, s.dh, s.N
    act, cdt = s.act, s.coeff
    init = inp if init is None else init
    U_all = decode(inp["basis"], act)
    out = {n: np.empty_like(np.asarray(init[n])) for n in ("w1", "b1", "w2", "b2")}
    loss = np.zeros((B, G, Hkv, steps + 1))
    for b in range(B):
        U = U_all[b]
        k = decode(inp["k"][b], act)
        v = decode(inp["v"][b], act)
        c = project(k.transpose(2, 0, 1, 3).reshape(N, -1), U)
        if cdt == I8:
            cq, cs = quantise(c, axis=0)
            cdeq = dequantise(cq, cs, axis=0)
        else:
            cdeq = decode(round_to(c, cdt), cdt)
        for l in range(G):
            for h in range(Hkv):
                khat = cdeq @ basis_slice(U, l, h, Hkv, dh).T
                w = [decode(init[n][b, l, h], act) for n in ("w1", "b1", "w2", "b2")]
                for st in range(steps + 1):
                    L, grads = predictor_loss_grad(khat, v[l, h], *w)
                    loss[b, l, h, st] = L
                    if st < steps:
                        w = [wi - lr * gi for wi, gi in zip(w, grads)]
                for n, wi in zip(("w1", "b1", "w2", "b2"), w):
                    out[n][b, l, h] = round_to(wi, act)
    out["loss"] = loss
    return out


# ============================================================================
# storage accounting
# ============================================================================
DTYPE_BYTES = {F64: 8, F32: 4, BF16: 2, F16: 2, I8: 1}


def m_kv(L: int, Hkv: int, dh: int, N: int, s_bytes: int) -> int:
    """M_KV = 2 L H_kv d_h N s (zicq.com English summary, "Core Mechanism")."""
    return 2 * L * Hkv * dh * N * s_bytes


def compressed_bytes(G, Hkv, dh, N, C, r, F, n_res, act, coeff, resid, rows=None) -> int:
    """Bytes of one sequence's compressed group: coefficients, basis, predictor,
    residual rows with their int32 token index, CSR pointers, fp32 landmarks
    and fp16 scales.  The uncompressed tail is identical on both sides and is
    not counted.  Residual storage is n_res rows for each of the G * Hkv heads,
    or, if `rows` is given, `rows` rows in all (the live rows of a cache whose
    heads hold different counts, e.g. after eviction)."""
    D = G * Hkv * dh
    n_c = N // C
    s, sc, sr = DTYPE_BYTES[act], DTYPE_BYTES[coeff], DTYPE_BYTES[resid]
    n_rows = G * Hkv * n_res if rows is None else rows
    total = N * r * sc + D * r * s + G * Hkv * (2 * F * dh + F + dh) * s
    total += n_rows * (dh * sr + 4) + G * Hkv * (n_c + 1) * 4 + n_c * r * 4
    if coeff == I8:
        total += r * 2
    if resid == I8:
        total += G * Hkv * dh * 2
    return total
