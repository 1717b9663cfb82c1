// Decode-side kernels for gfx950:
//   k_select      chunk scores in float64 and a deterministic per-(b, kv head) top-k
//   k_attend_valu rebuild-and-attend on the vector ALUs (float32 caches, and any
//                 shape the MFMA kernel does not cover), plus the uncompressed tail
//   k_combine     merge of split softmax partials with the hoisted second
//                 predictor layer
//   k_dense       uncompressed split-K decode attention (the comparator)
//
// Attention is softmax(q k^T / sqrt(d_h)) v (OjaKV page, section 3).  The
// chunk scorer maps the group-summed query into coefficient space and scores
// each chunk's mean coefficient; only the picked chunks are rebuilt (rit.work
// LowRAM page, generation section).  Values are the per-head predictor
// f(k) = W2 SiLU(W1 k + b1) + b2 plus the stored residual rows (zicq.com
// English summary, "Core Mechanism").  Because f's second layer is linear, the
// softmax-weighted sum of values equals W2 (sum p h) + b2 (sum p) + sum p delta;
// the split kernels accumulate sum p h and sum p delta and the combine applies
// W2 once per query head.
#include "common.hpp"
#include "internal.hpp"
#include "attend_common.hpp"

namespace lowram {

// ---------------------------------------------------------------------------
// D1-D3: q~ = U_{l,h}^T sum_g q_g; s_j = q~ . landmark_j (float64); top-k.
// grid (Hkv, B), 256 threads.  scores (optional) receives s[b][h][n_c].
// ---------------------------------------------------------------------------
template <typename TA>
__global__ __launch_bounds__(256) void k_select(const TA *__restrict__ q, long q_bstride,
                                                const TA *__restrict__ basis,
                                                const float *__restrict__ landmark, int Hq,
                                                int Hkv, int dh, int r, int n_c, int D, int layer,
                                                int k_eff, int32_t *__restrict__ sel,
                                                int32_t *__restrict__ sel_out,
                                                double *__restrict__ scores) {
  extern __shared__ __align__(16) unsigned char smem[];
  TopkSmem &tk = *reinterpret_cast<TopkSmem *>(smem);
  double *qsum = reinterpret_cast<double *>(smem + ((sizeof(TopkSmem) + 15) & ~15));
  double *qt = qsum + dh;
  double *sc = qt + r;
  int32_t *sl = reinterpret_cast<int32_t *>(sc + n_c);
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int grp = Hq / Hkv;
  const TA *qb = q + (long)b * q_bstride + (long)h * grp * dh;
  for (int d = tid; d < dh; d += 256) {
    double s = 0.0;
    for (int gi = 0; gi < grp; ++gi) s += to_f64(qb[gi * dh + d]);
    qsum[d] = s;
  }
  __syncthreads();
  const TA *U = basis + ((long)b * D + (long)(layer * Hkv + h) * dh) * r;
  for (int i = tid; i < r; i += 256) {
    double s = 0.0;
    for (int d = 0; d < dh; ++d) s = fma(to_f64(U[(long)d * r + i]), qsum[d], s);
    qt[i] = s;
  }
  __syncthreads();
  const float *L = landmark + (long)b * n_c * r;
  for (int j = wave; j < n_c; j += 256 / WAVE) {
    double s = 0.0;
    for (int i = lane; i < r; i += WAVE) s = fma((double)L[(long)j * r + i], qt[i], s);
    s = wave_sum(s);
    if (lane == 0) sc[j] = s;
  }
  __syncthreads();
  if (scores)
    for (int j = tid; j < n_c; j += 256) scores[((long)b * Hkv + h) * n_c + j] = sc[j];
  if (k_eff > 0) {
    block_topk<256>([&](int i) { return f64_order_key(sc[i]); }, n_c, k_eff, sl, tk, 0, nullptr);
    __syncthreads();
    for (int i = tid; i < k_eff; i += 256) {
      sel[((long)b * Hkv + h) * k_eff + i] = sl[i];
      if (sel_out) sel_out[((long)b * Hkv + h) * k_eff + i] = sl[i];
    }
  }
}

// ---------------------------------------------------------------------------
// D4-D6 on the vector ALUs.  grid (n_split + 1, Hkv, B), 256 threads; the last
// split of each (b, h) is the tail.  TT tokens per tile.
// ---------------------------------------------------------------------------
template <typename TA, typename TC, typename TR>
__global__ __launch_bounds__(256) void k_attend_valu(const AttendArgs a, int TT) {
  extern __shared__ __align__(16) float fsm[];
  const int h = blockIdx.y, b = blockIdx.z, split = blockIdx.x, tid = threadIdx.x;
  const int g = a.g, dh = a.dh, r = a.r, F = a.F, C = a.C;
  float *qs = fsm;                      // [g][dh]
  float *accV = qs + g * dh;            // [g][dh]
  float *accH = accV + g * dh;          // [g][F]
  float *ms = accH + g * F;             // [g]
  float *ls = ms + 16, *al = ls + 16;   // [g]
  float *lg = al + 16;                  // [g][TT]
  float *cb = lg + g * TT;              // [TT][r]
  float *kh = cb + TT * r;              // [TT][dh]
  float *hb = kh + TT * dh;             // [TT][F]

  const TA *qb = reinterpret_cast<const TA *>(a.q) + ((long)b * a.Hq + (long)h * g) * dh;
  for (int i = tid; i < g * dh; i += 256) { qs[i] = ldf(qb, i); accV[i] = 0.f; }
  for (int i = tid; i < g * F; i += 256) accH[i] = 0.f;
  if (tid < g) { ms[tid] = -INFINITY; ls[tid] = 0.f; al[tid] = 0.f; }
  __syncthreads();

  if (split == a.n_split) {
    tail_split<TA>(a, qs, lg, TT, accV, ms, ls, al);
    write_partial(a, split, ms, ls, nullptr, accV);
    return;
  }

  const int D = a.G * a.Hkv * dh;
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;
  const TA *U = reinterpret_cast<const TA *>(a.basis) + ((long)b * D + (long)(a.layer * a.Hkv + h) * dh) * r;
  const TA *W1 = reinterpret_cast<const TA *>(a.w1) + bh * F * dh;
  const TA *B1 = reinterpret_cast<const TA *>(a.b1) + bh * F;
  const TC *cf = reinterpret_cast<const TC *>(a.coeff) + (long)b * a.N * r;
  const uint16_t *csc = a.coeff_scale ? a.coeff_scale + (long)b * r : nullptr;
  const int32_t *rptr = a.res_ptr + bh * (a.N / C + 1);
  const int32_t *ridx = a.res_idx + bh * a.n_res;
  const TR *rval = reinterpret_cast<const TR *>(a.res_val) + bh * a.n_res * dh;
  const uint16_t *rsc = a.res_scale ? a.res_scale + bh * dh : nullptr;
  const int32_t *selp = a.sel + ((long)b * a.Hkv + h) * a.k_eff;

  const int s_end = min(a.k_eff, (split + 1) * a.cps);
  for (int slot = split * a.cps; slot < s_end; ++slot) {
    const int j = selp[slot];
    const int e0 = rptr[j], e1 = rptr[j + 1];
    for (int t0 = 0; t0 < C; t0 += TT) {
      const int nt = min(TT, C - t0);
      const long row0 = (long)j * C + t0;
      for (int idx = tid; idx < nt * r; idx += 256) {
        const int t = idx / r, i = idx % r;
        cb[idx] = ld_coeff(cf, (row0 + t) * r + i, csc, i);
      }
      __syncthreads();
      for (int idx = tid; idx < nt * dh; idx += 256) {
        const int t = idx / dh, d = idx % dh;
        const TA *ur = U + (long)d * r;
        float s = 0.f;
        for (int i = 0; i < r; ++i) s = fmaf(ldf(ur, i), cb[t * r + i], s);
        kh[idx] = s;
      }
      __syncthreads();
      for (int idx = tid; idx < g * nt; idx += 256) {
        const int gi = idx / nt, t = idx % nt;
        float s = 0.f;
        for (int d = 0; d < dh; ++d) s = fmaf(qs[gi * dh + d], kh[t * dh + d], s);
        lg[gi * TT + t] = s * a.scale_log2;
      }
      for (int idx = tid; idx < nt * F; idx += 256) {
        const int t = idx / F, f = idx % F;
        const TA *wr = W1 + (long)f * dh;
        float s = ldf(B1, f);
        for (int d = 0; d < dh; ++d) s = fmaf(ldf(wr, d), kh[t * dh + d], s);
        hb[idx] = silu_f(s);
      }
      __syncthreads();
      softmax_tile(lg, TT, nt, g, ms, ls, al);
      __syncthreads();
      for (int idx = tid; idx < g * F; idx += 256) {
        const int gi = idx / F, f = idx % F;
        float acc = accH[idx] * al[gi];
        for (int t = 0; t < nt; ++t) acc = fmaf(lg[gi * TT + t], hb[t * F + f], acc);
        accH[idx] = acc;
      }
      for (int idx = tid; idx < g * dh; idx += 256) {
        const int gi = idx / dh, d = idx % dh;
        float acc = accV[idx] * al[gi];
        for (int e = e0; e < e1; ++e) {
          const int t = ridx[e] - (int)row0;
          if (t >= 0 && t < nt)
            acc = fmaf(lg[gi * TT + t], ld_coeff(rval, (long)e * dh + d, rsc, d), acc);
        }
        accV[idx] = acc;
      }
      __syncthreads();
    }
  }
  write_partial(a, split, ms, ls, accH, accV);
}

// ---------------------------------------------------------------------------
// D7: merge the splits of each query head and apply W2 / b2 once.
// grid (Hq, B), 256 threads.
// ---------------------------------------------------------------------------
template <typename TA>
__global__ __launch_bounds__(256) void k_combine(const CombineArgs a) {
  extern __shared__ __align__(16) float csm[];
  const int gq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int h = (gq * a.Hkv) / a.Hq, gi = gq - h * a.g;
  float *wts = csm;                   // [n_total]
  float *accH = wts + a.n_total;      // [F]
  float *red = accH + a.F;            // [8]
  const float *p = a.part + ((long)b * a.Hkv + h) * a.n_total * a.g * a.PW + (long)gi * a.PW;
  const long sstride = (long)a.g * a.PW;
  // global max over splits (exact, order independent)
  float mx = -INFINITY;
  for (int s = tid; s < a.n_total; s += 256) mx = fmaxf(mx, p[s * sstride]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  for (int s = tid; s < a.n_total; s += 256) {
    const float m = p[s * sstride];
    wts[s] = (m == -INFINITY) ? 0.f : exp2f(m - M);
  }
  __syncthreads();
  float L = 0.f, mass = 0.f;  // same order in every thread: deterministic
  for (int s = 0; s < a.n_total; ++s) {
    const float wl = wts[s] * p[s * sstride + 1];
    L += wl;
    if (s < a.n_comp) mass += wl;
  }
  for (int f = tid; f < a.F; f += 256) {
    float acc = 0.f;
    for (int s = 0; s < a.n_comp; ++s) acc = fmaf(wts[s], p[s * sstride + 4 + f], acc);
    accH[f] = acc;
  }
  __syncthreads();
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;
  const bool hoisted = a.F > 0 && a.n_comp > 0;  // W2/b2 only when rebuilt chunks contributed
  const TA *W2 = hoisted ? reinterpret_cast<const TA *>(a.w2) + bh * a.dh * a.F : nullptr;
  const TA *B2 = hoisted ? reinterpret_cast<const TA *>(a.b2) + bh * a.dh : nullptr;
  TA *out = reinterpret_cast<TA *>(a.out) + ((long)b * a.Hq + gq) * a.dh;
  const float invL = 1.0f / L;
  for (int d = wave; d < a.dh; d += 256 / WAVE) {
    float s = 0.f;
    if (hoisted) {
      for (int f = lane; f < a.F; f += WAVE) s = fmaf(ldf(W2, (long)d * a.F + f), accH[f], s);
      s = wave_sum(s);
    }
    if (lane == 0) {
      float v = s;
      if (hoisted) v = fmaf(ldf(B2, d), mass, v);
      for (int sp = 0; sp < a.n_total; ++sp) v = fmaf(wts[sp], p[sp * sstride + 4 + a.F + d], v);
      store_f32(out + d, v * invL);
    }
  }
}

// ---------------------------------------------------------------------------
// Dense split-K decode attention over n tokens.  grid (n_split, Hkv, B).
// ---------------------------------------------------------------------------
template <typename TA>
__global__ __launch_bounds__(256) void k_dense(const TA *__restrict__ q, const TA *__restrict__ k,
                                               const TA *__restrict__ v, long bstride, int Hq,
                                               int Hkv, int dh, int n, int tps, int n_split,
                                               float *__restrict__ part, int PW, float scale_log2) {
  constexpr int TT = 64;
  extern __shared__ __align__(16) float dsm[];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int g = Hq / Hkv;
  const int kst = dh + 1;
  float *qs = dsm;                 // [g][dh]
  float *accV = qs + g * dh;       // [g][dh]
  float *ms = accV + g * dh, *ls = ms + 16, *al = ls + 16;
  float *lg = al + 16;             // [g][TT]
  float *ks = lg + g * TT;         // [TT][dh+1]
  const TA *qb = q + ((long)b * Hq + (long)h * g) * dh;
  for (int i = tid; i < g * dh; i += 256) { qs[i] = ldf(qb, i); accV[i] = 0.f; }
  if (tid < g) { ms[tid] = -INFINITY; ls[tid] = 0.f; al[tid] = 0.f; }
  __syncthreads();
  const TA *kb = k + (long)b * bstride + (long)h * n * dh;
  const TA *vb = v + (long)b * bstride + (long)h * n * dh;
  const int t_end = min(n, (split + 1) * tps);
  for (int t0 = split * tps; t0 < t_end; t0 += TT) {
    const int nt = min(TT, t_end - t0);
    for (int idx = tid; idx < nt * dh; idx += 256) {
      const int t = idx / dh, d = idx % dh;
      ks[t * kst + d] = ldf(kb, (long)(t0 + t) * dh + d);
    }
    __syncthreads();
    for (int idx = tid; idx < g * nt; idx += 256) {
      const int gi = idx / nt, t = idx % nt;
      float s = 0.f;
      for (int d = 0; d < dh; ++d) s = fmaf(qs[gi * dh + d], ks[t * kst + d], s);
      lg[gi * TT + t] = s * scale_log2;
    }
    __syncthreads();
    softmax_tile(lg, TT, nt, g, ms, ls, al);
    __syncthreads();
    for (int idx = tid; idx < g * dh; idx += 256) {
      const int gi = idx / dh, d = idx % dh;
      float acc = accV[idx] * al[gi];
      for (int t = 0; t < nt; ++t) acc = fmaf(lg[gi * TT + t], ldf(vb, (long)(t0 + t) * dh + d), acc);
      accV[idx] = acc;
    }
    __syncthreads();
  }
  float *pp = part + (((long)b * Hkv + h) * n_split + split) * g * PW;
  for (int gi = 0; gi < g; ++gi) {
    if (tid == 0) { pp[gi * PW] = ms[gi]; pp[gi * PW + 1] = ls[gi]; pp[gi * PW + 2] = 0.f; pp[gi * PW + 3] = 0.f; }
    for (int d = tid; d < dh; d += 256) pp[gi * PW + 4 + d] = accV[gi * dh + d];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_select(int act, const void *q, long q_bstride, const void *basis,
                         const float *landmark, int B, int Hq, int Hkv, int dh, int r, int n_c,
                         int D, int layer, int k_eff, int32_t *sel, int32_t *sel_out,
                         double *scores, hipStream_t st) {
  const size_t smem = ((sizeof(TopkSmem) + 15) & ~size_t(15)) + sizeof(double) * (dh + r + n_c) +
                      sizeof(int32_t) * (k_eff > 0 ? k_eff : 0);
  dim3 grid(Hkv, B);
  allow_dynamic_lds(act == LOWRAM_F32 ? (const void *)k_select<float> : (const void *)k_select<bf16>, smem);
  if (act == LOWRAM_F32)
    hipLaunchKernelGGL(k_select<float>, grid, dim3(256), smem, st, (const float *)q, q_bstride,
                       (const float *)basis, landmark, Hq, Hkv, dh, r, n_c, D, layer, k_eff, sel,
                       sel_out, scores);
  else
    hipLaunchKernelGGL(k_select<bf16>, grid, dim3(256), smem, st, (const bf16 *)q, q_bstride,
                       (const bf16 *)basis, landmark, Hq, Hkv, dh, r, n_c, D, layer, k_eff, sel,
                       sel_out, scores);
  return hipGetLastError();
}

size_t valu_smem_bytes(int g, int dh, int r, int F, int TT) {
  return sizeof(float) * ((size_t)2 * g * dh + (size_t)g * F + 48 + (size_t)g * TT +
                          (size_t)TT * (r + dh + F));
}

int valu_tile(int g, int dh, int r, int F) {
  int TT = 64;
  while (TT > 4 && valu_smem_bytes(g, dh, r, F, TT) > 64 * 1024) TT /= 2;
  return TT;
}

hipError_t launch_attend_valu(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st) {
  const int TT = valu_tile(a.g, a.dh, a.r, a.F);
  const size_t smem = valu_smem_bytes(a.g, a.dh, a.r, a.F, TT);
  dim3 grid(a.n_split + 1, a.Hkv, a.B);
  if (act == LOWRAM_F32) {
    hipLaunchKernelGGL((k_attend_valu<float, float, float>), grid, dim3(256), smem, st, a, TT);
  } else if (coeff == LOWRAM_BF16 && resid == LOWRAM_BF16) {
    hipLaunchKernelGGL((k_attend_valu<bf16, bf16, bf16>), grid, dim3(256), smem, st, a, TT);
  } else if (coeff == LOWRAM_I8 && resid == LOWRAM_I8) {
    hipLaunchKernelGGL((k_attend_valu<bf16, int8_t, int8_t>), grid, dim3(256), smem, st, a, TT);
  } else if (coeff == LOWRAM_I8) {
    hipLaunchKernelGGL((k_attend_valu<bf16, int8_t, bf16>), grid, dim3(256), smem, st, a, TT);
  } else {
    hipLaunchKernelGGL((k_attend_valu<bf16, bf16, int8_t>), grid, dim3(256), smem, st, a, TT);
  }
  return hipGetLastError();
}

hipError_t launch_combine(int act, const CombineArgs &a, hipStream_t st) {
  const size_t smem = sizeof(float) * ((size_t)a.n_total + a.F + 8);
  dim3 grid(a.Hq, a.B);
  if (act == LOWRAM_F32)
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), smem, st, a);
  else
    hipLaunchKernelGGL(k_combine<bf16>, grid, dim3(256), smem, st, a);
  return hipGetLastError();
}

hipError_t launch_dense(int act, const void *q, const void *k, const void *v, long batch_stride,
                        int B, int Hq, int Hkv, int dh, int n, int tps, int n_split, float *part,
                        int PW, hipStream_t st) {
  const int g = Hq / Hkv;
  const size_t smem = sizeof(float) * ((size_t)2 * g * dh + 48 + (size_t)g * 64 + (size_t)64 * (dh + 1));
  dim3 grid(n_split, Hkv, B);
  const float sl = 1.4426950408889634f / sqrtf((float)dh);
  if (act == LOWRAM_F32)
    hipLaunchKernelGGL(k_dense<float>, grid, dim3(256), smem, st, (const float *)q,
                       (const float *)k, (const float *)v, batch_stride, Hq, Hkv, dh, n, tps,
                       n_split, part, PW, sl);
  else
    hipLaunchKernelGGL(k_dense<bf16>, grid, dim3(256), smem, st, (const bf16 *)q, (const bf16 *)k,
                       (const bf16 *)v, batch_stride, Hq, Hkv, dh, n, tps, n_split, part, PW, sl);
  return hipGetLastError();
}

}  // namespace lowram
