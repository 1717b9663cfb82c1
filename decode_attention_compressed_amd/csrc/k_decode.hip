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
#include "select_partial.hpp"

namespace lowram {

// ---------------------------------------------------------------------------
// D1-D3 in two wide kernels (the scorer reads the basis slices of all heads
// and every landmark; spreading it over hundreds of workgroups keeps those
// reads in flight together):
//   k_select_partial q~_{b,h} = U_{l,h}^T sum_{g in group(h)} q_g, and the
//                    partial scores q~ . landmark_{b,j} of one rank block  (float64)
//   k_topk_small     n_c <= 256: s_{b,h,j}, the blocks' partials summed in block
//                    order, and the top min(k, n_c) chunks per (b, h) by
//                    (s desc, j asc), ascending
//   k_select_sum     n_c > 256: s_{b,h,j} as above, then k_topk selects
// Every score is reduced in the same fixed order (lane partials, then a
// butterfly), so equal landmark rows give equal scores.
// ---------------------------------------------------------------------------
// scores[b][h][j] = sum over rank blocks rb (in order) of part[b][h][rb][j].
// grid (ceil(n_c / 256), Hkv, B), 256 threads.
// p[0] + p[n] + p[2 n] + ... over NRB rank blocks, added in block order.  The
// loads go out eight at a time (NRB is a runtime count), so that the sum
// waits for one round trip per eight blocks rather than one per block.
__device__ __forceinline__ double sum_rank_blocks(const double *__restrict__ p, int NRB, int n) {
  double s = 0.0;
  for (int rb0 = 0; rb0 < NRB; rb0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = rb0 + u < NRB ? p[(long)(rb0 + u) * n] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (rb0 + u < NRB) s = rb0 + u == 0 ? v[u] : s + v[u];
  }
  return s;
}

__global__ __launch_bounds__(256) void k_select_sum(const double *__restrict__ part, int Hkv, int n_c,
                                                    int NRB, double *__restrict__ scores) {
  const int j = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (j >= n_c) return;
  scores[((long)b * Hkv + h) * n_c + j] = sum_rank_blocks(part + ((long)b * Hkv + h) * NRB * n_c + j, NRB, n_c);
}

constexpr int TK_NT = 1024;

// grid (Hkv, B), 1024 threads, any n_c.  dynamic LDS: keys [n_c] u64, sel [k].
__global__ __launch_bounds__(TK_NT) void k_topk(const double *__restrict__ scores, int Hkv, int n_c,
                                                int k_eff, int32_t *__restrict__ sel,
                                                int32_t *__restrict__ sel_out) {
  extern __shared__ __align__(16) unsigned char tsm[];
  __shared__ TopkSmem tk;
  uint64_t *key = reinterpret_cast<uint64_t *>(tsm);
  int32_t *sl = reinterpret_cast<int32_t *>(key + n_c);
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const double *sc = scores + ((long)b * Hkv + h) * n_c;
  for (int j = tid; j < n_c; j += TK_NT) key[j] = f64_order_key(sc[j]);
  __syncthreads();
  block_topk<TK_NT>([&](int i) { return key[i]; }, n_c, k_eff, sl, tk, 0, nullptr);
  __syncthreads();
  for (int i = tid; i < k_eff; i += TK_NT) {
    sel[((long)b * Hkv + h) * k_eff + i] = sl[i];
    if (sel_out) sel_out[((long)b * Hkv + h) * k_eff + i] = sl[i];
  }
}

// grid (Hkv, B), 1024 threads, n_c <= 256.  A chunk's score is the sum of its
// NRB rank-block partials in block order (the sum k_select_sum forms), taken
// here so that no separate launch is needed.  Four threads per chunk j each
// count, over a quarter of the chunks, those ranked above j (higher score, or
// equal score and lower index); j is kept iff fewer than k are in total.
// Positions in the output follow chunk order.
constexpr int TK_SMALL = 256;
__global__ __launch_bounds__(TK_NT) void k_topk_small(const double *__restrict__ part, int NRB, int Hkv,
                                                      int n_c, int k_eff, int32_t *__restrict__ sel,
                                                      int32_t *__restrict__ sel_out) {
  __shared__ __align__(16) double s[TK_SMALL];
  __shared__ int32_t cnt[4][TK_SMALL];
  __shared__ TopkSmem tk;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = tid % TK_SMALL, qp = tid / TK_SMALL;
  if (tid < TK_SMALL) s[tid] = tid < n_c ? sum_rank_blocks(part + ((long)b * Hkv + h) * NRB * n_c + tid, NRB, n_c)
                                         : -INFINITY;
  __syncthreads();
  const double mine = s[j];
  int above = 0;
#pragma unroll
  for (int i0 = 0; i0 < TK_SMALL / 4; i0 += 8) {
    double v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = s[qp * (TK_SMALL / 4) + i0 + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = qp * (TK_SMALL / 4) + i0 + e;
      above += (i < j) ? (v[e] >= mine) : (v[e] > mine);
    }
  }
  cnt[qp][j] = above;
  __syncthreads();
  const bool take = tid < n_c && (cnt[0][tid] + cnt[1][tid]) + (cnt[2][tid] + cnt[3][tid]) < k_eff;
  uint32_t pos, p2, tot, t2;
  block_exclusive_counts<TK_NT>(take, false, pos, p2, tot, t2, tk);
  if (take) {
    sel[((long)b * Hkv + h) * k_eff + pos] = tid;
    if (sel_out) sel_out[((long)b * Hkv + h) * k_eff + pos] = tid;
  }
}

// st(i, ld(i)) for i = threadIdx.x, + 256, ... < n, with eight of a thread's
// loads in flight at a time (ld is called on indices clamped into [0, n)).
template <typename Ld, typename St>
__device__ __forceinline__ void batched_copy(int n, Ld ld, St st) {
  constexpr int NB = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += 256 * NB) {
    float v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = ld(min(i0 + 256 * u, n - 1));
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i0 + 256 * u < n) st(i0 + 256 * u, v[u]);
  }
}

// ---------------------------------------------------------------------------
// D4-D6 on the vector ALUs.  grid (n_split + 1, Hkv, B), 256 threads; split
// slot * vsub + range takes one token range of the slot's chunk, and the last
// split of each (b, h) is the tail.  TT tokens per tile.  Global reads are
// issued several at a time (staging, coefficient tiles, residual rows), and
// the inner products are unrolled so that their LDS reads are in flight
// together (each still sums in index order).
// ---------------------------------------------------------------------------
template <typename TA, typename TC, typename TR, bool STAGE>
__global__ __launch_bounds__(256) void k_attend_valu(const AttendArgs a, int TT) {  // STAGE: U and W1 in LDS
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
    tail_split<TA>(a, h, b, qs, lg, TT, accV, ms, ls, al, cb, 0, a.T);
    write_partial(a, h, b, split, ms, ls, nullptr, accV);
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
  // with STAGE the basis slice [dh][r] and W1 [F][dh] are read once into LDS
  // (as fp32, after the tile region) instead of element by element per token.
  // Rows are padded by one word: neighbouring threads read neighbouring rows.
  float *Ul = hb + TT * F, *W1l = Ul + dh * (r + 1);
  if (STAGE) {
    batched_copy(dh * r, [&](int i) { return ldf(U, i); },
                 [&](int i, float v) { Ul[(i / r) * (r + 1) + i % r] = v; });
    batched_copy(F * dh, [&](int i) { return ldf(W1, i); },
                 [&](int i, float v) { W1l[(i / dh) * (dh + 1) + i % dh] = v; });
    __syncthreads();
  }

  // split = slot * vsub + range: tokens [range * C / vsub, (range + 1) * C / vsub)
  // of the slot's chunk
  const int cr = C / a.vsub, slot0 = split / a.vsub, tr0 = (split % a.vsub) * cr;
  for (int slot = slot0; slot < slot0 + 1 && slot < a.k_eff; ++slot) {
    const int j = selp[slot];
    const int e0 = rptr[j], e1 = rptr[j + 1];
    for (int t0 = tr0; t0 < tr0 + cr; t0 += TT) {
      const int nt = min(TT, tr0 + cr - t0);
      const long row0 = (long)j * C + t0;
      batched_copy(nt * r, [&](int idx) { return ld_coeff(cf, row0 * r + idx, csc, idx % r); },
                   [&](int idx, float v) { cb[idx] = v; });
      __syncthreads();
      for (int idx = tid; idx < nt * dh; idx += 256) {
        const int t = idx / dh, d = idx % dh;
        const TA *ur = U + (long)d * r;
        const float *ul = Ul + d * (r + 1);
        float s = 0.f;
#pragma unroll 8
        for (int i = 0; i < r; ++i) s = fmaf(STAGE ? ul[i] : ldf(ur, i), cb[t * r + i], s);
        kh[idx] = s;
      }
      __syncthreads();
      for (int idx = tid; idx < g * nt; idx += 256) {
        const int gi = idx / nt, t = idx % nt;
        float s = 0.f;
#pragma unroll 8
        for (int d = 0; d < dh; ++d) s = fmaf(qs[gi * dh + d], kh[t * dh + d], s);
        lg[gi * TT + t] = s * a.scale_log2;
      }
      for (int idx = tid; idx < nt * F; idx += 256) {
        const int t = idx / F, f = idx % F;
        const TA *wr = W1 + (long)f * dh;
        const float *wl = W1l + f * (dh + 1);
        float s = ldf(B1, f);
#pragma unroll 8
        for (int d = 0; d < dh; ++d) s = fmaf(STAGE ? wl[d] : ldf(wr, d), kh[t * dh + d], s);
        hb[idx] = silu_f(s);
      }
      __syncthreads();
      softmax_tile(lg, TT, nt, g, ms, ls, al);
      __syncthreads();
      for (int idx = tid; idx < g * F; idx += 256) {
        const int gi = idx / F, f = idx % F;
        float acc = accH[idx] * al[gi];
#pragma unroll 8
        for (int t = 0; t < nt; ++t) acc = fmaf(lg[gi * TT + t], hb[t * F + f], acc);
        accH[idx] = acc;
      }
      for (int idx = tid; idx < g * dh; idx += 256) {
        const int gi = idx / dh, d = idx % dh;
        float acc = accV[idx] * al[gi];
        for (int eb = e0; eb < e1; eb += 8) {  // eight rows' loads in flight, added in order
          int tr[8];
          float rv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int e = min(eb + u, e1 - 1);
            tr[u] = ridx[e] - (int)row0;
            rv[u] = ld_coeff(rval, (long)e * dh + d, rsc, d);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (eb + u < e1 && tr[u] >= 0 && tr[u] < nt) acc = fmaf(lg[gi * TT + tr[u]], rv[u], acc);
        }
        accV[idx] = acc;
      }
      __syncthreads();
    }
  }
  write_partial(a, h, b, split, ms, ls, accH, accV);
}

// ---------------------------------------------------------------------------
// D7: merge the splits of each query head and apply W2 / b2 once.
// grid (Hq, B), 256 threads.  Split partials pass through LDS in batches of
// CB splits, every load of a batch issued before any is used; all sums run in
// a fixed order.
// ---------------------------------------------------------------------------
constexpr int CB = 16;

template <typename TA>
__global__ __launch_bounds__(256) void k_combine(const CombineArgs a) {
  extern __shared__ __align__(16) float csm[];
  const int gq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int h = (gq * a.Hkv) / a.Hq, gi = gq - h * a.g;
  const int n_out = a.F + a.dh;
  float *wts = csm;                      // [n_total]
  float *ls = wts + a.n_total;           // [n_total]
  float *mc = ls + a.n_total;            // [n_total] part of l from rebuilt tokens
  float *acc = mc + a.n_total;           // [F + dh]: accH then accV
  float *red = acc + n_out;              // [8]
  float *stage = red + 8;                // [CB][n_out]
  const float *p = a.part + ((long)b * a.Hkv + h) * a.n_total * a.g * a.PW + (long)gi * a.PW;
  if (a.rclock && gi == 0 && tid == 0) a.rclock[((long)b * a.G + a.layer) * a.Hkv + h] += 1;
  const long sstride = (long)a.g * a.PW;
  float mx = -INFINITY;
  for (int s = tid; s < a.n_total; s += 256) {
    const float m = p[s * sstride];
    wts[s] = m;
    ls[s] = p[s * sstride + 1];
    mc[s] = p[s * sstride + 2];
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int s = tid; s < a.n_total; s += 256) wts[s] = (wts[s] == -INFINITY) ? 0.f : exp2f(wts[s] - M);
  for (int o = tid; o < n_out; o += 256) acc[o] = 0.f;
  // 16-byte pieces of one split's [accH | accV] row; threads are laid out as
  // (split offset, piece) with a power-of-two piece stride (no divisions)
  const int per_split = n_out / 4;
  const int pstride = per_split <= 64 ? 64 : (per_split <= 128 ? 128 : 256);
  const int sub = 256 / pstride, pc = tid % pstride, so = tid / pstride;
  const int bsz = CB * sub;  // splits per batch: each thread loads CB pieces
  for (int s0 = 0; s0 < a.n_total; s0 += bsz) {
    const int nb = min(bsz, a.n_total - s0);
    __syncthreads();
    u32x4 v[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {  // all of this thread's loads of the batch in flight together
      const int sl = min(s0 + so + u * sub, a.n_total - 1);
      v[u] = gld16(p + sl * sstride + 4 + 4 * min(pc, per_split - 1));
    }
#pragma unroll
    for (int u = 0; u < CB; ++u)
      if (so + u * sub < nb && pc < per_split) lst16(stage + (so + u * sub) * n_out + 4 * pc, v[u]);
    __syncthreads();
    for (int o = tid; o < n_out; o += 256) {
      // hidden sums only from the rows that rebuilt chunks (a tail-only row's
      // hidden sums are zero and its kernel need not write them)
      const int nu = o < a.F ? min(nb, max(a.n_comp - s0, 0)) : nb;
      float vv = acc[o];
      for (int u = 0; u < nu; ++u) vv = fmaf(wts[s0 + u], stage[u * n_out + o], vv);
      acc[o] = vv;
    }
  }
  __syncthreads();
  float L = 0.f, mass = 0.f;  // same order in every thread
  for (int s = 0; s < a.n_total; ++s) {
    L += wts[s] * ls[s];
    mass += wts[s] * mc[s];
  }
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;
  const bool hoisted = a.F > 0 && a.n_comp > 0;  // W2/b2 only when rebuilt chunks contributed
  const TA *W2 = hoisted ? reinterpret_cast<const TA *>(a.w2) + bh * a.dh * a.F : nullptr;
  const TA *B2 = hoisted ? reinterpret_cast<const TA *>(a.b2) + bh * a.dh : nullptr;
  TA *out = reinterpret_cast<TA *>(a.out) + ((long)b * a.Hq + gq) * a.dh;
  const float invL = 1.0f / L;
  // out[d] = (W2[d] . accH + b2[d] mass + accV[d]) / L.  The block splits each
  // W2 row into tpr contiguous segments; a thread dots its segment with accH
  // (16-byte loads, eight in flight), the segment sums of a row are added in a
  // fixed order through LDS.
  float *rs = stage;  // [256] partial row sums (stage is free now)
  const int tpr = 256 / a.dh;  // 1, 2 or 4 threads per row
  const int d = tid / tpr, sg = tid % tpr;
  float sv = 0.f;
  if (hoisted) {
    constexpr int PER = 16 / sizeof(TA);
    const int seg = a.F / tpr;  // a multiple of 16
    const TA *wr = W2 + (long)d * a.F + sg * seg;
    const float *hv = acc + sg * seg;
    for (int f0 = 0; f0 < seg; f0 += 8 * PER) {
      u32x4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = gld16(wr + min(f0 + u * PER, seg - PER));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const TA *e = reinterpret_cast<const TA *>(&raw[u]);
        if (f0 + u * PER < seg)
#pragma unroll
          for (int j = 0; j < PER; ++j) sv = fmaf(to_f32(e[j]), hv[f0 + u * PER + j], sv);
      }
    }
  }
  rs[tid] = sv;
  __syncthreads();
  if (sg == 0) {
    float v = 0.f;
    for (int k = 0; k < tpr; ++k) v += rs[tid + k];
    if (hoisted) v = fmaf(ldf(B2, d), mass, v);
    store_f32(out + d, (v + acc[a.F + d]) * invL);
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
// Dense split-K decode attention for bf16 caches on the matrix cores.
// grid (n_split, Hkv, B), 256 threads; 64-token tiles.  Logits: each wave
// feeds its 16 tokens' key rows straight from global memory as the A operand
// of a 16x16x32 bf16 MFMA against the zero-padded queries.  Values: each
// thread loads the rows of a token pair for 8 head dims and stores them
// transposed into LDS (fp16, one dword per head dim and token pair, so a
// wave's stores fall in distinct banks); p . V is then a 16x16x32 fp16 MFMA
// per 16 head dims and 32 tokens, with p rounded to fp16 (the softmax
// denominator sums the same rounded p).  The next tile's keys and values are
// in flight in registers while the current tile is reduced.
// ---------------------------------------------------------------------------
typedef __bf16 dbf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 df16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float df32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef u32x4 dvec4;

__device__ __forceinline__ uint32_t dense_h2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

template <int DH>
__global__ __launch_bounds__(256) void k_dense_mfma(const uint16_t *__restrict__ q,
                                                    const uint16_t *__restrict__ k,
                                                    const uint16_t *__restrict__ v, long bstride,
                                                    int Hq, int Hkv, int n, int tps, int n_split,
                                                    float *__restrict__ part, int PW, float scale_log2) {
  constexpr int TT = 64, NK = DH / 32;
  constexpr int VT_LD = TT + 8;                        // transposed V row (one head dim), fp16
  constexpr int NPP = DH / 8;                          // 8-dim parts of a row
  constexpr int NVI = (TT / 2) * NPP / 256;            // (token pair, part) items per thread
  constexpr int NDT = DH / 64;                         // 16-dim output tiles per wave
  __shared__ __align__(16) uint16_t Vt[DH * VT_LD];
  __shared__ __align__(16) uint16_t Pt[16 * VT_LD];    // p [head][token] fp16 (rows past the group zero)
  __shared__ float red[64], red2[64], ms[16], ls[16], al[16];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, gi = lane & 15, l16 = lane & 15, kg = lane >> 4;
  const int g = Hq / Hkv;
  const uint16_t *kb = k + (long)b * bstride + (long)h * n * DH;
  const uint16_t *vb = v + (long)b * bstride + (long)h * n * DH;
  dbf16x8 qf[NK];
  {
    const uint16_t *qr = q + ((long)b * Hq + (long)h * g + gi) * DH;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      u32x4 u = v4(0, 0, 0, 0);
      if (gi < g) u = gld16(qr + 32 * ks + 8 * kg);
      qf[ks] = __builtin_bit_cast(dbf16x8, u);
    }
  }
  if (tid < 16) { ms[tid] = -INFINITY; ls[tid] = 0.f; al[tid] = 0.f; }
  df32x4 oacc[NDT];   // out^T[d][head]: lane (head l16, dims 4 kg + v of tile dt)
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = df32x4{0.f, 0.f, 0.f, 0.f};
  const int t_beg = split * tps, t_end = min(n, t_beg + tps);
  dvec4 kr[NK], vr[NVI][2];
  auto fetch = [&](int t0) {
    // rows past the split's end are clamped to its last row: the loads stay
    // unconditional, and those rows get p = 0
    const int t = min(t0 + 16 * w + l16, t_end - 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      kr[ks] = *reinterpret_cast<const dvec4 *>(kb + (long)t * DH + 32 * ks + 8 * kg);
#pragma unroll
    for (int u = 0; u < NVI; ++u) {
      const int it = tid + 256 * u, j = it % (TT / 2), pt = it / (TT / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        vr[u][e] = *reinterpret_cast<const dvec4 *>(vb + (long)min(t0 + 2 * j + e, t_end - 1) * DH + 8 * pt);
    }
  };
  if (t_beg < t_end) fetch(t_beg);
  __syncthreads();
  for (int t0 = t_beg; t0 < t_end; t0 += TT) {
    df32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dbf16x8, kr[ks]), qf[ks], acc, 0, 0, 0);
    // values transposed into LDS: dword (d, token pair j) = (v[2j][d], v[2j + 1][d]) in fp16
#pragma unroll
    for (int u = 0; u < NVI; ++u) {
      const int it = tid + 256 * u, j = it % (TT / 2), pt = it / (TT / 2);
      const uint16_t *a0 = reinterpret_cast<const uint16_t *>(&vr[u][0]);
      const uint16_t *a1 = reinterpret_cast<const uint16_t *>(&vr[u][1]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t *>(Vt + (8 * pt + i) * VT_LD + 2 * j) =
            dense_h2(bf16_bits_to_f32(a0[i]), bf16_bits_to_f32(a1[i]));
    }
    if (t0 + TT < t_end) fetch(t0 + TT);
    float mx = -INFINITY;
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * w + 4 * kg + i;
      lg[i] = t < t_end ? acc[i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, lg[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lane < 16) red[w * 16 + gi] = mx;
    __syncthreads();
    const float m_old = ms[gi];
    const float m_new = fmaxf(m_old, fmaxf(fmaxf(red[gi], red[16 + gi]), fmaxf(red[32 + gi], red[48 + gi])));
    float psum = 0.f;
    {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (gi < g && lg[i] != -INFINITY) ? exp2f(lg[i] - m_new) : 0.f;
        pv[i] = (float)(_Float16)p;
        psum += pv[i];
      }
      *reinterpret_cast<uint2 *>(Pt + gi * VT_LD + 16 * w + 4 * kg) =
          make_uint2(dense_h2(pv[0], pv[1]), dense_h2(pv[2], pv[3]));
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (lane < 16) red2[w * 16 + gi] = psum;
    __syncthreads();
    if (tid < 16) {
      const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
      al[tid] = alpha;
      ls[tid] = ls[tid] * alpha + ((red2[tid] + red2[16 + tid]) + (red2[32 + tid] + red2[48 + tid]));
      ms[tid] = m_new;
    }
    __syncthreads();
    {  // out^T[d][head] = alpha out^T + V^T p^T over the tile's 64 tokens
      const float a_h = al[l16];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= a_h;
        const int d = (w * NDT + dt) * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < TT / 32; ++ks)
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              *reinterpret_cast<const df16x8 *>(Vt + d * VT_LD + 32 * ks + 8 * kg),
              *reinterpret_cast<const df16x8 *>(Pt + l16 * VT_LD + 32 * ks + 8 * kg), oacc[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  float *pp = part + (((long)b * Hkv + h) * n_split + split) * g * PW;
  if (tid < g) { pp[tid * PW] = ms[tid]; pp[tid * PW + 1] = ls[tid]; pp[tid * PW + 2] = 0.f; pp[tid * PW + 3] = 0.f; }
  if (l16 < g)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[l16 * PW + 4 + (w * NDT + dt) * 16 + 4 * kg + i] = oacc[dt][i];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename TA, int QG>
static void launch_partial_g(const TA *q, long q_bstride, const TA *basis, const float *landmark, int B,
                             int Hq, int Hkv, int dh, int r, int n_c, int D, int layer, double *part,
                             const QOut &qo, hipStream_t st, int k_eff = 0, int32_t *sel = nullptr,
                             int32_t *sel_out = nullptr) {
  const dim3 g(select_rank_blocks(r), Hkv, B);
  if (dh == 64)
    hipLaunchKernelGGL((k_select_partial<TA, 64, QG>), g, dim3(256), 0, st, q, q_bstride, basis, landmark, Hq, Hkv, r, n_c, D, layer, part, qo.qtg, qo.qfrag, qo.scale, qo.mode, k_eff, sel, sel_out);
  else if (dh == 128)
    hipLaunchKernelGGL((k_select_partial<TA, 128, QG>), g, dim3(256), 0, st, q, q_bstride, basis, landmark, Hq, Hkv, r, n_c, D, layer, part, qo.qtg, qo.qfrag, qo.scale, qo.mode, k_eff, sel, sel_out);
  else
    hipLaunchKernelGGL((k_select_partial<TA, 256, QG>), g, dim3(256), 0, st, q, q_bstride, basis, landmark, Hq, Hkv, r, n_c, D, layer, part, qo.qtg, qo.qfrag, qo.scale, qo.mode, k_eff, sel, sel_out);
}
template <typename TA>
static void launch_partial(const TA *q, long q_bstride, const TA *basis, const float *landmark, int B,
                           int Hq, int Hkv, int dh, int r, int n_c, int D, int layer, double *part,
                           const QOut &qo, hipStream_t st, int k_eff = 0, int32_t *sel = nullptr,
                           int32_t *sel_out = nullptr) {
  if (qo.qfrag && Hq / Hkv > QTG_G)
    launch_partial_g<TA, QTG_MAX>(q, q_bstride, basis, landmark, B, Hq, Hkv, dh, r, n_c, D, layer, part, qo, st,
                                  k_eff, sel, sel_out);
  else
    launch_partial_g<TA, QTG_G>(q, q_bstride, basis, landmark, B, Hq, Hkv, dh, r, n_c, D, layer, part, qo, st,
                                k_eff, sel, sel_out);
}

hipError_t launch_select(int act, const void *q, long q_bstride, const void *basis,
                         const float *landmark, int B, int Hq, int Hkv, int dh, int r, int n_c,
                         int D, int layer, int k_eff, int32_t *sel, int32_t *sel_out,
                         double *part, double *scores, hipStream_t st, const QOut &qo,
                         const AttendArgs *absorb) {
  // one rank block (r <= 64) and few chunks: the score kernel ranks its own
  // scores, one launch instead of two
  if (!absorb && scores && k_eff > 0 && n_c <= 4 * WAVE && select_rank_blocks(r) == 1) {
    if (act == LOWRAM_F32)
      launch_partial<float>((const float *)q, q_bstride, (const float *)basis, landmark, B, Hq, Hkv, dh, r, n_c, D,
                            layer, part, qo, st, k_eff, sel, sel_out);
    else
      launch_partial<bf16>((const bf16 *)q, q_bstride, (const bf16 *)basis, landmark, B, Hq, Hkv, dh, r, n_c, D,
                           layer, part, qo, st, k_eff, sel, sel_out);
    return hipGetLastError();
  }
  if (absorb) {
    const hipError_t e = launch_select_absorb(*absorb, landmark, part, q_bstride, st);
    if (e != hipSuccess) return e;
  } else if (act == LOWRAM_F32)
    launch_partial<float>((const float *)q, q_bstride, (const float *)basis, landmark, B, Hq, Hkv, dh, r, n_c, D, layer, part, qo, st);
  else
    launch_partial<bf16>((const bf16 *)q, q_bstride, (const bf16 *)basis, landmark, B, Hq, Hkv, dh, r, n_c, D, layer, part, qo, st);
  if (!scores) return k_eff > 0 ? hipErrorInvalidValue : hipGetLastError();
  if (k_eff > 0 && n_c <= TK_SMALL) {  // sums the partials itself
    hipLaunchKernelGGL(k_topk_small, dim3(Hkv, B), dim3(TK_NT), 0, st, part, select_rank_blocks(r), Hkv,
                       n_c, k_eff, sel, sel_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_select_sum, dim3((n_c + 255) / 256, Hkv, B), dim3(256), 0, st, part, Hkv, n_c,
                     select_rank_blocks(r), scores);
  if (k_eff > 0) {
    const size_t sm3 = (size_t)n_c * 8 + sizeof(int32_t) * (size_t)k_eff;
    allow_dynamic_lds(k_topk, sm3);
    hipLaunchKernelGGL(k_topk, dim3(Hkv, B), dim3(TK_NT), sm3, st, scores, Hkv, n_c, k_eff, sel,
                       sel_out);
  }
  return hipGetLastError();
}

size_t valu_smem_bytes(int g, int dh, int r, int F, int TT) {
  // the tail split reuses the tile region for 2*TT*(dh+1) floats of keys/values
  const size_t tile = (size_t)TT * (r + dh + F), tail = (size_t)2 * TT * (dh + 1);
  return sizeof(float) * ((size_t)2 * g * dh + (size_t)g * F + 48 + (size_t)g * TT +
                          (tile > tail ? tile : tail));
}

int valu_tile(int g, int dh, int r, int F) {
  int TT = 64;
  while (TT > 4 && valu_smem_bytes(g, dh, r, F, TT) > 64 * 1024) TT /= 2;
  return TT;
}

template <typename TA, typename TC, typename TR>
static void go_valu(const AttendArgs &a, int TT, size_t smem, bool stage, hipStream_t st) {
  dim3 grid(a.n_split + 1, a.Hkv, a.B);
  if (stage) {
    allow_dynamic_lds(k_attend_valu<TA, TC, TR, true>, smem);
    hipLaunchKernelGGL((k_attend_valu<TA, TC, TR, true>), grid, dim3(256), smem, st, a, TT);
  } else {
    hipLaunchKernelGGL((k_attend_valu<TA, TC, TR, false>), grid, dim3(256), smem, st, a, TT);
  }
}

hipError_t launch_attend_valu(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st) {
  const int TT = valu_tile(a.g, a.dh, a.r, a.F);
  size_t smem = valu_smem_bytes(a.g, a.dh, a.r, a.F, TT);
  const size_t staged = smem + sizeof(float) * ((size_t)a.dh * (a.r + 1) + (size_t)a.F * (a.dh + 1));
  const bool stage = staged <= 160 * 1024;
  if (stage) smem = staged;
  if (act == LOWRAM_F32) go_valu<float, float, float>(a, TT, smem, stage, st);
  else if (coeff == LOWRAM_BF16 && resid == LOWRAM_BF16) go_valu<bf16, bf16, bf16>(a, TT, smem, stage, st);
  else if (coeff == LOWRAM_I8 && resid == LOWRAM_I8) go_valu<bf16, int8_t, int8_t>(a, TT, smem, stage, st);
  else if (coeff == LOWRAM_I8) go_valu<bf16, int8_t, bf16>(a, TT, smem, stage, st);
  else go_valu<bf16, bf16, int8_t>(a, TT, smem, stage, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// D7 for d_h = 128 or 256, bf16, at most 4 query heads per kv head and F a
// multiple of 128: one workgroup per (sequence, kv head, 32 head dims) merges
// the splits of all query heads of the kv head and applies the rows of W2 it
// owns.  Every global read is issued before the first is used (split
// heads first, then W2 rows and b2, hidden sums, value sums): one memory
// round trip, and the split weights are formed while the rest is in flight.
// Sums run in split order, so the result is deterministic.
// grid (d_h / 32, Hkv, B), 256 threads.
// ---------------------------------------------------------------------------
constexpr int KV_DQ = 32;    // head dims per workgroup
constexpr int KV_SB = 16;    // splits whose loads are in flight together

template <int F, int DH>
__global__ __launch_bounds__(256) void k_combine_kv(const CombineArgs a) {
  constexpr int GM = 4, FP = F / 4;                   // float4 pieces of a hidden row
  constexpr int PPT = (GM * FP + 255) / 256;          // (g, piece) pairs per thread
  constexpr int WPT = F / 8 / 8;                      // 16-byte W2 pieces per thread (8 threads per row)
  __shared__ float wt[64][GM];                        // split weights
  __shared__ float fin[GM][3];                        // M, 1/L, mass
  // merged hidden sums
  __shared__ __align__(16) float accHm[GM][F];
  __shared__ float accVm[GM][KV_DQ];
  const int dq = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  // rows past the first n_comp hold tail tokens only: their hidden sums are
  // zero by definition and are neither written nor read
  const int g = a.g, S = a.n_total, nc = a.n_comp;
  const long sstride = (long)g * a.PW;
  const float *p0 = a.part + ((long)b * a.Hkv + h) * S * sstride;
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;
  if (a.rclock && dq == 0 && tid == 0) a.rclock[bh] += 1;  // the attend kernel has read it
  const uint16_t *W2 = reinterpret_cast<const uint16_t *>(a.w2) + (bh * DH + (long)dq * KV_DQ) * F;
  const uint16_t *B2 = reinterpret_cast<const uint16_t *>(a.b2) + bh * DH + dq * KV_DQ;

  // split heads (m, l, mass) first, thread (split tid / GM, head tid % GM):
  // the weights need only them.  Every load below is unconditional (indices
  // clamped into the partials of this (b, h), values past the counts unused),
  // so the wait for the heads covers nothing issued after them.
  static_assert(64 * GM <= 256, "one split head per thread");
  const int hs = tid / GM, hg = tid % GM;
  const bool h_ok = hs < S && hg < g;
  const u32x4 hv = gld16(p0 + (long)min(hs, S - 1) * sstride + (long)min(hg, g - 1) * a.PW);
  // W2 rows of this workgroup and b2 (independent of the partials): thread
  // (row wr, lane ws of 8) takes the 16-byte pieces ws, ws + 8, ... of its
  // row, so the eight threads of a row read 128 contiguous bytes per load
  const int wr = tid >> 3, ws = tid & 7;
  u32x4 w2r[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) w2r[i] = gld16(W2 + (long)wr * F + 8 * (8 * i + ws));
  const float b2v = bf16_bits_to_f32(B2[wr]);
  // hidden and value sums of the first KV_SB splits: thread pairs (gi, piece)
  // and (gi, dd), in flight while the split weights are formed
  const int vg = tid / KV_DQ, vd = tid % KV_DQ;
  f32v4 hp[PPT][KV_SB];
  float vv[KV_SB];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pr = tid + 256 * k, gi = min(pr / FP, g - 1), pc = pr % FP;
#pragma unroll
      for (int u = 0; u < KV_SB; ++u)
        hp[k][u] = *reinterpret_cast<const f32v4 *>(p0 + (long)min(s0 + u, nc - 1) * sstride + (long)gi * a.PW + 4 +
                                                     4 * pc);
    }
#pragma unroll
    for (int u = 0; u < KV_SB; ++u)
      vv[u] = p0[(long)min(s0 + u, S - 1) * sstride + (long)min(vg, g - 1) * a.PW + 4 + F + dq * KV_DQ + vd];
  };
  load_batch(0);
  // all four words of hv live until here: no register of the heads' load is
  // reused (which would wait for it) before the loads above are issued
  asm volatile("" ::"v"(hv.x), "v"(hv.y), "v"(hv.z), "v"(hv.w));
  __builtin_amdgcn_sched_barrier(0);   // and no use of hv is moved above them
  f32v4 hacc[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) hacc[k] = f32v4{0.f, 0.f, 0.f, 0.f};
  // common maximum per head: over the lanes of a wave with the same head
  // (lane bits 2..5), then over the waves
  __shared__ float red[3][4][GM];   // per wave: max, then partial L and mass
  const int lane = tid & 63, wv = tid >> 6;
  const float m_s = h_ok ? __uint_as_float(hv.x) : -INFINITY;
  float mx = m_s;
#pragma unroll
  for (int o = GM; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane < GM) red[0][wv][lane] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0][hg], red[0][1][hg]), fmaxf(red[0][2][hg], red[0][3][hg]));
  const float w_s = m_s == -INFINITY ? 0.f : exp2f(m_s - M);
  if (hs < 64) wt[hs][hg] = w_s;
  // L and the rebuilt-token mass: the same lane tree, then the waves in order
  float lsum = w_s * __uint_as_float(hv.y), msum = w_s * __uint_as_float(hv.z);
  if (!h_ok) lsum = msum = 0.f;
#pragma unroll
  for (int o = GM; o < 64; o <<= 1) {
    lsum += __shfl_xor(lsum, o, 64);
    msum += __shfl_xor(msum, o, 64);
  }
  if (lane < GM) {
    red[1][wv][lane] = lsum;
    red[2][wv][lane] = msum;
  }
  __syncthreads();
  if (tid < g) {
    fin[tid][0] = M;
    fin[tid][1] = 1.0f / (((red[1][0][tid] + red[1][1][tid]) + red[1][2][tid]) + red[1][3][tid]);
    fin[tid][2] = ((red[2][0][tid] + red[2][1][tid]) + red[2][2][tid]) + red[2][3][tid];
  }
  __syncthreads();
  float vsum = 0.f;
  for (int s0 = 0; s0 < S; s0 += KV_SB) {
    const int nb = min(KV_SB, S - s0);
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pr = tid + 256 * k, gi = pr / FP;
      if (gi < g) {
#pragma unroll
        for (int u = 0; u < KV_SB; ++u)
          if (u < nb && s0 + u < nc) {
            const float w = wt[s0 + u][gi];
            hacc[k].x = fmaf(w, hp[k][u].x, hacc[k].x);
            hacc[k].y = fmaf(w, hp[k][u].y, hacc[k].y);
            hacc[k].z = fmaf(w, hp[k][u].z, hacc[k].z);
            hacc[k].w = fmaf(w, hp[k][u].w, hacc[k].w);
          }
      }
    }
    if (vg < g) {
#pragma unroll
      for (int u = 0; u < KV_SB; ++u)
        if (u < nb) vsum = fmaf(wt[s0 + u][vg], vv[u], vsum);
    }
  }
  if (vg < g) accVm[vg][vd] = vsum;
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int pr = tid + 256 * k, gi = pr / FP, pc = pr % FP;
    if (gi < GM) *reinterpret_cast<f32v4 *>(&accHm[gi][4 * pc]) = hacc[k];
  }
  __syncthreads();
  // out[gi][d] = (W2[d] . accH[gi] + b2[d] mass[gi] + accV[gi][d]) / L[gi]
  float dot[GM] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int f0 = 8 * (8 * i + ws);
    const uint32_t wv[4] = {w2r[i].x, w2r[i].y, w2r[i].z, w2r[i].w};
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      const f32v4 h0 = *reinterpret_cast<const f32v4 *>(&accHm[gi][f0]);
      const f32v4 h1 = *reinterpret_cast<const f32v4 *>(&accHm[gi][f0 + 4]);
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot[gi] = fmaf(bf16_bits_to_f32(wv[e] & 0xFFFFu), hv[2 * e], dot[gi]);
        dot[gi] = fmaf(bf16_bits_to_f32(wv[e] >> 16), hv[2 * e + 1], dot[gi]);
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {  // the eight partial dots of a row, fixed order
    dot[gi] += __shfl_xor(dot[gi], 1, 64);
    dot[gi] += __shfl_xor(dot[gi], 2, 64);
    dot[gi] += __shfl_xor(dot[gi], 4, 64);
  }
  if (ws == 0) {
    bf16 *out = reinterpret_cast<bf16 *>(a.out) + ((long)b * a.Hq + (long)h * g) * DH + dq * KV_DQ + wr;
    for (int gi = 0; gi < g; ++gi)
      store_f32(out + (long)gi * DH, (dot[gi] + fmaf(b2v, fin[gi][2], accVm[gi][wr])) * fin[gi][1]);
  }
}

hipError_t launch_combine(int act, const CombineArgs &a, hipStream_t st) {
  if (act == LOWRAM_BF16 && a.F > 0 && a.n_comp > 0 && (a.dh == 128 || a.dh == 256) && a.g <= 4 &&
      a.n_total <= 64) {
    const dim3 grid(a.dh / KV_DQ, a.Hkv, a.B);
#define LOWRAM_COMBINE_KV(FF, DD)                                                   \
    if (a.F == FF && a.dh == DD) {                                                  \
      hipLaunchKernelGGL((k_combine_kv<FF, DD>), grid, dim3(256), 0, st, a);        \
      return hipGetLastError();                                                     \
    }
    LOWRAM_COMBINE_KV(128, 128) LOWRAM_COMBINE_KV(256, 128) LOWRAM_COMBINE_KV(512, 128)
    LOWRAM_COMBINE_KV(128, 256) LOWRAM_COMBINE_KV(256, 256) LOWRAM_COMBINE_KV(512, 256)
#undef LOWRAM_COMBINE_KV
  }
  // stage: CB * sub splits of (F + dh) floats, sub = 256 / (piece stride) <= 1024 / (F + dh)
  const int n_out = a.F + a.dh, per = n_out / 4;
  const int sub = 256 / (per <= 64 ? 64 : (per <= 128 ? 128 : 256));
  const size_t stage = (size_t)CB * sub * n_out > 256 ? (size_t)CB * sub * n_out : 256;
  const size_t smem = sizeof(float) * ((size_t)3 * a.n_total + n_out + 8 + stage);
  dim3 grid(a.Hq, a.B);
  allow_dynamic_lds(act == LOWRAM_F32 ? (const void *)k_combine<float> : (const void *)k_combine<bf16>, smem);
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
  else if (dh == 128)
    hipLaunchKernelGGL(k_dense_mfma<128>, grid, dim3(256), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, batch_stride, Hq, Hkv, n, tps,
                       n_split, part, PW, sl);
  else if (dh == 256)
    hipLaunchKernelGGL(k_dense_mfma<256>, grid, dim3(256), 0, st, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, batch_stride, Hq, Hkv, n, tps,
                       n_split, part, PW, sl);
  else
    hipLaunchKernelGGL(k_dense<bf16>, grid, dim3(256), smem, st, (const bf16 *)q, (const bf16 *)k,
                       (const bf16 *)v, batch_stride, Hq, Hkv, dh, n, tps, n_split, part, PW, sl);
  return hipGetLastError();
}

}  // namespace lowram
