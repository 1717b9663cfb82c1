// Partial chunk scores of the selection stage and q~ = U_{l,h}^T q, in a
// form both the selection launch and the absorbed-path launch (which runs it
// beside the formation of A) can call.
//
// Method: the chunk scorer maps the group-summed query into coefficient space
// and scores each chunk's mean coefficient (rit.work LowRAM page, generation
// section), in float64.
#pragma once
#include "common.hpp"
#include "internal.hpp"
#include "attend_common.hpp"

namespace lowram {

// 8 consecutive basis values of one row as float64
template <typename TA> struct Load8;
template <> struct Load8<bf16> {
  typedef u32x4 raw;
  static constexpr int N = 1;
  __device__ static void ld(const bf16 *p, raw *v) { v[0] = gld16(p); }
  __device__ static void f64(const raw *v, double *o) {
    const uint32_t w[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = (double)bf16_bits_to_f32(w[i] & 0xFFFFu);
      o[2 * i + 1] = (double)bf16_bits_to_f32(w[i] >> 16);
    }
  }
};
template <> struct Load8<float> {
  typedef u32x4 raw;
  static constexpr int N = 2;
  __device__ static void ld(const float *p, raw *v) { v[0] = gld16(p); v[1] = gld16(p + 4); }
  __device__ static void f64(const raw *v, double *o) {
    const uint32_t w[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (double)__uint_as_float(w[i]);
  }
};

// Sums R rows of per-lane partials over the lanes that differ in the log2 R
// lane bits OFF0, OFF0 / 2, ... (R a power of two).  Each step also
// transposes: over lane bit k a lane keeps the half of its rows that its bit
// selects and adds the partner's partials of those rows, so one value per
// lane remains.  Every row is summed by the same pairwise tree whatever its
// position, so equal inputs give equal sums.  On return a lane holds the row
// whose index has the lane's bits OFF0, OFF0 / 2, ... as its binary digits,
// most significant first.
template <int N, int OFF>
__device__ __forceinline__ void xpose_step(double *v, int lane) {
  if constexpr (N > 1) {
    const bool hi = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const double keep = hi ? v[N / 2 + i] : v[i];
      const double send = hi ? v[i] : v[N / 2 + i];
      v[i] = keep + __shfl_xor(send, OFF, WAVE);
    }
    xpose_step<N / 2, OFF / 2>(v, lane);
  }
}
template <int R, int OFF0>
__device__ __forceinline__ double xpose_sum(double (&v)[R], int lane) {
  static_assert((R & (R - 1)) == 0 && R <= 2 * OFF0, "R a power of two within the lane bits");
  xpose_step<R, OFF0>(v, lane);
  return v[0];
}
template <int N, int OFF>
__device__ __forceinline__ void xpose_step_f32(float *v, int lane) {
  if constexpr (N > 1) {
    const bool hi = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = hi ? v[N / 2 + i] : v[i];
      const float send = hi ? v[i] : v[N / 2 + i];
      v[i] = keep + __shfl_xor(send, OFF, WAVE);
    }
    xpose_step_f32<N / 2, OFF / 2>(v, lane);
  }
}
template <int R, int OFF0>
__device__ __forceinline__ float xpose_sum_f32(float (&v)[R], int lane) {
  xpose_step_f32<R, OFF0>(v, lane);
  return v[0];
}

// D1 and D2 per block of 64 ranks.  grid (ceil(r / 64), Hkv, B), 256 threads;
// block rb of (b, h) writes part[b][h][rb][j] = sum over its ranks i of
// q~_i landmark_{b,j,i}, with q~ = U_{l,h}^T sum_g q_g restricted to the block.
// The chunk score is the sum of the blocks' partials in block order (summed by
// the consumer).  Splitting the rank dimension reads every basis row once and
// each landmark row once per kv head; a split over chunks would make every
// workgroup rebuild the whole q~.
//
// q~ of the block: lane (rank group lane & 7, slice 8 w + (lane >> 3)) sums
// eight ranks over head dims slice + 32 k in ascending k; the wave's eight
// slices are added by a transposing butterfly and the four waves in order.
// Partials: 16 lanes per chunk, four ranks (one 16-byte landmark piece) each,
// sixteen chunk rows in flight per lane, then a transposing butterfly over
// the 16 lanes.  Blocks are regrouped so that the heads of one (sequence,
// rank block) share an XCD and its L2 copy of those landmark columns.
constexpr int SEL_RB = 64;

template <int DH, int QG>
struct SelectSmem {
  double qsum[DH];
  double qtp[4][SEL_RB];
  double qt[SEL_RB];
  float qg[QG][DH];            // q of each query head (q~ outputs only)
  float qtpg[4][QG][SEL_RB];   // per-wave parts of q~_g (q~ outputs only)
};

// (rank block rb, kv head h, sequence b) of block `lin` of NRB * Hkv * B, the
// linear ids taken in (rb, h, b) order.  Workgroups are dispatched round-robin
// over the 8 XCDs (linear id mod 8); the ids are regrouped so that the kv
// heads of one (sequence, rank block) share an XCD.
__device__ __forceinline__ void select_coords(int lin, int NRB, int Hkv, int B, int &rb, int &h, int &b) {
  const int P = NRB * B;  // (sequence, rank block) pairs
  if (P % 8 == 0) {
    const int xcd = lin % 8, i = lin / 8, pr = xcd * (P / 8) + i / Hkv;
    h = i % Hkv; b = pr / NRB; rb = pr % NRB;
  } else {
    rb = lin % NRB; h = (lin / NRB) % Hkv; b = lin / (NRB * Hkv);
  }
}

// One block (rb, h, b) of the partial scores (and of q~ when qtg or qfrag is
// set); 256 threads, all of which call it.
template <typename TA, int DH, int QG>
__device__ __forceinline__ void select_partial_block(SelectSmem<DH, QG> &sm, int rb, int h, int b, int NRB,
                                                     const TA *__restrict__ q, long q_bstride,
                                                     const TA *__restrict__ basis,
                                                     const float *__restrict__ landmark, int Hq,
                                                     int Hkv, int r, int n_c, int D, int layer,
                                                     double *__restrict__ part, float *__restrict__ qtg,
                                                     uint16_t *__restrict__ qfrag,
                                                     const uint16_t *__restrict__ qf_scale, int qf_mode,
                                                     double *lds_scores = nullptr) {
  constexpr int RPS = DH / 32;  // basis rows per slice
  double *qsum = sm.qsum, *qt = sm.qt;
  auto &qtp = sm.qtp;
  auto &qg = sm.qg;
  auto &qtpg = sm.qtpg;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int i0 = rb * SEL_RB, nr = min(SEL_RB, r - i0);  // ranks of this block (a multiple of 16)

  // the group's q values at head dim tid, the first eight heads in one batch
  // of unconditional loads (clamped indices, values past the group unused)
  const int grp = Hq / Hkv;
  const TA *qb = q + (long)b * q_bstride + (long)h * grp * DH;
  constexpr int QB = 8;
  float qg0[QB];
#pragma unroll
  for (int u = 0; u < QB; ++u) qg0[u] = to_f32(qb[min(u, grp - 1) * DH + min(tid, DH - 1)]);
  // basis rows of this thread: rank group rg, head dims sl + 32 k
  const int rg = lane & 7, sl = 8 * w + (lane >> 3);
  const bool rg_ok = 8 * rg < nr;
  const TA *U = basis + ((long)b * D + (long)(layer * Hkv + h) * DH) * r + i0 + 8 * (rg_ok ? rg : 0);
  typename Load8<TA>::raw raw[RPS][Load8<TA>::N];
#pragma unroll
  for (int k = 0; k < RPS; ++k) Load8<TA>::ld(U + (long)(sl + 32 * k) * r, raw[k]);
  // landmark pieces of the first 16 chunk rows (independent of q~)
  const int gq = lane >> 4, li = lane & 15;
  const bool li_ok = 4 * li < nr;
  const float *L = landmark + (long)b * n_c * r + i0 + 4 * (li_ok ? li : 0);
  constexpr int MB = 16;  // chunk rows per lane in flight
  u32x4 lv[MB];
  auto load_rows = [&](int j_base) {
#pragma unroll
    for (int m = 0; m < MB; ++m) lv[m] = gld16(L + (long)min(j_base + 16 * m + 4 * w + gq, n_c - 1) * r);
  };
  load_rows(0);
  if (tid < DH) {
    // summed in head order in float64 (each value is exact in float32); heads
    // past the first eight are loaded eight at a time
    double sq = 0.0;
    auto add = [&](int g0, const float (&v)[QB]) {
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        if (g0 + u < grp) sq += (double)v[u];
        if ((qtg || qfrag) && g0 + u < QG && g0 + u < grp) qg[g0 + u][tid] = v[u];
      }
    };
    add(0, qg0);
    for (int g0 = QB; g0 < grp; g0 += QB) {
      float v[QB];
#pragma unroll
      for (int u = 0; u < QB; ++u) v[u] = to_f32(qb[min(g0 + u, grp - 1) * DH + tid]);
      add(g0, v);
    }
    qsum[tid] = sq;
    if (qtg || qfrag)
      for (int gi = grp; gi < QG; ++gi) qg[gi][tid] = 0.f;
  }
  __syncthreads();
  // q~_g of each query head over the block's ranks, in float32, four heads at
  // a time (groups past the kv head's query heads are skipped: zero rows)
  const int ng4 = (min(grp, QG) + 3) / 4;
  if (qtg || qfrag)
    for (int g4 = 0; g4 < ng4; ++g4) {
      float acc[4][8];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
#pragma unroll
      for (int k = 0; k < RPS; ++k) {
        double u[8];
        Load8<TA>::f64(raw[k], u);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const float wq = qg[4 * g4 + gi][sl + 32 * k];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[gi][e] = fmaf((float)u[e], wq, acc[gi][e]);
        }
      }
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        qtpg[w][4 * g4 + gi][8 * rg + (lane >> 3)] = xpose_sum_f32<8, 32>(acc[gi], lane);  // rank 8 rg + (lane >> 3)
    }
  {
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int k = 0; k < RPS; ++k) {
      double u[8];
      Load8<TA>::f64(raw[k], u);
      const double wq = qsum[sl + 32 * k];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fma(u[e], wq, acc[e]);
    }
    const double v = xpose_sum<8, 32>(acc, lane);  // rank 8 rg + (lane >> 3), this wave's slices
    qtp[w][8 * rg + (lane >> 3)] = v;
  }
  __syncthreads();
  if (tid < SEL_RB) qt[tid] = ((qtp[0][tid] + qtp[1][tid]) + qtp[2][tid]) + qtp[3][tid];
  if (qtg)  // [b][h][QG][r]; rows past the group are zero
    for (int it = tid; it < QG * SEL_RB; it += 256) {
      const int gi = it / SEL_RB, ri = it % SEL_RB;
      if (ri < nr)
        qtg[(((long)b * Hkv + h) * QG + gi) * r + i0 + ri] =
            gi < 4 * ng4 ? ((qtpg[0][gi][ri] + qtpg[1][gi][ri]) + qtpg[2][gi][ri]) + qtpg[3][gi][ri] : 0.f;
    }
  if (qfrag) {
    // MFMA operand columns for the per-chunk kernel's coefficient-space logits,
    // [b][h][2][16][r] 16-bit.  x = q~_g (times the rank scale for int8 codes)
    // is split into hi = x rounded to the codes' MFMA type (bf16 for bf16
    // codes, fp16 for int8) and lo = (x - hi) rounded.  With 2g <= 16, tile 0
    // column c holds hi of head c (c < g) or lo of head c - g (c < 2g); with
    // g > 8, tile 0 holds the hi halves and tile 1 the lo halves.  Other
    // columns are zero.
    const bool two = grp > 8;
    for (int it = tid; it < 2 * 16 * SEL_RB; it += 256) {
      const int tile = it / (16 * SEL_RB), c = (it / SEL_RB) % 16, ri = it % SEL_RB;
      if (ri >= nr || (tile == 1 && !two)) continue;
      const bool ok = two ? c < grp : c < 2 * grp;
      const bool lo = two ? tile == 1 : c >= grp;
      const int gi = ok ? (two ? c : (lo ? c - grp : c)) : 0;
      float x = ok ? ((qtpg[0][gi][ri] + qtpg[1][gi][ri]) + qtpg[2][gi][ri]) + qtpg[3][gi][ri] : 0.f;
      uint16_t v;
      if (qf_mode == 2) {
        x *= f16_bits_to_f32(qf_scale[(long)b * r + i0 + ri]);
        const _Float16 xh = (_Float16)x;
        v = __builtin_bit_cast(uint16_t, lo ? (_Float16)(x - (float)xh) : xh);
      } else {
        const uint16_t xh = f32_to_bf16_bits(x);
        v = lo ? f32_to_bf16_bits(x - bf16_bits_to_f32(xh)) : xh;
      }
      qfrag[((((long)b * Hkv + h) * 2 + tile) * 16 + c) * r + i0 + ri] = v;
    }
  }
  __syncthreads();

  double qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) qv[e] = li_ok ? qt[4 * li + e] : 0.0;
  double *pb = part + (((long)b * Hkv + h) * NRB + rb) * n_c;
  for (int j_base = 0; j_base < n_c; j_base += 16 * MB) {
    if (j_base > 0) load_rows(j_base);
    double sacc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const uint32_t w4[4] = {lv[m].x, lv[m].y, lv[m].z, lv[m].w};
      sacc[m] = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[m] = fma((double)__uint_as_float(w4[e]), qv[e], sacc[m]);
    }
    const double tot = xpose_sum<MB, 8>(sacc, lane);  // chunk row li of lane group gq
    const int j = j_base + 16 * li + 4 * w + gq;
    if (j < n_c) pb[j] = tot;
    if (lds_scores && j < n_c) lds_scores[j] = tot;
  }
}

// With sel set (one rank block, r <= 64, and n_c <= 256 only), the block's
// partial scores are the chunk scores, and the workgroup ranks them itself:
// wave 0 writes the top k_eff chunks of (b, h) by (score desc, index asc), in
// ascending order, to sel (and sel_out), as the separate top-k launch would.
template <typename TA, int DH, int QG>
__global__ __launch_bounds__(256) void k_select_partial(const TA *__restrict__ q, long q_bstride,
                                                        const TA *__restrict__ basis,
                                                        const float *__restrict__ landmark, int Hq,
                                                        int Hkv, int r, int n_c, int D, int layer,
                                                        double *__restrict__ part, float *__restrict__ qtg,
                                                        uint16_t *__restrict__ qfrag,
                                                        const uint16_t *__restrict__ qf_scale, int qf_mode,
                                                        int k_eff, int32_t *__restrict__ sel,
                                                        int32_t *__restrict__ sel_out) {
  __shared__ SelectSmem<DH, QG> sm;
  __shared__ double scs[4 * WAVE];
  int rb, h, b;
  select_coords(blockIdx.x + gridDim.x * (blockIdx.y + Hkv * blockIdx.z), gridDim.x, Hkv, gridDim.z, rb, h, b);
  select_partial_block<TA, DH, QG>(sm, rb, h, b, gridDim.x, q, q_bstride, basis, landmark, Hq, Hkv, r, n_c, D,
                                   layer, part, qtg, qfrag, qf_scale, qf_mode, sel ? scs : nullptr);
  if (sel) {
    __syncthreads();
    if (threadIdx.x < WAVE) {
      const long o = ((long)b * Hkv + h) * k_eff;
      wave_topk<4>(scs, n_c, k_eff, [&](int pos, int c) {
        sel[o + pos] = c;
        if (sel_out) sel_out[o + pos] = c;
      });
    }
  }
}

}  // namespace lowram
