// Compress-side kernels for gfx950 (run once per context, before decoding):
//   k_project     c_t = U^T k_t^cat in float64 (matrix cores), rounded once to the storage type
//   k_colmax      per-channel max |x| -> fp16 scale = fp16(max / 127)
//   k_quant       q = clamp(rne(x / s), -127, 127)
//   k_landmark    mean dequantised coefficient of each chunk, float64 -> float32
//   k_pred        float64 predictor (matrix cores): k_hat = U_{l,h} c~, v_hat = W2 SiLU(W1 k_hat + b1) + b2,
//                 emitting either e_t = ||v_t - v_hat_t||^2 or delta = v - v_hat
//   k_err_topk    residual set: top n_res tokens by (e desc, t asc), ascending,
//                 with chunk CSR pointers
//   eviction      group score accumulation, top chunks, compaction
//
// Keys of a layer group are stored as per-token coefficients on a shared basis
// (zicq.com English summary, "Cross-Layer Low-Rank Key Compression"); values
// are predicted from keys and only the worst-reconstructed tokens keep their
// residual (same page, "Core Mechanism"; abstract of arXiv 2611.07025).  The
// ranking key is computed in float64 so that the chosen set does not depend
// on summation order.
#include "common.hpp"
#include "internal.hpp"

namespace lowram {

__device__ __forceinline__ double ldd(const float *p, long i) { return (double)p[i]; }
__device__ __forceinline__ double ldd(const bf16 *p, long i) { return to_f64(p[i]); }
__device__ __forceinline__ double ld_cdeq(const float *c, long i, const uint16_t *, int) { return (double)c[i]; }
__device__ __forceinline__ double ld_cdeq(const bf16 *c, long i, const uint16_t *, int) { return to_f64(c[i]); }
__device__ __forceinline__ double ld_cdeq(const int8_t *c, long i, const uint16_t *sc, int ch) {
  return (double)c[i] * (double)f16_bits_to_f32(sc[ch]);
}
__device__ __forceinline__ void st_round(float *p, double x) { *p = (float)x; }
__device__ __forceinline__ void st_round(bf16 *p, double x) { p->u = f64_to_bf16_bits(x); }
__device__ __forceinline__ void st_round(double *p, double x) { *p = x; }

// ---------------------------------------------------------------------------
// C1: out[b][o0 + t][i] = sum_kk K(b, t, kk) U[b][kk][i] for t < N, float64
// products and sums on the float64 matrix cores (v_mfma_f64_16x16x4_f64).
// K(b, t, kk) = k[b][l][h][t][d] with kk = (l*Hkv + h)*dh + d and Nk tokens per
// (l, h) block of k; out holds No rows per sequence.
// With S > 1 the reduction over kk is split in S slices of Dsl (a multiple of
// 16): slice s writes its float64 partial sums to out + s * s_stride (TO =
// double) and k_project_sum adds the slices in order.
// grid (ceil(r/64), ceil(N/64), B * S), 256 threads; each wave a 32 x 32
// quarter of the 64 x 64 tile, the next 16-wide slab's loads in flight during
// the current slab's products.
// ---------------------------------------------------------------------------
template <typename TA, typename TO>
__global__ __launch_bounds__(256) void k_project(const TA *__restrict__ k, const TA *__restrict__ U,
                                                 TO *__restrict__ out, int N, int D, int dh, int r,
                                                 int Nk, int No, int o0, int S, int Dsl,
                                                 long s_stride) {
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  __shared__ double As[16][64 + 1];
  __shared__ double Bs[16][64];
  const int b = blockIdx.z / S, sl = blockIdx.z % S;
  const int t0 = blockIdx.y * 64, i0 = blockIdx.x * 64, tid = threadIdx.x;
  const int kbeg = sl * Dsl, kend = min(D, kbeg + Dsl);
  out += sl * s_stride;
  const int lane = tid & (WAVE - 1), w = tid / WAVE, l16 = lane & 15, kg = lane >> 4;
  const int wr0 = (w >> 1) * 32, wc0 = (w & 1) * 32;  // this wave's quarter of the tile
  const TA *kb = k + (long)b * D * Nk;  // [G*Hkv][Nk][dh] blocks
  const TA *Ub = U + (long)b * D * r;
  f64x4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) acc[mi][nj] = f64x4{0.0, 0.0, 0.0, 0.0};
  // both slabs' loads in flight together: indices clamped into range, the
  // values outside it zeroed when stored
  double av0[4], bv0[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, kk = idx % 16, t = idx / 16;  // consecutive threads walk d
      const int gk = min(k0 + kk, kend - 1), tt = min(t0 + t, N - 1);
      av0[u] = ldd(kb, (long)(gk / dh) * Nk * dh + (long)tt * dh + gk % dh);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, kk = idx / 64, i = idx % 64;
      bv0[u] = ldd(Ub, (long)min(k0 + kk, kend - 1) * r + min(i0 + i, r - 1));
    }
  };
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, kk = idx % 16, t = idx / 16;
      As[kk][t] = (t0 + t < N && k0 + kk < kend) ? av0[u] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, kk = idx / 64, i = idx % 64;
      Bs[kk][i] = (k0 + kk < kend && i0 + i < r) ? bv0[u] : 0.0;
    }
    __syncthreads();
    if (k0 + 16 < kend) load(k0 + 16);
    // lane (l16, kg) holds A[row l16][k kg] and B[k kg][column l16]
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      double xa[2], xb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) xa[mi] = As[4 * k4 + kg][wr0 + 16 * mi + l16];
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) xb[nj] = Bs[4 * k4 + kg][wc0 + 16 * nj + l16];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[mi], xb[nj], acc[mi][nj], 0, 0, 0);
    }
    __syncthreads();
  }
  // item v of lane (l16, kg) is row kg + 4 v, column l16 of its 16 x 16 block
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tt = t0 + wr0 + 16 * mi + kg + 4 * v, ii = i0 + wc0 + 16 * nj + l16;
        if (tt < N && ii < r) st_round(out + ((long)b * No + o0 + tt) * r + ii, acc[mi][nj][v]);
      }
}

// out[b][o0 + t][i] = round(sum over s = 0..S-1 of part[s][b][t][i]), slices
// added in order.  part: [S][B][N][r] float64.  grid (ceil(B*N*r / 256)).
template <typename TO>
__global__ __launch_bounds__(256) void k_project_sum(const double *__restrict__ part,
                                                     TO *__restrict__ out, int B, int N, int r,
                                                     int S, int No, int o0) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x, per = (long)B * N * r;
  if (i >= per) return;
  double s = 0.0;
  for (int j = 0; j < S; ++j) s += part[j * per + i];
  const long b = i / ((long)N * r), rem = i - b * N * r;
  st_round(out + ((long)b * No + o0) * r + rem, s);
}

// ---------------------------------------------------------------------------
// Per-channel fp16 scale over rows: x[batch][rows][cols] -> s[batch][cols].
// grid (ceil(cols/64), batch), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_colmax(const double *__restrict__ x, uint16_t *__restrict__ s,
                                                int rows, int cols) {
  __shared__ double red[4][64];
  const int bt = blockIdx.y, c = blockIdx.x * 64 + threadIdx.x % 64, rg = threadIdx.x / 64;
  double m = 0.0;
  if (c < cols)
    for (int t = rg; t < rows; t += 4) m = fmax(m, fabs(x[((long)bt * rows + t) * cols + c]));
  red[rg][threadIdx.x % 64] = m;
  __syncthreads();
  if (rg == 0 && c < cols) {
    const double mx = fmax(fmax(red[0][threadIdx.x], red[1][threadIdx.x]),
                           fmax(red[2][threadIdx.x], red[3][threadIdx.x]));
    s[(long)bt * cols + c] = f64_to_f16_bits(mx / 127.0);
  }
}

// q = clamp(rne(x / s), -127, 127); zero where the scale is zero.
// x: [batch][rows][cols] float64, s: [batch][cols]; row t of batch bt is
// written to row o0 + t of a [batch][out_rows][cols] int8 array.
__global__ __launch_bounds__(256) void k_quant(const double *__restrict__ x,
                                               const uint16_t *__restrict__ s,
                                               int8_t *__restrict__ q, long rows, int cols,
                                               long total, long out_rows, long o0) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long bt = i / (rows * cols);
  const long rc = i - bt * rows * cols;
  const int c = (int)(i % cols);
  const double sc = (double)f16_bits_to_f32(s[bt * cols + c]);
  double v = 0.0;
  if (sc > 0.0) v = fmin(127.0, fmax(-127.0, rint(x[i] / sc)));
  q[(bt * out_rows + o0) * cols + rc] = (int8_t)v;
}

// C2: landmark[b][j][i] = float32(mean_t deq(coeff[b][jC + t][i])) for chunks
// j = j0 + blockIdx.y of an N-token cache, 64 channels i per workgroup: four
// row groups sum rows t = g, g+4, ... in float64 and are added in a fixed
// order.  grid (ceil(r/64), chunks, B), 256 threads.
template <typename TC>
__global__ __launch_bounds__(256) void k_landmark(const TC *__restrict__ coeff,
                                                  const uint16_t *__restrict__ cscale,
                                                  float *__restrict__ lm, int N, int C, int r, int j0) {
  __shared__ double red[4][64];
  const int j = j0 + blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % 64, g = threadIdx.x / 64, i = blockIdx.x * 64 + c;
  const TC *cb = coeff + ((long)b * N + (long)j * C) * r;
  const uint16_t *sc = cscale ? cscale + (long)b * r : nullptr;
  double s = 0.0;
  if (i < r)
    for (int t = g; t < C; t += 4) s += ld_cdeq(cb, (long)t * r + i, sc, i);
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && i < r)
    lm[((long)b * (N / C) + j) * r + i] =
        (float)(((red[0][c] + red[1][c]) + (red[2][c] + red[3][c])) / (double)C);
}

// ---------------------------------------------------------------------------
// C3 / C5: float64 predictor over a tile of TM rows of one (b, l, h).
// MODE 0: rows are tokens t, writes err[b][l][h][t] = ||v_t - v_hat_t||^2.
// MODE 1: rows are residual entries e, token res_idx[e]; writes delta rows
//         (rounded to TD) to dout[b][l][h][e][:].
// MODE 2: as MODE 0, and also writes every token's float64 delta row to
//         dout[b][l][h][t][:].
// Token t reads coefficient row c0 + t of a cache with Nc rows per sequence and
// value row t of v[b][l][h] (Nv rows per (b, l, h)); err has N entries per
// (b, l, h).
// grid (ceil(rows/TM), G*Hkv, B), 256 threads (4 waves).  The products run on
// the float64 matrix cores.  Every 16-wide slab of the three products is
// loaded into registers while the previous slab's products run, and stored to
// LDS after them.
// ---------------------------------------------------------------------------
template <int DH, int TM, int MODE, typename TA, typename TC, typename TD>
__global__ __launch_bounds__(256) void k_pred(const TC *__restrict__ coeff,
                                              const uint16_t *__restrict__ cscale,
                                              const TA *__restrict__ basis, const TA *__restrict__ w1,
                                              const TA *__restrict__ b1, const TA *__restrict__ w2,
                                              const TA *__restrict__ b2, const TA *__restrict__ v,
                                              const int32_t *__restrict__ res_idx,
                                              double *__restrict__ err, TD *__restrict__ dout,
                                              int Hkv, int N, int r, int F, int n_rows, int n_res,
                                              int Nc, int c0, int Nv) {
  constexpr int KS = DH + 1, HS = 64 + 1;
  extern __shared__ __align__(16) double psm[];
  double *Ks = psm;              // [TM][DH+1]
  double *Hs = Ks + TM * KS;     // [TM][65]
  double *As = Hs + TM * HS;     // [16][TM]   (GEMM1 A slab)
  double *Bs = As + 16 * TM;     // [16][DH]   (B slabs: U, W1 block, W2 block)
  __shared__ int tok[TM];
  const int lh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int l = lh / Hkv, h = lh % Hkv;
  const int G = gridDim.y / Hkv;
  const long bh = ((long)b * G + l) * Hkv + h;
  const int row0 = blockIdx.x * TM;
  const int D = G * Hkv * DH;
  const TA *Ul = basis + ((long)b * D + (long)lh * DH) * r;
  const TA *W1 = w1 + bh * F * DH;
  const TA *B1 = b1 + bh * F;
  const TA *W2 = w2 + bh * DH * F;
  const TA *B2 = b2 + bh * DH;
  const TA *V = v + bh * Nv * DH;
  const TC *cb = coeff + ((long)b * Nc + c0) * r;
  const uint16_t *sc = cscale ? cscale + (long)b * r : nullptr;
  for (int i = tid; i < TM; i += 256) {
    const int rr = row0 + i;
    int t = -1;
    if (rr < n_rows) t = MODE == 1 ? res_idx[bh * n_res + rr] : rr;
    tok[i] = t;
  }
  __syncthreads();

  // The three products run on the float64 matrix cores
  // (v_mfma_f64_16x16x4_f64: lane (l16, kg) holds A[row l16][k kg] and
  // B[k kg][column l16], and the 16 x 16 result's rows kg + 4 v of column l16;
  // the float32 and 16-bit variants hold rows 4 kg + v instead).
  // Each wave owns a quarter of the head dims of k_hat and v_hat (NW4 blocks of
  // 16 columns, all MB row blocks) and 16 columns of each 64-wide hidden block.
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  const int lane = tid & (WAVE - 1), w = tid / WAVE, l16 = lane & 15, kg = lane >> 4;
  constexpr int MB = TM / 16, NW4 = DH / 64;
  static_assert(DH % 64 == 0 && TM % 16 == 0, "whole blocks per wave");
  const int wc0 = w * (DH / 4);   // this wave's first head-dim column
  auto mma = [](double x, double y, f64x4 c) { return __builtin_amdgcn_mfma_f64_16x16x4f64(x, y, c, 0, 0, 0); };
  const f64x4 z4 = {0.0, 0.0, 0.0, 0.0};

  // GEMM1: k_hat[TM][DH] = deq(c)[TM][r] . U_{l,h}^T
  f64x4 acc[MB][NW4];
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int nj = 0; nj < NW4; ++nj) acc[mi][nj] = z4;
  static_assert(16 * TM % 256 == 0 && 16 * DH % 256 == 0, "whole slabs per thread");
  // slab registers: both slabs' loads in flight together, the next slab's
  // issued before the current one's products (rows of absent tokens read
  // token 0 and are zeroed when stored)
  double av0[16 * TM / 256], bv0[16 * DH / 256];
  auto load_slab = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 16 * TM / 256; ++u) {
      const int idx = tid + 256 * u, kk = idx % 16, t = tok[idx / 16];
      av0[u] = ld_cdeq(cb, (long)max(t, 0) * r + k0 + kk, sc, k0 + kk);
    }
#pragma unroll
    for (int u = 0; u < 16 * DH / 256; ++u) {
      const int idx = tid + 256 * u, kk = idx % 16, d = idx / 16;
      bv0[u] = ldd(Ul, (long)d * r + k0 + kk);
    }
  };
  load_slab(0);
  for (int k0 = 0; k0 < r; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 16 * TM / 256; ++u) {
      const int idx = tid + 256 * u, kk = idx % 16, m = idx / 16;
      As[kk * TM + m] = tok[m] >= 0 ? av0[u] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 16 * DH / 256; ++u) {
      const int idx = tid + 256 * u;
      Bs[(idx % 16) * DH + idx / 16] = bv0[u];
    }
    __syncthreads();
    if (k0 + 16 < r) load_slab(k0 + 16);
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      double xa[MB], xb[NW4];
#pragma unroll
      for (int mi = 0; mi < MB; ++mi) xa[mi] = As[(4 * k4 + kg) * TM + 16 * mi + l16];
#pragma unroll
      for (int nj = 0; nj < NW4; ++nj) xb[nj] = Bs[(4 * k4 + kg) * DH + wc0 + 16 * nj + l16];
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < NW4; ++nj) acc[mi][nj] = mma(xa[mi], xb[nj], acc[mi][nj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int nj = 0; nj < NW4; ++nj)
#pragma unroll
      for (int v = 0; v < 4; ++v) Ks[(16 * mi + kg + 4 * v) * KS + wc0 + 16 * nj + l16] = acc[mi][nj][v];
  __syncthreads();

  // GEMM2 + SiLU per 64-wide hidden block, GEMM3 accumulated: v_hat = H . W2^T
  f64x4 vacc[MB][NW4];
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int nj = 0; nj < NW4; ++nj) vacc[mi][nj] = z4;
  for (int f0 = 0; f0 < F; f0 += 64) {
    f64x4 hacc[MB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) hacc[mi] = z4;
    // W1 slabs: the next one's loads in flight during the current products
    double wv0[16 * 64 / 256];
    auto load_w1 = [&](int k0) {
#pragma unroll
      for (int u = 0; u < 16 * 64 / 256; ++u) {
        const int idx = tid + 256 * u;
        wv0[u] = ldd(W1, (long)(f0 + idx / 16) * DH + k0 + idx % 16);
      }
    };
    load_w1(0);
    for (int k0 = 0; k0 < DH; k0 += 16) {
#pragma unroll
      for (int u = 0; u < 16 * 64 / 256; ++u) {
        const int idx = tid + 256 * u;
        Bs[(idx % 16) * 64 + idx / 16] = wv0[u];
      }
      __syncthreads();
      if (k0 + 16 < DH) load_w1(k0 + 16);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const double xb = Bs[(4 * k4 + kg) * 64 + 16 * w + l16];
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
          hacc[mi] = mma(Ks[(16 * mi + l16) * KS + k0 + 4 * k4 + kg], xb, hacc[mi]);
      }
      __syncthreads();
    }
    {
      const double bias = ldd(B1, f0 + 16 * w + l16);
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double x = hacc[mi][v] + bias;
          Hs[(16 * mi + kg + 4 * v) * HS + 16 * w + l16] = x / (1.0 + exp(-x));
        }
    }
    __syncthreads();
    // W2 slabs of this hidden block, prefetched like W1's
    double w2v0[16 * DH / 256];
    auto load_w2 = [&](int k0) {
#pragma unroll
      for (int u = 0; u < 16 * DH / 256; ++u) {
        const int idx = tid + 256 * u;
        w2v0[u] = ldd(W2, (long)(idx / 16) * F + f0 + k0 + idx % 16);
      }
    };
    load_w2(0);
    for (int k0 = 0; k0 < 64; k0 += 16) {
#pragma unroll
      for (int u = 0; u < 16 * DH / 256; ++u) {
        const int idx = tid + 256 * u;
        Bs[(idx % 16) * DH + idx / 16] = w2v0[u];
      }
      __syncthreads();
      if (k0 + 16 < 64) load_w2(k0 + 16);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        double xa[MB], xb[NW4];
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) xa[mi] = Hs[(16 * mi + l16) * HS + k0 + 4 * k4 + kg];
#pragma unroll
        for (int nj = 0; nj < NW4; ++nj) xb[nj] = Bs[(4 * k4 + kg) * DH + wc0 + 16 * nj + l16];
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
          for (int nj = 0; nj < NW4; ++nj) vacc[mi][nj] = mma(xa[mi], xb[nj], vacc[mi][nj]);
      }
      __syncthreads();
    }
  }

  // epilogue: lane holds v_hat - b2 of rows m = 16 mi + kg + 4 v, head dims
  // wc0 + 16 nj + l16.  The squared error of a row is summed over the lane's
  // blocks, then over the 16 lanes of its row group, then over the 4 waves in
  // order.
  double *ered = As;  // [4][TM]: the first product's slab area, free since its last barrier
#pragma unroll
  for (int mi = 0; mi < MB; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * mi + kg + 4 * v;
      const int t = tok[m];
      if (MODE != 1) {
        double e = 0.0;
        if (t >= 0) {
#pragma unroll
          for (int nj = 0; nj < NW4; ++nj) {
            const int d = wc0 + 16 * nj + l16;
            const double dv = ldd(V, (long)t * DH + d) - (vacc[mi][nj][v] + ldd(B2, d));
            e = fma(dv, dv, e);
            if (MODE == 2) st_round(dout + (bh * N + t) * DH + d, dv);
          }
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) e += __shfl_xor(e, o, WAVE);
        if (l16 == 0) ered[w * TM + m] = e;
      } else if (t >= 0) {
        const int rr = row0 + m;
#pragma unroll
        for (int nj = 0; nj < NW4; ++nj) {
          const int d = wc0 + 16 * nj + l16;
          const double dv = ldd(V, (long)t * DH + d) - (vacc[mi][nj][v] + ldd(B2, d));
          st_round(dout + (bh * n_res + rr) * DH + d, dv);
        }
      }
    }
  if (MODE != 1) {
    __syncthreads();
    if (tid < TM && tok[tid] >= 0)
      err[bh * N + tok[tid]] = ((ered[tid] + ered[TM + tid]) + ered[2 * TM + tid]) + ered[3 * TM + tid];
  }
}

// C4: residual set and CSR pointers per (b, l, h).  grid (G*Hkv, B), 1024 threads.
__global__ __launch_bounds__(1024) void k_err_topk(const double *__restrict__ err, int N, int C,
                                                   int n_res, int32_t *__restrict__ res_idx,
                                                   int32_t *__restrict__ res_ptr) {
  __shared__ TopkSmem tk;
  const long bh = (long)blockIdx.y * gridDim.x + blockIdx.x;
  const double *e = err + bh * N;
  block_topk<1024>([&](int i) { return f64_order_key(e[i]); }, N, n_res, res_idx + bh * n_res, tk,
                   C, res_ptr + bh * (N / C + 1));
}

// ---------------------------------------------------------------------------
// eviction
// ---------------------------------------------------------------------------
// acc[b][j] += sum_h s[b][h][j], heads in ascending order (so over all calls
// acc = sum over w, then l, then h, in that order).  grid (ceil(n_c/256), B).
__global__ __launch_bounds__(256) void k_evict_accum(const double *__restrict__ s, double *__restrict__ acc,
                                                     int Hkv, int n_c, int first) {
  const int j = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (j >= n_c) return;
  double v = first ? 0.0 : acc[(long)b * n_c + j];
  for (int h = 0; h < Hkv; ++h) v += s[((long)b * Hkv + h) * n_c + j];
  acc[(long)b * n_c + j] = v;
}

// keep the top `keep` chunks by accumulated score.  grid (B), 1024 threads.
__global__ __launch_bounds__(1024) void k_evict_select(const double *__restrict__ acc, int n_c,
                                                       int keep, int32_t *__restrict__ keep_idx) {
  __shared__ TopkSmem tk;
  const int b = blockIdx.x;
  const double *ab = acc + (long)b * n_c;
  block_topk<1024>([&](int i) { return f64_order_key(ab[i]); }, n_c, keep,
                   keep_idx + (long)b * keep, tk, 0, nullptr);
}

// copy the kept chunks' coefficient rows and landmarks.  grid (keep, B).
__global__ __launch_bounds__(256) void k_evict_copy(const unsigned char *__restrict__ coeff,
                                                    const float *__restrict__ lm,
                                                    const int32_t *__restrict__ keep_idx,
                                                    unsigned char *__restrict__ d_coeff,
                                                    float *__restrict__ d_lm, int keep, int n_c,
                                                    long chunk_bytes, int r) {
  const int jn = blockIdx.x, b = blockIdx.y;
  const int jo = keep_idx[(long)b * keep + jn];
  const u32x4 *src = reinterpret_cast<const u32x4 *>(coeff + ((long)b * n_c + jo) * chunk_bytes);
  u32x4 *dst = reinterpret_cast<u32x4 *>(d_coeff + ((long)b * keep + jn) * chunk_bytes);
  for (long i = threadIdx.x; i < chunk_bytes / 16; i += 256) dst[i] = src[i];
  for (int i = threadIdx.x; i < r; i += 256)
    d_lm[((long)b * keep + jn) * r + i] = lm[((long)b * n_c + jo) * r + i];
}

// rebuild the residual CSR of the kept chunks.  grid (G*Hkv, B), 256 threads.
// dst holds d_cap rows per (b, l, h): rows past it are not copied and the
// pointers are clamped to it, so the new CSR never names a row it lacks.
// live (optional) receives each head's row count before clamping.  With
// d_ptr null only live is written.
__global__ __launch_bounds__(256) void k_evict_resid(const int32_t *__restrict__ ptr,
                                                     const int32_t *__restrict__ idx,
                                                     const unsigned char *__restrict__ val,
                                                     const int32_t *__restrict__ keep_idx,
                                                     int32_t *__restrict__ d_ptr,
                                                     int32_t *__restrict__ d_idx,
                                                     unsigned char *__restrict__ d_val,
                                                     int32_t *__restrict__ live, int n_c, int keep,
                                                     int C, int n_res, int d_cap, int row_bytes) {
  __shared__ int32_t part[257];
  const long bh = (long)blockIdx.y * gridDim.x + blockIdx.x;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int32_t *p = ptr + bh * (n_c + 1);
  const int32_t *kp = keep_idx + (long)b * keep;
  // each thread sums a contiguous run of kept chunks, then a serial scan of the runs
  const int per = (keep + 255) / 256;
  const int j0 = min(keep, tid * per), j1 = min(keep, j0 + per);
  int32_t s = 0;
  for (int jn = j0; jn < j1; ++jn) s += p[kp[jn] + 1] - p[kp[jn]];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int i = 0; i < 256; ++i) { const int32_t c = part[i]; part[i] = run; run += c; }
    part[256] = run;
    if (live) live[bh] = run;
  }
  __syncthreads();
  if (!d_ptr) return;
  int32_t *dp = d_ptr + bh * (keep + 1);
  int32_t run = part[tid];
  for (int jn = j0; jn < j1; ++jn) {
    dp[jn] = min(run, d_cap);
    const int jo = kp[jn];
    for (int e = p[jo]; e < p[jo + 1] && run < d_cap; ++e, ++run) {
      d_idx[bh * d_cap + run] = idx[bh * n_res + e] - jo * C + jn * C;
      const unsigned char *sr = val + (bh * n_res + e) * (long)row_bytes;
      unsigned char *dr = d_val + (bh * d_cap + run) * (long)row_bytes;
      for (int i = 0; i < row_bytes; i += 16)
        lst16(dr + i, gld16(sr + i));
    }
  }
  if (tid == 0) dp[keep] = min(part[256], d_cap);
}

// ---------------------------------------------------------------------------
// tail re-pack
// ---------------------------------------------------------------------------
// dst[b][0..words) = src[b][0..words) for b = blockIdx.y, in 8-byte words, with
// per-sequence strides src_stride / dst_stride (words).  grid (ceil(words/256), B).
__global__ __launch_bounds__(256) void k_copy_rows(const uint2 *__restrict__ src, long src_stride,
                                                   uint2 *__restrict__ dst, long dst_stride,
                                                   long words) {
  const long w = (long)blockIdx.x * 256 + threadIdx.x;
  if (w >= words) return;
  dst[(long)blockIdx.y * dst_stride + w] = src[(long)blockIdx.y * src_stride + w];
}

// Residual CSR of one (b, l, h) after appending a chunk: the source's n_c + 1
// pointers and its live rows (ptr[n_c] of them, read on the device and clamped
// to the capacity n_res), then the indices N + t_idx[e] of the m new rows
// (whose values k_repack_rows writes), then zeros up to the new capacity
// n_res + m.  Each workgroup moves RB rows in 8-byte words; the first also
// writes the pointers.
// grid (ceil((n_res + m) / RB), G*Hkv, B), 256 threads.
constexpr int REPACK_RB = 64;
__global__ __launch_bounds__(256) void k_repack_resid(
    const int32_t *__restrict__ ptr, const int32_t *__restrict__ idx,
    const unsigned char *__restrict__ val, const int32_t *__restrict__ t_idx,
    int32_t *__restrict__ d_ptr,
    int32_t *__restrict__ d_idx, unsigned char *__restrict__ d_val, int n_c, int N, int n_res,
    int m, int row_bytes) {
  const long bh = (long)blockIdx.z * gridDim.y + blockIdx.y;
  const int tid = threadIdx.x, cap = n_res + m, words = row_bytes / 8;
  const int e0 = blockIdx.x * REPACK_RB, e1 = min(cap, e0 + REPACK_RB);
  const int32_t *op = ptr + bh * (n_c + 1);
  const int live = min(max(op[n_c], 0), n_res);
  if (blockIdx.x == 0)
    for (int j = tid; j <= n_c + 1; j += 256) d_ptr[bh * (n_c + 2) + j] = j <= n_c ? op[j] : live + m;
  for (int e = e0 + tid; e < e1; e += 256) {
    int32_t x = 0;
    if (e < live) x = idx[bh * n_res + e];
    else if (e < live + m) x = N + t_idx[bh * m + (e - live)];
    d_idx[bh * cap + e] = x;
  }
  const uint2 *sv = reinterpret_cast<const uint2 *>(val + bh * n_res * row_bytes);
  uint2 *dv = reinterpret_cast<uint2 *>(d_val + bh * cap * row_bytes);
  for (long w = (long)e0 * words + tid; w < (long)e1 * words; w += 256) {
    const int e = (int)(w / words), o = (int)(w % words);
    if (e >= live && e < live + m) continue;
    dv[w] = e < live ? sv[(long)e * words + o] : make_uint2(0u, 0u);
  }
}

__device__ __forceinline__ void st_resid(float *p, double x, const uint16_t *) { *p = (float)x; }
__device__ __forceinline__ void st_resid(bf16 *p, double x, const uint16_t *) { p->u = f64_to_bf16_bits(x); }
__device__ __forceinline__ void st_resid(int8_t *p, double x, const uint16_t *sc) {
  const double s = (double)f16_bits_to_f32(*sc);
  *p = (int8_t)(s > 0.0 ? fmin(127.0, fmax(-127.0, rint(x / s))) : 0.0);
}

// The m new residual rows of one (b, l, h): row e is token t_idx[e]'s float64
// delta (dall, [B][G][Hkv][C][dh]) stored at row live + e of the grown cache,
// rounded to TR (int8: the existing per-dim scales rscale[b][l][h][:]).
// grid (G*Hkv, B), 256 threads.
template <typename TR>
__global__ __launch_bounds__(256) void k_repack_rows(const int32_t *__restrict__ ptr,
                                                     const int32_t *__restrict__ t_idx,
                                                     const double *__restrict__ dall,
                                                     const uint16_t *__restrict__ rscale,
                                                     TR *__restrict__ d_val, int n_c, int n_res,
                                                     int m, int C, int dh) {
  const long bh = (long)blockIdx.y * gridDim.x + blockIdx.x;
  const int live = min(max(ptr[bh * (n_c + 1) + n_c], 0), n_res);
  const long cap = n_res + m;
  for (int i = threadIdx.x; i < m * dh; i += 256) {
    const int e = i / dh, d = i % dh;
    const int t = t_idx[bh * m + e];
    st_resid(d_val + (bh * cap + live + e) * dh + d, dall[(bh * C + t) * dh + d],
             rscale ? rscale + bh * dh + d : nullptr);
  }
}

// ---------------------------------------------------------------------------
// host sequencing
// ---------------------------------------------------------------------------
// One predictor pass over the tokens of every (b, l, h): errors over n_tok
// tokens (coefficient rows c0.. of a cache with Nc rows per sequence, value
// rows of v with Nv rows per (b, l, h)), the residual set (top n_sel, with
// chunk CSR pointers), and the delta rows of that set -- float64 into d64 for
// int8 residuals (quantised afterwards), else rounded into val.  With
// delta_all the error pass also leaves every token's float64 delta row in d64
// ([B][G][Hkv][n_tok][dh]) and no second pass runs: the caller gathers the
// selected rows.
struct PredPass {
  const void *coeff; const uint16_t *cscale;
  const void *basis, *w1, *b1, *w2, *b2, *v;
  double *err; int32_t *idx, *ptr; void *val; double *d64;
  int B, G, Hkv, r, F, n_tok, C, n_sel, Nc, c0, Nv, resid_i8, delta_all;
};

template <int DH, int TM, int MODE, typename TA, typename TC, typename TD>
static void launch_pred(const PredPass &p, int n_rows, TD *dout, hipStream_t st) {
  const size_t smem = sizeof(double) * ((size_t)TM * (DH + 1) + (size_t)TM * 65 + 16 * TM + 16 * DH);
  dim3 grid((n_rows + TM - 1) / TM, p.G * p.Hkv, p.B);
  static const bool lds_ok = (allow_dynamic_lds(k_pred<DH, TM, MODE, TA, TC, TD>, smem), true);
  (void)lds_ok;
  hipLaunchKernelGGL((k_pred<DH, TM, MODE, TA, TC, TD>), grid, dim3(256), smem, st,
                     (const TC *)p.coeff, p.cscale, (const TA *)p.basis, (const TA *)p.w1,
                     (const TA *)p.b1, (const TA *)p.w2, (const TA *)p.b2, (const TA *)p.v,
                     p.idx, p.err, dout, p.Hkv, p.n_tok, p.r, p.F, n_rows, p.n_sel, p.Nc, p.c0,
                     p.Nv);
}

template <int DH, int TM, typename TA, typename TC, typename TR>
static void pred_both(const PredPass &p, hipStream_t st) {
  if (p.delta_all)
    launch_pred<DH, TM, 2, TA, TC, double>(p, p.n_tok, p.d64, st);
  else
    launch_pred<DH, TM, 0, TA, TC, double>(p, p.n_tok, nullptr, st);
  hipLaunchKernelGGL(k_err_topk, dim3(p.G * p.Hkv, p.B), dim3(1024), 0, st, p.err, p.n_tok, p.C,
                     p.n_sel, p.idx, p.ptr);
  if (p.n_sel > 0 && !p.delta_all) {
    if (p.resid_i8)
      launch_pred<DH, TM, 1, TA, TC, double>(p, p.n_sel, p.d64, st);
    else
      launch_pred<DH, TM, 1, TA, TC, TR>(p, p.n_sel, (TR *)p.val, st);
  }
}

template <typename TA, typename TC, typename TR>
static void pred_by_dh(int dh, const PredPass &p, hipStream_t st) {
  if (dh == 64) pred_both<64, 128, TA, TC, TR>(p, st);
  else if (dh == 128) pred_both<128, 64, TA, TC, TR>(p, st);
  else pred_both<256, 32, TA, TC, TR>(p, st);
}

// Residual rows are either float32 (act F32), bf16, or int8 whose float64
// deltas pred_both leaves in d64; the template argument only names the type
// non-int8 rows are rounded to.
static void pred_dispatch(int act, int coeff_dt, int dh, const PredPass &p, hipStream_t st) {
  if (act == LOWRAM_F32) pred_by_dh<float, float, float>(dh, p, st);
  else if (coeff_dt == LOWRAM_BF16) pred_by_dh<bf16, bf16, bf16>(dh, p, st);
  else pred_by_dh<bf16, int8_t, bf16>(dh, p, st);
}

static void launch_landmark(int act, int coeff_dt, const void *coeff, const uint16_t *cscale,
                            float *lm, int B, int N, int C, int r, int j0, int chunks,
                            hipStream_t st) {
  const dim3 grid((r + 63) / 64, chunks, B);
  if (act == LOWRAM_F32)
    hipLaunchKernelGGL(k_landmark<float>, grid, dim3(256), 0, st, (const float *)coeff, nullptr,
                       lm, N, C, r, j0);
  else if (coeff_dt == LOWRAM_BF16)
    hipLaunchKernelGGL(k_landmark<bf16>, grid, dim3(256), 0, st, (const bf16 *)coeff, nullptr,
                       lm, N, C, r, j0);
  else
    hipLaunchKernelGGL(k_landmark<int8_t>, grid, dim3(256), 0, st, (const int8_t *)coeff, cscale,
                       lm, N, C, r, j0);
}

// Projection of N tokens (Nk per (l, h) block of k) into rows o0.. of a cache
// with No rows per sequence, the reduction over D split in S slices
// (project_splits; partial sums in part, [S][B][N][r] float64, when S > 1).
// int8 coefficients go through c64 ([B][N][r]) and are quantised with the
// scales in cscale.
template <typename TA, typename TO>
static void project_typed(const void *k, const void *basis, TO *out, double *part, int B, int N,
                          int D, int dh, int r, int Nk, int No, int o0, int S, hipStream_t st) {
  const int Dsl = ((D + S - 1) / S + 15) / 16 * 16;
  const dim3 grid((r + 63) / 64, (N + 63) / 64, B * S);
  if (S == 1) {
    hipLaunchKernelGGL((k_project<TA, TO>), grid, dim3(256), 0, st, (const TA *)k,
                       (const TA *)basis, out, N, D, dh, r, Nk, No, o0, 1, Dsl, 0L);
    return;
  }
  const long per = (long)B * N * r;
  hipLaunchKernelGGL((k_project<TA, double>), grid, dim3(256), 0, st, (const TA *)k,
                     (const TA *)basis, part, N, D, dh, r, Nk, N, 0, S, Dsl, per);
  hipLaunchKernelGGL(k_project_sum<TO>, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, st,
                     (const double *)part, out, B, N, r, S, No, o0);
}

static void launch_project(int act, int coeff_dt, const void *k, const void *basis, void *coeff,
                           double *c64, double *part, const uint16_t *cscale, int B, int N, int D,
                           int dh, int r, int Nk, int No, int o0, int S, hipStream_t st) {
  if (act == LOWRAM_F32) {
    project_typed<float, float>(k, basis, (float *)coeff, part, B, N, D, dh, r, Nk, No, o0, S, st);
  } else if (coeff_dt == LOWRAM_BF16) {
    project_typed<bf16, bf16>(k, basis, (bf16 *)coeff, part, B, N, D, dh, r, Nk, No, o0, S, st);
  } else {
    project_typed<bf16, double>(k, basis, c64, part, B, N, D, dh, r, Nk, N, 0, S, st);
    const long total = (long)B * N * r;
    hipLaunchKernelGGL(k_quant, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, c64,
                       cscale, (int8_t *)coeff, (long)N, r, total, (long)No, (long)o0);
  }
}

// C1 (+ Q1 for int8 coefficients: scales over the N tokens first) into
// a.coeff / a.coeff_scale; a.c64 is the int8 staging buffer.
void compress_coefficients(const CompressArgs &a, hipStream_t st) {
  const int D = a.G * a.Hkv * a.dh;
  if (a.act != LOWRAM_F32 && a.coeff_dt == LOWRAM_I8) {
    project_typed<bf16, double>(a.k, a.basis, a.c64, nullptr, a.B, a.N, D, a.dh, a.r, a.N, a.N, 0,
                                1, st);
    hipLaunchKernelGGL(k_colmax, dim3((a.r + 63) / 64, a.B), dim3(256), 0, st, a.c64,
                       a.coeff_scale, a.N, a.r);
    const long total = (long)a.B * a.N * a.r;
    hipLaunchKernelGGL(k_quant, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a.c64,
                       a.coeff_scale, (int8_t *)a.coeff, (long)a.N, a.r, total, (long)a.N, 0L);
  } else {
    launch_project(a.act, a.coeff_dt, a.k, a.basis, a.coeff, nullptr, nullptr, nullptr, a.B, a.N, D,
                   a.dh, a.r, a.N, a.N, 0, 1, st);
  }
}

hipError_t run_compress(const CompressArgs &a, hipStream_t st) {
  const int n_c = a.N / a.C;
  compress_coefficients(a, st);
  // C2
  launch_landmark(a.act, a.coeff_dt, a.coeff, a.coeff_scale, a.landmark, a.B, a.N, a.C, a.r, 0,
                  n_c, st);
  // C3, C4, C5
  PredPass p;
  p.coeff = a.coeff; p.cscale = a.coeff_scale;
  p.basis = a.basis; p.w1 = a.w1; p.b1 = a.b1; p.w2 = a.w2; p.b2 = a.b2; p.v = a.v;
  p.err = a.err; p.idx = a.res_idx; p.ptr = a.res_ptr; p.val = a.res_val; p.d64 = a.d64;
  p.B = a.B; p.G = a.G; p.Hkv = a.Hkv; p.r = a.r; p.F = a.F;
  p.n_tok = a.N; p.C = a.C; p.n_sel = a.n_res; p.Nc = a.N; p.c0 = 0; p.Nv = a.N;
  p.resid_i8 = a.resid_dt == LOWRAM_I8;
  p.delta_all = 0;
  pred_dispatch(a.act, a.coeff_dt, a.dh, p, st);
  // Q1 on residual rows
  if (a.resid_dt == LOWRAM_I8 && a.n_res > 0) {
    const int bl = a.B * a.G * a.Hkv;
    hipLaunchKernelGGL(k_colmax, dim3((a.dh + 63) / 64, bl), dim3(256), 0, st, a.d64, a.res_scale,
                       a.n_res, a.dh);
    const long total = (long)bl * a.n_res * a.dh;
    hipLaunchKernelGGL(k_quant, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a.d64,
                       a.res_scale, (int8_t *)a.res_val, (long)a.n_res, a.dh, total,
                       (long)a.n_res, 0L);
  } else if (a.resid_dt == LOWRAM_I8) {
    const int bl = a.B * a.G * a.Hkv;
    hipLaunchKernelGGL(k_colmax, dim3((a.dh + 63) / 64, bl), dim3(256), 0, st, a.d64, a.res_scale,
                       0, a.dh);
  }
  return hipGetLastError();
}

hipError_t run_evict(const EvictArgs &a, hipStream_t st) {
  const int n_c = a.N / a.C, D = a.G * a.Hkv * a.dh;
  const int esz = dtype_bytes(a.act);
  for (int w = 0; w < a.n_obs; ++w)
    for (int l = 0; l < a.G; ++l) {
      const unsigned char *qb = reinterpret_cast<const unsigned char *>(a.obs_q) +
                                ((long)w * a.B * a.G + l) * a.Hq * a.dh * esz;
      hipError_t e = launch_select(a.act, qb, (long)a.G * a.Hq * a.dh, a.basis, a.landmark, a.B,
                                   a.Hq, a.Hkv, a.dh, a.r, n_c, D, l, 0, nullptr, nullptr,
                                   a.spart, a.scores, st);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_evict_accum, dim3((n_c + 255) / 256, a.B), dim3(256), 0, st, a.scores,
                         a.acc, a.Hkv, n_c, (w == 0 && l == 0) ? 1 : 0);
    }
  if (a.n_obs == 0)
    hipLaunchKernelGGL(k_evict_accum, dim3((n_c + 255) / 256, a.B), dim3(256), 0, st, a.scores,
                       a.acc, 0, n_c, 1);
  hipLaunchKernelGGL(k_evict_select, dim3(a.B), dim3(1024), 0, st, a.acc, n_c, a.keep, a.keep_out);
  if (a.d_coeff) {
    const long chunk_bytes = (long)a.C * a.r * dtype_bytes(a.coeff_dt);
    hipLaunchKernelGGL(k_evict_copy, dim3(a.keep, a.B), dim3(256), 0, st,
                       (const unsigned char *)a.coeff, a.landmark, a.keep_out,
                       (unsigned char *)a.d_coeff, a.d_landmark, a.keep, n_c, chunk_bytes, a.r);
  }
  if (a.d_coeff || a.live_out)
    hipLaunchKernelGGL(k_evict_resid, dim3(a.G * a.Hkv, a.B), dim3(256), 0, st, a.res_ptr, a.res_idx,
                       (const unsigned char *)a.res_val, a.keep_out, a.d_coeff ? a.d_res_ptr : nullptr,
                       a.d_res_idx, (unsigned char *)a.d_res_val, a.live_out, n_c, a.keep, a.C, a.n_res,
                       a.d_n_res, a.dh * dtype_bytes(a.resid_dt));
  return hipGetLastError();
}

// Batched copy of `bytes` per sequence (a multiple of 8) between arrays with
// per-sequence strides in bytes (multiples of 8); nothing when bytes is 0.
static void copy_rows(const void *src, long src_stride, void *dst, long dst_stride, long bytes,
                      int B, hipStream_t st) {
  const long words = bytes / 8;
  if (words <= 0 || B <= 0) return;
  hipLaunchKernelGGL(k_copy_rows, dim3((unsigned)((words + 255) / 256), B), dim3(256), 0, st,
                     (const uint2 *)src, src_stride / 8, (uint2 *)dst, dst_stride / 8, words);
}

hipError_t run_repack(const RepackArgs &a, hipStream_t st) {
  const int D = a.G * a.Hkv * a.dh, n_c = a.N / a.C, Nd = a.N + a.C;
  const int bl = a.B * a.G * a.Hkv;
  const long cb = dtype_bytes(a.coeff_dt), rb = (long)a.dh * dtype_bytes(a.resid_dt);
  // the existing chunks: coefficient rows, landmarks, scales
  copy_rows(a.coeff, (long)a.N * a.r * cb, a.d_coeff, (long)Nd * a.r * cb, (long)a.N * a.r * cb,
            a.B, st);
  copy_rows(a.landmark, (long)n_c * a.r * 4, a.d_landmark, (long)(n_c + 1) * a.r * 4,
            (long)n_c * a.r * 4, a.B, st);
  if (a.coeff_dt == LOWRAM_I8 && a.d_coeff_scale != a.coeff_scale)
    copy_rows(a.coeff_scale, 0, a.d_coeff_scale, 0, (long)a.B * a.r * 2, 1, st);
  if (a.resid_dt == LOWRAM_I8 && a.d_res_scale != a.res_scale)
    copy_rows(a.res_scale, 0, a.d_res_scale, 0, (long)bl * a.dh * 2, 1, st);
  // C1 on the oldest C tail tokens into rows N.. (int8: the existing scales)
  launch_project(a.act, a.coeff_dt, a.k_tail, a.basis, a.d_coeff, a.c64, a.part, a.coeff_scale,
                 a.B, a.C, D, a.dh, a.r, a.T, Nd, a.N, project_splits(a.B, a.C, D, a.r), st);
  // C2 for the new chunk
  launch_landmark(a.act, a.coeff_dt, a.d_coeff, a.coeff_scale, a.d_landmark, a.B, Nd, a.C, a.r,
                  n_c, 1, st);
  // C3-C5 over the new chunk: errors and delta rows of its C tokens, its top m
  if (a.m > 0) {
    PredPass p;
    p.coeff = a.d_coeff; p.cscale = a.coeff_scale;
    p.basis = a.basis; p.w1 = a.w1; p.b1 = a.b1; p.w2 = a.w2; p.b2 = a.b2; p.v = a.v_tail;
    p.err = a.err; p.idx = a.t_idx; p.ptr = a.t_ptr; p.val = nullptr; p.d64 = a.dall;
    p.B = a.B; p.G = a.G; p.Hkv = a.Hkv; p.r = a.r; p.F = a.F;
    p.n_tok = a.C; p.C = a.C; p.n_sel = a.m; p.Nc = Nd; p.c0 = a.N; p.Nv = a.T;
    p.resid_i8 = a.resid_dt == LOWRAM_I8;
    p.delta_all = 1;
    pred_dispatch(a.act, a.coeff_dt, a.dh, p, st);
  }
  // the residual CSR with one more chunk, then the new rows (Q1 on the existing scales)
  const int n_blk = (a.n_res + a.m + REPACK_RB - 1) / REPACK_RB;
  hipLaunchKernelGGL(k_repack_resid, dim3(n_blk > 0 ? n_blk : 1, a.G * a.Hkv, a.B), dim3(256), 0,
                     st, a.res_ptr, a.res_idx, (const unsigned char *)a.res_val, a.t_idx,
                     a.d_res_ptr, a.d_res_idx, (unsigned char *)a.d_res_val, n_c, a.N, a.n_res,
                     a.m, (int)rb);
  if (a.m > 0) {
    const dim3 grid(a.G * a.Hkv, a.B);
    if (a.resid_dt == LOWRAM_I8)
      hipLaunchKernelGGL(k_repack_rows<int8_t>, grid, dim3(256), 0, st, a.res_ptr, a.t_idx, a.dall,
                         a.res_scale, (int8_t *)a.d_res_val, n_c, a.n_res, a.m, a.C, a.dh);
    else if (a.act == LOWRAM_F32)
      hipLaunchKernelGGL(k_repack_rows<float>, grid, dim3(256), 0, st, a.res_ptr, a.t_idx, a.dall,
                         nullptr, (float *)a.d_res_val, n_c, a.n_res, a.m, a.C, a.dh);
    else
      hipLaunchKernelGGL(k_repack_rows<bf16>, grid, dim3(256), 0, st, a.res_ptr, a.t_idx, a.dall,
                         nullptr, (bf16 *)a.d_res_val, n_c, a.n_res, a.m, a.C, a.dh);
  }
  return hipGetLastError();
}

}  // namespace lowram
