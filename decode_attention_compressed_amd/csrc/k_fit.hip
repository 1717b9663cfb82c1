// Test-time fitting of the per-head value predictor (gfx950, float32).
//
// The abstract fits a lightweight per-head predictor V_hat = f(K) at test
// time, from scratch or from a meta-learned start that needs fewer steps; the
// rit.work page (values section) trains it during prefill on the context's
// keys.  Here: `steps` steps of full-batch gradient descent on
//   L = (1/N) sum_t ||v_t - f(k_hat_t)||^2,  f(k) = W2 SiLU(W1 k + b1) + b2,
// per (sequence, layer, kv head), with k_hat = U_{l,h} deq(c~) built from the
// coefficients compress stores, float32 master weights, and the act dtype
// written once at the end.
//
// One gradient step of head z is a chain of batched products over its N
// tokens (64 x 64 output tiles, 4 x 4 per thread, float32 accumulate):
//   A = K_hat W1^T + b1, H = SiLU(A)             (epilogue keeps A and H)
//   R = H W2^T + b2 - V                          (epilogue subtracts the values)
//   loss = sum R^2 / N                           (fixed-order float64 sum)
//   G = (2/N) (R W2) . SiLU'(A)                  (written over A)
//   W2 -= lr (2/N) R^T H,  b2 -= lr (2/N) sum_t R (products over the N tokens)
//   W1 -= lr G^T K_hat,    b1 -= lr sum_t G
// Every sum runs in a fixed order, so the result is bitwise reproducible.
#include <cstring>

#include "common.hpp"
#include "gemm_f32.hpp"
#include "internal.hpp"

namespace lowram {
namespace fit {

using namespace f32gemm;

// Stored coefficients of head z's sequence, dequantised: A(z, t, i) = deq(c~[b][t][i]).
template <typename TC>
struct CoefOp {
  static constexpr bool KC = true;
  const TC *p; const uint16_t *scale; int GH, N, r;
  __device__ float operator()(int z, int t, int i) const {
    const int b = z / GH;
    const long o = ((long)b * N + t) * r + i;
    if constexpr (sizeof(TC) == 1) return (float)p[o] * f16_bits_to_f32(scale[(long)b * r + i]);
    else return ldf(p, o);
  }
};

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

struct EpStore {  // X[z][i][j] = c
  float *x; int ld; long zs;
  __device__ void operator()(int z, int i, int j, float c) const { x[z * zs + (long)i * ld + j] = c; }
};
struct EpHidden {  // A = c + b1, H = SiLU(A)
  float *apre, *hid; const float *b1; int F; long zs;
  __device__ void operator()(int z, int i, int j, float c) const {
    const float x = c + b1[(long)z * F + j];
    const long o = z * zs + (long)i * F + j;
    apre[o] = x;
    hid[o] = x * sigmoid(x);
  }
};
template <typename TA>
struct EpResidual {  // R = c + b2 - v
  float *res; const float *b2; const TA *v; int dh; long zs;
  __device__ void operator()(int z, int i, int j, float c) const {
    const long o = z * zs + (long)i * dh + j;
    res[o] = c + b2[(long)z * dh + j] - ldf(v, o);
  }
};
struct EpSiluGrad {  // G = scale c SiLU'(A), written over A
  float *ag; float scale; int F; long zs;
  __device__ void operator()(int z, int i, int j, float c) const {
    const long o = z * zs + (long)i * F + j;
    const float a = ag[o], s = sigmoid(a);
    ag[o] = scale * c * (s * (1.0f + a * (1.0f - s)));
  }
};
struct EpUpdate {  // W[z][i][j] -= step c
  float *w; float step; int ld; long zs;
  __device__ void operator()(int z, int i, int j, float c) const {
    w[z * zs + (long)i * ld + j] -= step * c;
  }
};

// Sums over the N tokens run in two fixed-order levels: NPART parts of
// consecutive rows per head, then the parts in order.
constexpr int NPART = 64;

// part[z][p][c] = sum over rows of part p of X[z][t][c] (float64; four row
// groups t = g, g+4, ... added in a fixed order).  grid (ceil(cols/64), NPART, Z).
__global__ __launch_bounds__(256) void k_colsum_part(const float *__restrict__ x, int rows, int cols,
                                                     double *__restrict__ part) {
  __shared__ double red[4][64];
  const int z = blockIdx.z, p = blockIdx.y, c = blockIdx.x * 64 + threadIdx.x % 64, g = threadIdx.x / 64;
  const int per = (rows + NPART - 1) / NPART, t0 = p * per, t1 = min(rows, t0 + per);
  const float *xz = x + (long)z * rows * cols;
  double s = 0.0;
  if (c < cols)
    for (int t = t0 + g; t < t1; t += 4) s += (double)xz[(long)t * cols + c];
  red[g][threadIdx.x % 64] = s;
  __syncthreads();
  if (g == 0 && c < cols)
    part[((long)z * NPART + p) * cols + c] = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                                             (red[2][threadIdx.x] + red[3][threadIdx.x]);
}

// bias[z][c] -= step * sum_p part[z][p][c].  grid (ceil(cols/64), Z), 64 threads.
__global__ __launch_bounds__(64) void k_colsum_update(const double *__restrict__ part, int cols,
                                                      float *__restrict__ bias, float step) {
  const int z = blockIdx.y, c = blockIdx.x * 64 + threadIdx.x;
  if (c >= cols) return;
  double s = 0.0;
  for (int p = 0; p < NPART; ++p) s += part[((long)z * NPART + p) * cols + c];
  bias[(long)z * cols + c] -= step * (float)s;
}

// part[z][p] = sum of squares over part p of R[z] (float64, fixed order).
// grid (NPART, Z), 256 threads.
__global__ __launch_bounds__(256) void k_sumsq_part(const float *__restrict__ res, long n,
                                                    double *__restrict__ part) {
  __shared__ double red[256];
  const int z = blockIdx.y, p = blockIdx.x, tid = threadIdx.x;
  const long per = (n + NPART - 1) / NPART, i0 = p * per, i1 = min(n, i0 + per);
  const float *rz = res + (long)z * n;
  double s = 0.0;
  for (long i = i0 + tid; i < i1; i += 256) {
    const double x = rz[i];
    s = fma(x, x, s);
  }
  red[tid] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) part[(long)z * NPART + p] = red[0];
}

// loss[z * stride + st] = sum_p part[z][p] / N.  grid (ceil(Z/64)), 64 threads.
__global__ __launch_bounds__(64) void k_loss(const double *__restrict__ part, int Z, double inv_n,
                                             double *__restrict__ loss, int stride, int st) {
  const int z = blockIdx.x * 64 + threadIdx.x;
  if (z >= Z) return;
  double s = 0.0;
  for (int p = 0; p < NPART; ++p) s += part[(long)z * NPART + p];
  loss[(long)z * stride + st] = s * inv_n;
}

// float32 masters from the act-dtype weights, and back (round to nearest even).
template <typename TA>
__global__ __launch_bounds__(256) void k_to_master(const TA *__restrict__ w, float *__restrict__ m, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) m[i] = ldf(w, i);
}
template <typename TA>
__global__ __launch_bounds__(256) void k_from_master(const float *__restrict__ m, TA *__restrict__ w, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) store_f32(w + i, m[i]);
}

static inline unsigned blocks(long n) { return (unsigned)((n + 255) / 256); }

static void colsum_update(const float *x, int rows, int cols, float *bias, float step, double *part, int Z,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_colsum_part, dim3((cols + 63) / 64, NPART, Z), dim3(256), 0, st, x, rows, cols, part);
  hipLaunchKernelGGL(k_colsum_update, dim3((cols + 63) / 64, Z), dim3(64), 0, st, (const double *)part, cols,
                     bias, step);
}

template <typename TA, typename TC>
static void fit_typed(const FitArgs &a, hipStream_t st) {
  const int Z = a.B * a.G * a.Hkv, GH = a.G * a.Hkv, N = a.N, dh = a.dh, F = a.F, r = a.r;
  const int D = GH * dh;
  const long nw1 = (long)Z * F * dh, nb1 = (long)Z * F, nw2 = (long)Z * dh * F, nb2 = (long)Z * dh;
  // master weights
  hipLaunchKernelGGL(k_to_master<TA>, dim3(blocks(nw1)), dim3(256), 0, st, (const TA *)a.w1, a.m_w1, nw1);
  hipLaunchKernelGGL(k_to_master<TA>, dim3(blocks(nb1)), dim3(256), 0, st, (const TA *)a.b1, a.m_b1, nb1);
  hipLaunchKernelGGL(k_to_master<TA>, dim3(blocks(nw2)), dim3(256), 0, st, (const TA *)a.w2, a.m_w2, nw2);
  hipLaunchKernelGGL(k_to_master<TA>, dim3(blocks(nb2)), dim3(256), 0, st, (const TA *)a.b2, a.m_b2, nb2);
  // K_hat[z][t][d] = sum_i deq(c~[b][t][i]) U[b][(l, h, d)][i]
  {
    CoefOp<TC> A{(const TC *)a.coeff, a.coeff_scale, GH, N, r};
    BOp<TA, true> Ub{(const TA *)a.basis, ZOff{GH, (long)D * r, (long)dh * r}, r};
    gemm(A, Ub, EpStore{a.khat, dh, (long)N * dh}, N, dh, r, Z, st);
  }
  const long zsd = (long)N * dh, zsf = (long)N * F;
  const float two_n = 2.0f / (float)N;
  AOp<float, true> Khat{a.khat, ZOff{1, zsd, 0}, dh};
  AOp<float, true> Hrow{a.hid, ZOff{1, zsf, 0}, F};
  AOp<float, true> Rrow{a.res, ZOff{1, zsd, 0}, dh};
  BOp<float, true> W1t{a.m_w1, ZOff{1, (long)F * dh, 0}, dh};   // B(d, f) = W1[f][d]
  BOp<float, true> W2t{a.m_w2, ZOff{1, (long)dh * F, 0}, F};    // B(f, e) = W2[e][f]
  BOp<float, false> W2n{a.m_w2, ZOff{1, (long)dh * F, 0}, F};   // B(e, f) = W2[e][f]
  AOp<float, false> Rcol{a.res, ZOff{1, zsd, 0}, dh};           // A(e, t) = R[t][e]
  AOp<float, false> Gcol{a.apre, ZOff{1, zsf, 0}, F};           // A(f, t) = G[t][f]
  BOp<float, false> Hn{a.hid, ZOff{1, zsf, 0}, F};              // B(t, f) = H[t][f]
  BOp<float, false> Kn{a.khat, ZOff{1, zsd, 0}, dh};            // B(t, d) = K_hat[t][d]
  for (int s = 0; s <= a.steps; ++s) {
    gemm(Khat, W1t, EpHidden{a.apre, a.hid, a.m_b1, F, zsf}, N, F, dh, Z, st);
    gemm(Hrow, W2t, EpResidual<TA>{a.res, a.m_b2, (const TA *)a.v, dh, zsd}, N, dh, F, Z, st);
    if (a.loss) {
      hipLaunchKernelGGL(k_sumsq_part, dim3(NPART, Z), dim3(256), 0, st, (const float *)a.res, zsd, a.part);
      hipLaunchKernelGGL(k_loss, dim3((Z + 63) / 64), dim3(64), 0, st, (const double *)a.part, Z, 1.0 / N,
                         a.loss, a.steps + 1, s);
    }
    if (s == a.steps) break;
    gemm(Rrow, W2n, EpSiluGrad{a.apre, two_n, F, zsf}, N, F, dh, Z, st);
    gemm(Rcol, Hn, EpUpdate{a.m_w2, a.lr * two_n, F, (long)dh * F}, dh, F, N, Z, st);
    colsum_update(a.res, N, dh, a.m_b2, a.lr * two_n, a.part, Z, st);
    gemm(Gcol, Kn, EpUpdate{a.m_w1, a.lr, dh, (long)F * dh}, F, dh, N, Z, st);
    colsum_update(a.apre, N, F, a.m_b1, a.lr, a.part, Z, st);
  }
  hipLaunchKernelGGL(k_from_master<TA>, dim3(blocks(nw1)), dim3(256), 0, st, (const float *)a.m_w1, (TA *)a.o_w1, nw1);
  hipLaunchKernelGGL(k_from_master<TA>, dim3(blocks(nb1)), dim3(256), 0, st, (const float *)a.m_b1, (TA *)a.o_b1, nb1);
  hipLaunchKernelGGL(k_from_master<TA>, dim3(blocks(nw2)), dim3(256), 0, st, (const float *)a.m_w2, (TA *)a.o_w2, nw2);
  hipLaunchKernelGGL(k_from_master<TA>, dim3(blocks(nb2)), dim3(256), 0, st, (const float *)a.m_b2, (TA *)a.o_b2, nb2);
}

}  // namespace fit

hipError_t run_fit(const FitArgs &a, hipStream_t st) {
  CompressArgs c;
  memset(&c, 0, sizeof c);
  c.k = a.k; c.basis = a.basis; c.coeff = a.coeff; c.coeff_scale = a.coeff_scale; c.c64 = a.c64;
  c.B = a.B; c.G = a.G; c.Hkv = a.Hkv; c.dh = a.dh; c.r = a.r; c.N = a.N;
  c.act = a.act; c.coeff_dt = a.coeff_dt;
  compress_coefficients(c, st);
  if (a.act == LOWRAM_F32) fit::fit_typed<float, float>(a, st);
  else if (a.coeff_dt == LOWRAM_I8) fit::fit_typed<bf16, int8_t>(a, st);
  else fit::fit_typed<bf16, bf16>(a, st);
  return hipGetLastError();
}

}  // namespace lowram
