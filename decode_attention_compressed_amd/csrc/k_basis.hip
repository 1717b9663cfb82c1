// The group key basis at prefill (gfx950, float32).
//
// xKV finds a few principal directions of the keys and shares the basis
// across adjacent layers (rit.work page, keys section; zicq.com English
// summary, "Cross-Layer Low-Rank Key Compression").  Here, per sequence:
//   G = K_cat^T K_cat over the N prefill tokens (D x D, float32 sums; only
//       the upper tiles are computed, the epilogue writes both triangles; on
//       the matrix cores for bf16 keys);
//   Q = orth(Omega), Omega a counter-hash pseudo-random r x D start;
//   `iterations` times: Q = orth(Q G)   (subspace iteration, rows of Q^T);
//   U = Q^T rounded to the act dtype.
// orth() orthonormalises blocks of NB rows in order, each twice: the block is
// projected off the finished rows with two products, then orthonormalised in
// itself by a Cholesky factorisation of its NB x NB Gram matrix M = V V^T
// (float64, summed over column slices in a fixed order): with M = L L^T the
// rows of L^{-1} V (forward substitution) are orthonormal.  In the first pass a row whose pivot
// (its remainder after the block's earlier rows, squared) falls below TAU^2
// of its squared norm is numerically in the span before it: it is left out of
// the factorisation and replaced by a pseudo-random row, which the second
// pass orthogonalises like any other.  The result spans the dominant
// r-dimensional subspace; no rotation within it is made (reconstructions
// U U^T k do not depend on one).
#include <cstring>
#include <type_traits>

#include "common.hpp"
#include "gemm_f32.hpp"
#include "internal.hpp"

namespace lowram {
namespace basis {

using namespace f32gemm;

constexpr int NB = 32;          // rows per orthonormalisation block
constexpr int MAXD = 8192;      // largest group key dim D
constexpr int GW = 256;         // columns per slice of the in-block Gram matrix
constexpr int KSPLIT = 16;      // most column slices of the block dots
constexpr double TAU = 1e-4;    // remainder / norm below which a row counts as dependent

// K_cat(b, t, i) = k[b][i / dh][t][i % dh], read as A(b, i, t) = K_cat(b, t, i)
// and B(b, t, j) = K_cat(b, t, j); consecutive dims of one (layer, head) block
// are contiguous, so neither operand is contiguous in its k index.
template <typename TA>
__device__ __forceinline__ float kcat(const TA *p, int N, int dh, int D, int b, int t, int i) {
  return ldf(p, (long)b * D * N + (long)(i / dh) * N * dh + (long)t * dh + i % dh);
}
template <typename TA>
struct KcatA {
  static constexpr bool KC = false;
  const TA *p; int N, dh, D;
  __device__ float operator()(int b, int i, int t) const { return kcat(p, N, dh, D, b, t, i); }
};
template <typename TA>
struct KcatB {
  static constexpr bool KC = false;
  const TA *p; int N, dh, D;
  __device__ float operator()(int b, int t, int j) const { return kcat(p, N, dh, D, b, t, j); }
};
struct EpSym {  // G[b][i][j] = G[b][j][i] = c
  float *g; int D;
  __device__ void operator()(int b, int i, int j, float c) const {
    float *gb = g + (long)b * D * D;
    gb[(long)i * D + j] = c;
    gb[(long)j * D + i] = c;
  }
};
struct EpSub {  // X[b][row0 + i][j] -= c
  float *x; long zs; int ld, row0;
  __device__ void operator()(int b, int i, int j, float c) const {
    x[b * zs + (long)(row0 + i) * ld + j] -= c;
  }
};
struct EpPut {  // X[b][i][j] = c
  float *x; long zs; int ld;
  __device__ void operator()(int b, int i, int j, float c) const { x[b * zs + (long)i * ld + j] = c; }
};

// Counter-hash uniform in [-1, 1) for (b, row, column, salt).  The four
// counters are combined with multiplicative-hashing constants (the 32-bit
// golden-ratio constant 0x9E3779B1, the low word of the 64-bit golden gamma
// 0x9E3779B97F4A7C15, and the 32-bit primes of the xxHash32 specification),
// then mixed by the published "lowbias32" finaliser (Chris Wellons'
// hash-prospector: xorshift 16, multiply, xorshift 15, multiply, xorshift 16).
// The top 24 bits give the uniform value.
__device__ __forceinline__ float hash_uniform(uint32_t b, uint32_t row, uint32_t col, uint32_t salt) {
  uint32_t x = b * 0x9E3779B1u ^ (row + 0x7F4A7C15u) * 0x85EBCA77u ^ (col + salt * 0x165667B1u) * 0xC2B2AE3Du;
  x ^= x >> 16; x *= 0x7FEB352Du;
  x ^= x >> 15; x *= 0x846CA68Bu;
  x ^= x >> 16;
  return (float)(x >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

// Yt[b][j][i] = hash_uniform(b, j, i, 0).  grid (ceil(D/256), r, B).
__global__ __launch_bounds__(256) void k_start(float *__restrict__ yt, int r, int D) {
  const int i = blockIdx.x * 256 + threadIdx.x, j = blockIdx.y, b = blockIdx.z;
  if (i < D) yt[((long)b * r + j) * D + i] = hash_uniform(b, j, i, 0);
}

// nrm[b][a] = || X[b][row0 + a] ||, float64, fixed order.  grid (NB, B), 256 threads.
__global__ __launch_bounds__(256) void k_rownorm(const float *__restrict__ x, int r, int D, int row0,
                                                 double *__restrict__ nrm) {
  __shared__ double red[256];
  const int a = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float *row = x + ((long)b * r + row0 + a) * D;
  double s = 0.0;
  for (int i = tid; i < D; i += 256) s = fma((double)row[i], (double)row[i], s);
  red[tid] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) nrm[(long)b * NB + a] = sqrt(red[0]);
}

// G[b] = K_cat^T K_cat of bf16 keys on the matrix cores: bf16 x bf16
// products are exact in float32 and the sums accumulate in float32, the
// precision of the vector-ALU product it replaces.  One workgroup of 4 waves
// per 128 x 128 tile of G with i0 <= j0 (the epilogue writes both triangles;
// a diagonal tile writes only i <= j, so no element is stored twice); each
// wave owns a 64 x 64 quarter, 16 blocks of v_mfma_f32_16x16x32_bf16.  Per
// step of 32 tokens the tile's key columns (rows i and rows j of K_cat^T) are
// staged through LDS token-contiguous per column, two tokens per dword, so a
// lane reads its 8 consecutive tokens of a column as one MFMA operand; the
// next step's keys are loaded into registers while the current step's
// products run.  Tokens past N and columns past D are zero.
// grid (ceil(D / 128), ceil(D / 128), B), 256 threads.
namespace gram {
constexpr int TI = 128, KS = 32, LD = KS + 8;  // tile, tokens per step, LDS row stride (elements)
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
}  // namespace gram

__global__ __launch_bounds__(256) void k_gram_mfma(const uint16_t *__restrict__ k, float *__restrict__ g,
                                                   int N, int dh, int D) {
  using namespace gram;
  __shared__ __align__(16) uint16_t As[2][TI * LD], Bs[2][TI * LD];
  const int b = blockIdx.z, i0 = blockIdx.y * TI, j0 = blockIdx.x * TI;
  if (i0 > j0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const uint16_t *kb = k + (long)b * D * N;
  // staging: thread (token pair tp, column group cg) loads tokens 2 tp, 2 tp + 1
  // of columns 8 cg .. 8 cg + 7 of the A (rows i) and B (rows j) tiles
  const int tp = tid >> 4, cg = tid & 15;
  auto col_ptr = [&](int c) -> const uint16_t * {  // K_cat(t = 0, column c)
    return kb + (long)(c / dh) * N * dh + c % dh;
  };
  const int ca = i0 + 8 * cg, cb = j0 + 8 * cg;
  const uint16_t *pa = col_ptr(ca < D ? ca : 0), *pb = col_ptr(cb < D ? cb : 0);
  const bool oka = ca < D, okb = cb < D;
  u32x4 ra[2], rb[2];
  auto load = [&](int t0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + 2 * tp + u;
      ra[u] = (oka && t < N) ? gld16(pa + (long)t * dh) : v4(0, 0, 0, 0);
      rb[u] = (okb && t < N) ? gld16(pb + (long)t * dh) : v4(0, 0, 0, 0);
    }
  };
  // column c = 8 cg + e of a tile gets the dword (token 2 tp, token 2 tp + 1)
  auto stage = [&](uint16_t *dst, const u32x4 (&r)[2]) {
    const uint32_t x0[4] = {r[0].x, r[0].y, r[0].z, r[0].w}, x1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t lo = (x0[m] & 0xFFFFu) | (x1[m] << 16);          // column 8 cg + 2 m
      const uint32_t hi = (x0[m] >> 16) | (x1[m] & 0xFFFF0000u);      // column 8 cg + 2 m + 1
      *reinterpret_cast<uint32_t *>(dst + (8 * cg + 2 * m) * LD + 2 * tp) = lo;
      *reinterpret_cast<uint32_t *>(dst + (8 * cg + 2 * m + 1) * LD + 2 * tp) = hi;
    }
  };
  const int wi = (w >> 1) * 64, wj = (w & 1) * 64;  // this wave's quarter of the tile
  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int steps = (N + KS - 1) / KS;
  load(0);
  stage(As[0], ra);
  stage(Bs[0], rb);
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    if (st + 1 < steps) load((st + 1) * KS);
    bf16x8 af[4], bf[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      af[mi] = *reinterpret_cast<const bf16x8 *>(As[buf] + (wi + 16 * mi + l16) * LD + 8 * kg);
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
      bf[nj] = *reinterpret_cast<const bf16x8 *>(Bs[buf] + (wj + 16 * nj + l16) * LD + 8 * kg);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int nj = 0; nj < 4; ++nj)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bf[nj], acc[mi][nj], 0, 0, 0);
    if (st + 1 < steps) {
      stage(As[buf ^ 1], ra);
      stage(Bs[buf ^ 1], rb);
    }
    __syncthreads();
  }
  // lane holds G[i0 + wi + 16 mi + 4 kg + v][j0 + wj + 16 nj + l16]
  float *gb = g + (long)b * D * D;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + wi + 16 * mi + 4 * kg + v, j = j0 + wj + 16 * nj + l16;
        if (i < D && j < D && (i0 != j0 || i <= j)) {
          gb[(long)i * D + j] = acc[mi][nj][v];
          gb[(long)j * D + i] = acc[mi][nj][v];
        }
      }
}

// In-block Gram matrix of rows row0 .. row0 + nb - 1 of x over the GW
// columns of slice s: mpart[b][s][a][c] = sum_i x[a][i] x[c][i] in float64
// (float32 products are exact in float64), columns in ascending order.  Both
// triangles are written.  grid (ceil(D / GW), B), 256 threads.
__global__ __launch_bounds__(256) void k_bgram(const float *__restrict__ x, int r, int D, int row0, int nb,
                                               double *__restrict__ mpart) {
  __shared__ float xs[NB][GW + 1];
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, S = gridDim.x;
  const int c0 = s * GW;
  {  // every load of the slice is issued before any is stored
    constexpr int PER = NB * GW / 256;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + 256 * u, a = idx / GW, i = idx % GW;
      v[u] = (a < nb && c0 + i < D) ? x[((long)b * r + row0 + a) * D + c0 + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + 256 * u;
      xs[idx / GW][idx % GW] = v[u];
    }
  }
  __syncthreads();
  double *mp = mpart + ((long)b * S + s) * NB * NB;
  for (int p = tid; p < NB * NB; p += 256) {
    const int a = p / NB, c = p % NB;
    if (c > a) continue;
    double acc = 0.0;
    for (int i = 0; i < GW; ++i) acc = fma((double)xs[a][i], (double)xs[c][i], acc);
    mp[a * NB + c] = acc;
    mp[c * NB + a] = acc;
  }
}

// Per sequence: M = sum over the S slices (in order) of mpart, then the
// Cholesky factor M = L L^T column by column.  fac receives L below the
// diagonal and 1 / L[a][a] on it.  DETECT: a row whose pivot is <=
// (TAU nrm0[a])^2 is left out (its column of L and its reciprocal pivot are
// zero, so no later row is projected on it and it solves to zero) and flagged
// in dep for replacement; without DETECT only a pivot <= 0 is left out.  The
// slice sums use every thread (eight slices' loads at a time); the
// factorisation runs on the first wave, lane x holding row x of M in
// registers, with the pivot and column values passed between lanes by
// shuffles.  grid (B), NB * NB threads.
template <bool DETECT>
__global__ __launch_bounds__(NB * NB) void k_chol(const double *__restrict__ mpart, int S, int nb,
                                                  const double *__restrict__ nrm0, double *__restrict__ fac,
                                                  int32_t *__restrict__ dep) {
  __shared__ double M[NB][NB + 1];
  const int b = blockIdx.x, tid = threadIdx.x, x = tid / NB, y = tid % NB;
  {
    const double *mp = mpart + (long)b * S * NB * NB + x * NB + y;
    double acc = 0.0;
    for (int s0 = 0; s0 < S; s0 += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = s0 + u < S ? mp[(long)(s0 + u) * NB * NB] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < S) acc += v[u];
    }
    M[x][y] = acc;
  }
  __syncthreads();
  if (tid >= WAVE) return;
  const int lane = tid;
  double mrow[NB];  // row `lane` of M (lanes past nb: zero), updated in place
#pragma unroll
  for (int c = 0; c < NB; ++c) mrow[c] = lane < nb ? M[lane][c] : 0.0;
  // row `lane` of fac is written into M's row as each column is formed (the
  // row's registers hold what is still needed)
  uint32_t dropped = 0u;
#pragma unroll
  for (int a = 0; a < NB; ++a) {
    if (a >= nb) continue;  // (uniform) keeps the loop fully unrolled, rows in registers
    const double d = __shfl(mrow[a], a, WAVE);  // the updated pivot, held by lane a
    const double t = DETECT ? TAU * nrm0[(long)b * NB + a] : 0.0;
    const bool drop = !(d > t * t);
    dropped |= drop ? 1u << a : 0u;
    const double la = drop ? 0.0 : sqrt(d);
    const double ra = drop ? 0.0 : 1.0 / la;
    // column a of L: L[lane][a] for lanes below the pivot
    const double lx = lane > a && lane < nb ? mrow[a] * ra : 0.0;
    if (lane < NB) M[lane][a] = lane == a ? ra : lx;
    // trailing update of this lane's row: M[lane][c] -= L[lane][a] L[c][a]
#pragma unroll
    for (int c = a + 1; c < NB; ++c) {
      const double lc = __shfl(lx, c, WAVE);
      mrow[c] = fma(-lx, lc, mrow[c]);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < NB) {
#pragma unroll
    for (int c = 0; c < NB; ++c) fac[((long)b * NB + lane) * NB + c] = c <= lane && lane < nb ? M[lane][c] : 0.0;
    dep[(long)b * NB + lane] = DETECT && lane < nb ? (int)((dropped >> lane) & 1u) : 0;
  }
}

// Rows row0 .. row0 + nb - 1 of q = L^{-1} (rows of src), column by column, by
// forward substitution with the factor from k_chol (L below the diagonal, the
// reciprocal pivots on it; left-out rows solve to zero).  src may be q: a
// thread reads its column of every row before writing it.  Rows flagged in
// dep get the pseudo-random values of (b, row, column, salt).
// grid (ceil(D / 256), B), 256 threads.
__global__ __launch_bounds__(256) void k_apply_tri(const float *src, float *q, int r, int D, int row0, int nb,
                                                   const double *__restrict__ fac, const int32_t *__restrict__ dep,
                                                   uint32_t salt) {
  __shared__ double T[NB][NB];
  __shared__ int dp[NB];
  const int b = blockIdx.y, tid = threadIdx.x, i = blockIdx.x * 256 + tid;
  for (int idx = tid; idx < NB * NB; idx += 256) T[idx / NB][idx % NB] = fac[(long)b * NB * NB + idx];
  if (tid < NB) dp[tid] = dep[(long)b * NB + tid];
  __syncthreads();
  if (i >= D) return;
  const long base = ((long)b * r + row0) * D + i;
  double v[NB];
#pragma unroll
  for (int a = 0; a < NB; ++a) v[a] = a < nb ? (double)src[base + (long)a * D] : 0.0;
#pragma unroll
  for (int a = 0; a < NB; ++a) {
    if (a >= nb) continue;
    double s = v[a];
#pragma unroll
    for (int c = 0; c < a; ++c) s = fma(-T[a][c], v[c], s);
    v[a] = s * T[a][a];  // the solved value replaces row a's input
    q[base + (long)a * D] = dp[a] ? hash_uniform(b, row0 + a, i, salt) : (float)v[a];
  }
}

// C[b][a][c] = sum over slices s of part[b * S + s][a][c], in order.
// grid (ceil(nb * j0 / 256), B), 256 threads.
__global__ __launch_bounds__(256) void k_sum_slices(const float *__restrict__ part, float *__restrict__ c, int S,
                                                    int nb, int j0, int r) {
  const int idx = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (idx >= nb * j0) return;
  const int a = idx / j0, cc = idx % j0;
  float s = 0.f;
  for (int k = 0; k < S; ++k) s += part[(((long)b * S + k) * NB + a) * r + cc];
  c[((long)b * NB + a) * r + cc] = s;
}

// U[b][i][j] = round(Qt[b][j][i]).  grid (ceil(r/64), ceil(D/4), B), 256 threads.
template <typename TA>
__global__ __launch_bounds__(256) void k_store_basis(const float *__restrict__ qt, TA *__restrict__ u, int r,
                                                     int D) {
  const int j = blockIdx.x * 64 + threadIdx.x % 64, i = blockIdx.y * 4 + threadIdx.x / 64, b = blockIdx.z;
  if (j < r && i < D) store_f32(u + ((long)b * D + i) * r + j, qt[((long)b * r + j) * D + i]);
}

// rows of src -> orthonormal rows of q (block Gram-Schmidt, twice).
// Slices of D for the block dots: about 256 columns each, at most KSPLIT.
static int dot_slices(int D) {
  int S = 1;
  while (S < KSPLIT && D / (2 * S) >= 256 && D % (2 * S * 16) == 0) S *= 2;
  return S;
}

static void orth(float *src, float *q, float *cbuf, float *cpart, double *nrm, double *mpart, double *tri,
                 int32_t *dep, int B, int r, int D, uint32_t salt, hipStream_t st) {
  const long zs = (long)r * D;
  const int S = dot_slices(D), Dsl = D / S;
  const int SG = (D + GW - 1) / GW;
  for (int j0 = 0; j0 < r; j0 += NB) {
    const int nb = min(NB, r - j0);
    hipLaunchKernelGGL(k_rownorm, dim3(nb, B), dim3(256), 0, st, (const float *)src, r, D, j0, nrm);
    for (int pass = 0; pass < 2; ++pass) {
      float *blk = pass == 0 ? src : q;  // pass 0 reads the block from src, pass 1 from q
      if (j0 > 0) {
        // C[b][a][c] = <blk row j0 + a, q row c> (S slices of the columns, added
        // in order), then blk rows -= C q[:j0]
        AOp<float, true> Ab{blk + (long)j0 * D, ZOff{S, zs, Dsl}, D};
        BOp<float, true> Qk{q, ZOff{S, zs, Dsl}, D};
        gemm(Ab, Qk, EpPut{cpart, (long)NB * r, r}, nb, j0, Dsl, B * S, st);
        hipLaunchKernelGGL(k_sum_slices, dim3((nb * j0 + 255) / 256, B), dim3(256), 0, st,
                           (const float *)cpart, cbuf, S, nb, j0, r);
        AOp<float, true> Ac{cbuf, ZOff{1, (long)NB * r, 0}, r};
        BOp<float, false> Qn{q, ZOff{1, zs, 0}, D};
        gemm(Ac, Qn, EpSub{blk, zs, D, j0}, nb, D, j0, B, st);
      }
      hipLaunchKernelGGL(k_bgram, dim3(SG, B), dim3(256), 0, st, (const float *)blk, r, D, j0, nb, mpart);
      if (pass == 0)
        hipLaunchKernelGGL(k_chol<true>, dim3(B), dim3(NB * NB), 0, st, (const double *)mpart, SG, nb,
                           (const double *)nrm, tri, dep);
      else
        hipLaunchKernelGGL(k_chol<false>, dim3(B), dim3(NB * NB), 0, st, (const double *)mpart, SG, nb,
                           (const double *)nrm, tri, dep);
      hipLaunchKernelGGL(k_apply_tri, dim3((D + 255) / 256, B), dim3(256), 0, st, (const float *)blk, q, r, D,
                         j0, nb, (const double *)tri, (const int32_t *)dep, salt);
    }
  }
}

template <typename TA>
static void basis_typed(const BasisArgs &a, hipStream_t st) {
  const int B = a.B, D = a.G * a.Hkv * a.dh, r = a.r, N = a.N;
  const long zs = (long)r * D;
  // Gram matrix, upper tiles
  KcatA<TA> Ka{(const TA *)a.k, N, a.dh, D};
  KcatB<TA> Kb{(const TA *)a.k, N, a.dh, D};
  if (std::is_same<TA, bf16>::value && a.dh % 8 == 0) {
    const int nt = (D + gram::TI - 1) / gram::TI;
    hipLaunchKernelGGL(k_gram_mfma, dim3(nt, nt, B), dim3(256), 0, st, (const uint16_t *)a.k, a.gram, N, a.dh, D);
  } else {
    gemm<true>(Ka, Kb, EpSym{a.gram, D}, D, D, N, B, st);
  }
  // start
  hipLaunchKernelGGL(k_start, dim3((D + 255) / 256, r, B), dim3(256), 0, st, a.yt, r, D);
  orth(a.yt, a.qt, a.cbuf, a.cpart, a.nrm, a.mpart, a.tri, a.dep, B, r, D, 1u, st);
  AOp<float, true> Qa{a.qt, ZOff{1, zs, 0}, D};
  BOp<float, false> Gb{a.gram, ZOff{1, (long)D * D, 0}, D};
  for (int it = 0; it < a.iterations; ++it) {
    gemm(Qa, Gb, EpPut{a.yt, zs, D}, r, D, D, B, st);   // Yt = Qt G
    orth(a.yt, a.qt, a.cbuf, a.cpart, a.nrm, a.mpart, a.tri, a.dep, B, r, D, 2u + it, st);
  }
  hipLaunchKernelGGL(k_store_basis<TA>, dim3((r + 63) / 64, (D + 3) / 4, B), dim3(256), 0, st,
                     (const float *)a.qt, (TA *)a.basis, r, D);
}

}  // namespace basis

int basis_max_dim() { return basis::MAXD; }

hipError_t run_basis(const BasisArgs &a, hipStream_t st) {
  if (a.act == LOWRAM_F32) basis::basis_typed<float>(a, st);
  else basis::basis_typed<bf16>(a, st);
  return hipGetLastError();
}

}  // namespace lowram
