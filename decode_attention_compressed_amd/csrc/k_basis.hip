// The group key basis at prefill (gfx950, float32).
//
// xKV finds a few principal directions of the keys and shares the basis
// across adjacent layers (rit.work page, keys section; zicq.com English
// summary, "Cross-Layer Low-Rank Key Compression").  Here, per sequence:
//   G = K_cat^T K_cat over the N prefill tokens (D x D, float32; only the
//       upper tiles are computed, the epilogue writes both triangles);
//   Q = orth(Omega), Omega a counter-hash pseudo-random r x D start;
//   `iterations` times: Q = orth(Q G)   (subspace iteration, rows of Q^T);
//   U = Q^T rounded to the act dtype.
// orth() is block Gram-Schmidt run twice (blocks of NB rows): each block is
// projected off the finished rows with two products, then its rows are
// orthonormalised one by one inside one workgroup (each thread owns a fixed
// set of columns, so it only ever reads back what it wrote).  In the first
// pass a row whose remainder falls below TAU of its norm (numerically in the
// span of the rows before it) is replaced by a pseudo-random row, which the
// second pass orthogonalises like any other.  The result spans the dominant r-dimensional
// subspace; no rotation within it is made (reconstructions U U^T k do not
// depend on one).
#include <cstring>

#include "common.hpp"
#include "gemm_f32.hpp"
#include "internal.hpp"

namespace lowram {
namespace basis {

using namespace f32gemm;

constexpr int NB = 32;          // rows per Gram-Schmidt block
constexpr int ONT = 1024;       // threads of the in-block kernel
constexpr int MAXE = 8;         // columns per thread (D <= ONT * MAXE)
constexpr int PBATCH = 16;      // rows whose dots are reduced together (8 when D > 4 ONT)
constexpr int KSPLIT = 16;      // most column slices of the block dots
constexpr float TAU = 1e-4f;    // remainder / norm below which a row counts as dependent

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

// Block sums of NV values per thread, in a fixed order; every thread gets the totals.
template <int NV>
__device__ void block_sums(float (&v)[NV], float *red /* [ONT / 64][NV] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v[k] += __shfl_xor(v[k], o, 64);
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < NV; ++k) red[w * NV + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < ONT / 64; ++ww) s += red[ww * NV + k];
    v[k] = s;
  }
  __syncthreads();
}

// v -= sum_c <v, q row c> q row c over rows first .. first + count - 1, in
// batches of PB rows: the batch's rows (the thread's ME columns of each) are
// loaded into registers at once, so a batch costs one round trip to memory;
// each wave reduces its partial dot of a row with shuffles and leaves it in
// LDS; after one barrier every thread adds the waves' parts in order and
// updates v from the rows it holds.  Thread t holds columns t + ONT e of v.
// red: [PB][ONT / 64].
template <int PB, int ME>
__device__ __forceinline__ void project_rows(float (&v)[ME], const float *q, long base, int D, int first,
                                             int count, float *red) {
  constexpr int NWV = ONT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int c0 = first; c0 < first + count; c0 += PB) {
    const int nc = min(PB, first + count - c0);
    float rw[PB][ME];
#pragma unroll
    for (int c = 0; c < PB; ++c) {
      const float *row = q + base + (long)min(c0 + c, first + count - 1) * D;
#pragma unroll
      for (int e = 0; e < ME; ++e) {
        const int i = tid + ONT * e;
        rw[c][e] = i < D ? row[i] : 0.f;
      }
    }
#pragma unroll
    for (int c = 0; c < PB; ++c) {
      if (c < nc) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < ME; ++e) s = fmaf(rw[c][e], v[e], s);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (lane == 0) red[c * NWV + w] = s;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < PB; ++c) {
      if (c < nc) {
        float d = 0.f;
#pragma unroll
        for (int ww = 0; ww < NWV; ++ww) d += red[c * NWV + ww];
#pragma unroll
        for (int e = 0; e < ME; ++e) v[e] = fmaf(-d, rw[c][e], v[e]);
      }
    }
    __syncthreads();
  }
}

template <int ME>
__device__ __forceinline__ float row_norm(const float (&v)[ME], float *red) {
  float n2[1] = {0.f};
#pragma unroll
  for (int e = 0; e < ME; ++e) n2[0] = fmaf(v[e], v[e], n2[0]);
  block_sums<1>(n2, red);
  return sqrtf(n2[0]);
}

// Rows row0 .. row0 + nb - 1 of src orthonormalised one by one against the
// rows before them inside the block (two passes each) and written to rows
// row0.. of q (src may be q).  DETECT: a row whose remainder is <= TAU *
// nrm0[a] is replaced by a pseudo-random row, orthogonalised here against the
// block's earlier rows; the second block pass projects it off the earlier
// blocks (a random row is far from their span, so one projection suffices).
// Thread t owns columns t + ONT e (e < ME, ME = ceil(D / ONT)) and only reads
// back columns it wrote itself.  grid (B), ONT threads.
template <bool DETECT, int ME>
__global__ __launch_bounds__(ONT) void k_intra(const float *src, float *q, int r, int D, int row0, int nb,
                                               const double *__restrict__ nrm0, uint32_t salt) {
  constexpr int PB = ME <= 4 ? PBATCH : PBATCH / 2;  // the batch's columns stay within the registers
  __shared__ float red[PB * (ONT / 64)];
  const int b = blockIdx.x, tid = threadIdx.x;
  const long base = (long)b * r * D;
  for (int a = 0; a < nb; ++a) {
    float v[ME];
#pragma unroll
    for (int e = 0; e < ME; ++e) {
      const int i = tid + ONT * e;
      v[e] = i < D ? src[base + (long)(row0 + a) * D + i] : 0.f;
    }
    project_rows<PB>(v, q, base, D, row0, a, red);
    project_rows<PB>(v, q, base, D, row0, a, red);
    float nrm = row_norm(v, red);
    if (DETECT && (double)nrm <= (double)TAU * nrm0[(long)b * NB + a]) {
#pragma unroll
      for (int e = 0; e < ME; ++e) {
        const int i = tid + ONT * e;
        v[e] = i < D ? hash_uniform(b, row0 + a, i, salt) : 0.f;
      }
      project_rows<PB>(v, q, base, D, row0, a, red);
      project_rows<PB>(v, q, base, D, row0, a, red);
      nrm = row_norm(v, red);
    }
    const float inv = nrm > 0.f ? 1.0f / nrm : 0.f;
#pragma unroll
    for (int e = 0; e < ME; ++e) {
      const int i = tid + ONT * e;
      if (i < D) q[base + (long)(row0 + a) * D + i] = v[e] * inv;
    }
  }
}

template <bool DETECT>
static void launch_intra(const float *src, float *q, int B, int r, int D, int row0, int nb, const double *nrm,
                         uint32_t salt, hipStream_t st) {
  const int me = (D + ONT - 1) / ONT;
  if (me <= 1)
    hipLaunchKernelGGL((k_intra<DETECT, 1>), dim3(B), dim3(ONT), 0, st, src, q, r, D, row0, nb, nrm, salt);
  else if (me <= 2)
    hipLaunchKernelGGL((k_intra<DETECT, 2>), dim3(B), dim3(ONT), 0, st, src, q, r, D, row0, nb, nrm, salt);
  else if (me <= 4)
    hipLaunchKernelGGL((k_intra<DETECT, 4>), dim3(B), dim3(ONT), 0, st, src, q, r, D, row0, nb, nrm, salt);
  else
    hipLaunchKernelGGL((k_intra<DETECT, MAXE>), dim3(B), dim3(ONT), 0, st, src, q, r, D, row0, nb, nrm, salt);
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

static void orth(float *src, float *q, float *cbuf, float *cpart, double *nrm, int B, int r, int D,
                 uint32_t salt, hipStream_t st) {
  const long zs = (long)r * D;
  const int S = dot_slices(D), Dsl = D / S;
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
      if (pass == 0)
        launch_intra<true>(blk, q, B, r, D, j0, nb, nrm, salt, st);
      else
        launch_intra<false>(blk, q, B, r, D, j0, nb, nrm, salt, st);
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
  gemm<true>(Ka, Kb, EpSym{a.gram, D}, D, D, N, B, st);
  // start
  hipLaunchKernelGGL(k_start, dim3((D + 255) / 256, r, B), dim3(256), 0, st, a.yt, r, D);
  orth(a.yt, a.qt, a.cbuf, a.cpart, a.nrm, B, r, D, 1u, st);
  AOp<float, true> Qa{a.qt, ZOff{1, zs, 0}, D};
  BOp<float, false> Gb{a.gram, ZOff{1, (long)D * D, 0}, D};
  for (int it = 0; it < a.iterations; ++it) {
    gemm(Qa, Gb, EpPut{a.yt, zs, D}, r, D, D, B, st);   // Yt = Qt G
    orth(a.yt, a.qt, a.cbuf, a.cpart, a.nrm, B, r, D, 2u + it, st);
  }
  hipLaunchKernelGGL(k_store_basis<TA>, dim3((r + 63) / 64, (D + 3) / 4, B), dim3(256), 0, st,
                     (const float *)a.qt, (TA *)a.basis, r, D);
}

}  // namespace basis

int basis_max_dim() { return basis::ONT * basis::MAXE; }

hipError_t run_basis(const BasisArgs &a, hipStream_t st) {
  if (a.act == LOWRAM_F32) basis::basis_typed<float>(a, st);
  else basis::basis_typed<bf16>(a, st);
  return hipGetLastError();
}

}  // namespace lowram
