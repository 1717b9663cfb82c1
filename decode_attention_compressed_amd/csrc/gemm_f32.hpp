// Batched float32 products on the matrix cores (v_mfma_f32_16x16x4_f32,
// float32 operands and sums): 64 x 64 output tiles per workgroup, k-steps of 16
// or 64 staged through LDS, each of the 4 waves a 32 x 32 quarter (2 x 2 blocks of
// 16 x 16); the next step's operands are read into registers while the
// current step's products run.  Operands are read through loader functors, outputs handed to an
// epilogue functor, so one kernel serves every product shape and fused
// elementwise step.
#pragma once

#include "common.hpp"

namespace lowram {
namespace f32gemm {

// Offset of head z's block in an array: (z / div) * hi + (z % div) * lo.
struct ZOff {
  int div;
  long hi, lo;
  __device__ long operator()(int z) const { return (long)(z / div) * hi + (long)(z % div) * lo; }
};

__device__ __forceinline__ float ldf(const float *p, long i) { return p[i]; }
__device__ __forceinline__ float ldf(const bf16 *p, long i) { return bf16_bits_to_f32(p[i].u); }

// A(z, i, k) operands.  KC: k is the contiguous index.
template <typename T, bool KC_>
struct AOp {
  static constexpr bool KC = KC_;
  const T *p; ZOff zo; int ld;
  __device__ float operator()(int z, int i, int k) const {
    return ldf(p, zo(z) + (KC ? (long)i * ld + k : (long)k * ld + i));
  }
};
// B(z, k, j) operands.  KC: k is the contiguous index.
template <typename T, bool KC_>
struct BOp {
  static constexpr bool KC = KC_;
  const T *p; ZOff zo; int ld;
  __device__ float operator()(int z, int k, int j) const {
    return ldf(p, zo(z) + (KC ? (long)j * ld + k : (long)k * ld + j));
  }
};
// C(z)[i][j] = sum_k A(z, i, k) B(z, k, j) handed to ep(z, i, j, c).
// grid (ceil(N/64), ceil(M/64), Z), 256 threads.
// UPPER: only tiles with i0 <= j0 run (for symmetric products whose epilogue
// writes both triangles).
template <class LA, class LB, class EP, bool UPPER, int KT>
__global__ __launch_bounds__(256) void k_gemm(LA A, LB Bm, EP ep, int M, int N, int K) {
  // KT: k per staged step
  constexpr int PER = KT * 64 / 256;     // operand values per thread and step
  __shared__ float As[KT][64 + 1];
  __shared__ float Bs[KT][64 + 1];
  const int z = blockIdx.z, i0 = blockIdx.y * 64, j0 = blockIdx.x * 64, tid = threadIdx.x;
  if (UPPER && i0 > j0) return;
  const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, kg = lane >> 4;
  const int wi = (w >> 1) * 32, wj = (w & 1) * 32;  // this wave's quarter of the tile
  typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
  f32x4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next step's operands are read into registers while this step's
  // products run
  float ra[PER], rb[PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + 256 * u;
      const int kk = LA::KC ? idx % KT : idx / 64, m = LA::KC ? idx / KT : idx % 64;
      const int gi = i0 + m, gk = k0 + kk;
      ra[u] = (gi < M && gk < K) ? A(z, gi, gk) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + 256 * u;
      const int kk = LB::KC ? idx % KT : idx / 64, n = LB::KC ? idx / KT : idx % 64;
      const int gj = j0 + n, gk = k0 + kk;
      rb[u] = (gj < N && gk < K) ? Bm(z, gk, gj) : 0.f;
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + 256 * u;
      const int kk = LA::KC ? idx % KT : idx / 64, m = LA::KC ? idx / KT : idx % 64;
      As[kk][m] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + 256 * u;
      const int kk = LB::KC ? idx % KT : idx / 64, n = LB::KC ? idx / KT : idx % 64;
      Bs[kk][n] = rb[u];
    }
  };
  fetch(0);
  put();
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += KT) {
    const bool more = k0 + KT < K;
    if (more) fetch(k0 + KT);
    // 4-wide k-steps: lane (l16, kg) holds A[row l16][k kg] and B[k kg][column l16]
#pragma unroll
    for (int k4 = 0; k4 < KT / 4; ++k4) {
      float av[2], bv[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) av[mi] = As[4 * k4 + kg][wi + 16 * mi + l16];
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) bv[nj] = Bs[4 * k4 + kg][wj + 16 * nj + l16];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi], bv[nj], acc[mi][nj], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      put();
      __syncthreads();
    }
  }
  // lane holds C[wi + 16 mi + 4 kg + v][wj + 16 nj + l16]
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + wi + 16 * mi + 4 * kg + v, j = j0 + wj + 16 * nj + l16;
        if (i < M && j < N) ep(z, i, j, acc[mi][nj][v]);
      }
}

// Deep contractions (K >= 2048: the reductions over tokens) stage 64 k per
// step, so fewer round trips; shorter ones 16, which keeps the registers low
// and many workgroups per CU hiding each other's loads (their grids are large).
template <bool UPPER = false, class LA, class LB, class EP>
inline void gemm(LA A, LB Bm, EP ep, int M, int N, int K, int Z, hipStream_t st) {
  if (M <= 0 || N <= 0 || Z <= 0) return;
  const dim3 grid((N + 63) / 64, (M + 63) / 64, Z);
  if (K >= 2048)
    hipLaunchKernelGGL((k_gemm<LA, LB, EP, UPPER, 64>), grid, dim3(256), 0, st, A, Bm, ep, M, N, K);
  else
    hipLaunchKernelGGL((k_gemm<LA, LB, EP, UPPER, 16>), grid, dim3(256), 0, st, A, Bm, ep, M, N, K);
}


}  // namespace f32gemm
}  // namespace lowram
