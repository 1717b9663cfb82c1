// Batched float32 products on the vector ALUs: 64 x 64 output tiles per
// workgroup, 4 x 4 per thread, k-steps of 16 staged through LDS.  Operands are
// read through loader functors, outputs handed to an epilogue functor, so one
// kernel serves every product shape and fused elementwise step.
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
template <class LA, class LB, class EP, bool UPPER = false>
__global__ __launch_bounds__(256) void k_gemm(LA A, LB Bm, EP ep, int M, int N, int K) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int z = blockIdx.z, i0 = blockIdx.y * 64, j0 = blockIdx.x * 64, tid = threadIdx.x;
  if (UPPER && i0 > j0) return;
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int idx = tid; idx < 16 * 64; idx += 256) {
      const int kk = LA::KC ? idx % 16 : idx / 64, m = LA::KC ? idx / 16 : idx % 64;
      const int gi = i0 + m, gk = k0 + kk;
      As[kk][m] = (gi < M && gk < K) ? A(z, gi, gk) : 0.f;
    }
    for (int idx = tid; idx < 16 * 64; idx += 256) {
      const int kk = LB::KC ? idx % 16 : idx / 64, n = LB::KC ? idx / 16 : idx % 64;
      const int gj = j0 + n, gk = k0 + kk;
      Bs[kk][n] = (gj < N && gk < K) ? Bm(z, gk, gj) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[kk][ty + 16 * a];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[kk][tx + 16 * c];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(av[a], bv[c], acc[a][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = i0 + ty + 16 * a, j = j0 + tx + 16 * c;
      if (i < M && j < N) ep(z, i, j, acc[a][c]);
    }
}

template <bool UPPER = false, class LA, class LB, class EP>
inline void gemm(LA A, LB Bm, EP ep, int M, int N, int K, int Z, hipStream_t st) {
  if (M <= 0 || N <= 0 || Z <= 0) return;
  hipLaunchKernelGGL((k_gemm<LA, LB, EP, UPPER>), dim3((N + 63) / 64, (M + 63) / 64, Z), dim3(256), 0, st,
                     A, Bm, ep, M, N, K);
}


}  // namespace f32gemm
}  // namespace lowram
