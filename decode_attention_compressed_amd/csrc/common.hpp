// Device helpers shared by the gfx950 kernels: number formats, wave/block
// reductions and a deterministic block-wide top-k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowram {

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
struct bf16 { uint16_t u; };   // bfloat16 bit pattern
struct f16 { uint16_t u; };    // IEEE half bit pattern

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u) { return __uint_as_float(u << 16); }

// float32 -> bfloat16, round to nearest even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float64 -> bfloat16 with a single rounding (RNE on 8 significant bits)
__device__ inline uint16_t f64_to_bf16_bits(double x) {
  if (fabs(x) < 0x1p-126) {  // subnormal bf16 range: grid 2^-133
    const double y = rint(x * 0x1p133) * 0x1p-133;
    return (uint16_t)(__float_as_uint((float)y) >> 16);
  }
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += 0xFFFFFFFFFFFull + ((u >> 45) & 1ull);   // half - 1 + lsb, 45 dropped bits
  u &= ~0x1FFFFFFFFFFFull;
  const float f = (float)__longlong_as_double((long long)u);  // exact, or inf past the range
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// float64 -> float16 with a single rounding (RNE on 11 significant bits)
__device__ inline uint16_t f64_to_f16_bits(double x) {
  double y;
  if (fabs(x) < 0x1p-14) {  // subnormal half range: grid 2^-24
    y = rint(x * 0x1p24) * 0x1p-24;
  } else {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    u += 0x1FFFFFFFFFFull + ((u >> 42) & 1ull);  // 42 dropped bits
    u &= ~0x3FFFFFFFFFFull;
    y = __longlong_as_double((long long)u);
  }
  const _Float16 h = (_Float16)(float)y;  // exact on the half grid; inf past 65504
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return bf16_bits_to_f32(x.u); }
__device__ __forceinline__ double to_f64(float x) { return (double)x; }
__device__ __forceinline__ double to_f64(bf16 x) { return (double)bf16_bits_to_f32(x.u); }

__device__ __forceinline__ void store_f32(float *p, float x) { *p = x; }
__device__ __forceinline__ void store_f32(bf16 *p, float x) { p->u = f32_to_bf16_bits(x); }

// ---------------------------------------------------------------------------
// 16-byte payloads as native vectors.  (HIP's uint4/float4 are classes; whole
// copies of them out of register arrays are lowered through stack memory and
// serialise the loads.)
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 gld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void lst16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ u32x4 v4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 r;
  r.x = a; r.y = b; r.z = c; r.w = d;
  return r;
}

// ---------------------------------------------------------------------------
// reductions
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, WAVE));
  return v;
}

// order-preserving map of a float64 to uint64 (larger double -> larger key)
// (-0.0 is mapped to +0.0 first, so the two compare equal as doubles do)
__device__ __forceinline__ uint64_t f64_order_key(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (WAVE - 1);
  return lane ? (~0ull >> (WAVE - lane)) : 0ull;
}

// ---------------------------------------------------------------------------
// deterministic block top-k
//
// Selects the k indices in [0, n) with the largest key(i), the lowest index
// winning among equal keys, and writes them in ascending index order to
// out[0..k).  Keys are uint64 (use f64_order_key for float64).  All NT threads
// of the block must call it.  Scratch (shared): TopkSmem.  When ptr_out is not
// null, n is a multiple of C and ptr_out[j] (j = 0..n/C) receives the number of
// selected indices below j*C (chunk CSR pointers).
// ---------------------------------------------------------------------------
struct TopkSmem {
  uint32_t hist[256];
  uint32_t wave_cnt[2][16];
  uint64_t prefix;
  uint32_t need;
  uint32_t base_sel, base_eq;
};

template <int NT>
__device__ inline void block_exclusive_counts(bool a, bool b, uint32_t &pa, uint32_t &pb,
                                              uint32_t &ta, uint32_t &tb, TopkSmem &sm) {
  // Exclusive prefix counts of two flags over the block, in thread order.
  const int w = threadIdx.x / WAVE;
  const uint64_t ma = __ballot(a), mb = __ballot(b);
  const uint64_t lt = lanemask_lt();
  if ((threadIdx.x & (WAVE - 1)) == 0) {
    sm.wave_cnt[0][w] = (uint32_t)__popcll(ma);
    sm.wave_cnt[1][w] = (uint32_t)__popcll(mb);
  }
  __syncthreads();
  uint32_t oa = 0, ob = 0;
  ta = tb = 0;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) {
    const uint32_t ca = sm.wave_cnt[0][i], cb = sm.wave_cnt[1][i];
    if (i < w) { oa += ca; ob += cb; }
    ta += ca; tb += cb;
  }
  pa = oa + (uint32_t)__popcll(ma & lt);
  pb = ob + (uint32_t)__popcll(mb & lt);
  __syncthreads();
}

template <int NT, typename KeyF>
__device__ void block_topk(KeyF key, int n, int k, int32_t *out, TopkSmem &sm, int C,
                           int32_t *ptr_out) {
  const int tid = threadIdx.x;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) out[i] = i;
    if (ptr_out)
      for (int j = tid; j <= n / C; j += NT) ptr_out[j] = j * C;
    return;
  }
  if (k <= 0) {
    if (ptr_out)
      for (int j = tid; j <= n / C; j += NT) ptr_out[j] = 0;
    return;
  }
  // 1. radix-select the k-th largest key, 8 bits per pass from the top
  if (tid == 0) { sm.prefix = 0; sm.need = (uint32_t)k; }
  __syncthreads();
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
    __syncthreads();
    const uint64_t hi_mask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
    const uint64_t prefix = sm.prefix;
    for (int i = tid; i < n; i += NT) {
      const uint64_t kv = key(i);
      if ((kv & hi_mask) == prefix) atomicAdd(&sm.hist[(kv >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < WAVE) {
      // lane l owns digits 255-4l .. 252-4l (high to low); find the digit
      // where the running count from the top reaches `need`.
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = sm.hist[255 - 4 * tid - j]; loc += c[j]; }
      uint32_t incl = loc;  // inclusive prefix over lanes 0..l (higher digits first)
#pragma unroll
      for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, WAVE);
        if (tid >= o) incl += t;
      }
      const uint32_t above = incl - loc;
      const uint32_t need = sm.need;
      if (above < need && need <= incl) {
        uint32_t run = above;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < need && need <= run + c[j]) {
            const uint32_t d = 255 - 4 * tid - j;
            sm.prefix = prefix | ((uint64_t)d << shift);
            sm.need = need - run;
          }
          run += c[j];
        }
      }
    }
    __syncthreads();
  }
  const uint64_t thr = sm.prefix;
  const uint32_t need_eq = sm.need;  // how many keys equal to thr are taken
  // 2. one ordered pass: take keys above thr and the first need_eq equal ones
  if (tid == 0) { sm.base_sel = 0; sm.base_eq = 0; }
  __syncthreads();
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + tid;
    const uint64_t kv = i < n ? key(i) : 0ull;
    const bool eq = i < n && kv == thr;
    const bool gt = i < n && kv > thr;
    uint32_t p_eq, dummy_p, t_eq, dummy_t;
    block_exclusive_counts<NT>(eq, false, p_eq, dummy_p, t_eq, dummy_t, sm);
    const uint32_t base_eq = sm.base_eq;
    const bool take = gt || (eq && base_eq + p_eq < need_eq);
    uint32_t p_sel, p2, t_sel, t2;
    block_exclusive_counts<NT>(take, false, p_sel, p2, t_sel, t2, sm);
    const uint32_t base_sel = sm.base_sel;
    if (take) out[base_sel + p_sel] = i;
    if (ptr_out && i < n && i % C == 0) ptr_out[i / C] = (int32_t)(base_sel + p_sel);
    __syncthreads();
    if (tid == 0) { sm.base_sel = base_sel + t_sel; sm.base_eq = base_eq + t_eq; }
    __syncthreads();
  }
  if (ptr_out && tid == 0) ptr_out[n / C] = k;
}

}  // namespace lowram
