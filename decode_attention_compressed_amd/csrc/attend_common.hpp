// Pieces shared by the two rebuild-and-attend kernels: loaders, the online
// softmax tile update, the uncompressed tail split and the partial writer.
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace lowram {

// SiLU with the hardware reciprocal (about 1 ulp); callers round the result
// to 11 or fewer significant bits
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

template <typename T> __device__ __forceinline__ float ldf(const T *p, long i) { return to_f32(p[i]); }
__device__ __forceinline__ float ld_coeff(const float *c, long i, const uint16_t *, int) { return c[i]; }
__device__ __forceinline__ float ld_coeff(const bf16 *c, long i, const uint16_t *, int) { return to_f32(c[i]); }
__device__ __forceinline__ float ld_coeff(const int8_t *c, long i, const uint16_t *sc, int ch) {
  return (float)c[i] * f16_bits_to_f32(sc[ch]);
}

// ---------------------------------------------------------------------------
// Online-softmax update of one tile: lg[gi*ld + t] holds scaled logits (log2
// units) for t < nt; replaced by p = 2^(lg - m_new).  Updates m, l and writes
// the rescale factor alpha = 2^(m_old - m_new).  Whole block calls; each wave
// owns query heads gi = wave, wave + 4, ...
// ---------------------------------------------------------------------------
__device__ inline void softmax_tile(float *lg, int ld, int nt, int g, float *ms, float *ls,
                                    float *al) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  for (int gi = wave; gi < g; gi += 256 / WAVE) {
    float mx = -INFINITY;
    for (int t = lane; t < nt; t += WAVE) mx = fmaxf(mx, lg[gi * ld + t]);
    mx = wave_max(mx);
    const float m_old = ms[gi];
    const float m_new = fmaxf(m_old, mx);
    float sum = 0.f;
    for (int t = lane; t < nt; t += WAVE) {
      const float p = exp2f(lg[gi * ld + t] - m_new);
      lg[gi * ld + t] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
      al[gi] = alpha;
      ls[gi] = ls[gi] * alpha + sum;
      ms[gi] = m_new;
    }
  }
}

// ---------------------------------------------------------------------------
// Uncompressed tail of one (b, h): dense softmax over tail tokens [t_begin,
// t_end) (shared by the VALU and MFMA kernels).  qs[g][dh] floats already
// loaded; lg scratch [g][TT]; accV [g][dh]; ms/ls/al [g]; kv scratch of
// 2*TT*(dh+1) floats where each tile's keys and values are staged with 16-byte
// loads.
// ---------------------------------------------------------------------------
template <typename TA>
__device__ void tail_split(const AttendArgs &a, int h, int b, const float *qs, float *lg, int TT,
                           float *accV, float *ms, float *ls, float *al, float *kv, int t_begin,
                           int t_end) {
  const int tid = threadIdx.x;
  const int g = a.g, dh = a.dh, ld = dh + 1;
  const long base = ((((long)b * a.G + a.layer) * a.Hkv + h) * a.T) * dh;
  const TA *kt = reinterpret_cast<const TA *>(a.k_tail) + base;
  const TA *vt = reinterpret_cast<const TA *>(a.v_tail) + base;
  float *ks = kv, *vs = kv + TT * ld;
  constexpr int PER = 16 / sizeof(TA);  // elements per 16-byte piece
  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    const int nt = min(TT, t_end - t0);
    for (int pc = tid; pc < nt * dh / PER; pc += 256) {
      const int t = pc / (dh / PER), d0 = (pc % (dh / PER)) * PER;
      const u32x4 kr = gld16(kt + (long)(t0 + t) * dh + d0);
      const u32x4 vr = gld16(vt + (long)(t0 + t) * dh + d0);
      const TA *ke = reinterpret_cast<const TA *>(&kr), *ve = reinterpret_cast<const TA *>(&vr);
#pragma unroll
      for (int j = 0; j < PER; ++j) { ks[t * ld + d0 + j] = to_f32(ke[j]); vs[t * ld + d0 + j] = to_f32(ve[j]); }
    }
    __syncthreads();
    for (int idx = tid; idx < g * nt; idx += 256) {
      const int gi = idx / nt, t = idx % nt;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < dh; ++d) s = fmaf(qs[gi * dh + d], ks[t * ld + d], s);
      lg[gi * TT + t] = s * a.scale_log2;
    }
    __syncthreads();
    softmax_tile(lg, TT, nt, g, ms, ls, al);
    __syncthreads();
    for (int idx = tid; idx < g * dh; idx += 256) {
      const int gi = idx / dh, d = idx % dh;
      float acc = accV[idx] * al[gi];
#pragma unroll 8
      for (int t = 0; t < nt; ++t) acc = fmaf(lg[gi * TT + t], vs[t * ld + d], acc);
      accV[idx] = acc;
    }
    __syncthreads();
  }
}

// Eight int8 codes (two dwords, lowest byte first) as fp16, exactly.  Each
// code x is biased to the byte u = x + 128 (a sign-bit flip) and placed as
// the low mantissa byte of the fp16 word 0x64uu, which is the value 1024 + u
// (fp16 has unit spacing in [1024, 2048)); subtracting 1152 leaves x.  One
// byte permute and one packed fp16 subtraction per pair of codes.
typedef _Float16 attend_h2 __attribute__((ext_vector_type(2)));
typedef _Float16 attend_f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
__device__ __forceinline__ attend_f16x8 i8x8_to_f16x8(uint32_t lo, uint32_t hi) {
  const uint32_t w[2] = {lo ^ 0x80808080u, hi ^ 0x80808080u};
  const attend_h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  attend_f16x8 o;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // bytes (u_2i, 0x64, u_2i+1, 0x64): selector bytes 0-3 take the second
    // operand's bytes, 4 the first operand's byte 0
    const attend_h2 a = __builtin_bit_cast(attend_h2, __builtin_amdgcn_perm(0x64646464u, w[j], 0x04010400u)) - bias;
    const attend_h2 b = __builtin_bit_cast(attend_h2, __builtin_amdgcn_perm(0x64646464u, w[j], 0x04030402u)) - bias;
    o[4 * j] = a.x;
    o[4 * j + 1] = a.y;
    o[4 * j + 2] = b.x;
    o[4 * j + 3] = b.y;
  }
  return o;
}

// ---------------------------------------------------------------------------
// Top-k chunk selection by one wave: the k chunks of [0, n_c) with the largest
// fp64 score in scL (LDS, NSL * 64 entries readable; those past n_c are
// ignored), the lowest index first among equal scores.  Lane l holds the
// order keys of chunks 64 i + l in slot i; the k-th largest key is found by a
// bitwise search on the top 32 bits, then on the low 32 bits among the chunks
// that tie there (a uniform branch, rare outside crafted ties).  Every count
// is a 64-lane compare mask and a popcount.  emit(pos, c) is called once per
// selected chunk c, pos its rank in ascending chunk order.  1 <= k <= n_c <=
// 64 NSL; lanes of the wave call it together.
// ---------------------------------------------------------------------------
template <int NSL, typename Emit>
__device__ __forceinline__ void wave_topk(const double *scL, int n_c, int k, Emit emit) {
  const int lane = threadIdx.x & (WAVE - 1);
  uint32_t khi[NSL], klo[NSL];
  uint64_t valid[NSL];
  double sv[NSL];  // the caller's score area holds NSL * 64 entries: read all, mask later
#pragma unroll
  for (int i = 0; i < NSL; ++i) sv[i] = scL[WAVE * i + lane];
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int c = WAVE * i + lane;
    const uint64_t key = c < n_c ? f64_order_key(sv[i]) : 0ull;
    khi[i] = (uint32_t)(key >> 32);
    klo[i] = (uint32_t)key;
    valid[i] = __ballot(c < n_c);
  }
  // count of chunks with top half >= x, summed as a tree.  Lanes past n_c
  // hold key 0 and every x searched below is at least 1, so they never count.
  auto count_hi = [&](uint32_t x) {
    int c8[NSL];
#pragma unroll
    for (int i = 0; i < NSL; ++i) c8[i] = __popcll(__ballot(khi[i] >= x));
#pragma unroll
    for (int n = NSL / 2; n > 0; n /= 2)
#pragma unroll
      for (int i = 0; i < n; ++i) c8[i] += c8[i + n];
    return c8[0];
  };
  // the k-th largest top half, highest bit first; stops as soon as exactly
  // k chunks lie at or above the bits fixed so far (further low bits could
  // only drop chunks below k)
  uint32_t th = 0u;
  for (uint32_t m = 0x80000000u; m != 0u; m >>= 1) {
    const uint32_t cand = th | m;
    const int cnt = count_hi(cand);
    if (cnt >= k) th = cand;
    if (cnt == k) break;
  }
  uint64_t eq_hi[NSL], sel[NSL];
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    sel[i] = __ballot(khi[i] > th) & valid[i];
    eq_hi[i] = __ballot(khi[i] == th) & valid[i];
    n_gt += __popcll(sel[i]);
    n_eq += __popcll(eq_hi[i]);
  }
  if (n_gt + n_eq == k) {  // the threshold's top half is shared by exactly the missing chunks
#pragma unroll
    for (int i = 0; i < NSL; ++i) sel[i] |= eq_hi[i];
  } else {  // more chunks share that top half than are missing: decide on the low halves
    const int need = k - n_gt;
    auto count_lo = [&](uint32_t x) {
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NSL; ++i) cnt += __popcll(__ballot(klo[i] >= x) & eq_hi[i]);
      return cnt;
    };
    uint32_t tl = 0u;
    for (uint32_t m = 0x80000000u; m != 0u; m >>= 1) {
      const uint32_t cand = tl | m;
      const int cnt = count_lo(cand);
      if (cnt >= need) tl = cand;
      if (cnt == need) break;
    }
    int rem = need;
    uint64_t eq[NSL];
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      const uint64_t gt = __ballot(klo[i] > tl) & eq_hi[i];
      sel[i] |= gt;
      rem -= __popcll(gt);
      eq[i] = __ballot(klo[i] == tl) & eq_hi[i];
    }
#pragma unroll
    for (int i = 0; i < NSL; ++i) {  // equal keys: lowest chunk index first
      uint64_t e = eq[i];
      while (rem > 0 && e) {
        const uint64_t low = e & (~e + 1ull);
        sel[i] |= low;
        e ^= low;
        --rem;
      }
    }
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    if ((sel[i] >> lane) & 1ull) emit(base + __popcll(sel[i] & lanemask_lt()), WAVE * i + lane);
    base += __popcll(sel[i]);
  }
}

// Partial of one split for each query head: m, l, the part of l from rebuilt
// tokens (all of it for a rebuilt split, none for the tail), 0, then accH[F]
// (zero for the tail) and accV[dh].
__device__ inline void write_partial(const AttendArgs &a, int h, int b, int split, const float *ms,
                                     const float *ls, const float *accH, const float *accV) {
  const int tid = threadIdx.x;
  float *p = a.part + (((long)b * a.Hkv + h) * (a.n_split + 1) + split) * a.g * a.PW;
  for (int gi = 0; gi < a.g; ++gi) {
    float *pg = p + (long)gi * a.PW;
    if (tid == 0) { pg[0] = ms[gi]; pg[1] = ls[gi]; pg[2] = accH ? ls[gi] : 0.f; pg[3] = 0.f; }
    for (int f = tid; f < a.F; f += 256) pg[4 + f] = accH ? accH[gi * a.F + f] : 0.f;
    for (int d = tid; d < a.dh; d += 256) pg[4 + a.F + d] = accV[gi * a.dh + d];
  }
}

}  // namespace lowram
