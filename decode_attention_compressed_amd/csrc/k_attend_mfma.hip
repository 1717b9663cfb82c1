// Fused rebuild-and-attend on gfx950 matrix cores (bf16/fp16 MFMA, fp32 accumulate).
//
// One workgroup (4 waves) owns one (sequence b, kv head h) and a run of the
// chunks selected for it.  For each 128-token tile of a selected chunk:
//   1. K_hat[128][dh] = deq(coeff tile)[128][r] . U_{l,h}^T   (32x32x16 MFMA,
//      coefficient and basis slabs staged through LDS; bf16 operands as
//      stored; int8 coefficients are exact in fp16 and their per-channel
//      scale is folded into an fp16 basis slab)
//   2. logits = K_hat . q^T for the g query heads of h (16x16x32 MFMA, g padded
//      to 16), online softmax in log2 units, p rounded to fp16 in LDS
//   3. H = SiLU(K_hat . W1^T + b1) in 64-wide hidden blocks (32x32x16 MFMA)
//   4. accH += p . H (16x16x32 MFMA), kept in registers across tiles
//   5. accV += p . delta for the residual rows of the tile (CSR of the chunk)
// The second predictor layer is linear, so W2 and b2 are applied once per
// query head in the combine: sum_t p_t v_t = W2 accH + b2 sum_t p_t + accV.
//
// Method: keys rebuilt from per-token coefficients on a group basis (zicq.com
// English summary, "Cross-Layer Low-Rank Key Compression"); values from the
// per-head predictor plus residuals of the worst tokens ("Core Mechanism");
// only query-selected chunks are rebuilt (rit.work page, generation section);
// attention softmax(q K^T / sqrt(d_h)) V (OjaKV page, section 3).
#include "attend_common.hpp"

namespace lowram {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int TM = 128;   // tokens per tile
constexpr int RS = 32;    // rank slab of step 1
constexpr int PAD = 8;    // bf16 pad per LDS row (keeps 16-byte rows, spreads banks)
constexpr int CS_LD = RS + PAD, HS_LD = TM + PAD, PS_LD = TM + PAD;

// 16-byte LDS fragment loads
__device__ __forceinline__ bf16x8 ldb8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f16x8 ldh8(const uint16_t *p) { return *reinterpret_cast<const f16x8 *>(p); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Operands produced inside the kernel (rebuilt keys, hidden activations,
// softmax weights, queries, first-layer weights) are fp16: 11 significant
// bits instead of bf16's 8 at the same MFMA rate.  The stored bf16
// coefficients and basis feed step 1 exactly as stored.
__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)h16(lo) | ((uint32_t)h16(hi) << 16);
}

template <typename TC> struct Step1 { typedef bf16x8 frag; static __device__ frag ld(const uint16_t *p) { return ldb8(p); } };
template <> struct Step1<int8_t> { typedef f16x8 frag; static __device__ frag ld(const uint16_t *p) { return ldh8(p); } };

template <int DH>
struct MfmaSmem {
  static constexpr int KS_LD = DH + PAD, W1S_LD = DH + PAD;
  static constexpr int A1 = TM * CS_LD + DH * CS_LD;            // step 1 staging
  static constexpr int A3 = 64 * W1S_LD + 64 * HS_LD;           // steps 3/4
  static constexpr int REGION_A = A1 > A3 ? A1 : A3;            // bf16 elements
  static constexpr int KS_OFF = REGION_A;
  static constexpr int QS_OFF = KS_OFF + TM * KS_LD;
  static constexpr int PS_OFF = QS_OFF + 16 * KS_LD;
  static constexpr int END16 = PS_OFF + 16 * PS_LD;             // bf16 elements
  static constexpr int FLOATS = 4 * 16 * 2 + 16 * 3;            // red, red2, ms, ls, al
  static constexpr size_t BYTES = (size_t)END16 * 2 + FLOATS * 4;
};

// staging of one rank slab: coefficient rows and basis rows (16-byte pieces)
template <int DH>
__device__ __forceinline__ void stage_slab(const bf16 *cf, const uint16_t *, const bf16 *U,
                                           long row0, int r, int r0, uint16_t *Cs, uint16_t *Us) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < (TM * RS / 8) / 256; ++u) {
    const int c = tid + 256 * u, row = c / (RS / 8), part = c % (RS / 8);
    const uint4 v = *reinterpret_cast<const uint4 *>(cf + (row0 + row) * r + r0 + part * 8);
    *reinterpret_cast<uint4 *>(Cs + row * CS_LD + part * 8) = v;
  }
#pragma unroll
  for (int u = 0; u < (DH * RS / 8) / 256; ++u) {
    const int c = tid + 256 * u, row = c / (RS / 8), part = c % (RS / 8);
    const uint4 v = *reinterpret_cast<const uint4 *>(U + (long)row * r + r0 + part * 8);
    *reinterpret_cast<uint4 *>(Us + row * CS_LD + part * 8) = v;
  }
}

template <int DH>
__device__ __forceinline__ void stage_slab(const int8_t *cf, const uint16_t *csc, const bf16 *U,
                                           long row0, int r, int r0, uint16_t *Cs, uint16_t *Us) {
  const int tid = threadIdx.x;
  // int8 coefficient rows: 32 bytes per row, two 16-byte pieces; |q| <= 127 is exact in fp16
  {
    const int row = tid / 2, part = tid % 2;
    const uint4 v = *reinterpret_cast<const uint4 *>(cf + (row0 + row) * r + r0 + part * 16);
    const int8_t *b8 = reinterpret_cast<const int8_t *>(&v);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack2((float)b8[2 * i], (float)b8[2 * i + 1]);
    *reinterpret_cast<uint4 *>(Cs + row * CS_LD + part * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4 *>(Cs + row * CS_LD + part * 16 + 8) = make_uint4(w[4], w[5], w[6], w[7]);
  }
  // basis rows scaled by the coefficient channel scales, rounded once to fp16
#pragma unroll
  for (int u = 0; u < (DH * RS / 8) / 256; ++u) {
    const int c = tid + 256 * u, row = c / (RS / 8), part = c % (RS / 8);
    const uint4 v = *reinterpret_cast<const uint4 *>(U + (long)row * r + r0 + part * 8);
    const uint16_t *u16 = reinterpret_cast<const uint16_t *>(&v);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = r0 + part * 8 + 2 * i;
      w[i] = pack2(bf16_bits_to_f32(u16[2 * i]) * f16_bits_to_f32(csc[ch]),
                   bf16_bits_to_f32(u16[2 * i + 1]) * f16_bits_to_f32(csc[ch + 1]));
    }
    *reinterpret_cast<uint4 *>(Us + row * CS_LD + part * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ float ld_res(const bf16 *p, long i, const uint16_t *, int) { return to_f32(p[i]); }
__device__ __forceinline__ float ld_res(const int8_t *p, long i, const uint16_t *sc, int d) {
  return (float)p[i] * f16_bits_to_f32(sc[d]);
}

template <int DH, int NF64, typename TC, typename TR>
__global__ __launch_bounds__(256) void k_attend_mfma(const AttendArgs a) {
  using S = MfmaSmem<DH>;
  constexpr int KS_LD = S::KS_LD, W1S_LD = S::W1S_LD;
  constexpr int NT1 = DH / 64;                 // 32-wide N tiles per wave in step 1
  constexpr int PAIRS = (16 * DH + 255) / 256; // (query head, dim) pairs per thread
  extern __shared__ __align__(16) unsigned char msm[];
  uint16_t *sm16 = reinterpret_cast<uint16_t *>(msm);
  uint16_t *Cs = sm16, *Us = sm16 + TM * CS_LD;               // step 1
  uint16_t *W1s = sm16, *Hs = sm16 + 64 * W1S_LD;             // steps 3/4
  uint16_t *Ks = sm16 + S::KS_OFF, *Qs = sm16 + S::QS_OFF, *Ps = sm16 + S::PS_OFF;
  float *fl = reinterpret_cast<float *>(sm16 + S::END16);
  float *red = fl, *red2 = fl + 64, *ms = fl + 128, *ls = ms + 16, *al = ls + 16;

  const int h = blockIdx.y, b = blockIdx.z, split = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int g = a.g, r = a.r, C = a.C;

  if (split == a.n_split) {  // uncompressed tail on the vector ALUs
    float *qs = reinterpret_cast<float *>(msm), *accV = qs + g * DH, *lgs = accV + g * DH;
    float *tms = lgs + g * 64, *tls = tms + 16, *tal = tls + 16;
    const bf16 *qb = reinterpret_cast<const bf16 *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
    for (int i = tid; i < g * DH; i += 256) { qs[i] = to_f32(qb[i]); accV[i] = 0.f; }
    if (tid < 16) { tms[tid] = -INFINITY; tls[tid] = 0.f; tal[tid] = 0.f; }
    __syncthreads();
    tail_split<bf16>(a, qs, lgs, 64, accV, tms, tls, tal);
    write_partial(a, split, tms, tls, nullptr, accV);
    return;
  }

  const int D = a.G * a.Hkv * DH;
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;
  const bf16 *U = reinterpret_cast<const bf16 *>(a.basis) + ((long)b * D + (long)(a.layer * a.Hkv + h) * DH) * r;
  const bf16 *W1 = reinterpret_cast<const bf16 *>(a.w1) + bh * (long)(NF64 * 64) * DH;
  const bf16 *B1 = reinterpret_cast<const bf16 *>(a.b1) + bh * (NF64 * 64);
  const TC *cf = reinterpret_cast<const TC *>(a.coeff) + (long)b * a.N * r;
  const uint16_t *csc = a.coeff_scale ? a.coeff_scale + (long)b * r : nullptr;
  const int32_t *rptr = a.res_ptr + bh * (a.N / C + 1);
  const int32_t *ridx = a.res_idx + bh * a.n_res;
  const TR *rval = reinterpret_cast<const TR *>(a.res_val) + bh * a.n_res * DH;
  const uint16_t *rsc = a.res_scale ? a.res_scale + bh * DH : nullptr;
  const int32_t *selp = a.sel + ((long)b * a.Hkv + h) * a.k_eff;

  // query rows of this kv head, zero-padded to 16
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
    for (int i = tid; i < 16 * DH; i += 256) {
      const int gi = i / DH, d = i % DH;
      Qs[gi * KS_LD + d] = gi < g ? h16(bf16_bits_to_f32(qb[gi * DH + d])) : (uint16_t)0;
    }
  }
  if (tid < 16) { ms[tid] = -INFINITY; ls[tid] = 0.f; al[tid] = 0.f; }

  f32x4 accH[NF64];
#pragma unroll
  for (int i = 0; i < NF64; ++i) accH[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float accV[PAIRS];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) accV[p] = 0.f;
  __syncthreads();

  const int s_end = min(a.k_eff, (split + 1) * a.cps);
  for (int slot = split * a.cps; slot < s_end; ++slot) {
    const int j = selp[slot];
    const int e0 = rptr[j], e1 = rptr[j + 1];
    for (int t0 = 0; t0 < C; t0 += TM) {
      const long row0 = (long)j * C + t0;
      // ---- step 1: K_hat = C . U^T --------------------------------------
      f32x16 acc1[2][NT1];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT1; ++ni)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc1[mi][ni][i] = 0.f;
      for (int r0 = 0; r0 < r; r0 += RS) {
        stage_slab<DH>(cf, csc, U, row0, r, r0, Cs, Us);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < RS / 16; ++ks) {
          const int kof = 16 * ks + 8 * (lane >> 5);
          typename Step1<TC>::frag af[2];
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) af[mi] = Step1<TC>::ld(Cs + (64 * wm + 32 * mi + (lane & 31)) * CS_LD + kof);
#pragma unroll
          for (int ni = 0; ni < NT1; ++ni) {
            const typename Step1<TC>::frag bfr = Step1<TC>::ld(Us + (wn * (DH / 2) + 32 * ni + (lane & 31)) * CS_LD + kof);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) acc1[mi][ni] = mfma32(af[mi], bfr, acc1[mi][ni]);
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT1; ++ni)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            const int col = wn * (DH / 2) + 32 * ni + (lane & 31);
            Ks[row * KS_LD + col] = h16(acc1[mi][ni][i]);
          }
      __syncthreads();

      // ---- step 2: logits and online softmax ----------------------------
      f32x4 acc2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) {
        const int kof = 32 * ks + 8 * (lane >> 4);
        const f16x8 bq = ldh8(Qs + (lane & 15) * KS_LD + kof);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          acc2[mi] = mfma16(ldh8(Ks + (32 * w + 16 * mi + (lane & 15)) * KS_LD + kof), bq, acc2[mi]);
      }
      const int gi = lane & 15;
      float mx = -INFINITY;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc2[mi][i] *= a.scale_log2;
          mx = fmaxf(mx, acc2[mi][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lane < 16) red[w * 16 + gi] = mx;
      __syncthreads();
      const float m_old = ms[gi];
      const float m_new = fmaxf(m_old, fmaxf(fmaxf(red[gi], red[16 + gi]), fmaxf(red[32 + gi], red[48 + gi])));
      float psum = 0.f;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = gi < g ? exp2f(acc2[mi][i] - m_new) : 0.f;
          pv[i] = f16f(h16(p));
          psum += pv[i];
        }
        const int t = 32 * w + 16 * mi + 4 * (lane >> 4);
        *reinterpret_cast<uint2 *>(Ps + gi * PS_LD + t) = make_uint2(pack2(pv[0], pv[1]), pack2(pv[2], pv[3]));
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

      // ---- step 5: residual rows of this tile, and rescale of accH ----------
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) {
        const int idx = tid + 256 * p;
        if (idx < g * DH) {
          const int gq = idx / DH, d = idx % DH;
          float acc = accV[p] * al[gq];
          for (int e = e0; e < e1; ++e) {
            const int t = ridx[e] - (int)row0;
            if (t >= 0 && t < TM)
              acc = fmaf(f16f(Ps[gq * PS_LD + t]), ld_res(rval, (long)e * DH + d, rsc, d), acc);
          }
          accV[p] = acc;
        }
      }
#pragma unroll
      for (int fb = 0; fb < NF64; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) accH[fb][i] *= al[4 * (lane >> 4) + i];

      // ---- steps 3 and 4 per 64-wide hidden block ---------------------------
#pragma unroll 1
      for (int fb = 0; fb < NF64; ++fb) {
        for (int c = tid; c < 64 * DH / 8; c += 256) {
          const int f = c / (DH / 8), part = c % (DH / 8);
          const uint4 v = *reinterpret_cast<const uint4 *>(W1 + (long)(fb * 64 + f) * DH + part * 8);
          const uint32_t *u = reinterpret_cast<const uint32_t *>(&v);
          uint32_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = pack2(bf16_bits_to_f32(u[i] & 0xFFFFu), bf16_bits_to_f32(u[i] >> 16));
          *reinterpret_cast<uint4 *>(W1s + f * W1S_LD + part * 8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        __syncthreads();
        f32x16 acc3[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc3[mi][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DH / 16; ++ks) {
          const int kof = 16 * ks + 8 * (lane >> 5);
          const f16x8 bw = ldh8(W1s + (32 * wn + (lane & 31)) * W1S_LD + kof);
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            acc3[mi] = mfma32(ldh8(Ks + (64 * wm + 32 * mi + (lane & 31)) * KS_LD + kof), bw, acc3[mi]);
        }
        const int fl_ = 32 * wn + (lane & 31);
        const float bias = to_f32(B1[fb * 64 + fl_]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int row = 64 * wm + 32 * mi + 8 * q4 + 4 * (lane >> 5);
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = silu_f(acc3[mi][4 * q4 + i] + bias);
            *reinterpret_cast<uint2 *>(Hs + fl_ * HS_LD + row) = make_uint2(pack2(hv[0], hv[1]), pack2(hv[2], hv[3]));
          }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < TM / 32; ++ks) {
          const int kof = 32 * ks + 8 * (lane >> 4);
          accH[fb] = mfma16(ldh8(Ps + (lane & 15) * PS_LD + kof),
                            ldh8(Hs + (16 * w + (lane & 15)) * HS_LD + kof), accH[fb]);
        }
      }
      __syncthreads();
    }
  }

  // ---- partials ---------------------------------------------------------------
  float *p = a.part + (((long)b * a.Hkv + h) * (a.n_split + 1) + split) * g * a.PW;
  if (tid < g) { p[tid * a.PW] = ms[tid]; p[tid * a.PW + 1] = ls[tid]; p[tid * a.PW + 2] = 0.f; p[tid * a.PW + 3] = 0.f; }
#pragma unroll
  for (int fb = 0; fb < NF64; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gq = 4 * (lane >> 4) + i;
      if (gq < g) p[gq * a.PW + 4 + fb * 64 + 16 * w + (lane & 15)] = accH[fb][i];
    }
#pragma unroll
  for (int pp = 0; pp < PAIRS; ++pp) {
    const int idx = tid + 256 * pp;
    if (idx < g * DH) p[(idx / DH) * a.PW + 4 + a.F + idx % DH] = accV[pp];
  }
}

hipError_t launch_attend_valu(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st);

template <int DH, int NF64, typename TC, typename TR>
static hipError_t go(const AttendArgs &a, hipStream_t st) {
  const size_t smem = MfmaSmem<DH>::BYTES;
  static const bool lds_ok = (allow_dynamic_lds(k_attend_mfma<DH, NF64, TC, TR>, smem), true);
  (void)lds_ok;
  hipLaunchKernelGGL((k_attend_mfma<DH, NF64, TC, TR>), dim3(a.n_split + 1, a.Hkv, a.B), dim3(256),
                     smem, st, a);
  return hipGetLastError();
}

template <typename TC, typename TR>
static hipError_t dispatch_shape(const AttendArgs &a, hipStream_t st) {
  if (a.dh == 128 && a.F == 256) return go<128, 4, TC, TR>(a, st);
  if (a.dh == 128 && a.F == 128) return go<128, 2, TC, TR>(a, st);
  if (a.dh == 128 && a.F == 512) return go<128, 8, TC, TR>(a, st);
  if (a.dh == 256 && a.F == 512) return go<256, 8, TC, TR>(a, st);
  return hipErrorInvalidValue;
}

bool mfma_supported(const AttendArgs &a, int act, int coeff, int resid) {
  if (act != LOWRAM_BF16 || coeff != resid) return false;
  const bool shape = (a.dh == 128 && (a.F == 128 || a.F == 256 || a.F == 512)) || (a.dh == 256 && a.F == 512);
  return shape && a.C % TM == 0 && a.r % RS == 0 && a.g <= 16;
}

hipError_t launch_attend(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st) {
  if (!mfma_supported(a, act, coeff, resid)) return launch_attend_valu(act, coeff, resid, a, st);
  if (coeff == LOWRAM_I8) return dispatch_shape<int8_t, int8_t>(a, st);
  return dispatch_shape<bf16, bf16>(a, st);
}

}  // namespace lowram
