// Rebuild-and-attend with register-chained matrix tiles (gfx950, 16x16x32 MFMA).
//
// One workgroup of 8 waves owns one (sequence b, kv head h, split s).  A split
// is a run of 64-token tiles of the chunks selected for h; each wave takes one
// tile at a time and keeps everything about it in its own registers:
//   1. K_hat^T[128 d][64 t] = U_{l,h} . deq(coeff)^T, contracted over the rank
//      in 32-wide steps.  The basis slab of a step is shared by the 8 waves
//      through LDS (double-buffered, one barrier per step, loaded two steps
//      ahead); every lane loads its coefficient fragments straight from global
//      memory into the MFMA operand, two steps ahead.
//   2. logits[t][g] = K_hat[t] . q_g: the key accumulators rounded to fp16 are
//      the A operand exactly as the step-1 output leaves them; online softmax
//      per wave; p rounded to fp16.
//   3. H^T[t][f] = SiLU(K_hat W1^T + b1) per 16-wide hidden tile: the same key
//      registers are the A operand, W1 stays in LDS (fp16) for the whole
//      workgroup and b1 enters as the initial accumulator.
//   4. accH[g][f] += p . H^T: p (from the logits' output layout) and SiLU(H^T)
//      (from step 3's output layout) are operands as they stand.
//   5. accV[g][d] += p[g][t] delta[t][d] over the tile's residual rows on the
//      vector ALUs (about one token in eight carries a row).
// The order of a contracted index inside one MFMA is free, so both operands of
// a product use the same permutation of it: the head dims in steps 2 and 3
// follow the step-1 output layout (W1 and q are stored permuted), the tokens
// in step 4 follow the step-3 output layout.
//
// The workgroup also attends its share of the uncompressed tail (staged in LDS
// at the start, vector ALUs), then merges the 8 waves and the tail into one
// partial: (m, l, mass of rebuilt tokens, accH[F], accV[d_h]) per query head.
// The second predictor layer is linear and is applied once per query head in
// the combine: sum_t p_t v_t = W2 accH + b2 mass + accV.
//
// Method: keys rebuilt from per-token coefficients on a group basis (zicq.com
// English summary, "Cross-Layer Low-Rank Key Compression"); values from the
// per-head predictor plus residuals of the worst tokens ("Core Mechanism");
// only query-selected chunks are rebuilt (rit.work page, generation section);
// attention softmax(q K^T / sqrt(d_h)) V (OjaKV page, section 3).
#include <type_traits>

#include "attend_common.hpp"

namespace lowram {
namespace chain {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int DH = 128;           // head dim handled here
constexpr int NW = 8;             // waves per workgroup
constexpr int NTH = NW * WAVE;
constexpr int TT = 64;            // tokens per wave tile
constexpr int NTT = TT / 16;      // 16-token tiles
constexpr int NDT = DH / 16;      // 16-row head-dim tiles
constexpr int NJ = DH / 32;       // 32-wide head-dim steps
constexpr int KS = 32;            // ranks per step-1 k-step
constexpr int ULD = KS + 8;       // basis slab row stride, 16-bit elements (80 bytes)
constexpr int WLD = DH + 8;       // W1 / q row stride, 16-bit elements (272 bytes)
constexpr int GQ = 4;             // query heads per kv head (at most)
constexpr int RP = 16;            // residual rows of a tile held in registers
constexpr int DC = 3;             // coefficient k-steps in registers (2 ahead)
constexpr int LU = 2;             // basis slabs are loaded LU steps before use
constexpr int NU = 4;             // basis register ring (divides the step count)
constexpr int TP = 32;            // tail tokens staged per piece
constexpr int CPT = 2;            // tiles per chunk: 128-token chunks

template <int I, int N, typename Fn>
__device__ __forceinline__ void sfor_impl(Fn &f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor_impl<I + 1, N>(f);
  }
}
template <int N, typename Fn>
__device__ __forceinline__ void sfor(Fn &&f) { sfor_impl<0, N>(f); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)h16(lo) | ((uint32_t)h16(hi) << 16);
}
__device__ __forceinline__ f16x8 ldh8(const uint16_t *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ bf16x8 ldb8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Position of head dim d inside the permuted order: within each 32-wide step,
// lane group kg of the step-1 output holds dims 4kg..4kg+3 and 16+4kg..16+4kg+3,
// which become its eight consecutive k positions 8kg..8kg+7.
__device__ __forceinline__ int dpos(int d) {
  return (d & ~31) + 8 * ((d & 15) >> 2) + 4 * ((d >> 4) & 1) + (d & 3);
}

// LDS layout (bytes).  The merge area at the end reuses W1 and the basis slabs;
// each wave's running accH stays in LDS across its tiles.
template <int F>
struct Smem {
  static constexpr int W1S = 0;                          // [F][WLD] fp16, dims permuted
  static constexpr int US = W1S + F * WLD * 2;           // 2 x [DH][ULD] basis slabs
  static constexpr int QS = US + 2 * DH * ULD * 2;       // [16][WLD] fp16 q, dims permuted
  static constexpr int QF = QS + 16 * WLD * 2;           // [GQ][DH] fp32 q (tail)
  static constexpr int B1 = QF + GQ * DH * 4;            // [F] fp32 b1
  static constexpr int PS = B1 + F * 4;                  // [NW][GQ][TT] fp32 p
  static constexpr int TK = PS + NW * GQ * TT * 4;       // [TP][DH] bf16 tail keys
  static constexpr int TV = TK + TP * DH * 2;            // [TP][DH] bf16 tail values
  static constexpr int TL = TV + TP * DH * 2;            // [GQ][TP] fp32 tail logits / p
  static constexpr int TS = TL + GQ * TP * 4;            // [4][GQ] fp32 tail m, l, alpha
  static constexpr int AH = TS + 4 * GQ * 4;             // [NW][GQ][F] fp32 running accH per wave
  static constexpr int BYTES = AH + NW * GQ * F * 4;
  // merge area (after the last tile): m, l [NW+1][GQ], accV [NW+1][GQ][DH]
  static constexpr int MM = 0, ML = MM + (NW + 1) * GQ * 4, MV = ML + (NW + 1) * GQ * 4;
  static_assert(MV + (NW + 1) * GQ * DH * 4 <= QS, "merge area does not fit");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Block -> (sequence b, kv head h, split s).  Workgroups are dispatched
// round-robin over the 8 XCDs (linear id mod 8), each with its own L2.  The
// linear id is remapped so that each XCD receives a contiguous run of the
// (b, s, h) order: all kv heads of a sequence's low splits on one XCD, its
// high splits on the next.  Each sequence's coefficient tiles are then shared
// in one or two L2s, and a head's basis slice and W1 stay L2-resident.
__device__ __forceinline__ void coords(const AttendArgs &a, int &b, int &h, int &s) {
  const int n = gridDim.x;
  int u = blockIdx.x;
  if (n % 8 == 0) u = (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8;
  h = u % a.Hkv;
  s = (u / a.Hkv) % a.n_split;
  b = u / (a.Hkv * a.n_split);
}

// Buffer resources: an SGPR descriptor per tensor and one 32-bit lane offset
// per access pattern keep the per-lane address state small; the uniform parts
// of an address (tile row, k-step, residual row) go in the scalar offset.
// Reads past num_records bytes return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// coefficient fragments: lane (token l16 of a 16-token tile, rank group kg)
template <typename TC> struct Coef;
template <> struct Coef<bf16> {
  typedef u32x4 raw;   // 8 bf16 ranks of one token
  typedef bf16x8 op;
  static constexpr int ES = 2;
  __device__ static raw ld(rsrc_t r, uint32_t voff, uint32_t soff) { return bld16(r, voff, soff); }
  __device__ static op get(raw v) { return __builtin_bit_cast(bf16x8, v); }
};
template <> struct Coef<int8_t> {
  typedef uint2 raw;   // 8 int8 ranks of one token
  typedef f16x8 op;
  static constexpr int ES = 1;
  __device__ static raw ld(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return make_uint2(v.x, v.y);
  }
  __device__ static op get(raw v) {  // int8 is exact in fp16
    const int8_t *b = reinterpret_cast<const int8_t *>(&v);
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)(float)b[i];
    return o;
  }
};

// basis slab pieces: thread tid stages 8 ranks of head-dim row tid / 4
// (lane offset ((tid / 4) * r + 8 (tid % 4)) * 2 bytes, k-step in the scalar offset)
template <typename TC> struct Slab;
template <> struct Slab<bf16> {
  typedef bf16x8 op;
  __device__ static void ld(rsrc_t U, const uint16_t *, uint32_t voff, int k0, u32x4 &u, u32x4 &) {
    u = bld16(U, voff, 2u * k0);
  }
  __device__ static void st(uint16_t *Ub, const u32x4 &u, const u32x4 &) {
    const int tid = threadIdx.x;
    lst16(Ub + (tid >> 2) * ULD + 8 * (tid & 3), u);
  }
  __device__ static op get(const uint16_t *p) { return ldb8(p); }
};
template <> struct Slab<int8_t> {  // fp16 slab with the coefficient scale folded in
  typedef f16x8 op;
  __device__ static void ld(rsrc_t U, const uint16_t *csc, uint32_t voff, int k0, u32x4 &u, u32x4 &sc) {
    u = bld16(U, voff, 2u * k0);
    sc = gld16(csc + k0 + 8 * (threadIdx.x & 3));
  }
  __device__ static void st(uint16_t *Ub, const u32x4 &u, const u32x4 &sc) {
    const int tid = threadIdx.x;
    const uint16_t *u16 = reinterpret_cast<const uint16_t *>(&u);
    const uint16_t *s16 = reinterpret_cast<const uint16_t *>(&sc);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack2(bf16_bits_to_f32(u16[2 * i]) * f16_bits_to_f32(s16[2 * i]),
                   bf16_bits_to_f32(u16[2 * i + 1]) * f16_bits_to_f32(s16[2 * i + 1]));
    lst16(Ub + (tid >> 2) * ULD + 8 * (tid & 3), v4(w[0], w[1], w[2], w[3]));
  }
  __device__ static op get(const uint16_t *p) { return ldh8(p); }
};

// residual row pieces: lane holds head dims 2*lane and 2*lane + 1
template <typename TR> struct Res;
template <> struct Res<bf16> {
  typedef uint32_t raw;
  static constexpr int ES = 2;
  __device__ static raw ld(rsrc_t rv, int e, int lane) {
    return __builtin_amdgcn_raw_buffer_load_b32(rv, 4u * lane, (uint32_t)e * DH * 2u, 0);
  }
  __device__ static void get(raw v, float, float, float &d0, float &d1) {
    d0 = bf16_bits_to_f32(v & 0xFFFFu);
    d1 = bf16_bits_to_f32(v >> 16);
  }
};
template <> struct Res<int8_t> {
  typedef uint32_t raw;
  static constexpr int ES = 1;
  __device__ static raw ld(rsrc_t rv, int e, int lane) {
    return __builtin_amdgcn_raw_buffer_load_b16(rv, 2u * lane, (uint32_t)e * DH, 0);
  }
  __device__ static void get(raw v, float s0, float s1, float &d0, float &d1) {
    d0 = (float)(int8_t)(v & 0xFFu) * s0;
    d1 = (float)(int8_t)((v >> 8) & 0xFFu) * s1;
  }
};

template <typename TC, int NR, int NF>
__global__ __launch_bounds__(NTH, 1) void k_attend_chain(const AttendArgs a) {
  static_assert(NR % NU == 0, "the basis register ring must divide the k-step count");
  constexpr int F = NF * 16;
  using S = Smem<F>;
  using CT = Coef<TC>;
  using ST = Slab<TC>;
  extern __shared__ __align__(16) unsigned char sm[];
  uint16_t *W1s = reinterpret_cast<uint16_t *>(sm + S::W1S);
  uint16_t *Us = reinterpret_cast<uint16_t *>(sm + S::US);
  uint16_t *Qs = reinterpret_cast<uint16_t *>(sm + S::QS);
  float *Qf = reinterpret_cast<float *>(sm + S::QF);
  float *B1s = reinterpret_cast<float *>(sm + S::B1);
  float *Ps = reinterpret_cast<float *>(sm + S::PS);
  uint16_t *Tk = reinterpret_cast<uint16_t *>(sm + S::TK);
  uint16_t *Tv = reinterpret_cast<uint16_t *>(sm + S::TV);
  float *Tl = reinterpret_cast<float *>(sm + S::TL);
  float *Ts = reinterpret_cast<float *>(sm + S::TS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile offsets stay scalar
  const int l16 = lane & 15, kg = lane >> 4;
  float *AHw = reinterpret_cast<float *>(sm + S::AH) + w * GQ * F;  // this wave's running accH
  int b, h, s;
  coords(a, b, h, s);
  const int g = a.g, r = NR * KS, C = a.C;

  const int D = a.G * a.Hkv * DH;
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;
  const bf16 *U = reinterpret_cast<const bf16 *>(a.basis) + ((long)b * D + (long)(a.layer * a.Hkv + h) * DH) * r;
  const rsrc_t Ur = make_rsrc(U, (uint32_t)(DH * r * 2));
  const uint32_t u_voff = (uint32_t)(((tid >> 2) * r + 8 * (tid & 3)) * 2);
  const uint16_t *W1 = reinterpret_cast<const uint16_t *>(a.w1) + bh * (long)F * DH;
  const uint16_t *B1 = reinterpret_cast<const uint16_t *>(a.b1) + bh * F;
  const TC *cf = reinterpret_cast<const TC *>(a.coeff) + (long)b * a.N * r;
  const rsrc_t Cr = make_rsrc(cf, (uint32_t)((long)a.N * r * CT::ES));
  const uint32_t c_voff = (uint32_t)((l16 * r + 8 * kg) * CT::ES);  // + (row0 + 16 tt) r + 32 ks
  const uint16_t *csc = a.coeff_scale ? a.coeff_scale + (long)b * r : nullptr;
  const int32_t *rptr = a.res_ptr + bh * (a.N / C + 1);
  const int32_t *ridx = a.res_idx + bh * a.n_res;
  const TC *rval = reinterpret_cast<const TC *>(a.res_val) + bh * (long)a.n_res * DH;
  const rsrc_t Rr = make_rsrc(rval, (uint32_t)((long)a.n_res * DH * Res<TC>::ES));
  const int32_t *selp = a.sel + ((long)b * a.Hkv + h) * a.k_eff;

  constexpr int cpt = CPT;                     // tiles per chunk (C == 128)
  const int n_tiles = a.k_eff * cpt;           // tiles of this (b, h)
  const int t_begin = s * a.tps;
  const int t_end = min(n_tiles, t_begin + a.tps);
  const int iters = (a.tps + NW - 1) / NW;

  // ---- prologue: W1 (in flight first), basis slabs, q, b1, tail piece ------
  constexpr int W1P = F * DH / 8 / NTH;        // 16-byte W1 pieces per thread
  u32x4 w1r[W1P];
#pragma unroll
  for (int k = 0; k < W1P; ++k) {
    const int p = tid + NTH * k;
    w1r[k] = gld16(W1 + (long)(p / (DH / 8)) * DH + 8 * (p % (DH / 8)));
  }
  u32x4 ur[NU], us_[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) { ur[k] = v4(0, 0, 0, 0); us_[k] = v4(0, 0, 0, 0); }
  // slabs 0..LU-1: slab 0 goes straight to LDS, 1..LU-1 stay in the ring
#pragma unroll
  for (int q = 0; q < LU; ++q) ST::ld(Ur, csc, u_voff, q * KS, ur[q % NU], us_[q % NU]);

  // the first tile's coordinates and coefficient fragments
  const int tau0 = t_begin + w;
  auto tile_row = [&](int tau) -> long {
    const int j = selp[tau / cpt];
    return (long)j * C + (long)(tau % cpt) * TT;
  };
  typename CT::raw cr[DC][NTT];
  long row0 = tau0 < t_end ? tile_row(tau0) : 0;
  // scalar offset of k-step q of token tile tt
  auto c_soff = [&](int tt, int q) -> uint32_t {
    return (uint32_t)(((row0 + 16 * tt) * r + q * KS) * CT::ES);
  };
  if (tau0 < t_end) {
#pragma unroll
    for (int q = 0; q < DC - 1; ++q)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) cr[q][tt] = CT::ld(Cr, c_voff, c_soff(tt, q));
  }

  // tail share of this split: tokens [tb, te), first piece staged now
  const int tb = min(a.T, s * a.tail_per_split), te = min(a.T, tb + a.tail_per_split);
  const long tail_base = ((((long)b * a.G + a.layer) * a.Hkv + h) * a.T) * DH;
  const uint16_t *kt = reinterpret_cast<const uint16_t *>(a.k_tail) + tail_base;
  const uint16_t *vt = reinterpret_cast<const uint16_t *>(a.v_tail) + tail_base;
  auto stage_tail = [&](int t0) {  // one piece: TP rows of keys and values, 16 bytes per thread each
    const int nt = min(TP, te - t0);
    const int row = tid >> 4, c8 = (tid & 15) * 8;
    u32x4 kv = v4(0, 0, 0, 0), vv = v4(0, 0, 0, 0);
    if (row < nt) {
      kv = gld16(kt + (long)(t0 + row) * DH + c8);
      vv = gld16(vt + (long)(t0 + row) * DH + c8);
    }
    return std::make_pair(kv, vv);
  };
  auto tail0 = stage_tail(tb);

  // W1 -> fp16, head dims permuted (two 4-dim runs per piece)
#pragma unroll
  for (int k = 0; k < W1P; ++k) {
    const int p = tid + NTH * k, f = p / (DH / 8), d0 = 8 * (p % (DH / 8));
    const u32x4 v = w1r[k];
    const uint2 lo = make_uint2(pack2(bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16)),
                                pack2(bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16)));
    const uint2 hi = make_uint2(pack2(bf16_bits_to_f32(v.z & 0xFFFFu), bf16_bits_to_f32(v.z >> 16)),
                                pack2(bf16_bits_to_f32(v.w & 0xFFFFu), bf16_bits_to_f32(v.w >> 16)));
    *reinterpret_cast<uint2 *>(W1s + f * WLD + dpos(d0)) = lo;
    *reinterpret_cast<uint2 *>(W1s + f * WLD + dpos(d0 + 4)) = hi;
  }
  {  // q rows of this kv head: fp16 permuted (zero rows up to 16) and fp32 natural
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
    for (int i = tid; i < 16 * DH; i += NTH) {
      const int gi = i / DH, d = i % DH;
      const float x = gi < g ? bf16_bits_to_f32(qb[gi * DH + d]) : 0.f;
      Qs[gi * WLD + dpos(d)] = h16(x);
      if (gi < GQ) Qf[gi * DH + d] = x;
    }
    for (int f = tid; f < F; f += NTH) B1s[f] = bf16_bits_to_f32(B1[f]);
  }
  {
    const int row = tid >> 4, c8 = (tid & 15) * 8;
    lst16(Tk + row * DH + c8, tail0.first);
    lst16(Tv + row * DH + c8, tail0.second);
  }
  ST::st(Us, ur[0], us_[0]);   // slab 0 -> buffer 0
  __syncthreads();

  // per-wave softmax state: lane holds query head l16 (rows >= g are padding)
  float m_run = -INFINITY, l_run = 0.f;
  bool first = true;  // no tile attended yet: the running accH in LDS is undefined
  float accV[GQ][2];
#pragma unroll
  for (int i = 0; i < GQ; ++i) accV[i][0] = accV[i][1] = 0.f;
  float rs0 = 1.f, rs1 = 1.f;  // int8 residual scales of the lane's two dims
  if (sizeof(TC) == 1 && a.res_scale) {
    const uint16_t *rsc = a.res_scale + bh * DH;
    rs0 = f16_bits_to_f32(rsc[2 * lane]);
    rs1 = f16_bits_to_f32(rsc[2 * lane + 1]);
  }

  for (int it = 0; it < iters; ++it) {
    const int tau = t_begin + w + NW * it;
    const bool has = tau < t_end;
    if (it > 0 && has) {
      row0 = tile_row(tau);
#pragma unroll
      for (int q = 0; q < DC - 1; ++q)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) cr[q][tt] = CT::ld(Cr, c_voff, c_soff(tt, q));
    }
    // this tile's residual rows: CSR range of the chunk, then the tile's part
    int e0 = 0, e1 = 0;
    if (has) {
      const int j = (int)(row0 / C);
      e0 = rptr[j];
      e1 = rptr[j + 1];
    }
    int rtok[CPT] = {-1, -1};                  // token - row0 of entries e0 + lane + 64m
    int r_lo = 0, r_n = 0;                     // first row and count of this tile's rows
    typename Res<TC>::raw dr[RP];

    // ---- step 1: K_hat^T = U . C^T over NR k-steps ------------------------
    f32x4 acc[NDT][NTT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) acc[dt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    sfor<NR>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      // basis slab ks + LU into the ring (wraps to the next tile's first slabs);
      // issued before this step's coefficient loads so that waiting for it
      // LU - 1 steps later waits for nothing newer than the coefficients then due
      if (it + 1 < iters || ks + LU < NR)
        ST::ld(Ur, csc, u_voff, ((ks + LU) % NR) * KS, ur[(ks + LU) % NU], us_[(ks + LU) % NU]);
      // coefficients DC - 1 steps ahead
      if constexpr (ks + DC - 1 < NR) {
        if (has) {
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) cr[(ks + DC - 1) % DC][tt] = CT::ld(Cr, c_voff, c_soff(tt, ks + DC - 1));
        }
      }
      // residual entries of the chunk (their CSR range arrived by now)
      if constexpr (ks == 1) {
        if (has) {
          const int cnt = e1 - e0;
#pragma unroll
          for (int m = 0; m < CPT; ++m)
            if (lane + 64 * m < cnt) rtok[m] = ridx[e0 + lane + 64 * m] - (int)row0;
        }
      }
      if constexpr (ks == 3 || (NR <= 3 && ks == NR - 1)) {
        if (has) {
          const int cnt = e1 - e0;
          int below = 0, inside = 0;
#pragma unroll
          for (int m = 0; m < CPT; ++m) {
            const bool valid = lane + 64 * m < cnt;
            below += __popcll(__ballot(valid && rtok[m] < 0));
            inside += __popcll(__ballot(valid && rtok[m] >= 0 && rtok[m] < TT));
          }
          r_lo = e0 + below;
          r_n = inside;
#pragma unroll
          for (int k = 0; k < RP; ++k)
            if (k < r_n) dr[k] = Res<TC>::ld(Rr, r_lo + k, lane);
        }
      }
      // basis slab ks + 1 -> LDS (its load was issued LU - 1 steps ago)
      if constexpr (ks + 1 < NR) {
        ST::st(Us + ((ks + 1) & 1) * DH * ULD, ur[(ks + 1) % NU], us_[(ks + 1) % NU]);
      } else {
        if (it + 1 < iters) ST::st(Us, ur[0], us_[0]);  // the next tile's slab 0
      }
      if (has) {
        const uint16_t *ub = Us + (ks & 1) * DH * ULD + l16 * ULD + 8 * kg;
        typename CT::op bc[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) bc[tt] = CT::get(cr[ks % DC][tt]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const typename ST::op au = ST::get(ub + 16 * dt * ULD);
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) acc[dt][tt] = mfma(au, bc[tt], acc[dt][tt]);
        }
      }
      __syncthreads();
    });
    if (!has) continue;

    // ---- rebuilt keys as fp16 A operands --------------------------------------
    f16x8 KA[NJ][NTT];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          KA[jj][tt][v] = (_Float16)acc[2 * jj][tt][v];
          KA[jj][tt][4 + v] = (_Float16)acc[2 * jj + 1][tt][v];
        }

    // ---- step 2: logits and online softmax ------------------------------------
    f32x4 lg[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) lg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const f16x8 qf = ldh8(Qs + l16 * WLD + 32 * jj + 8 * kg);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) lg[tt] = mfma(KA[jj][tt], qf, lg[tt]);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        lg[tt][v] *= a.scale_log2;
        mt = fmaxf(mt, lg[tt][v]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    f16x8 PA[NTT / 2];
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const _Float16 p = (_Float16)exp2f(lg[tt][v] - m_new);
        PA[tt >> 1][4 * (tt & 1) + v] = p;
        lg[tt][v] = (float)p;
        psum += (float)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // p of this tile for the residual pass: Ps[w][g][t]
    if (l16 < GQ) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        *reinterpret_cast<f32x4 *>(Ps + (w * GQ + l16) * TT + 16 * tt + 4 * kg) = lg[tt];
    }
    // rescale the running sums: accV here, accH (rows g = v of lanes 0..15)
    // when this tile's hidden sums are folded into LDS
    float ah[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) ah[v] = __shfl(alpha, v, 64);
    {
#pragma unroll
      for (int gi = 0; gi < GQ; ++gi) {
        const float av = __shfl(alpha, gi, 64);
        accV[gi][0] *= av;
        accV[gi][1] *= av;
      }
    }

    // ---- step 5: residual rows (vector ALUs) -------------------------------------
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const int below = r_lo - e0;
      auto row = [&](int k, typename Res<TC>::raw raw) {
        const int pos = below + k;
        const int tsel = pos < 64 ? rtok[0] : rtok[1];
        const int t = __shfl(tsel, pos & 63, 64);
        float d0, d1;
        Res<TC>::get(raw, rs0, rs1, d0, d1);
        const float *pt = Ps + w * GQ * TT + t;
#pragma unroll
        for (int gi = 0; gi < GQ; ++gi) {
          const float p = pt[gi * TT];
          accV[gi][0] = fmaf(p, d0, accV[gi][0]);
          accV[gi][1] = fmaf(p, d1, accV[gi][1]);
        }
      };
#pragma unroll
      for (int k = 0; k < RP; ++k)
        if (k < r_n) row(k, dr[k]);
      for (int k = RP; k < r_n; ++k) row(k, Res<TC>::ld(Rr, r_lo + k, lane));
    }

    // ---- steps 3 and 4 per 16-wide hidden tile ------------------------------------
    // accH[g][f] of this tile: lane holds column f = 16 fi + l16, rows g = 4 kg + v;
    // each hidden tile is folded into the wave's running accH in LDS right away
    // (the real rows g < GQ live in lanes 0..15)
#pragma unroll
    for (int fi = 0; fi < NF; ++fi) {
      const float bias = B1s[16 * fi + l16];
      f32x4 hc[NTT];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) hc[tt] = f32x4{bias, bias, bias, bias};
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const f16x8 bw = ldh8(W1s + (16 * fi + l16) * WLD + 32 * jj + 8 * kg);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) hc[tt] = mfma(KA[jj][tt], bw, hc[tt]);
      }
      f32x4 ahc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NTT / 2; ++i) {
        f16x8 hb;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hb[v] = (_Float16)silu_f(hc[2 * i][v]);
          hb[4 + v] = (_Float16)silu_f(hc[2 * i + 1][v]);
        }
        ahc = mfma(PA[i], hb, ahc);
      }
      if (kg == 0) {
#pragma unroll
        for (int v = 0; v < GQ; ++v) {
          float *pa = AHw + v * F + 16 * fi + l16;
          *pa = first ? ahc[v] : fmaf(*pa, ah[v], ahc[v]);
        }
      }
    }
    first = false;
  }
  if (first && kg == 0) {  // a wave with no tile contributes zeros
#pragma unroll
    for (int fi = 0; fi < NF; ++fi)
#pragma unroll
      for (int v = 0; v < GQ; ++v) AHw[v * F + 16 * fi + l16] = 0.f;
  }

  // ---- the split's share of the uncompressed tail (vector ALUs) ---------------
  __syncthreads();
  float *mm = reinterpret_cast<float *>(sm + S::MM), *ml = reinterpret_cast<float *>(sm + S::ML);
  float *mv = reinterpret_cast<float *>(sm + S::MV);
  const float *AH = reinterpret_cast<const float *>(sm + S::AH);
  if (tid < GQ) { Ts[tid] = -INFINITY; Ts[GQ + tid] = 0.f; }
  float tacc = 0.f;   // thread (gi, d) = (tid / DH, tid % DH) of the tail's p . V
  for (int t0 = tb; t0 < te; t0 += TP) {
    const int nt = min(TP, te - t0);
    if (t0 > tb) {
      __syncthreads();
      auto piece = stage_tail(t0);
      const int row = tid >> 4, c8 = (tid & 15) * 8;
      lst16(Tk + row * DH + c8, piece.first);
      lst16(Tv + row * DH + c8, piece.second);
      __syncthreads();
    }
    if (tid < GQ * TP) {  // logits: thread (gi, t)
      const int gi = tid / TP, t = tid % TP;
      if (gi < g && t < nt) {
        float sdot = 0.f;
        for (int d = 0; d < DH; ++d) sdot = fmaf(Qf[gi * DH + d], bf16_bits_to_f32(Tk[t * DH + d]), sdot);
        Tl[gi * TP + t] = sdot * a.scale_log2;
      }
    }
    __syncthreads();
    if (tid < g) {  // online softmax of the piece
      float mx = -INFINITY;
      for (int t = 0; t < nt; ++t) mx = fmaxf(mx, Tl[tid * TP + t]);
      const float m_old = Ts[tid], mn = fmaxf(m_old, mx);
      const float al = (m_old == -INFINITY) ? 0.f : exp2f(m_old - mn);
      float sum = 0.f;
      for (int t = 0; t < nt; ++t) {
        const float p = exp2f(Tl[tid * TP + t] - mn);
        Tl[tid * TP + t] = p;
        sum += p;
      }
      Ts[tid] = mn;
      Ts[GQ + tid] = Ts[GQ + tid] * al + sum;
      Ts[2 * GQ + tid] = al;
    }
    __syncthreads();
    {
      const int gi = tid / DH, d = tid % DH;
      if (gi < g) {
        float v = tacc * Ts[2 * GQ + gi];
        for (int t = 0; t < nt; ++t) v = fmaf(Tl[gi * TP + t], bf16_bits_to_f32(Tv[t * DH + d]), v);
        tacc = v;
      }
    }
  }
  __syncthreads();  // W1, the basis slabs and the tail scratch are free from here

  // ---- merge the waves and the tail into one partial ------------------------------
  {
    float lt = l_run;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (lane < GQ) { mm[w * GQ + lane] = m_run; ml[w * GQ + lane] = lt; }
    float *aw = mv + w * GQ * DH;
#pragma unroll
    for (int gi = 0; gi < GQ; ++gi) {
      aw[gi * DH + 2 * lane] = accV[gi][0];
      aw[gi * DH + 2 * lane + 1] = accV[gi][1];
    }
    // the tail as a ninth contributor (no hidden sums)
    float *at = mv + NW * GQ * DH;
    if (tid < GQ) {
      mm[NW * GQ + tid] = tb < te && tid < g ? Ts[tid] : -INFINITY;
      ml[NW * GQ + tid] = tb < te && tid < g ? Ts[GQ + tid] : 0.f;
    }
    {
      const int gi = tid / DH, d = tid % DH;
      if (gi < GQ) at[gi * DH + d] = (tb < te && gi < g) ? tacc : 0.f;
    }
  }
  __syncthreads();
  float *part = a.part + (((long)b * a.Hkv + h) * a.n_split + s) * g * a.PW;
  constexpr int PWC = 4 + F + DH;
  for (int i = tid; i < g * PWC; i += NTH) {
    const int gi = i / PWC, c = i % PWC;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k <= NW; ++k) M = fmaxf(M, mm[k * GQ + gi]);
    float wt[NW + 1];
#pragma unroll
    for (int k = 0; k <= NW; ++k) wt[k] = mm[k * GQ + gi] == -INFINITY ? 0.f : exp2f(mm[k * GQ + gi] - M);
    float v = 0.f;
    if (c == 0) {
      v = M;
    } else if (c == 1 || c == 2) {  // l over everything, mass over rebuilt tokens
#pragma unroll
      for (int k = 0; k < NW; ++k) v = fmaf(wt[k], ml[k * GQ + gi], v);
      if (c == 1) v = fmaf(wt[NW], ml[NW * GQ + gi], v);
    } else if (c >= 4 && c < 4 + F) {
#pragma unroll
      for (int k = 0; k < NW; ++k) v = fmaf(wt[k], AH[(k * GQ + gi) * F + c - 4], v);
    } else if (c >= 4 + F) {
#pragma unroll
      for (int k = 0; k <= NW; ++k) v = fmaf(wt[k], mv[(k * GQ + gi) * DH + c - 4 - F], v);
    }
    part[(long)gi * a.PW + c] = v;
  }
}

template <typename TC, int NR, int NF>
static hipError_t go(const AttendArgs &a, hipStream_t st) {
  const size_t smem = Smem<NF * 16>::BYTES;
  static const bool lds_ok = (allow_dynamic_lds(k_attend_chain<TC, NR, NF>, smem), true);
  (void)lds_ok;
  hipLaunchKernelGGL((k_attend_chain<TC, NR, NF>), dim3(a.B * a.Hkv * a.n_split), dim3(NTH), smem, st, a);
  return hipGetLastError();
}

}  // namespace chain

// (rank, hidden, coefficient type) combinations compiled for this kernel; all
// need d_h = 128, bf16 activations, at most 4 query heads per kv head,
// 128-token chunks and residuals stored like the coefficients.
#define LOWRAM_CHAIN_SHAPES(X) \
  X(512, 256, bf16)            \
  X(256, 256, bf16)            \
  X(512, 128, bf16)            \
  X(256, 256, int8_t)          \
  X(512, 256, int8_t)

bool chain_supported(int act, int coeff, int resid, int dh, int F, int r, int C, int g, int k_eff) {
  if (act != LOWRAM_BF16 || coeff != resid || dh != chain::DH || g > chain::GQ ||
      C != chain::CPT * chain::TT || k_eff < 1)
    return false;
  const bool i8 = coeff == LOWRAM_I8;
#define X(r_, f_, t_) \
  if (r == r_ && F == f_ && i8 == (sizeof(t_) == 1)) return true;
  LOWRAM_CHAIN_SHAPES(X)
#undef X
  return false;
}

// Splits per (b, h) and tiles per split: about one workgroup per CU (256) when
// the batch allows, at most 8 tiles per wave; every split gets at least one tile.
void chain_plan(int B, int Hkv, int k_eff, int C, int T, int &n_split, int &tps, int &tail_per_split) {
  const int n_tiles = k_eff * (C / chain::TT);
  const int bh = B * Hkv;
  int want = (256 + bh - 1) / bh;                 // splits for about 256 workgroups
  const int max_split = (n_tiles + chain::NW - 1) / chain::NW;  // >= 8 tiles each
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  int iters = (n_tiles + want * chain::NW - 1) / (want * chain::NW);
  if (iters > 8) iters = 8;
  tps = iters * chain::NW;
  n_split = (n_tiles + tps - 1) / tps;
  tail_per_split = (T + n_split - 1) / n_split;
}

hipError_t launch_attend_chain(int coeff, const AttendArgs &a, hipStream_t st) {
  const bool i8 = coeff == LOWRAM_I8;
#define X(r_, f_, t_) \
  if (a.r == r_ && a.F == f_ && i8 == (sizeof(t_) == 1)) return chain::go<t_, r_ / chain::KS, f_ / 16>(a, st);
  LOWRAM_CHAIN_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace lowram
