// Fused rebuild-and-attend on gfx950 matrix cores (bf16/fp16 MFMA, fp32 accumulate).
//
// One workgroup (4 waves) owns one (sequence b, kv head h), a run of the
// chunks selected for it and an equal share of the uncompressed tail (on the
// vector ALUs after the chunks, merged into the same partial).  For each
// 128-token tile of a selected chunk:
//   1. K_hat^T[dh][128] = U_{l,h}[dh][r] . deq(coeff tile)^T  (32x32x16 MFMA).
//      Rank slabs of 64 are staged through LDS while the next slab is already
//      in flight in registers.  bf16 coefficients and basis enter as stored;
//      int8 coefficients are exact in fp16 and their per-channel scale is
//      folded into an fp16 basis slab.
//   2. logits in coefficient space, q_g . k_hat_t = (U^T q_g) . c_t, on the
//      coefficient slabs staged for step 1 (16x16x32 MFMA, heads padded to 16)
//      with U^T q_g from the select stage split into hi/lo halves; online
//      softmax in log2 units; p rounded to fp16 in LDS.
//   5. residual rows of the tile scattered into a dense, transposed delta
//      tile; accV += p . delta (16x16x32 MFMA).
//   3. H = SiLU(K_hat . W1^T + b1) per 64-wide hidden block (32x32x16 MFMA),
//      the next block's W1 already in flight.
//   4. accH += p . H (16x16x32 MFMA), kept in registers across tiles.
// The second predictor layer is linear, so W2 and b2 are applied once per
// query head in the combine: sum_t p_t v_t = W2 accH + b2 sum_t p_t + accV.
// Operands produced in the kernel (rebuilt keys, hidden activations, p, q,
// W1, delta) are fp16: 11 significant bits at the bf16 MFMA rate.
//
// Method: keys rebuilt from per-token coefficients on a group basis (zicq.com
// English summary, "Cross-Layer Low-Rank Key Compression"); values from the
// per-head predictor plus residuals of the worst tokens ("Core Mechanism");
// only query-selected chunks are rebuilt (rit.work page, generation section);
// attention softmax(q K^T / sqrt(d_h)) V (OjaKV page, section 3).
#include <type_traits>

#include "attend_common.hpp"

namespace lowram {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));


constexpr int TM = 128;   // tokens per tile
constexpr int RS = 64;    // rank slab of step 1
constexpr int PAD = 8;    // fp16/bf16 pad per LDS row (16-byte rows, spread banks)
constexpr int PF = 3;     // rank slabs in flight in registers (at most)
constexpr int CS_LD = RS + PAD, HS_LD = TM + PAD, PS_LD = TM + PAD;

// Two workgroups share a CU when the (head dim, hidden) pair leaves room in
// 256 registers per lane: one group's loads then run under the other's matrix
// work.  Larger shapes keep one group per CU, deeper register rings instead.
template <int DH, int NF64> constexpr bool dual_occupancy() { return DH == 128 && NF64 <= 4; }

// compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F &f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) { static_for_impl<0, N>(f); }

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
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)h16(lo) | ((uint32_t)h16(hi) << 16);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return v4(pack2(bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16)),
            pack2(bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16)),
            pack2(bf16_bits_to_f32(v.z & 0xFFFFu), bf16_bits_to_f32(v.z >> 16)),
            pack2(bf16_bits_to_f32(v.w & 0xFFFFu), bf16_bits_to_f32(v.w >> 16)));
}

// tokens per tail tile: keys and values of one tile staged as floats
template <int DH> constexpr int tail_tile() { return 32; }

template <int DH>
struct MfmaSmem {
  static constexpr int KS_LD = DH + PAD;
  static constexpr int A1 = (TM + DH) * CS_LD;                  // step 1 staging
  static constexpr int A3 = 64 * KS_LD + 64 * HS_LD;            // W1 block + H block
  static constexpr int A5 = DH * HS_LD;                         // transposed delta tile
  static constexpr int M13 = A1 > A3 ? A1 : A3;
  static constexpr int REGION_A = M13 > A5 ? M13 : A5;          // 16-bit elements
  static constexpr int KS_OFF = REGION_A;
  static constexpr int PS_OFF = KS_OFF + TM * KS_LD;
  static constexpr int END16 = PS_OFF + 16 * PS_LD;
  static constexpr int FLOATS = 4 * 16 * 2 + 16 * 3;            // red, red2, ms, ls, al
  static constexpr size_t BYTES = (size_t)END16 * 2 + FLOATS * 4;
};

// ---------------------------------------------------------------------------
// step 1 slab staging: global -> registers (several slabs in flight) -> LDS.
// The register ring is indexed only by compile-time constants so that it
// stays in registers.
// ---------------------------------------------------------------------------
template <int DH, typename TC> struct SlabT;
template <int DH> struct SlabT<DH, bf16> {
  static constexpr int NC = TM * RS / 8 / 256, NU = DH * RS / 8 / 256, NS = 0;  // 16-byte pieces
  typedef bf16x8 frag;
  __device__ static frag ld(const uint16_t *p) { return ldb8(p); }
};
template <int DH> struct SlabT<DH, int8_t> {
  static constexpr int NC = TM * RS / 16 / 256, NU = DH * RS / 8 / 256, NS = 1;
  typedef f16x8 frag;
  __device__ static frag ld(const uint16_t *p) { return ldh8(p); }
};

template <int DH>
__device__ __forceinline__ void slab_fetch(const bf16 *cf, const uint16_t *, const bf16 *U, long row0,
                                           int r, int r0, u32x4 *c, u32x4 *u, u32x4 *) {
  const int tid = threadIdx.x;
  constexpr int NC = SlabT<DH, bf16>::NC, NU = SlabT<DH, bf16>::NU;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 8), part = p % (RS / 8);
    c[k] = *reinterpret_cast<const u32x4 *>(cf + (row0 + row) * r + r0 + part * 8);
  }
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 8), part = p % (RS / 8);
    u[k] = *reinterpret_cast<const u32x4 *>(U + (long)row * r + r0 + part * 8);
  }
}
template <int DH>
__device__ __forceinline__ void slab_store(const bf16 *, const u32x4 *c, const u32x4 *u, const u32x4 *,
                                           uint16_t *Cs, uint16_t *Us) {
  const int tid = threadIdx.x;
  constexpr int NC = SlabT<DH, bf16>::NC, NU = SlabT<DH, bf16>::NU;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 8), part = p % (RS / 8);
    *reinterpret_cast<u32x4 *>(Cs + row * CS_LD + part * 8) = c[k];
  }
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 8), part = p % (RS / 8);
    *reinterpret_cast<u32x4 *>(Us + row * CS_LD + part * 8) = u[k];
  }
}
template <int DH>
__device__ __forceinline__ void slab_fetch(const int8_t *cf, const uint16_t *csc, const bf16 *U,
                                           long row0, int r, int r0, u32x4 *c, u32x4 *u, u32x4 *sc) {
  const int tid = threadIdx.x;
  constexpr int NC = SlabT<DH, int8_t>::NC, NU = SlabT<DH, int8_t>::NU;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 16), part = p % (RS / 16);
    c[k] = *reinterpret_cast<const u32x4 *>(cf + (row0 + row) * r + r0 + part * 16);
  }
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 8), part = p % (RS / 8);
    u[k] = *reinterpret_cast<const u32x4 *>(U + (long)row * r + r0 + part * 8);
  }
  sc[0] = *reinterpret_cast<const u32x4 *>(csc + r0 + (tid % (RS / 8)) * 8);  // part is tid % 8
}
template <int DH>
__device__ __forceinline__ void slab_store(const int8_t *, const u32x4 *c, const u32x4 *u,
                                           const u32x4 *sc, uint16_t *Cs, uint16_t *Us) {
  const int tid = threadIdx.x;
  constexpr int NC = SlabT<DH, int8_t>::NC, NU = SlabT<DH, int8_t>::NU;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 16), part = p % (RS / 16);
    const int8_t *b8 = reinterpret_cast<const int8_t *>(&c[k]);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack2((float)b8[2 * i], (float)b8[2 * i + 1]);  // exact
    *reinterpret_cast<u32x4 *>(Cs + row * CS_LD + part * 16) = v4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<u32x4 *>(Cs + row * CS_LD + part * 16 + 8) = v4(w[4], w[5], w[6], w[7]);
  }
  const uint16_t *s16 = reinterpret_cast<const uint16_t *>(sc);
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int p = tid + 256 * k, row = p / (RS / 8), part = p % (RS / 8);
    const uint16_t *u16 = reinterpret_cast<const uint16_t *>(&u[k]);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack2(bf16_bits_to_f32(u16[2 * i]) * f16_bits_to_f32(s16[2 * i]),
                   bf16_bits_to_f32(u16[2 * i + 1]) * f16_bits_to_f32(s16[2 * i + 1]));
    *reinterpret_cast<u32x4 *>(Us + row * CS_LD + part * 8) = v4(w[0], w[1], w[2], w[3]);
  }
}

// residual row pieces: 16 bytes of one row per thread per round
template <typename TR> struct ResRow;
template <> struct ResRow<bf16> {
  static constexpr int VALS = 8;  // values per 16-byte piece
  __device__ static void to_f16(u32x4 v, const uint16_t *, int, uint16_t *o) {
    const uint16_t *u = reinterpret_cast<const uint16_t *>(&v);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = h16(bf16_bits_to_f32(u[j]));
  }
};
template <> struct ResRow<int8_t> {
  static constexpr int VALS = 16;
  __device__ static void to_f16(u32x4 v, const uint16_t *sc, int d0, uint16_t *o) {
    const int8_t *q = reinterpret_cast<const int8_t *>(&v);
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = h16((float)q[j] * f16_bits_to_f32(sc[d0 + j]));
  }
};

// Block -> (kv head, sequence, split).  Workgroups are dispatched round-robin
// over the 8 XCDs (linear id mod 8), each with its own L2.  The linear id is
// remapped so that every split of one (sequence, kv head) lands on the same
// XCD, next to the other heads of that sequence: the head's basis slice and
// first predictor layer then stay L2-resident, and chunks picked by several
// heads of a sequence are fetched once per XCD.  Every split also attends its
// share of the tail, so the grid holds no tail-only workgroups (which would
// exceed one workgroup per CU at B Hkv n_split = 256); with no chunk selected
// there is one tail workgroup per (sequence, kv head), split 0 = n_split.
__device__ __forceinline__ void block_coords(const AttendArgs &a, int &h, int &b, int &split) {
  const int S = a.n_split, BH = a.B * a.Hkv;
  if (S == 0) {
    const int bh = blockIdx.x;
    b = bh / a.Hkv; h = bh % a.Hkv; split = 0;
    return;
  }
  const int lin = blockIdx.x;
  int bh;
  if (BH % 8 == 0) {
    const int xcd = lin % 8, i = lin / 8;
    bh = xcd * (BH / 8) + i / S;
    split = i % S;
  } else {
    bh = lin / S;
    split = lin % S;
  }
  b = bh / a.Hkv; h = bh % a.Hkv;
}

template <int DH, int NF64, int NSLAB, typename TC, typename TR>
__global__ __launch_bounds__(256, (dual_occupancy<DH, NF64>() ? 2 : 1)) void k_attend_mfma(const AttendArgs a) {
  constexpr bool OCC2 = dual_occupancy<DH, NF64>();
  using S = MfmaSmem<DH>;
  constexpr int KS_LD = S::KS_LD;
  constexpr int NT1 = DH / 64;        // 32-row d tiles per wave in step 1
  constexpr int NVT = DH / 64;        // 16-wide d tiles per wave for accV
  constexpr int RPR = DH / ResRow<TR>::VALS;   // 16-byte pieces per residual row
  constexpr int W1P = 64 * DH / 8 / 256;       // W1 16-byte pieces per thread per block
  extern __shared__ __align__(16) unsigned char msm[];
  uint16_t *sm16 = reinterpret_cast<uint16_t *>(msm);
  uint16_t *Cs = sm16, *Us = sm16 + TM * CS_LD;               // step 1
  uint16_t *W1s = sm16, *Hs = sm16 + 64 * KS_LD;              // steps 3/4
  uint16_t *Dt = sm16;                                         // step 5: delta^T [DH][TM+8]
  uint16_t *Ks = sm16 + S::KS_OFF, *Ps = sm16 + S::PS_OFF;
  float *fl = reinterpret_cast<float *>(sm16 + S::END16);
  float *red = fl, *red2 = fl + 64, *ms = fl + 128, *ls = ms + 16, *al = ls + 16;

  const int tid = threadIdx.x;
  int h, b, split;
  block_coords(a, h, b, split);
  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int g = a.g, r = a.r, C = a.C;
  constexpr int TAIL_TT = tail_tile<DH>();
  // the tail scratch ends below the float area (m, l, alpha of the rebuilt tokens)
  static_assert((2 * 16 * DH + 16 * TAIL_TT + 48 + 2 * TAIL_TT * (DH + 1)) * 4 <= S::END16 * 2,
                "tail split does not fit the LDS of the rebuild kernel");

  if (split == a.n_split) {  // no chunk selected: the whole tail on the vector ALUs
    float *qs = reinterpret_cast<float *>(msm), *accV = qs + g * DH, *lgs = accV + g * DH;
    float *tms = lgs + g * TAIL_TT, *tls = tms + 16, *tal = tls + 16, *kv = tal + 16;
    const bf16 *qb = reinterpret_cast<const bf16 *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
    for (int i = tid; i < g * DH; i += 256) { qs[i] = to_f32(qb[i]); accV[i] = 0.f; }
    if (tid < 16) { tms[tid] = -INFINITY; tls[tid] = 0.f; tal[tid] = 0.f; }
    __syncthreads();
    tail_split<bf16>(a, h, b, qs, lgs, TAIL_TT, accV, tms, tls, tal, kv, 0, a.T);
    write_partial(a, h, b, split, tms, tls, nullptr, accV);
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

  // Logit operand (16x16x32 B operand: column lane & 15, ranks 8 (lane >> 4)
  // .. + 8 of each k-step), written by the select stage: x = U^T q_g (times
  // the int8 rank scales) as hi = x rounded to the codes' MFMA type and lo =
  // (x - hi) rounded, so hi + lo carries x to about 2^-16 (bf16) or 2^-22
  // (fp16) relative where a key rebuilt and rounded to fp16 would move logits
  // in the hundreds by ~0.1.  With 2g <= 16 column c of tile 0 holds hi of
  // head c or lo of head c - g, added after the MFMAs; with g > 8 tile 1 holds
  // the lo halves and accumulates into the same logits.
  const bool q_two = g > 8;
  // (wave-uniform base, 32-bit lane offset: one VGPR for the address)
  const uint16_t *qfb = a.qfrag + ((long)b * a.Hkv + h) * 2 * 16 * r;
  uint32_t qfo = (uint32_t)((lane & 15) * r + 8 * (lane >> 4));
  if (tid < 16) { ms[tid] = -INFINITY; ls[tid] = 0.f; al[tid] = 0.f; }

  f32x4 accH[NF64], accV[NVT];
#pragma unroll
  for (int i = 0; i < NF64; ++i) accH[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NVT; ++i) accV[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const int s_end = min(a.k_eff, (split + 1) * a.cps);
  for (int slot = split * a.cps; slot < s_end; ++slot) {
    const int j = selp[slot];
    for (int t0 = 0; t0 < C; t0 += TM) {
      const long row0 = (long)j * C + t0;
      // the operand loads are the same for every tile: an opaque offset keeps
      // them in the tile loop rather than hoisted into 8 NSLAB live registers
      asm volatile("" : "+v"(qfo));
      // ---- step 1: K_hat^T = U . C^T --------------------------------------
      f32x16 acc1[NT1][2];
#pragma unroll
      for (int mi = 0; mi < NT1; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc1[mi][ni][i] = 0.f;
      // logits of the wave's 32 tokens (rows 32 w + 16 mi ..)
      f32x4 acc2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      // ring of PFD slabs in flight, PFD-1 ahead of the one being multiplied
      int e0, e1, rt = -1;
      u32x4 rv = v4(0, 0, 0, 0);
      auto res_head = [&]() {
        e0 = rptr[j];
        e1 = rptr[j + 1];
        const int e = e0 + tid / RPR;
        if (e < e1) {
          rt = ridx[e] - (int)row0;
          rv = gld16(rval + (long)e * DH + (tid % RPR) * ResRow<TR>::VALS);
        }
      };
      {
        using ST = SlabT<DH, TC>;
        constexpr int PFD_MAX = OCC2 ? 2 : (DH > 128 ? 2 : PF);
        constexpr int PFD = NSLAB < PFD_MAX ? NSLAB : PFD_MAX;
        u32x4 rc[PFD][ST::NC], ru[PFD][ST::NU], rs[PFD][ST::NS > 0 ? ST::NS : 1];
#pragma unroll
        for (int u = 0; u < PFD - 1; ++u) slab_fetch<DH>(cf, csc, U, row0, r, u * RS, rc[u], ru[u], rs[u]);
        // this chunk's residual rows: CSR range, then the first round of pieces
        // (after step 1 instead when registers are tight)
        if constexpr (!OCC2) res_head();
        static_for<NSLAB>([&](auto sc_) {
          constexpr int s = decltype(sc_)::value;
          constexpr int cur_slot = s % PFD, next_slot = (s + PFD - 1) % PFD;
          slab_store<DH>(cf, rc[cur_slot], ru[cur_slot], rs[cur_slot], Cs, Us);
          __syncthreads();
          if constexpr (s + PFD - 1 < NSLAB)
            slab_fetch<DH>(cf, csc, U, row0, r, (s + PFD - 1) * RS, rc[next_slot], ru[next_slot], rs[next_slot]);
          if constexpr (OCC2) {  // the other workgroup covers LDS latency
#pragma unroll
            for (int ks = 0; ks < RS / 16; ++ks) {
              const int kof = 16 * ks + 8 * (lane >> 5);
              typename ST::frag bc[2], au[NT1];
#pragma unroll
              for (int ni = 0; ni < 2; ++ni) bc[ni] = ST::ld(Cs + (64 * wn + 32 * ni + (lane & 31)) * CS_LD + kof);
#pragma unroll
              for (int mi = 0; mi < NT1; ++mi) au[mi] = ST::ld(Us + (wm * (DH / 2) + 32 * mi + (lane & 31)) * CS_LD + kof);
#pragma unroll
              for (int mi = 0; mi < NT1; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) acc1[mi][ni] = mfma32(au[mi], bc[ni], acc1[mi][ni]);
            }
          } else {
            typename ST::frag bc[2][2], au[2][NT1];
  #pragma unroll
            for (int ni = 0; ni < 2; ++ni) bc[0][ni] = ST::ld(Cs + (64 * wn + 32 * ni + (lane & 31)) * CS_LD + 8 * (lane >> 5));
  #pragma unroll
            for (int mi = 0; mi < NT1; ++mi) au[0][mi] = ST::ld(Us + (wm * (DH / 2) + 32 * mi + (lane & 31)) * CS_LD + 8 * (lane >> 5));
  #pragma unroll
            for (int ks = 0; ks < RS / 16; ++ks) {
              const int cur = ks & 1, nxt = cur ^ 1;
              if (ks + 1 < RS / 16) {  // next k-step's fragments in flight under this k-step's MFMAs
                const int kof = 16 * (ks + 1) + 8 * (lane >> 5);
  #pragma unroll
                for (int ni = 0; ni < 2; ++ni) bc[nxt][ni] = ST::ld(Cs + (64 * wn + 32 * ni + (lane & 31)) * CS_LD + kof);
  #pragma unroll
                for (int mi = 0; mi < NT1; ++mi) au[nxt][mi] = ST::ld(Us + (wm * (DH / 2) + 32 * mi + (lane & 31)) * CS_LD + kof);
              }
  #pragma unroll
              for (int mi = 0; mi < NT1; ++mi)
  #pragma unroll
                for (int ni = 0; ni < 2; ++ni) acc1[mi][ni] = mfma32(au[cur][mi], bc[cur][ni], acc1[mi][ni]);
            }
          }
          // step 2's logits over this slab's ranks: coefficient rows of the wave's tokens
#pragma unroll
          for (int ks = 0; ks < RS / 32; ++ks) {
            const int kof = 32 * ks + 8 * (lane >> 4);
            const typename ST::frag qb = __builtin_bit_cast(typename ST::frag, gld16(qfb + (qfo + (uint32_t)(s * RS + 32 * ks))));
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
              acc2[mi] = mfma16(ST::ld(Cs + (32 * w + 16 * mi + (lane & 15)) * CS_LD + kof), qb, acc2[mi]);
          }
          if (q_two) {  // lo halves of g > 8 heads (second operand tile)
#pragma unroll
            for (int ks = 0; ks < RS / 32; ++ks) {
              const int kof = 32 * ks + 8 * (lane >> 4);
              const typename ST::frag ql =
                  __builtin_bit_cast(typename ST::frag, gld16(qfb + (qfo + (uint32_t)(16 * r + s * RS + 32 * ks))));
#pragma unroll
              for (int mi = 0; mi < 2; ++mi)
                acc2[mi] = mfma16(ST::ld(Cs + (32 * w + 16 * mi + (lane & 15)) * CS_LD + kof), ql, acc2[mi]);
            }
          }
          __syncthreads();
        });
      }
      if constexpr (OCC2) res_head();
      // the first WD blocks of W1 go in flight behind steps 2 and 5
      constexpr int WD_MAX = OCC2 ? 1 : 16 / W1P;
      constexpr int WD = WD_MAX < NF64 ? WD_MAX : NF64;
      u32x4 w1r[WD][W1P];
      static_for<WD>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int k = 0; k < W1P; ++k) {
          const int p = tid + 256 * k, f = p / (DH / 8), part = p % (DH / 8);
          w1r[i][k] = gld16(W1 + (long)(i * 64 + f) * DH + part * 8);
        }
      });
#pragma unroll
      for (int mi = 0; mi < NT1; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int t = 64 * wn + 32 * ni + (lane & 31);
            const int d = wm * (DH / 2) + 32 * mi + 8 * q4 + 4 * (lane >> 5);
            *reinterpret_cast<uint2 *>(Ks + t * KS_LD + d) =
                make_uint2(pack2(acc1[mi][ni][4 * q4], acc1[mi][ni][4 * q4 + 1]),
                           pack2(acc1[mi][ni][4 * q4 + 2], acc1[mi][ni][4 * q4 + 3]));
          }
      __syncthreads();

      // ---- step 2: online softmax ----------------------------------------
      // with 2g <= 16: hi (column gi) + lo (column g + gi) of each head's logit
      if (!q_two)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc2[mi][i] += __shfl_down(acc2[mi][i], g, 16);
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
      // delta^T tile: clear it while the maxima settle
      const bool has_res = e1 > e0;
      if (has_res)
        for (int i = tid; i < DH * HS_LD / 8; i += 256) reinterpret_cast<u32x4 *>(Dt)[i] = v4(0, 0, 0, 0);
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
      // residual rows into delta^T: row e fills column t of its dims
      if (has_res) {
        int first = 1;
        for (int e = e0 + tid / RPR; e < e1; e += 256 / RPR, first = 0) {
          u32x4 v = rv;
          int t = rt;
          if (!first) {
            t = ridx[e] - (int)row0;
            v = gld16(rval + (long)e * DH + (tid % RPR) * ResRow<TR>::VALS);
          }
          if (t >= 0 && t < TM) {
            uint16_t o[ResRow<TR>::VALS];
            const int d0 = (tid % RPR) * ResRow<TR>::VALS;
            ResRow<TR>::to_f16(v, rsc, d0, o);
#pragma unroll
            for (int jv = 0; jv < ResRow<TR>::VALS; ++jv) Dt[(d0 + jv) * HS_LD + t] = o[jv];
          }
        }
      }
      __syncthreads();
      if (tid < 16) {
        const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
        al[tid] = alpha;
        ls[tid] = ls[tid] * alpha + ((red2[tid] + red2[16 + tid]) + (red2[32 + tid] + red2[48 + tid]));
        ms[tid] = m_new;
      }
      __syncthreads();

      // ---- rescale, then step 5: accV += p . delta -----------------------
      float alr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) alr[i] = al[4 * (lane >> 4) + i];
#pragma unroll
      for (int fb = 0; fb < NF64; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) accH[fb][i] *= alr[i];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i) accV[vt][i] *= alr[i];
      if (has_res) {
#pragma unroll
        for (int ks = 0; ks < TM / 32; ++ks) {
          const int kof = 32 * ks + 8 * (lane >> 4);
          const f16x8 ap = ldh8(Ps + (lane & 15) * PS_LD + kof);
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt)
            accV[vt] = mfma16(ap, ldh8(Dt + (16 * (w * NVT + vt) + (lane & 15)) * HS_LD + kof), accV[vt]);
        }
        __syncthreads();
      }

      // ---- steps 3 and 4 per 64-wide hidden block ---------------------------
      static_for<NF64>([&](auto fbc) {
        constexpr int fb = decltype(fbc)::value, slot_w = fb % WD;
#pragma unroll
        for (int k = 0; k < W1P; ++k) {
          const int p = tid + 256 * k, f = p / (DH / 8), part = p % (DH / 8);
          lst16(W1s + f * KS_LD + part * 8, bf16x8_to_f16x8(w1r[slot_w][k]));
        }
        __syncthreads();
        if constexpr (fb + WD < NF64) {
#pragma unroll
          for (int k = 0; k < W1P; ++k) {
            const int p = tid + 256 * k, f = p / (DH / 8), part = p % (DH / 8);
            w1r[slot_w][k] = gld16(W1 + (long)((fb + WD) * 64 + f) * DH + part * 8);
          }
        }
        f32x16 acc3[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc3[mi][i] = 0.f;
        {  // fragments of k-step ks+1 in flight under the MFMAs of k-step ks
          f16x8 bw[2], ak[2][2];
          bw[0] = ldh8(W1s + (32 * wn + (lane & 31)) * KS_LD + 8 * (lane >> 5));
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) ak[0][mi] = ldh8(Ks + (64 * wm + 32 * mi + (lane & 31)) * KS_LD + 8 * (lane >> 5));
#pragma unroll
          for (int ks = 0; ks < DH / 16; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            if (ks + 1 < DH / 16) {
              const int kof = 16 * (ks + 1) + 8 * (lane >> 5);
              bw[nxt] = ldh8(W1s + (32 * wn + (lane & 31)) * KS_LD + kof);
#pragma unroll
              for (int mi = 0; mi < 2; ++mi) ak[nxt][mi] = ldh8(Ks + (64 * wm + 32 * mi + (lane & 31)) * KS_LD + kof);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) acc3[mi] = mfma32(ak[cur][mi], bw[cur], acc3[mi]);
          }
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
      });
      __syncthreads();
    }
  }

  // ---- this split's share of the tail, on the vector ALUs ----------------------
  // Tokens [tb, te) of the T tail tokens; the LDS below the float area is free
  // once the last tile is done.  Its own softmax state (m, l, accV over the
  // tail tokens) is merged with the rebuilt tokens' below.
  const int tshare = (a.T + a.n_split - 1) / a.n_split;
  const int tb = min(a.T, split * tshare), te = min(a.T, tb + tshare);
  float *qt = reinterpret_cast<float *>(msm), *accVt = qt + g * DH, *lgt = accVt + g * DH;
  float *tms = lgt + g * TAIL_TT, *tls = tms + 16, *tal = tls + 16, *kvt = tal + 16;
  {
    const bf16 *qb = reinterpret_cast<const bf16 *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
    for (int i = tid; i < g * DH; i += 256) { qt[i] = to_f32(qb[i]); accVt[i] = 0.f; }
    if (tid < 16) { tms[tid] = -INFINITY; tls[tid] = 0.f; tal[tid] = 0.f; }
    __syncthreads();
    tail_split<bf16>(a, h, b, qt, lgt, TAIL_TT, accVt, tms, tls, tal, kvt, tb, te);
  }
  // merge weights: rebuilt tokens 2^(m_c - M), tail tokens 2^(m_t - M)
  float *wc = red, *wt = red + 16;
  if (tid < g) {
    const float mc = ms[tid], mt = tms[tid], M = fmaxf(mc, mt);
    wc[tid] = mc == -INFINITY ? 0.f : exp2f(mc - M);
    wt[tid] = mt == -INFINITY ? 0.f : exp2f(mt - M);
  }
  __syncthreads();

  // ---- partials ---------------------------------------------------------------
  float *p = a.part + (((long)b * a.Hkv + h) * a.n_split + split) * g * a.PW;
  if (tid < g) {
    const float lc = wc[tid] * ls[tid];
    p[tid * a.PW] = fmaxf(ms[tid], tms[tid]);
    p[tid * a.PW + 1] = fmaf(wt[tid], tls[tid], lc);
    p[tid * a.PW + 2] = lc;
    p[tid * a.PW + 3] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gq = 4 * (lane >> 4) + i;
    if (gq < g) {
      const float c = wc[gq], u = wt[gq];
#pragma unroll
      for (int fb = 0; fb < NF64; ++fb) p[gq * a.PW + 4 + fb * 64 + 16 * w + (lane & 15)] = c * accH[fb][i];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const int d = 16 * (w * NVT + vt) + (lane & 15);
        p[gq * a.PW + 4 + a.F + d] = fmaf(u, accVt[gq * DH + d], c * accV[vt][i]);
      }
    }
  }
}

hipError_t launch_attend_valu(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st);

template <int DH, int NF64, int NSLAB, typename TC, typename TR>
static hipError_t go(const AttendArgs &a, hipStream_t st) {
  if (a.n_split > 0 && !a.qfrag) return hipErrorInvalidValue;  // logits need the select stage's U^T q
  const size_t smem = MfmaSmem<DH>::BYTES;
  static const bool lds_ok = (allow_dynamic_lds(k_attend_mfma<DH, NF64, NSLAB, TC, TR>, smem), true);
  (void)lds_ok;
  hipLaunchKernelGGL((k_attend_mfma<DH, NF64, NSLAB, TC, TR>), dim3((a.n_split > 0 ? a.n_split : 1) * a.Hkv * a.B),
                     dim3(256), smem, st, a);
  return hipGetLastError();
}

// (head dim, hidden, rank, coefficient/residual type) combinations compiled for
// the matrix cores; every other valid shape runs on the vector-ALU kernel.
#define LOWRAM_MFMA_SHAPES(X)        \
  X(128, 256, 512, bf16)             \
  X(128, 256, 256, bf16)             \
  X(128, 128, 512, bf16)             \
  X(128, 512, 512, bf16)             \
  X(256, 512, 384, bf16)             \
  X(256, 512, 512, bf16)             \
  X(128, 256, 256, int8_t)           \
  X(128, 256, 512, int8_t)           \
  X(256, 512, 384, int8_t)

bool mfma_supported(const AttendArgs &a, int act, int coeff, int resid) {
  if (act != LOWRAM_BF16 || coeff != resid || a.C % TM != 0 || a.g > 16) return false;
  const bool i8 = coeff == LOWRAM_I8;
#define X(dh_, f_, r_, t_) \
  if (a.dh == dh_ && a.F == f_ && a.r == r_ && i8 == (sizeof(t_) == 1)) return true;
  LOWRAM_MFMA_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_attend(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st) {
  if (a.path == LOWRAM_PATH_CHAIN) return launch_attend_chain(coeff, a, st);
  if (a.path == LOWRAM_PATH_ABSORB) return launch_attend_absorb(coeff, a, st);
  if (!mfma_supported(a, act, coeff, resid)) return launch_attend_valu(act, coeff, resid, a, st);
  const bool i8 = coeff == LOWRAM_I8;
#define X(dh_, f_, r_, t_) \
  if (a.dh == dh_ && a.F == f_ && a.r == r_ && i8 == (sizeof(t_) == 1)) return go<dh_, f_ / 64, r_ / RS, t_, t_>(a, st);
  LOWRAM_MFMA_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace lowram
