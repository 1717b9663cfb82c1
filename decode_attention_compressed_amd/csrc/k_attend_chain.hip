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
// While wave 0 selects the chunks, the other waves convert W1 into LDS and
// attend the split's share of the uncompressed tail on the vector ALUs; after
// the tiles the 8 waves merge into one partial per query head:
// (m, l, mass of rebuilt tokens, accH[F], accV[d_h]).
// The second predictor layer is linear and is applied once per query head in
// the combine: sum_t p_t v_t = W2 accH + b2 mass + accV.
//
// The REUSE variant also keeps rebuilt keys across decode steps: wave 0 maps
// the selected chunks to slots of a per-head table right after selecting them
// (reuse_assign_wave); a workgroup whose tiles all hit reads its keys back and
// skips the step-1 products (its coefficient loads point past the buffer end),
// and tiles given a slot on a miss store their keys after step 1.
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
constexpr int NW = 8;             // waves per workgroup (two per SIMD)
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
constexpr int NU = 2;             // basis register ring (divides the step count)
constexpr int SP = DH * KS / 8 / NTH;  // 16-byte basis pieces per thread and slab
constexpr int TP = 32;            // tail tokens staged in LDS per split
constexpr int CPT = 2;            // tiles per chunk: 128-token chunks
constexpr int MAXIT = 8;          // tiles per wave and split (at most)
constexpr int MAXSLOT = MAXIT * NW / CPT;  // selected chunks per split (at most)
// A cached tile: the rebuilt keys KA[NJ][NTT] (fp16) in 16-byte words, laid
// out as the registers hold them (lane fastest).
constexpr int KA_W = NJ * NTT * WAVE;


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
__device__ __forceinline__ u32x4 lds16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ bf16x8 ldb8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// The hidden pre-activation is kept in units of -log2(e): W1 and b1 are scaled
// by -log2(e) when staged, so with y = -log2(e) x, SiLU(x) = x / (1 + e^-x)
// becomes -ln(2) * y / (1 + 2^y): one exp2, one reciprocal and one product.
// The factor -ln(2) is applied once, to the merged hidden sums.
constexpr float NEG_LOG2E = -1.4426950408889634f;
constexpr float NEG_LN2 = -0.6931471805599453f;
__device__ __forceinline__ float silu_scaled(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
}

// Position of head dim d inside the permuted order: within each 32-wide step,
// lane group kg of the step-1 output holds dims 4kg..4kg+3 and 16+4kg..16+4kg+3,
// which become its eight consecutive k positions 8kg..8kg+7.
__device__ __forceinline__ int dpos(int d) {
  return (d & ~31) + 8 * ((d & 15) >> 2) + 4 * ((d >> 4) & 1) + (d & 3);
}

// Sums R rows of per-lane partials over the lanes that differ in the log2 R
// lane bits OFF0, OFF0 / 2, ..., then over the remaining lower lane bits.
// Each transposing step keeps the half of a lane's rows that its lane bit
// selects and adds the partner's values of those rows.  On return every lane
// holds the wave total of row (lane >> (6 - log2 R)) when OFF0 = 32.
template <int N, int OFF>
__device__ __forceinline__ void xpose_step_f(float *v, int lane) {
  if constexpr (N > 1) {
    const bool hi = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = hi ? v[N / 2 + i] : v[i];
      const float send = hi ? v[i] : v[N / 2 + i];
      v[i] = keep + __shfl_xor(send, OFF, 64);
    }
    xpose_step_f<N / 2, OFF / 2>(v, lane);
  } else if constexpr (OFF > 0) {
    v[0] += __shfl_xor(v[0], OFF, 64);
    xpose_step_f<1, OFF / 2>(v, lane);
  }
}
template <int R, int OFF0>
__device__ __forceinline__ float xpose_sum_f(float (&v)[R], int lane) {
  static_assert((R & (R - 1)) == 0 && R <= 2 * OFF0, "R a power of two within the lane bits");
  xpose_step_f<R, OFF0>(v, lane);
  return v[0];
}

// LDS layout (bytes).  The merge area at the end reuses W1 and the basis slabs;
// each wave's running accH stays in LDS across its tiles.
template <int F, int R>
struct Smem {
  static constexpr int W1S = 0;                          // [F][WLD] fp16, dims permuted
  static constexpr int US = W1S + F * WLD * 2;           // 2 x [DH][ULD] basis slabs
  static constexpr int QS = US + 2 * DH * ULD * 2;       // [16][WLD] fp16 q, dims permuted
  static constexpr int B1 = QS + 16 * WLD * 2;           // [F] fp32 b1
  static constexpr int PS = B1 + F * 4;                  // [NW][TT][GQ] fp32 p
  static constexpr int TK = PS + NW * GQ * TT * 4;       // [TP][DH] bf16 tail keys
  static constexpr int TV = TK + TP * DH * 2;            // [TP][DH] bf16 tail values
  static constexpr int AH = TV + TP * DH * 2;            // [NW][F][GQ] fp32 running accH per wave
  static constexpr int SEL = AH + NW * GQ * F * 4;       // [MAXSLOT] chunks of this split, [NW] counts
  static constexpr int TLS = SEL + (MAXSLOT + NW) * 4;   // [2][NW][GQ] tail l and the m it is taken at
  static constexpr int RCODE = TLS + 2 * NW * GQ * 4;    // [MAXSLOT] reuse slot codes of this split's chunks
  // logits in coefficient space: q~_g (int8: times the rank scales), hi then lo parts [2][GQ][R]
  static constexpr int QSC = (RCODE + MAXSLOT * 4 + 15) / 16 * 16;
  static constexpr int BYTES = QSC + 2 * GQ * R * 2;
  // reuse, prologue only: the whole selection after the chunk scores in the p
  // area, the slot table of (b, l, h) in the accH area
  static constexpr int SELALL = PS + CHAIN_SELECT_MAX_NC * 8;
  static_assert(CHAIN_SELECT_MAX_NC * 12 <= NW * GQ * TT * 4, "selection staging does not fit");
  static_assert((3 * REUSE_MAX_SLOTS + CHAIN_SELECT_MAX_NC) * 4 <= NW * GQ * F * 4,
                "slot table staging does not fit");
  // the chunk scores of the in-kernel selection use the p area (free until the first softmax)
  static_assert(CHAIN_SELECT_MAX_NC * 8 <= NW * GQ * TT * 4, "score staging does not fit");
  // merge area (after the last tile): per wave and query head m, l of rebuilt
  // tokens, l of tail tokens; then accV
  static constexpr int MM = 0, MLC = MM + NW * GQ * 4, MLT = MLC + NW * GQ * 4;
  static constexpr int MV = MLT + NW * GQ * 4;
  static constexpr int MWT = MV + NW * GQ * DH * 4, MWH = MWT + NW * GQ * 4;  // merge weights
  static_assert(MWH + NW * GQ * 4 <= QS, "merge area does not fit");
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
  __device__ static op get(raw v) { return i8x8_to_f16x8(v.x, v.y); }  // |code| <= 127: exact
};

// basis slab pieces: thread tid stages 8 ranks of head-dim rows tid / 4 + 64 i
// (lane offset ((tid / 4) * r + 8 (tid % 4)) * 2 bytes; piece and k-step in the
// scalar offset)
template <typename TC> struct Slab;
template <> struct Slab<bf16> {
  typedef bf16x8 op;
  __device__ static void ld(rsrc_t U, const uint16_t *, uint32_t voff, int r, int k0, u32x4 *u, u32x4 &,
                            uint32_t skip = 0u) {
#pragma unroll
    for (int i = 0; i < SP; ++i) u[i] = bld16(U, voff, 2u * (k0 + i * (NTH / 4) * r) + skip);
  }
  __device__ static void st(uint16_t *Ub, const u32x4 *u, const u32x4 &) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < SP; ++i) lst16(Ub + ((tid >> 2) + i * (NTH / 4)) * ULD + 8 * (tid & 3), u[i]);
  }
  __device__ static op get(const uint16_t *p) { return ldb8(p); }
};
template <> struct Slab<int8_t> {  // fp16 slab with the coefficient scale folded in
  typedef f16x8 op;
  __device__ static void ld(rsrc_t U, const uint16_t *csc, uint32_t voff, int r, int k0, u32x4 *u, u32x4 &sc,
                            uint32_t skip = 0u) {
#pragma unroll
    for (int i = 0; i < SP; ++i) u[i] = bld16(U, voff, 2u * (k0 + i * (NTH / 4) * r) + skip);
    sc = gld16(csc + k0 + 8 * (threadIdx.x & 3));
  }
  __device__ static void st(uint16_t *Ub, const u32x4 *u, const u32x4 &sc) {
    const int tid = threadIdx.x;
    const uint16_t *s16 = reinterpret_cast<const uint16_t *>(&sc);
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      const uint16_t *u16 = reinterpret_cast<const uint16_t *>(&u[i]);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack2(bf16_bits_to_f32(u16[2 * e]) * f16_bits_to_f32(s16[2 * e]),
                     bf16_bits_to_f32(u16[2 * e + 1]) * f16_bits_to_f32(s16[2 * e + 1]));
      lst16(Ub + ((tid >> 2) + i * (NTH / 4)) * ULD + 8 * (tid & 3), v4(w[0], w[1], w[2], w[3]));
    }
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

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reuse slots for the k selected chunks of one (b, l, h), by one wave (lane
// order fixes every decision): a chunk held by a slot of the table's current
// half is a hit (code slot | REUSE_HIT); the others, in ascending chunk order,
// take the free slots (not hit this step) by (stamp, slot index) and are
// stored there (code slot), or get no slot (code -1) when none is left.
// Codes of selection positions [q0, q0 + MAXSLOT) go to codeL; with `write`
// the updated table goes to the other half and the hit count to hits_out.
// Slot j lives in lane j % 64, register j / 64; selected chunk i is read from
// LDS as a broadcast.  Scratch: 3 S + k int32 of LDS.
__device__ void reuse_assign_wave(const int32_t *selAll, int k, const int32_t *chunk_in,
                                  const int32_t *stamp_in, int32_t *chunk_out, int32_t *stamp_out, int S,
                                  int t, int32_t *scr, int32_t *codeL, int q0, bool write,
                                  int32_t *hits_out) {
  constexpr int SPL = REUSE_MAX_SLOTS / WAVE;  // slots per lane
  const int lane = threadIdx.x & (WAVE - 1);
  int32_t *ch = scr, *stp = scr + S, *by_rank = scr + 2 * S, *held = scr + 3 * S;
  int myc[SPL], mys[SPL];
  bool myhit[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    const int j = u * WAVE + lane;
    myc[u] = j < S ? chunk_in[j] : -1;
    mys[u] = j < S ? stamp_in[j] : 0;
    myhit[u] = false;
  }
  // hits: one ballot per selected chunk and slot register
  int hits = 0;
  for (int i = 0; i < k; ++i) {
    const int c = selAll[i];
    int found = -1;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      if (u * WAVE >= S) break;
      const uint64_t m = __ballot(myc[u] == c && u * WAVE + lane < S);
      if (found < 0 && m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        found = u * WAVE + l;
        if (lane == l) myhit[u] = true;
      }
    }
    hits += found >= 0;
    if (lane == 0) {
      held[i] = found >= 0;
      if (i >= q0 && i < q0 + MAXSLOT) codeL[i - q0] = found >= 0 ? (found | REUSE_HIT) : -1;
    }
  }
  // free slots ranked by (stamp, index): each lane ranks its own slots
  int n_free = 0;
#pragma unroll
  for (int u = 0; u < SPL; ++u)
    if (u * WAVE < S) n_free += __popcll(__ballot(!myhit[u] && u * WAVE + lane < S));
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    if (u * WAVE >= S) break;
    const int j = u * WAVE + lane;
    int rank = 0;
#pragma unroll
    for (int u2 = 0; u2 < SPL; ++u2) {
      if (u2 * WAVE >= S) break;
      for (int l2 = 0; l2 < WAVE; ++l2) {
        const int s2 = __shfl(mys[u2], l2, WAVE);
        const bool f2 = __shfl((int)!myhit[u2], l2, WAVE) != 0;
        const int j2 = u2 * WAVE + l2;
        rank += (j2 < S && f2 && (s2 < mys[u] || (s2 == mys[u] && j2 < j))) ? 1 : 0;
      }
    }
    if (j < S && !myhit[u]) by_rank[rank] = j;
    if (j < S) {
      ch[j] = myc[u];
      stp[j] = myhit[u] ? t : mys[u];
    }
  }
  wave_lds_fence();
  // misses, in ascending chunk order, take the free slots in rank order
  int before = 0;
  for (int i0 = 0; i0 < k; i0 += WAVE) {
    const int i = i0 + lane;
    const bool miss = i < k && !held[i];
    const uint64_t mm = __ballot(miss);
    const int m = before + __popcll(mm & lanemask_lt());
    if (miss) {
      const int v = m < n_free ? by_rank[m] : -1;
      if (i >= q0 && i < q0 + MAXSLOT) codeL[i - q0] = v;
      if (v >= 0) {
        ch[v] = selAll[i];
        stp[v] = t;
      }
    }
    before += __popcll(mm);
  }
  wave_lds_fence();
  if (write) {
    for (int j = lane; j < S; j += WAVE) {
      chunk_out[j] = ch[j];
      stamp_out[j] = stp[j];
    }
    if (lane == 0 && hits_out) *hits_out = hits;
  }
}

template <typename TC, int NR, int NF, bool REUSE>
__global__ __launch_bounds__(NTH, 1) void k_attend_chain(const AttendArgs a) {
  static_assert(NR % NU == 0, "the basis register ring must divide the k-step count");
  static_assert(NR >= 4, "step 1 needs at least four k-steps");
  constexpr int F = NF * 16;
  constexpr int TILE_W = KA_W;
  constexpr bool I8 = sizeof(TC) == 1;
  using S = Smem<F, NR * KS>;
  using CT = Coef<TC>;
  using ST = Slab<TC>;
  extern __shared__ __align__(16) unsigned char sm[];
  uint16_t *W1s = reinterpret_cast<uint16_t *>(sm + S::W1S);
  uint16_t *Us = reinterpret_cast<uint16_t *>(sm + S::US);
  uint16_t *Qs = reinterpret_cast<uint16_t *>(sm + S::QS);
  float *B1s = reinterpret_cast<float *>(sm + S::B1);
  float *Ps = reinterpret_cast<float *>(sm + S::PS);
  uint16_t *Tk = reinterpret_cast<uint16_t *>(sm + S::TK);
  uint16_t *Tv = reinterpret_cast<uint16_t *>(sm + S::TV);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile offsets stay scalar
  const int l16 = lane & 15, kg = lane >> 4;
  float *AHw = reinterpret_cast<float *>(sm + S::AH) + w * F * GQ;  // this wave's running accH, [f][g]
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
  const rsrc_t Ir = make_rsrc(ridx, (uint32_t)a.n_res * 4u);
  const TC *rval = reinterpret_cast<const TC *>(a.res_val) + bh * (long)a.n_res * DH;
  const rsrc_t Rr = make_rsrc(rval, (uint32_t)((long)a.n_res * DH * Res<TC>::ES));
  const int32_t *selp = a.sel + ((long)b * a.Hkv + h) * a.k_eff;

  constexpr int cpt = CPT;                     // tiles per chunk (C == 128)
  const int n_tiles = a.k_eff * cpt;           // tiles of this (b, h)
  const int t_begin = s * a.tps;
  const int t_end = min(n_tiles, t_begin + a.tps);
  const int iters = (a.tps + NW - 1) / NW;

  // ---- prologue -------------------------------------------------------------
  int32_t *selL = reinterpret_cast<int32_t *>(sm + S::SEL);   // chunks of this split's slots
  const int q0 = t_begin / cpt;                                 // first slot of this split
  auto tile_row = [&](int tau) -> long {
    const int j = selL[tau / cpt - q0];
    return (long)j * C + (long)(tau % cpt) * TT;
  };
  const int tau0 = t_begin + w;
  long row0 = (long)a.N;  // set once the selection is known; a wave without a tile reads out of range
  auto c_soff = [&](int tt, int q) -> uint32_t {  // scalar offset of k-step q of token tile tt
    return (uint32_t)(((row0 + 16 * tt) * r + q * KS) * CT::ES);
  };
  // the selection inputs are read first.  A chunk's score is its rank blocks'
  // partials summed in block order; the sum is taken only after every other
  // prologue load is issued, so that their round trips overlap.
  static_assert(CHAIN_SELECT_MAX_NC <= NTH, "one chunk score per thread");
  const int n_c = a.N / C;
  constexpr int NRB = NR * KS / 64;
  static_assert(NR * KS % 64 == 0, "whole rank blocks");
  double spv[NRB];
#pragma unroll
  for (int k = 0; k < NRB; ++k) spv[k] = 0.0;
  int selv = 0;
  if (a.score_part) {
    if (tid < n_c) {
      const double *sp = a.score_part + ((long)b * a.Hkv + h) * NRB * n_c + tid;
#pragma unroll
      for (int k = 0; k < NRB; ++k) spv[k] = sp[(long)k * n_c];
    }
  } else if (tid < MAXSLOT && q0 + tid < a.k_eff) {
    selv = selp[q0 + tid];
  }
  const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
  const u32x4 qraw = tid < g * (DH / 8) ? gld16(qb + 8 * tid) : v4(0, 0, 0, 0);
  const u32x4 braw = tid < F / 8 ? gld16(B1 + 8 * tid) : v4(0, 0, 0, 0);
  // tail share of this split: tokens [tb, te); its first TP rows are staged now
  const int tb = min(a.T, s * a.tail_per_split), te = min(a.T, tb + a.tail_per_split);
  const long tail_base = ((((long)b * a.G + a.layer) * a.Hkv + h) * a.T) * DH;
  const uint16_t *kt = reinterpret_cast<const uint16_t *>(a.k_tail) + tail_base;
  const uint16_t *vt = reinterpret_cast<const uint16_t *>(a.v_tail) + tail_base;
  constexpr int TPP = TP * (DH / 8) / NTH;   // tail pieces per thread
  u32x4 tkr[TPP], tvr[TPP];
#pragma unroll
  for (int i = 0; i < TPP; ++i) {
    const int p = tid + NTH * i, row = p >> 4, c8 = (p & 15) * 8;
    tkr[i] = v4(0, 0, 0, 0);
    tvr[i] = v4(0, 0, 0, 0);
    if (tb + row < te) {
      tkr[i] = gld16(kt + (long)(tb + row) * DH + c8);
      tvr[i] = gld16(vt + (long)(tb + row) * DH + c8);
    }
  }

  // U^T q_g of the kv head's query heads (fp32, from the select stage), split
  // by waves 1..NW-1 into MFMA halves below: all of a thread's values are
  // loaded here at once (wave 0 and spare items read past the end: zeros)
  constexpr int W1T = NTH - WAVE;                             // threads of waves 1..NW-1
  constexpr int QTP = (GQ * NR * KS + W1T - 1) / W1T;         // q~ values per such thread
  static_assert(QTG_G == GQ, "q~ rows per kv head");
  const int tw = tid - WAVE;
  float qtv[QTP];
  uint16_t qts[QTP];  // int8 codes: the rank scale of each value
  {
    const rsrc_t Qr = make_rsrc(a.qtg + ((long)b * a.Hkv + h) * QTG_G * r, (uint32_t)(GQ * r * 4));
#pragma unroll
    for (int k = 0; k < QTP; ++k) {
      const int i = tw + W1T * k;
      const bool ok = w != 0 && i < GQ * r;
      qtv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(Qr, ok ? 4u * (uint32_t)i : 0x80000000u, 0u, 0));
    }
    if constexpr (I8) {
      const rsrc_t Sr = make_rsrc(csc, (uint32_t)(r * 2));
#pragma unroll
      for (int k = 0; k < QTP; ++k) {
        const int i = tw + W1T * k;
        const bool ok = w != 0 && i < GQ * r;
        qts[k] = __builtin_amdgcn_raw_buffer_load_b16(Sr, ok ? 2u * (uint32_t)(i % r) : 0x80000000u, 0u, 0);
      }
    }
  }

  u32x4 ur[NU][SP], us_[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
#pragma unroll
    for (int i = 0; i < SP; ++i) ur[k][i] = v4(0, 0, 0, 0);
    us_[k] = v4(0, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < LU; ++q) ST::ld(Ur, csc, u_voff, r, q * KS, ur[q % NU], us_[q % NU]);
  // W1 is read and converted by waves 1..NW-1 while wave 0 selects.  These
  // loads and the basis slabs' are issued after the scores, q and the tail
  // rows, which the first barrier waits for: loads complete in issue order, and
  // the W1 loads are unconditional (wave 0 and spare pieces read past the end:
  // zeros, no memory traffic) so that the waits before the barrier need not
  // cover them.
  constexpr int W1N = F * DH / 8;                             // 16-byte W1 pieces
  constexpr int W1P = (W1N + W1T - 1) / W1T;                  // pieces per such thread
  const rsrc_t W1r = make_rsrc(W1, (uint32_t)(F * DH * 2));
  u32x4 w1r[W1P];
#pragma unroll
  for (int k = 0; k < W1P; ++k) {
    const int p = tw + W1T * k;  // W1 rows are contiguous: piece p starts at byte 16 p
    w1r[k] = bld16(W1r, (w != 0 && p < W1N) ? 16u * (uint32_t)p : 0x80000000u, 0u);
  }
  // q rows of this kv head as fp16 with permuted dims (rows g..15 zero), and the
  // tail rows: both are read while wave 0 selects
  for (int i = tid; i < (16 - g) * (DH / 2); i += NTH)
    reinterpret_cast<uint32_t *>(Qs)[(g + i / (DH / 2)) * (WLD / 2) + i % (DH / 2)] = 0u;
  if (tid < g * (DH / 8)) {
    const int gi = tid / (DH / 8), d0 = 8 * (tid % (DH / 8));
    const uint2 lo = make_uint2(pack2(bf16_bits_to_f32(qraw.x & 0xFFFFu), bf16_bits_to_f32(qraw.x >> 16)),
                                pack2(bf16_bits_to_f32(qraw.y & 0xFFFFu), bf16_bits_to_f32(qraw.y >> 16)));
    const uint2 hi = make_uint2(pack2(bf16_bits_to_f32(qraw.z & 0xFFFFu), bf16_bits_to_f32(qraw.z >> 16)),
                                pack2(bf16_bits_to_f32(qraw.w & 0xFFFFu), bf16_bits_to_f32(qraw.w >> 16)));
    *reinterpret_cast<uint2 *>(Qs + gi * WLD + dpos(d0)) = lo;
    *reinterpret_cast<uint2 *>(Qs + gi * WLD + dpos(d0 + 4)) = hi;
  }
#pragma unroll
  for (int i = 0; i < TPP; ++i) {
    const int p = tid + NTH * i, row = p >> 4, c8 = (p & 15) * 8;
    lst16(Tk + row * DH + c8, tkr[i]);
    lst16(Tv + row * DH + c8, tvr[i]);
  }
  // per-wave softmax state: lane holds query head l16 (rows >= g are padding)
  float m_run = -INFINITY, l_run = 0.f;
  float accV[GQ][2];
#pragma unroll
  for (int i = 0; i < GQ; ++i) accV[i][0] = accV[i][1] = 0.f;
  // tail part of l per wave and query head, with the running maximum it is
  // relative to; the merge brings it to the wave's final maximum
  float *tl_l = reinterpret_cast<float *>(sm + S::TLS), *tl_m = tl_l + NW * GQ;
  // ---- chunk selection of (b, h): the top k_eff chunks by (score desc, index
  // asc), in ascending index order.  With the scores at hand every workgroup
  // selects them itself, on wave 0 (wave_topk); split 0 also writes the whole
  // selection to sel_out.  The other waves attend the tail meanwhile.
  double *scL = reinterpret_cast<double *>(sm + S::PS);
  if (a.score_part && tid < n_c) {
    double scv = spv[0];
#pragma unroll
    for (int k = 1; k < NRB; ++k) scv += spv[k];
    scL[tid] = scv;
  }
  __syncthreads();
  if (w == 0) {
    if (a.score_part) {
      // NSL key slots per lane: four while n_c <= 256, so that no count spends
      // compares and popcounts on empty slots
      auto emit = [&](int pos, int c) {
        if (pos >= q0 && pos < q0 + MAXSLOT) selL[pos - q0] = c;
        if constexpr (REUSE) reinterpret_cast<int32_t *>(sm + S::SELALL)[pos] = c;
        if (s == 0 && a.sel_out) a.sel_out[((long)b * a.Hkv + h) * a.k_eff + pos] = c;
      };
      static_assert(CHAIN_SELECT_MAX_NC % (4 * WAVE) == 0, "slot counts");
      if (n_c <= 4 * WAVE)
        wave_topk<4>(scL, n_c, a.k_eff, emit);
      else
        wave_topk<CHAIN_SELECT_MAX_NC / WAVE>(scL, n_c, a.k_eff, emit);
    } else if (tid < MAXSLOT && q0 + tid < a.k_eff) {
      selL[tid] = selv;
    }
    if constexpr (REUSE) {  // slots of this step's chunks (every split decides the same)
      int32_t *selAll = reinterpret_cast<int32_t *>(sm + S::SELALL);
      if (!a.score_part)
        for (int i = lane; i < a.k_eff; i += WAVE) selAll[i] = selp[i];
      wave_lds_fence();
      const long trow = ((long)b * a.G + a.layer) * a.Hkv + h;
      const int clk = a.rclock[trow], half = clk & 1;
      const long tin = (trow * 2 + half) * a.rslots, tout = (trow * 2 + (half ^ 1)) * a.rslots;
      reuse_assign_wave(selAll, a.k_eff, a.rt_chunk + tin, a.rt_stamp + tin, a.rt_chunk + tout,
                        a.rt_stamp + tout, a.rslots, clk + 1, reinterpret_cast<int32_t *>(sm + S::AH),
                        reinterpret_cast<int32_t *>(sm + S::RCODE), q0, s == 0,
                        a.rhits ? a.rhits + (long)b * a.Hkv + h : nullptr);
    }
    if (lane < GQ) {  // wave 0 attends no tail tokens
      tl_l[lane] = 0.f;
      tl_m[lane] = -INFINITY;
    }
  } else {
    // W1 -> fp16, head dims permuted (two 4-dim runs per piece)
#pragma unroll
    for (int k = 0; k < W1P; ++k) {
      const int p = tw + W1T * k, f = p / (DH / 8), d0 = 8 * (p % (DH / 8));
      if (p >= W1N) break;
      const u32x4 v = w1r[k];
      auto sc = [](uint32_t u) { return bf16_bits_to_f32(u) * NEG_LOG2E; };
      const uint2 lo = make_uint2(pack2(sc(v.x & 0xFFFFu), sc(v.x >> 16)), pack2(sc(v.y & 0xFFFFu), sc(v.y >> 16)));
      const uint2 hi = make_uint2(pack2(sc(v.z & 0xFFFFu), sc(v.z >> 16)), pack2(sc(v.w & 0xFFFFu), sc(v.w >> 16)));
      *reinterpret_cast<uint2 *>(W1s + f * WLD + dpos(d0)) = lo;
      *reinterpret_cast<uint2 *>(W1s + f * WLD + dpos(d0 + 4)) = hi;
    }
    {
      // Logits are taken in coefficient space: q_g . k_hat_t = sum_r
      // (U^T q_g)_r s_r c_t,r with the stored coefficients c (bf16 as stored;
      // int8 codes, exact in fp16, with their rank scales s; s = 1 for bf16).
      // x = (U^T q_g)_r s_r (U^T q_g in float32 from the select stage) is split
      // into a hi part in the codes' MFMA type and the rounding of the
      // remainder, so a logit carries the fp32 product to about 2^-16 (bf16) or
      // 2^-22 (fp16) relative: a key rebuilt and rounded to fp16 would move
      // logits in the hundreds by ~0.1.
      uint16_t *qsh = reinterpret_cast<uint16_t *>(sm + S::QSC), *qsl = qsh + GQ * r;
#pragma unroll
      for (int k = 0; k < QTP; ++k) {
        const int i = tw + W1T * k;
        if (i >= GQ * r) break;
        const int gi = i / r;
        const float v = gi < g ? qtv[k] * (I8 ? f16_bits_to_f32(qts[k]) : 1.f) : 0.f;
        uint16_t hi, lo;
        if constexpr (I8) {
          const _Float16 hv = (_Float16)v;
          hi = __builtin_bit_cast(uint16_t, hv);
          lo = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)hv));
        } else {
          hi = f32_to_bf16_bits(v);
          lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
        }
        qsh[i] = hi;
        qsl[i] = lo;
      }
    }
    // ---- the split's share of the uncompressed tail, attended while wave 0
    // selects: wave w takes tokens tb + w - 1, tb + w - 1 + (NW - 1), ..., two
    // at a time, logits and p . v on the vector ALUs (lane: head dims 2 lane,
    // 2 lane + 1).  The eight partial logits of a pair (token u, head gi) are
    // summed over the wave by a transposing butterfly.  Nothing has been added
    // to the hidden sums yet, so the tiles' rescaling covers everything.
    constexpr int NTW = NW - 1;  // tail waves
    float l_t = 0.f;             // partials over the lane groups kg, like l_run
    float qd[GQ][2];  // q of the kv head's query heads at the lane's dims (fp16 values)
#pragma unroll
    for (int gi = 0; gi < GQ; ++gi) {
      const uint32_t qq = *reinterpret_cast<const uint32_t *>(Qs + gi * WLD + dpos(2 * lane));
      qd[gi][0] = f16_bits_to_f32(qq & 0xFFFFu);
      qd[gi][1] = f16_bits_to_f32(qq >> 16);
    }
    auto row = [&](const uint16_t *lds, const uint16_t *glb, int t, float &x0, float &x1) {
      const int tl = t - tb;
      const uint32_t v2 = tl < TP ? *reinterpret_cast<const uint32_t *>(lds + tl * DH + 2 * lane)
                                  : *reinterpret_cast<const uint32_t *>(glb + (long)t * DH + 2 * lane);
      x0 = bf16_bits_to_f32(v2 & 0xFFFFu);
      x1 = bf16_bits_to_f32(v2 >> 16);
    };
    for (int t0 = tb + w - 1; t0 < te; t0 += 2 * NTW) {
      const bool two = t0 + NTW < te;
      float k0[2][2], v0[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = u == 0 || two ? t0 + NTW * u : t0;
        row(Tk, kt, t, k0[u][0], k0[u][1]);
        row(Tv, vt, t, v0[u][0], v0[u][1]);
      }
      float pl[2 * GQ];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int gi = 0; gi < GQ; ++gi) pl[GQ * u + gi] = fmaf(qd[gi][0], k0[u][0], qd[gi][1] * k0[u][1]);
      // lane l ends with the logit of pair (l >> 3): token (l >> 5), head (l >> 3) & 3
      const float lsum = xpose_sum_f<2 * GQ, 32>(pl, lane);
      const int hq = l16 & (GQ - 1);  // this lane's head (lanes past g are padding)
      float lt2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) lt2[u] = __shfl(lsum, 32 * u + 8 * hq, 64) * a.scale_log2;
      if (!two) lt2[1] = -INFINITY;
      const float m_new = fmaxf(m_run, fmaxf(lt2[0], lt2[1]));
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float p2[2], ps = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        p2[u] = lt2[u] == -INFINITY ? 0.f : (float)(_Float16)__builtin_amdgcn_exp2f(lt2[u] - m_new);
        ps += p2[u];
      }
      l_t = l_t * alpha + (kg == 0 ? ps : 0.f);
      m_run = m_new;
#pragma unroll
      for (int gi = 0; gi < GQ; ++gi) {
        const float av = __shfl(alpha, gi, 64);
        const float pa = __shfl(p2[0], gi, 64), pb = __shfl(p2[1], gi, 64);
        accV[gi][0] = fmaf(pb, v0[1][0], fmaf(pa, v0[0][0], accV[gi][0] * av));
        accV[gi][1] = fmaf(pb, v0[1][1], fmaf(pa, v0[0][1], accV[gi][1] * av));
      }
    }
    l_t += __shfl_xor(l_t, 16, 64);
    l_t += __shfl_xor(l_t, 32, 64);
    if (lane < GQ) {
      tl_l[w * GQ + lane] = l_t;
      tl_m[w * GQ + lane] = m_run;
    }
  }
  __syncthreads();
  if (tau0 < t_end) row0 = tile_row(tau0);
  typename CT::raw cr[DC][NTT];
#pragma unroll
  for (int q = 0; q < DC - 1; ++q)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) cr[q][tt] = CT::ld(Cr, c_voff, c_soff(tt, q));

  if (tid < F / 8) {
    float *bo = B1s + 8 * tid;
    auto sc = [](uint32_t u) { return bf16_bits_to_f32(u) * NEG_LOG2E; };
    *reinterpret_cast<f32x4 *>(bo) = f32x4{sc(braw.x & 0xFFFFu), sc(braw.x >> 16), sc(braw.y & 0xFFFFu), sc(braw.y >> 16)};
    *reinterpret_cast<f32x4 *>(bo + 4) = f32x4{sc(braw.z & 0xFFFFu), sc(braw.z >> 16), sc(braw.w & 0xFFFFu), sc(braw.w >> 16)};
  }
  // the wave's running accH starts at zero (a wave without a tile leaves it so)
#pragma unroll
  for (int i = 0; i < F * GQ / (4 * WAVE); ++i)
    *reinterpret_cast<f32x4 *>(AHw + 4 * (lane + WAVE * i)) = f32x4{0.f, 0.f, 0.f, 0.f};
  ST::st(Us, ur[0], us_[0]);   // slab 0 -> buffer 0
  __syncthreads();

  float rs0 = 1.f, rs1 = 1.f;  // int8 residual scales of the lane's two dims
  if (sizeof(TC) == 1 && a.res_scale) {
    const uint16_t *rsc = a.res_scale + bh * DH;
    rs0 = f16_bits_to_f32(rsc[2 * lane]);
    rs1 = f16_bits_to_f32(rsc[2 * lane + 1]);
  }
  // accV += p[g][t] row[t] for this wave's p in Ps and rows of d_h values
  // (lane: dims 2 lane, 2 lane + 1)
  static_assert(GQ == 4, "p rows are read as one 16-byte vector");
  auto add_row = [&](int t, float d0, float d1) {
    const f32x4 pv = *reinterpret_cast<const f32x4 *>(Ps + (w * TT + t) * GQ);
#pragma unroll
    for (int gi = 0; gi < GQ; ++gi) {
      accV[gi][0] = fmaf(pv[gi], d0, accV[gi][0]);
      accV[gi][1] = fmaf(pv[gi], d1, accV[gi][1]);
    }
  };
  auto wave_lds_sync = []() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Restart of the coefficient and basis pipelines for iteration it_next: issued
  // on every path at the end of an iteration (also after the last one, where the
  // coefficient reads fall out of range), so that the registers carried around
  // the loop always hold fresh loads and nothing of step 1 stays live through
  // the softmax and hidden phases.
  auto restart = [&](int it_next) {
    const int tau_n = t_begin + w + NW * it_next;
    row0 = tau_n < t_end ? tile_row(tau_n) : (long)a.N;
#pragma unroll
    for (int q = 0; q < DC - 1; ++q)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) cr[q][tt] = CT::ld(Cr, c_voff, c_soff(tt, q));
#pragma unroll
    for (int q = 0; q < LU; ++q) ST::ld(Ur, csc, u_voff, r, q * KS, ur[q % NU], us_[q % NU]);
  };

  for (int it = 0; it < iters; ++it) {
    const int tau = t_begin + w + NW * it;
    const bool has = tau < t_end;
    if (it > 0) {
      ST::st(Us, ur[0], us_[0]);   // slab 0 -> buffer 0 (last read two barriers ago)
      __syncthreads();
    }
    // this tile's residual rows: CSR range of the chunk (loads issued here, read
    // late in step 1), then the tile's part of it
    const int jc = has ? (int)(row0 >> 7) : 0;  // 128-token chunks
    static_assert(CPT * TT == 128, "chunk index by shift");
    const int e0r = rptr[jc], e1r = rptr[jc + 1];
    int e0 = 0, e1 = 0;
    constexpr int RM = CPT * TT / WAVE;         // chunk entries per lane (C <= 64 RM)
    int rtok[RM];                              // token of entries e0 + lane + 64m (raw)
#pragma unroll
    for (int m = 0; m < RM; ++m) rtok[m] = 0;
    int r_lo = 0, r_n = 0;                     // first row and count of this tile's rows
    typename Res<TC>::raw dr[RP];

    // residual entries of the chunk: their tokens (issued two k-steps before the
    // end of step 1), then the tile's rows (issued after step 1, read after the
    // softmax)
    auto res_tokens = [&]() {
      e0 = has ? e0r : 0;
      e1 = has ? e1r : 0;
      const int cnt = e1 - e0;
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        const int i = lane + 64 * m;
        rtok[m] = (int)__builtin_amdgcn_raw_buffer_load_b32(Ir, 4u * (uint32_t)(i < cnt ? e0 + i : a.n_res), 0u, 0);
      }
    };
    auto res_rows = [&]() {  // this tile's rows: a contiguous run of the chunk's
      const int cnt = e1 - e0;
      int below = 0, inside = 0;
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        const bool valid = lane + 64 * m < cnt;
        rtok[m] -= (int)row0;  // token within the tile
        below += __popcll(__ballot(valid && rtok[m] < 0));
        inside += __popcll(__ballot(valid && rtok[m] >= 0 && rtok[m] < TT));
      }
      r_lo = e0 + below;
      r_n = inside;
#pragma unroll
      for (int k = 0; k < RP; ++k) dr[k] = Res<TC>::ld(Rr, k < r_n ? r_lo + k : a.n_res, lane);
    };

    // reuse: the slot code of this tile's chunk (wave-uniform; read again after
    // step 1 so that nothing of it stays live there).  A wave whose tile hits
    // skips its step-1 products and coefficient loads and reads its rebuilt keys
    // back; the basis slabs are shared, so only a workgroup whose tiles all hit
    // skips their loads too.
    auto slot_code = [&]() -> int {
      return has ? reinterpret_cast<const int32_t *>(sm + S::RCODE)[tau / cpt - q0] : -1;
    };
    bool skip1 = false, skip_all = false;
    if constexpr (REUSE) {
      const int code = slot_code();
      const bool hit = !has || (code >= 0 && (code & REUSE_HIT) != 0);
      skip1 = __builtin_amdgcn_readfirstlane((int)hit) != 0;
      skip_all = __syncthreads_and(hit);
    } else {
      // always false, but opaque: each k-step's products then sit behind a
      // branch, which keeps the scheduler from stretching register lifetimes
      // across k-steps (the unbranched form spills)
      int sk = 0;
      asm volatile("" : "+s"(sk));
      skip1 = sk != 0;
    }
    // coefficient loads are never skipped: the logits come from them
    (void)skip1;
    const uint32_t uskip = skip_all ? 0x80000000u : 0u;

    // logits[t][g] of the tile (int8: accumulated during step 1)
    f32x4 lg[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) lg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // ---- step 1: K_hat^T = U . C^T over NR k-steps ------------------------
    const uint16_t *u_rd = Us + l16 * ULD + 8 * kg;  // lane's basis fragment, head-dim tile 0
    f32x4 acc[NDT][NTT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) acc[dt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    sfor<NR>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      __builtin_amdgcn_sched_barrier(0);  // keep each k-step's loads and MFMAs in place
      // basis slab ks + LU into the ring; issued before this step's coefficient
      // loads so that waiting for it LU - 1 steps later waits for nothing newer
      // than the coefficients then due
      if constexpr (ks + LU < NR)
        ST::ld(Ur, csc, u_voff, r, (ks + LU) * KS, ur[(ks + LU) % NU], us_[(ks + LU) % NU], uskip);
      // coefficients DC - 1 steps ahead.
      // Every load here is unconditional (a wave without a tile reads out of
      // range), so the wait counts stay exact across steps; a wave whose tile
      // is read back (reuse) points them past the end (zeros, no memory
      // traffic) and skips the products.
      if constexpr (ks + DC - 1 < NR) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) cr[(ks + DC - 1) % DC][tt] = CT::ld(Cr, c_voff, c_soff(tt, ks + DC - 1));
      }
      if constexpr (ks == NR - 3) res_tokens();
      __builtin_amdgcn_sched_barrier(0);  // this step's loads go out before its MFMAs
      // basis slab ks + 1 -> LDS (its load was issued LU - 1 steps ago)
      if constexpr (ks + 1 < NR) ST::st(Us + ((ks + 1) & 1) * DH * ULD, ur[(ks + 1) % NU], us_[(ks + 1) % NU]);
      {  // logits from the coefficients: B operand column l16 < GQ is q~ hi of
         // head l16, column GQ + g' its lo part; the two are added after step 1
        const uint16_t *qsb = reinterpret_cast<const uint16_t *>(sm + S::QSC) + l16 * r + ks * KS + 8 * kg;
        typedef typename CT::op OP;
        const OP qhl = l16 < 2 * GQ ? __builtin_bit_cast(OP, lds16(qsb)) : __builtin_bit_cast(OP, v4(0, 0, 0, 0));
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) lg[tt] = mfma(CT::get(cr[ks % DC][tt]), qhl, lg[tt]);
      }
      if (!skip1) {  // basis fragments one head-dim tile ahead of the MFMAs that use them
        const uint16_t *ub = u_rd + (ks & 1) * DH * ULD;
        typename CT::op bc[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) bc[tt] = CT::get(cr[ks % DC][tt]);
        typename ST::op au[2];
        au[0] = ST::get(ub);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          if (dt + 1 < NDT) au[(dt + 1) & 1] = ST::get(ub + 16 * (dt + 1) * ULD);
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) acc[dt][tt] = mfma(au[dt & 1], bc[tt], acc[dt][tt]);
        }
      }
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    });
    // this tile's residual rows: issued now, read after the softmax (their
    // registers are not held through step 1)
    res_rows();
    if (!has) {
      restart(it + 1);
      continue;
    }

    // ---- rebuilt keys as fp16 A operands --------------------------------------
    int rslot = -1;
    bool rhit = false;
    const u32x4 *rtile = nullptr;
    if constexpr (REUSE) {
      const int code = slot_code();
      rhit = code >= 0 && (code & REUSE_HIT) != 0;
      rslot = code < 0 ? -1 : (code & ~REUSE_HIT);
      if (rslot >= 0)
        rtile = reinterpret_cast<const u32x4 *>(a.rtiles) +
                ((((long)b * a.G + a.layer) * a.Hkv + h) * a.rslots + rslot) * (long)(CPT * TILE_W) +
                (long)(tau % cpt) * TILE_W;
    }
    // ---- rebuilt keys as fp16 A operands of the hidden layer (the logits were
    // taken during step 1)
    f16x8 KA[NJ][NTT];
    if (skip1) {  // this wave's tile is cached: the operands as stored
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
          KA[jj][tt] = __builtin_bit_cast(f16x8, rtile[(jj * NTT + tt) * WAVE + lane]);
    } else {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            KA[jj][tt][v] = (_Float16)acc[2 * jj][tt][v];
            KA[jj][tt][4 + v] = (_Float16)acc[2 * jj + 1][tt][v];
          }
      if (REUSE && rslot >= 0 && !rhit) {
        u32x4 *wt = const_cast<u32x4 *>(rtile);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) wt[(jj * NTT + tt) * WAVE + lane] = __builtin_bit_cast(u32x4, KA[jj][tt]);
      }
    }
    // logit of head g (lane l16 = g < GQ): hi column plus the lo column GQ + g
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) lg[tt][v] += __shfl_down(lg[tt][v], GQ, 16);
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
        const _Float16 p = (_Float16)__builtin_amdgcn_exp2f(lg[tt][v] - m_new);
        PA[tt >> 1][4 * (tt & 1) + v] = p;
        lg[tt][v] = (float)p;
        psum += (float)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // p of this tile for the residual pass: Ps[w][t][g]
    if (l16 < GQ) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) Ps[(w * TT + 16 * tt + 4 * kg + v) * GQ + l16] = lg[tt][v];
    }
    // rescale the running sums: accV here, accH (rows g = v of lanes 0..15)
    // when this tile's hidden sums are folded into LDS
    float ah[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) ah[v] = __shfl(alpha, v, 64);
#pragma unroll
    for (int gi = 0; gi < GQ; ++gi) {
      const float av = __shfl(alpha, gi, 64);
      accV[gi][0] *= av;
      accV[gi][1] *= av;
    }

    // ---- step 5: residual rows (vector ALUs) -------------------------------------
    // Branch-free over the RP rows held in registers: rows past r_n were read
    // out of range as zeros and add nothing, so every p read can be batched.
    wave_lds_sync();
    {
      const int below = r_lo - e0;
#pragma unroll
      for (int k = 0; k < RP; ++k) {
        const int pos = below + k;
        const int tsel = pos < 64 ? rtok[0] : rtok[1];
        const int t = min(max(__shfl(tsel, pos & 63, 64), 0), TT - 1);
        float d0, d1;
        Res<TC>::get(dr[k], rs0, rs1, d0, d1);
        add_row(t, d0, d1);
      }
      for (int k = RP; k < r_n; ++k) {  // rare: more than RP rows in the tile
        const int pos = below + k;
        const int tsel = pos < 64 ? rtok[0] : rtok[1];
        const int t = __shfl(tsel, pos & 63, 64);
        float d0, d1;
        Res<TC>::get(Res<TC>::ld(Rr, r_lo + k, lane), rs0, rs1, d0, d1);
        add_row(t, d0, d1);
      }
    }

    // ---- steps 3 and 4 per 16-wide hidden tile ------------------------------------
    // accH[g][f] of this tile: lane holds column f = 16 fi + l16, rows g = 4 kg + v;
    // each hidden tile is folded into the wave's running accH in LDS right away
    // (the real rows g < GQ live in lanes 0..15, whose four values are one
    // 16-byte word of the [f][g] layout, read before the products that update
    // it).  The running accH starts at zero and the first tile's rescale factor
    // is zero, so the fold needs no first-tile case.  Software-pipelined: the
    // W1 products of tile fi + 1 are issued before the SiLU of tile fi, so the
    // matrix cores work while the vector ALUs evaluate SiLU.
    // Lane offsets of the hidden phase are formed here, in every tile, from an
    // offset the compiler cannot see through: hoisted out of the tile loop
    // they would be held through step 1, where no register is left for them.
    int hl = lane;
    asm volatile("" : "+v"(hl));
    const int hl16 = hl & 15, hkg = hl >> 4;
    const uint16_t *w1_rd = W1s + hl16 * WLD + 8 * hkg;   // + 16 fi WLD + 32 jj
    const float *b1_rd = B1s + hl16;
    f32x4 *ah_rw = reinterpret_cast<f32x4 *>(AHw) + hl16;  // + 16 fi
    const f32x4 ahv = f32x4{ah[0], ah[1], ah[2], ah[3]};
    // W1 fragments and b1 of a hidden tile are read from LDS one tile before
    // the products that use them; both buffers are indexed by the tile's
    // parity, a constant in the unrolled loop, so nothing is copied
    f16x8 bw[2][NJ];
    float bias[2];
    auto load_w1 = [&](int fi) {
      bias[fi & 1] = b1_rd[16 * fi];
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) bw[fi & 1][jj] = ldh8(w1_rd + 16 * fi * WLD + 32 * jj);
    };
    f32x4 hc[2][NTT];
    auto hidden_mfma = [&](int fi) {
      const float bv = bias[fi & 1];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) hc[fi & 1][tt] = f32x4{bv, bv, bv, bv};
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)  // head-dim step outer: four independent chains
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) hc[fi & 1][tt] = mfma(KA[jj][tt], bw[fi & 1][jj], hc[fi & 1][tt]);
    };
    load_w1(0);
    if (NF > 1) load_w1(1);
    hidden_mfma(0);
#pragma unroll
    for (int fi = 0; fi < NF; ++fi) {
      f32x4 prev = f32x4{0.f, 0.f, 0.f, 0.f};
      if (kg == 0) prev = ah_rw[16 * fi];
      if (fi + 1 < NF) hidden_mfma(fi + 1);
      if (fi + 2 < NF) load_w1(fi + 2);
      f32x4 ahc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NTT / 2; ++i) {
        f16x8 hb;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hb[v] = (_Float16)silu_scaled(hc[fi & 1][2 * i][v]);
          hb[4 + v] = (_Float16)silu_scaled(hc[fi & 1][2 * i + 1][v]);
        }
        ahc = mfma(PA[i], hb, ahc);
      }
      if (kg == 0)
        ah_rw[16 * fi] = f32x4{fmaf(prev[0], ahv[0], ahc[0]), fmaf(prev[1], ahv[1], ahc[1]),
                               fmaf(prev[2], ahv[2], ahc[2]), fmaf(prev[3], ahv[3], ahc[3])};
    }
    restart(it + 1);
  }

  // ---- merge the waves into one partial --------------------------------------------
  __syncthreads();  // W1 and the basis slabs are free from here
  float *mm = reinterpret_cast<float *>(sm + S::MM), *mlc = reinterpret_cast<float *>(sm + S::MLC);
  float *mlt = reinterpret_cast<float *>(sm + S::MLT);
  float *mv = reinterpret_cast<float *>(sm + S::MV);
  const float *AH = reinterpret_cast<const float *>(sm + S::AH);
  {
    float lc = l_run;
    lc += __shfl_xor(lc, 16, 64);
    lc += __shfl_xor(lc, 32, 64);
    if (lane < GQ) {
      const float lt = tl_l[w * GQ + lane];  // the tail's l, brought to this wave's final maximum
      mm[w * GQ + lane] = m_run;
      mlc[w * GQ + lane] = lc;
      mlt[w * GQ + lane] = lt == 0.f ? 0.f : lt * __builtin_amdgcn_exp2f(tl_m[w * GQ + lane] - m_run);
    }
    float *aw = mv + w * GQ * DH;
#pragma unroll
    for (int gi = 0; gi < GQ; ++gi)
      *reinterpret_cast<float2 *>(aw + gi * DH + 2 * lane) = make_float2(accV[gi][0], accV[gi][1]);
  }
  __syncthreads();
  float *part = a.part + (((long)b * a.Hkv + h) * a.n_split + s) * g * a.PW;
  // wave weights exp2(m_k - M) per query head, and the same times the rescale
  // the wave still owes its hidden sums; zero for padded heads
  float *mwt = reinterpret_cast<float *>(sm + S::MWT), *mwh = reinterpret_cast<float *>(sm + S::MWH);
  if (tid < NW * GQ) {
    const int k = tid / GQ, gi = tid % GQ;
    float M = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < NW; ++kk) M = fmaxf(M, mm[kk * GQ + gi]);
    const float mk = mm[k * GQ + gi];
    const float wt = (gi >= g || mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
    mwt[k * GQ + gi] = wt;
    mwh[k * GQ + gi] = wt * NEG_LN2;  // hidden sums were accumulated in -log2(e) units
    if (k == 0 && gi < g) part[(long)gi * a.PW + 0] = M;
  }
  __syncthreads();
  if (tid < g) {
    float L = 0.f, mass = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      L = fmaf(mwt[k * GQ + tid], mlc[k * GQ + tid] + mlt[k * GQ + tid], L);
      mass = fmaf(mwt[k * GQ + tid], mlc[k * GQ + tid], mass);
    }
    part[(long)tid * a.PW + 1] = L;
    part[(long)tid * a.PW + 2] = mass;
    part[(long)tid * a.PW + 3] = 0.f;
  }
  // items [0, F): hidden column f for every query head (one 16-byte [f][g] word
  // per wave); items [F, F + g DH / 4): four value dims of one query head
  for (int i = tid; i < F + g * (DH / 4); i += NTH) {
    if (i < F) {
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(AH + (k * F + i) * GQ);
        const f32x4 wh = *reinterpret_cast<const f32x4 *>(mwh + k * GQ);
#pragma unroll
        for (int gi = 0; gi < GQ; ++gi) v[gi] = fmaf(wh[gi], x[gi], v[gi]);
      }
#pragma unroll
      for (int gi = 0; gi < GQ; ++gi)
        if (gi < g) part[(long)gi * a.PW + 4 + i] = v[gi];
    } else {
      const int gi = (i - F) / (DH / 4), c4 = 4 * ((i - F) % (DH / 4));
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const float wt = mwt[k * GQ + gi];
        const f32x4 x = *reinterpret_cast<const f32x4 *>(mv + (k * GQ + gi) * DH + c4);
        v = f32x4{fmaf(wt, x[0], v[0]), fmaf(wt, x[1], v[1]), fmaf(wt, x[2], v[2]), fmaf(wt, x[3], v[3])};
      }
      *reinterpret_cast<f32x4 *>(part + (long)gi * a.PW + 4 + F + c4) = v;
    }
  }
}

template <typename TC, int NR, int NF, bool REUSE>
static hipError_t go(const AttendArgs &a, hipStream_t st) {
  const size_t smem = Smem<NF * 16, NR * KS>::BYTES;
  static const bool lds_ok = (allow_dynamic_lds(k_attend_chain<TC, NR, NF, REUSE>, smem), true);
  (void)lds_ok;
  hipLaunchKernelGGL((k_attend_chain<TC, NR, NF, REUSE>), dim3(a.B * a.Hkv * a.n_split), dim3(NTH), smem, st, a);
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
  if (iters > chain::MAXIT) iters = chain::MAXIT;
  tps = iters * chain::NW;
  n_split = (n_tiles + tps - 1) / tps;
  tail_per_split = (T + n_split - 1) / n_split;
}

hipError_t launch_attend_chain(int coeff, const AttendArgs &a, hipStream_t st) {
  const bool i8 = coeff == LOWRAM_I8;
#define X(r_, f_, t_)                                                              \
  if (a.r == r_ && a.F == f_ && i8 == (sizeof(t_) == 1))                           \
    return a.rtiles ? chain::go<t_, r_ / chain::KS, f_ / 16, true>(a, st)           \
                    : chain::go<t_, r_ / chain::KS, f_ / 16, false>(a, st);
  LOWRAM_CHAIN_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

size_t chain_tile_bytes(int) { return (size_t)chain::CPT * 16 * chain::KA_W; }

}  // namespace lowram
