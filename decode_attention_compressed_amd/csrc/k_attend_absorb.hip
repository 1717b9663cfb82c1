// Rebuild-and-attend at head dim 256 with the first predictor layer absorbed
// into the basis (gfx950, 16x16x32 MFMA, fp32 accumulate).
//
// With k_hat_t = U_{l,h} c_t, both products that read the rebuilt key are
// re-associated exactly:
//   logits   q_g . k_hat_t     = (U_{l,h}^T q_g) . c_t = q~_g . c_t
//   hidden   W1 k_hat_t + b1   = (W1 U_{l,h}) c_t + b1 = A c_t + b1
// so no key is ever rebuilt.  At d_h = 256, F = 512, r = 384 the hidden layer
// costs F r = 196608 MACs per token-head against d_h r + F d_h = 229376 for
// rebuilding the key first, and it is one GEMM with nothing between two
// products.  (At d_h = 128 the plain form is cheaper, which is why the chained
// kernel keeps it there.)
//
// k_select_absorb (the launch of the partial chunk scores, before the attend
// kernel) also forms, per (sequence, kv head) of the layer,
// A = -log2(e) W1 U_{l,h} (rounded to fp16 once; int8 caches fold the per-rank
// scale in) and q~_g = U_{l,h}^T q_g for the g query heads (fp32, split into
// an fp16 part and the fp16 rounding of the remainder).
//
// The attend kernel ranks the chunk scores itself in its prologue (wave 0,
// while the other waves stage A).
//
// k_attend_absorb: one workgroup of 4 waves (one per SIMD) per (sequence b,
// kv head h, split s, quarter q of F).  Its quarter of A (128 hidden units x r,
// 96 KB at r = 384) is copied into LDS once and stays there; a split is a run
// of 64-token slices of the chunks selected for h and a round gives one slice
// to each wave (256 tokens).  Per round, over the rank in 32-wide k-steps and
// without a barrier:
//   H^T[t][f] += C[t][r] A^T[r][f] on fp16 MFMAs: the wave's coefficient
//     fragments go straight from global memory into a register ring several
//     k-steps deep (bf16 coefficients are exact in fp16's range, int8 codes
//     always) and A's fragments are read from LDS (16-byte granules XOR-
//     swizzled by row, so the 16 rows of a fragment fall in distinct banks);
//     fp16 A (11 significant bits) keeps the hidden pre-activations at the
//     accuracy of an fp16 rebuilt key;
//   logits[t][g] += C[t][r] q~^T[r][g] with q~ as fp16 hi and lo parts in one
//     operand (columns 0..3 hi, 4..7 lo), so each logit carries the fp32 q~ to
//     about 2^-22 relative against exact coefficients.
// Then: a workgroup-wide online softmax per query head (p in fp16), SiLU of
// the hidden pre-activations (held in -log2(e) units: one exp2, one
// reciprocal), accH^T[g][f] += p^T H^T on the matrix cores, and the residual
// rows of the round's tokens on the vector ALUs (each quarter a quarter of the
// head dims, the rows' loads in flight under the p . H products).
// The four quarters compute the same logits bit for bit, so their softmax
// states agree; each writes its quarter of the hidden sums and of the value
// sums into the split's partial row and quarter 0 writes (m, l, mass).
// Quarters 1..3 then attend a third each of the split's share of the
// uncompressed tail into partial rows of their own (hidden sums zero), so the
// combine merges 4 n_split rows per (b, h).
//
// Method: keys as per-token coefficients on a group basis (zicq.com English
// summary, "Cross-Layer Low-Rank Key Compression"); values from the per-head
// predictor plus residuals of the worst tokens ("Core Mechanism"); only
// query-selected chunks are rebuilt (rit.work page, generation section);
// attention softmax(q K^T / sqrt(d_h)) V (OjaKV page, section 3).
#include <type_traits>

#include "attend_common.hpp"
#include "select_partial.hpp"

namespace lowram {
namespace absorb {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int DH = 256;          // head dim handled here
constexpr int FF = 512;          // predictor hidden width handled here
constexpr int NQ = 4;            // quarters of F (one workgroup each)
constexpr int FQ = FF / NQ;      // hidden units per workgroup (128)
constexpr int NW = 4;            // waves per workgroup
constexpr int NTH = NW * WAVE;
constexpr int TT = 64;           // tokens per wave slice
constexpr int RT = NW * TT;      // tokens per round
constexpr int NTT = TT / 16;     // 16-token blocks of a slice
constexpr int NFB = FQ / 16;     // 16-wide hidden blocks of a quarter
constexpr int KS = 32;           // ranks per k-step
constexpr int GQ = 4;            // query heads per kv head (at most)
// coefficient k-steps in the register ring (DC - 1 ahead; DC divides the
// k-step count, so the ring runs on across rounds); four fit the register
// file next to the accumulators without scratch (six measured slower)
template <int NK> constexpr int dc_of() { return 4; }
constexpr int MAXSEL = 512;      // selected chunks staged per (b, h)
constexpr int TCH = 64;          // tail tokens per staged chunk (one 16-token tile per wave)
constexpr int NTQ = NQ - 1;      // quarters that attend the tail (1 .. 3), one partial row each
constexpr int DQ = DH / NQ;      // head dims of the residual pass per quarter (64)
constexpr int RB = 8;            // residual rows per thread whose loads are in flight together
// A granule (8 ranks, 16 bytes) k8 of hidden unit f sits at granule k8 ^ (f & 15)
__host__ __device__ constexpr int swz(int f, int k8) { return k8 ^ (f & 15); }
constexpr float NEG_LOG2E = -1.4426950408889634f;
constexpr float NEG_LN2 = -0.6931471805599453f;

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
__device__ __forceinline__ bf16x8 ldb8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f16x8 ldh8(const uint16_t *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return (uint32_t)h16(lo) | ((uint32_t)h16(hi) << 16);
}
// SiLU in -log2(e) units: y = -log2(e) x gives -log2(e) SiLU(x) = y / (1 + 2^y)
__device__ __forceinline__ float silu_scaled(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// coefficient fragments: lane (token l16 of a 16-token block, rank group kg)
// holds 8 consecutive ranks; buffer loads past the end return zeros
template <typename TC> struct Coef;
template <> struct Coef<bf16> {
  typedef u32x4 raw;
  static constexpr int ES = 2;
  __device__ static raw ld(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  }
  // bf16 -> fp16: exact for |c| in [2^-14, 65504] (8 significant bits fit in
  // 11); smaller values lose bits below 2^-24 as fp16 subnormals
  __device__ static f16x8 get(raw v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = (_Float16)bf16_bits_to_f32(w[i] & 0xFFFFu);
      o[2 * i + 1] = (_Float16)bf16_bits_to_f32(w[i] >> 16);
    }
    return o;
  }
};
template <> struct Coef<int8_t> {
  typedef uint2 raw;
  static constexpr int ES = 1;
  __device__ static raw ld(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return make_uint2(v.x, v.y);
  }
  __device__ static f16x8 get(raw v) { return i8x8_to_f16x8(v.x, v.y); }  // |code| <= 127: exact
};
// head dim d of residual row e as stored (int8 codes: before their scale)
template <typename TR> struct ResRow;
template <> struct ResRow<bf16> {
  __device__ static float get1(const void *rv, long e, int d) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(rv)[e * DH + d]);
  }
};
template <> struct ResRow<int8_t> {
  __device__ static float get1(const void *rv, long e, int d) {
    return (float)reinterpret_cast<const int8_t *>(rv)[e * DH + d];
  }
};

// ---------------------------------------------------------------------------
// A = -log2(e) W1 U_{l,h} (fp16, rows swizzled as the attend kernel's LDS
// copy) and q~_g = U_{l,h}^T q_g (fp16 hi, lo) for one 64 x 64 tile of
// (hidden unit, rank); (F / 64) (r / 64) B Hkv workgroups, 256 threads.  int8
// caches: both carry the per-rank scale of the codes.
// All of a wave's W1 fragments are loaded first, under the staging of the
// U^T tile (whole 128-byte row segments loaded, dword LDS writes of two head
// dims);
// the q~ products are bf16 x bf16 (exact) accumulated in fp32 on the matrix
// cores, like A's; the A tile leaves through LDS in 16-byte rows.
// ---------------------------------------------------------------------------
constexpr int AK = 64;
constexpr int UT_LD = DH + 8;     // U^T tile row (rank) stride, 16-bit elements
constexpr int OT_LD = AK + 8;     // output tile row (hidden unit) stride
struct AbsorbSmem {
  uint16_t ut[AK][UT_LD];         // U^T tile, bf16 (rank rows, head dims contiguous)
  uint16_t ot[AK][OT_LD];         // A tile, fp16 (hidden-unit rows, ranks contiguous)
};

// Tile `lin` of the n = (F / 64) (r / 64) B Hkv tiles, lin counted from a
// workgroup id that is a multiple of 8.
__device__ __forceinline__ void absorb_tile(const AttendArgs &a, int lin, int n, AbsorbSmem &sm) {
  // Workgroups are dispatched round-robin over the 8 XCDs (linear id mod 8),
  // each with its own L2.  The id is remapped so that an XCD receives a
  // contiguous run of (hidden tile, rank tile, (b, h)): all tiles of one or
  // two (b, h), whose W1 and basis slice it then reads from HBM once.
  constexpr int NFT = FF / AK;
  const int nrt = a.r / AK;
  int u = lin;
  if (n % 8 == 0) u = (lin % 8) * (n / 8) + lin / 8;
  const int ft = u % NFT, rt = (u / NFT) % nrt, bh = u / (NFT * nrt);
  const int b = bh / a.Hkv, h = bh % a.Hkv, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = a.r, D = a.G * a.Hkv * DH, g = a.g;
  const uint16_t *U = reinterpret_cast<const uint16_t *>(a.basis) + ((long)b * D + (long)(a.layer * a.Hkv + h) * DH) * r;
  const uint16_t *W1 = reinterpret_cast<const uint16_t *>(a.w1) + (((long)b * a.G + a.layer) * a.Hkv + h) * (long)FF * DH;
  const int wf = w >> 1, wr = w & 1, l16 = lane & 15, kg = lane >> 4;
  // W1 fragments of the wave: rows ft 64 + 32 wf + 16 mi + l16, head dims 32 ks + 8 kg
  constexpr int NKS = DH / 32;
  u32x4 w1f[NKS][2];
  const uint16_t *w1r = W1 + (long)(ft * AK + 32 * wf + l16) * DH + 8 * kg;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) w1f[ks][mi] = gld16(w1r + (long)16 * mi * DH + 32 * ks);
  // q of the group as bf16 A fragments (rows = query heads l16 < g), q~ tiles only
  const bool do_q = ft == 0;
  u32x4 qf[NKS];
  if (do_q) {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + ((long)b * a.Hq + (long)h * g + (l16 < g ? l16 : 0)) * DH + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = l16 < g ? gld16(qb + 32 * ks) : v4(0, 0, 0, 0);
  }
  // U^T tile: item (head-dim pair dp, rank octet oc) loads U[2 dp][8 oc ..] and
  // U[2 dp + 1][8 oc ..] and writes eight dwords ut[8 oc + i][2 dp .. 2 dp + 1].
  // The octets of a row are consecutive items, so a wave's load covers eight
  // whole 128-byte row segments.
  constexpr int NIT = (DH / 2) * (AK / 8) / 256;   // items per thread (4)
  u32x4 ua[NIT], ub[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int it = tid + 256 * k, oc = it % (AK / 8), dp = it / (AK / 8);
    const uint16_t *up = U + (long)(2 * dp) * r + rt * AK + 8 * oc;
    ua[k] = gld16(up);
    ub[k] = gld16(up + r);
  }
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int it = tid + 256 * k, oc = it % (AK / 8), dp = it / (AK / 8);
    const uint32_t x[4] = {ua[k].x, ua[k].y, ua[k].z, ua[k].w}, y[4] = {ub[k].x, ub[k].y, ub[k].z, ub[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint32_t *>(&sm.ut[8 * oc + 2 * i][2 * dp]) = (x[i] & 0xFFFFu) | (y[i] << 16);
      *reinterpret_cast<uint32_t *>(&sm.ut[8 * oc + 2 * i + 1][2 * dp]) = (x[i] >> 16) | (y[i] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  // A tile: wave (wf, wr) computes 32 x 32 outputs as 2 x 2 blocks
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    bf16x8 bfr[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bfr[ni] = ldb8(&sm.ut[32 * wr + 16 * ni + l16][32 * ks + 8 * kg]);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma(__builtin_bit_cast(bf16x8, w1f[ks][mi]), bfr[ni], acc[mi][ni]);
  }
  const uint16_t *csc = a.coeff_scale ? a.coeff_scale + (long)b * r : nullptr;
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int cl = 32 * wr + 16 * ni + l16;   // rank within the tile
    const float sc = NEG_LOG2E * (csc ? f16_bits_to_f32(csc[rt * AK + cl]) : 1.f);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.ot[32 * wf + 16 * mi + 4 * kg + v][cl] = h16(acc[mi][ni][v] * sc);
  }
  if (do_q) {  // q~ of the tile's ranks 16 w .. 16 w + 15: rows = heads, columns = ranks
    f32x4 qa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qa = mfma(__builtin_bit_cast(bf16x8, qf[ks]), ldb8(&sm.ut[16 * w + l16][32 * ks + 8 * kg]), qa);
    if (kg == 0) {   // lane holds heads v = 0..3 of rank 16 w + l16
      const int col = rt * AK + 16 * w + l16;
      const float s = csc ? f16_bits_to_f32(csc[col]) : 1.f;
      uint16_t *Q = a.absQ + (long)bh * 2 * GQ * r;
#pragma unroll
      for (int v = 0; v < GQ; ++v) {
        const float x = v < g ? qa[v] * s : 0.f;
        const _Float16 hv = (_Float16)x;
        Q[(long)v * r + col] = __builtin_bit_cast(uint16_t, hv);
        Q[(long)(GQ + v) * r + col] = h16(x - (float)hv);
      }
    }
  }
  __syncthreads();
  // rows of A as the attend kernel keeps them in LDS: granule k8 of unit f at swz(f, k8)
  uint16_t *A = a.absA + (long)bh * FF * r;
#pragma unroll
  for (int k = 0; k < AK * AK / 8 / 256; ++k) {
    const int pc = tid + 256 * k, row = pc / (AK / 8), part = pc % (AK / 8);
    const int f = ft * AK + row;
    *reinterpret_cast<u32x4 *>(A + (long)f * r + 8 * swz(f, rt * (AK / 8) + part)) =
        *reinterpret_cast<const u32x4 *>(&sm.ot[row][8 * part]);
  }
}

// The selection stage of the absorbed path in one launch: workgroups
// [0, n_sel) compute the partial chunk scores (select_partial_block, bf16,
// d_h = 256; no q~ output: the tiles below form it), up to the next multiple
// of 8 idle, the rest form A and q~ (absorb_tile).  The two roles share
// nothing but the launch.
struct SelectAbsorbArgs {
  const float *landmark;  // [B][n_c][r]
  double *part;           // [B][Hkv][r / 64][n_c] partial chunk scores
  long q_bstride;         // elements between the query rows of consecutive sequences
  int n_sel;              // r / 64 * Hkv * B
};

__global__ __launch_bounds__(256) void k_select_absorb(const AttendArgs a, const SelectAbsorbArgs x) {
  __shared__ __align__(16) union {
    SelectSmem<DH, QTG_G> s;
    AbsorbSmem t;
  } sm;
  const int n_pad = (x.n_sel + 7) & ~7;
  const int id = blockIdx.x;
  if (id < n_pad) {
    if (id < x.n_sel) {
      const int NRB = a.r / SEL_RB;
      int rb, h, b;
      select_coords(id, NRB, a.Hkv, a.B, rb, h, b);
      select_partial_block<bf16, DH, QTG_G>(sm.s, rb, h, b, NRB, reinterpret_cast<const bf16 *>(a.q), x.q_bstride,
                                            reinterpret_cast<const bf16 *>(a.basis), x.landmark, a.Hq, a.Hkv, a.r,
                                            a.N / a.C, a.G * a.Hkv * DH, a.layer, x.part, nullptr, nullptr,
                                            nullptr, 0);
    }
    return;
  }
  absorb_tile(a, id - n_pad, gridDim.x - n_pad, sm.t);
}

// ---------------------------------------------------------------------------
// LDS of the attend kernel (bytes)
// ---------------------------------------------------------------------------
template <int R>
struct Smem {
  static constexpr int QLD = R + 16;                      // q~ row stride (16-bit): rows in distinct banks
  static constexpr int AQ = 0;                            // [FQ][R] fp16 A quarter (swizzled granules)
  static constexpr int QT = AQ + FQ * R * 2;              // [8][QLD] fp16 q~ hi rows 0..3, lo rows 4..7
  static constexpr int B1S = QT + 8 * QLD * 2;            // [FQ] fp32 -log2(e) b1 of this quarter
  static constexpr int LG = B1S + FQ * 4;                 // [RT][GQ] fp32 logits of the round
  static constexpr int PS = LG + RT * GQ * 4;             // [RT][GQ] fp32 p of the round
  static constexpr int P16 = PS + RT * GQ * 4;            // [GQ][RT] fp16 p (MFMA operand)
  static constexpr int ST = P16 + GQ * RT * 2;            // [3][GQ] m, l, alpha
  static constexpr int RC = ST + 3 * GQ * 4;              // [2][NW] residual rows of the wave slices
  static constexpr int RL = RC + 2 * NW * 4;              // [2][NW][TT] residual rows (entry << 8 | token in round)
  static constexpr int SEL = RL + 2 * NW * TT * 4;        // [MAXSEL] selected chunks of (b, h)
  static constexpr int BYTES = SEL + MAXSEL * 4;
  // after the rounds the A area holds the per-wave hidden sums [NW][FQ][GQ]
  // of the merge, then the tail's staged V rows
  static constexpr int TVS = 0;
  static_assert(TVS + TCH * DH * 2 <= QT, "tail staging does not fit");
  static constexpr int AHM = 0;
  static constexpr int RVR = AHM + NW * FQ * GQ * 4;     // [NW row groups][GQ][DQ] value sums
  static_assert(RVR + NW * GQ * DQ * 4 <= QT, "merge area does not fit");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Block -> (b, h, split, quarter).  Workgroups are dispatched round-robin over
// the 8 XCDs; the linear id is remapped so that each XCD receives a contiguous
// run of (b, h, split, quarter): the quarters of a split share the
// coefficient tiles and the splits of a (b, h) share A in one L2.
__device__ __forceinline__ void coords(const AttendArgs &a, int &b, int &h, int &s, int &fq) {
  const int n = gridDim.x;
  int u = blockIdx.x;
  if (n % 8 == 0) u = (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8;
  fq = u % NQ;
  s = (u / NQ) % a.n_split;
  const int bh = (u / NQ) / a.n_split;
  h = bh % a.Hkv;
  b = bh / a.Hkv;
}

template <typename TC, int NK>
__global__ __launch_bounds__(NTH, 1) void k_attend_absorb(const AttendArgs a) {
  constexpr int R = NK * KS;
  constexpr int DC = dc_of<NK>();
  using S = Smem<R>;
  using CT = Coef<TC>;
  static_assert(NK % DC == 0, "the coefficient ring must divide the k-step count");
  extern __shared__ __align__(16) unsigned char sm[];
  const uint16_t *Aq = reinterpret_cast<const uint16_t *>(sm + S::AQ);
  const uint16_t *Qt = reinterpret_cast<const uint16_t *>(sm + S::QT);
  float *B1s = reinterpret_cast<float *>(sm + S::B1S);
  float *Lg = reinterpret_cast<float *>(sm + S::LG);
  float *Ps = reinterpret_cast<float *>(sm + S::PS);
  uint16_t *P16 = reinterpret_cast<uint16_t *>(sm + S::P16);
  float *st = reinterpret_cast<float *>(sm + S::ST);   // m [GQ], l [GQ], alpha [GQ]
  int32_t *rc = reinterpret_cast<int32_t *>(sm + S::RC);
  int32_t *rl = reinterpret_cast<int32_t *>(sm + S::RL);
  int32_t *selS = reinterpret_cast<int32_t *>(sm + S::SEL);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, kg = lane >> 4;
  int b, h, s, fq;
  coords(a, b, h, s, fq);
  const int g = a.g, C = a.C;
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;   // (b, layer, h)
  const long bhs = (long)b * a.Hkv + h;                      // (b, h)

  // ---- prologue: selection, A quarter, q~, b1 ---------------------------------
  // With the partial chunk scores at hand (n_c <= NTH), each workgroup ranks
  // them itself: their loads go first, so that the sum waits for nothing else.
  // A chunk's score is its rank blocks' partials summed in block order.
  const int k_eff = a.k_eff, n_c = a.N / C;
  constexpr int NRB = R / 64;
  double spv[NRB];
  if (a.score_part && tid < n_c) {
    const double *sp = a.score_part + bhs * NRB * n_c + tid;
#pragma unroll
    for (int k = 0; k < NRB; ++k) spv[k] = sp[(long)k * n_c];
  }
  // A quarter: every piece in flight at once
  constexpr int NP = FQ * R * 2 / 16 / NTH;   // 16-byte pieces per thread
  u32x4 apc[NP];
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.absA + bhs * (long)FF * R + (long)fq * FQ * R);
#pragma unroll
    for (int i = 0; i < NP; ++i) apc[i] = src[i * NTH + tid];
  }
  if (a.score_part) {
    // the top k_eff chunks by (score desc, index asc) in ascending index
    // order, ranked by wave 0 (wave_topk) while the others stage q~, b1 and
    // their part of A; the (split 0, quarter 0) workgroup writes sel_out.
    // The scores sit in the round buffers, unused until the first round.
    static_assert(ABSORB_SELECT_MAX_NC <= NTH && ABSORB_SELECT_MAX_NC == 4 * WAVE, "one chunk per thread");
    static_assert(S::PS - S::LG >= ABSORB_SELECT_MAX_NC * 8, "score staging");
    double *scL = reinterpret_cast<double *>(sm + S::LG);
    if (tid < n_c) {
      double v = spv[0];
#pragma unroll
      for (int k = 1; k < NRB; ++k) v += spv[k];
      scL[tid] = v;
    }
    __syncthreads();
    if (w == 0) {
      int32_t *so = (s == 0 && fq == 0 && a.sel_out) ? a.sel_out + bhs * k_eff : nullptr;
      wave_topk<4>(scL, n_c, k_eff, [&](int pos, int c) {
        selS[pos] = c;
        if (so) so[pos] = c;
      });
    }
  } else {
    const int32_t *selp = a.sel + bhs * k_eff;
    for (int i = tid; i < k_eff; i += NTH) selS[i] = selp[i];
  }
  {  // q~ hi and lo rows of this (b, h): absQ [2][GQ][R] -> rows 0..7 of QT
    // (a thread's pieces loaded together)
    constexpr int NQP = 2 * GQ * R / 8, QPT = (NQP + NTH - 1) / NTH;
    const uint16_t *Qg = a.absQ + bhs * 2 * GQ * R;
    uint16_t *qd = reinterpret_cast<uint16_t *>(sm + S::QT);
    u32x4 qp[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + NTH * k;
      if (i < NQP) qp[k] = gld16(Qg + 8 * i);
    }
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + NTH * k;
      if (i < NQP) lst16(qd + ((8 * i) / R) * S::QLD + (8 * i) % R, qp[k]);
    }
  }
  const uint16_t *B1 = reinterpret_cast<const uint16_t *>(a.b1) + bh * FF + fq * FQ;
  for (int i = tid; i < FQ; i += NTH) B1s[i] = bf16_bits_to_f32(B1[i]) * NEG_LOG2E;
  if (tid < GQ) {
    st[tid] = -INFINITY;
    st[GQ + tid] = 0.f;
    st[2 * GQ + tid] = 0.f;
  }
  {
    u32x4 *dst = reinterpret_cast<u32x4 *>(sm + S::AQ);
#pragma unroll
    for (int i = 0; i < NP; ++i) dst[i * NTH + tid] = apc[i];
  }

  const int n_slices = k_eff * (C / TT);
  const int sl0 = s * a.tps, sl1 = min(n_slices, sl0 + a.tps);
  const int rounds = a.tps / NW;
  const int r = R;
  const TC *cf = reinterpret_cast<const TC *>(a.coeff) + (long)b * a.N * r;
  const rsrc_t Cr = make_rsrc(cf, (uint32_t)((long)a.N * r * CT::ES));
  const uint32_t c_voff = (uint32_t)((l16 * r + 8 * kg) * CT::ES);   // + (row + 16 tt) r + 32 ks
  const int32_t *rptr = a.res_ptr + bh * (a.N / C + 1);
  const int32_t *ridx = a.res_idx + bh * a.n_res;
  const TC *rval = reinterpret_cast<const TC *>(a.res_val) + bh * (long)a.n_res * DH;
  // residual pass: thread (row group rg: rows rg, rg + NW, ... of the round;
  // head dim vd of this quarter's DQ), all query heads
  const int rg = w, vd = fq * DQ + lane, vg = tid >> 6;
  const float rsv = (sizeof(TC) == 1 && a.res_scale) ? f16_bits_to_f32(a.res_scale[bh * DH + vd]) : 1.f;
  float accV[GQ] = {0.f, 0.f, 0.f, 0.f};
  f32x4 accH[NFB];   // hidden sums [16 g][16 f] per block (rows g < GQ live)
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) accH[fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // token row of slice sig (a slice past the split reads zeros)
  auto slice_row = [&](int sig) -> long {
    return sig < sl1 ? (long)selS[(sig * TT) / C] * C + (sig * TT) % C : (long)a.N;
  };
  auto c_soff = [&](long row, int tt, int ks) -> uint32_t {
    return (uint32_t)(((row + 16 * tt) * r + ks * KS) * CT::ES);
  };
  // residual rows of the wave's slice at token row `row` (past the split: none)
  // into list buffer buf, as (entry << 8 | token in round); x0 = the index
  // entry e0 + lane, already loaded
  auto list_res = [&](long row, int x0, int e0, int e1, int buf) {
    int cnt = 0;
    if (row < a.N) {
      const int jc = (int)(row / C), t0 = (int)(row % C);
      for (int base = e0; base < e1; base += WAVE) {
        const int e = base + lane;
        const int x = base == e0 ? x0 : (e < e1 ? ridx[e] : -1);
        const int t = e < e1 ? x - jc * C - t0 : -1;
        const bool in = e < e1 && t >= 0 && t < TT;
        const uint64_t m = __ballot(in);
        const int pos = cnt + __popcll(m & lanemask_lt());
        if (in && pos < TT) rl[(buf * NW + w) * TT + pos] = (e << 8) | (TT * w + t);
        cnt += __popcll(m);
      }
    }
    if (lane == 0) rc[buf * NW + w] = min(cnt, TT);
  };
  __syncthreads();
  long row0 = slice_row(sl0 + w);
  typename CT::raw cr[DC][NTT];   // coefficient ring: k-step ks in cr[ks % DC]
#pragma unroll
  for (int q = 0; q < DC - 1; ++q)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) cr[q][tt] = CT::ld(Cr, c_voff, c_soff(row0, tt, q));
  {  // round 0's list
    int e0 = 0, e1 = 0, x0 = -1;
    if (row0 < a.N) {
      const int jc = (int)(row0 / C);
      e0 = rptr[jc];
      e1 = rptr[jc + 1];
      x0 = e0 + lane < e1 ? ridx[e0 + lane] : -1;
    }
    list_res(row0, x0, e0, e1, 0);
  }
  __syncthreads();   // every wave's round-0 list before any wave reads them

  // A fragment of k-step ks, block fb: unit 16 fb + l16, ranks 32 ks + 8 kg .. + 8;
  // q~ fragment: row l16 (< 8) of the q~ table.  The offsets are made opaque
  // once per round: the fragments are the same in every round, and hoisted out
  // of the round loop they would hold 12 k-steps of registers.
  uint32_t a_off = (uint32_t)(l16 * R), q_off = (uint32_t)((l16 & 7) * S::QLD + 8 * kg);
  const f16x8 z8 = __builtin_bit_cast(f16x8, v4(0, 0, 0, 0));

  for (int rd = 0; rd < rounds; ++rd) {
    const int sig = sl0 + NW * rd + w;
    const bool has = sig < sl1;
    const bool more = rd + 1 < rounds;
    const long row0n = more ? slice_row(sig + NW) : (long)a.N;
    // the next round's slice: its chunk's residual range now, its first 64
    // index entries under this round's k-loop (listed after the round)
    int e0n = 0, e1n = 0, xn = -1;
    if (row0n < a.N) {
      const int jcn = (int)(row0n / C);
      e0n = rptr[jcn];
      e1n = rptr[jcn + 1];
    }
    // residual rows of the round (listed at the end of the previous round): the
    // first RB rows' values of this thread's head dim, in flight under the
    // k-loop (row k of the round: list wl, entry k - rows of the lists before wl)
    const int *rcb = rc + (rd & 1) * NW, *rlb = rl + (rd & 1) * NW * TT;
    const int rn0 = rcb[0], rn1 = rcb[1], rn2 = rcb[2], rn3 = rcb[3];
    const int n_rows = rn0 + rn1 + rn2 + rn3;
    auto res_code = [&](int k) -> int {
      const int k1 = k - rn0, k2 = k1 - rn1, k3 = k2 - rn2;
      return rlb[k < rn0 ? k : k1 < rn1 ? TT + k1 : k2 < rn2 ? 2 * TT + k2 : 3 * TT + k3];
    };
    // this thread's rows: k0 + rg + NW u, u < RB
    float rx[RB];
    int rcode[RB];
    auto res_load = [&](int k0) {
#pragma unroll
      for (int u = 0; u < RB; ++u) rcode[u] = res_code(min(k0 + rg + NW * u, n_rows - 1));
#pragma unroll
      for (int u = 0; u < RB; ++u) rx[u] = ResRow<TC>::get1(rval, (long)(rcode[u] >> 8), vd);
    };
    if (n_rows > 0) res_load(0);
    // ---- k-loop: hidden pre-activations and logits ----------------------------
    f32x4 acc[NTT][NFB];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) acc[tt][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 lg[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) lg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // lane values of the swizzle, opaque per round for the same reason (the
    // twelve per-k-step granule offsets would otherwise be hoisted and spilled)
    uint32_t sw_l = (uint32_t)l16, sw_k = (uint32_t)kg;
    asm volatile("" : "+v"(a_off), "+v"(q_off), "+v"(sw_l), "+v"(sw_k));
    const uint16_t *a_rd = Aq + a_off;
    const uint16_t *q_rd = Qt + q_off;
    // A and q~ fragments double-buffered: k-step ks + 1's read under k-step ks's products
    f16x8 af[2][NFB + 1];   // [NFB] is the q~ operand
    auto load_af = [&](int ks, f16x8 *dst) {
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) dst[fb] = ldh8(a_rd + 16 * fb * R + 8 * (((uint32_t)(4 * ks) + sw_k) ^ sw_l));
      dst[NFB] = l16 < 8 ? ldh8(q_rd + ks * KS) : z8;
    };
    load_af(0, af[0]);
    sfor<NK>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      __builtin_amdgcn_sched_barrier(0);
      // coefficients DC - 1 k-steps ahead; past the round's end, the next
      // round's first k-steps (k-step kl of this round and kl - NK of the next
      // share ring slot kl % DC because DC divides NK)
      constexpr int kl = ks + DC - 1;
      if constexpr (kl < NK) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) cr[kl % DC][tt] = CT::ld(Cr, c_voff, c_soff(row0, tt, kl));
      } else {
        if (more) {
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) cr[kl % DC][tt] = CT::ld(Cr, c_voff, c_soff(row0n, tt, kl - NK));
        }
      }
      if constexpr (ks + 1 < NK) load_af(ks + 1, af[(ks + 1) & 1]);
      if constexpr (ks == 1) xn = e0n + lane < e1n ? ridx[e0n + lane] : -1;
      f16x8 c8[NTT];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) c8[tt] = CT::get(cr[ks % DC][tt]);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) acc[tt][fb] = mfma(c8[tt], af[ks & 1][fb], acc[tt][fb]);
        lg[tt] = mfma(c8[tt], af[ks & 1][NFB], lg[tt]);
      }
    });
    __builtin_amdgcn_sched_barrier(0);
    row0 = row0n;
    // ---- logits of the round: hi (column gi) + lo (column 4 + gi) -------------
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float x = lg[tt][v] + __shfl_down(lg[tt][v], GQ, 16);
        if (l16 < GQ) Lg[(TT * w + 16 * tt + 4 * kg + v) * GQ + l16] = x;
      }
    __syncthreads();
    // ---- softmax of the round, workgroup-wide: wave w takes query head w -----
    if (w < g) {
      const int gi = w;
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = lane + WAVE * u;            // token of the round (slice u)
        const int sl = sl0 + NW * rd + u;
        x[u] = sl < sl1 ? Lg[t * GQ + gi] * a.scale_log2 : -INFINITY;
      }
      const float mx = wave_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      const float m_old = st[gi], m_new = fmaxf(m_old, mx);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = lane + WAVE * u;
        const float p = x[u] == -INFINITY ? 0.f : (float)(_Float16)__builtin_amdgcn_exp2f(x[u] - m_new);
        Ps[t * GQ + gi] = p;
        P16[gi * RT + t] = h16(p);
        ps += p;
      }
      ps = wave_sum(ps);
      if (lane == 0) {
        const float alpha = (m_old == -INFINITY || m_new == -INFINITY) ? (m_old == m_new ? 1.f : 0.f)
                                                                       : __builtin_amdgcn_exp2f(m_old - m_new);
        st[2 * GQ + gi] = alpha;
        st[GQ + gi] = st[GQ + gi] * alpha + ps;
        st[gi] = m_new;
      }
    } else if (lane < RT / NW) {   // heads past the group: p = 0
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = (lane + (RT / NW) * u);
        Ps[t * GQ + w] = 0.f;
        P16[w * RT + t] = 0;
      }
      if (lane == 0) st[2 * GQ + w] = 1.f;
    }
    __syncthreads();
    // ---- accH^T[g][f] += p^T H^T: rescale, then two 32-token k-steps ----------
    {
      f32x4 al;
#pragma unroll
      for (int v = 0; v < 4; ++v) al[v] = kg == 0 ? st[2 * GQ + v] : 0.f;
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int v = 0; v < 4; ++v) accH[fb][v] *= al[v];
      // p^T A operand: lane (head l16, kg) holds p at the tokens of the H
      // operand's k positions: 16 (2 i) + 4 kg + v, then 16 (2 i + 1) + 4 kg + v
#pragma unroll
      for (int i = 0; i < NTT / 2; ++i) {
        f16x8 pa = z8;
        if (l16 < GQ) {
          const uint16_t *pr = P16 + l16 * RT + TT * w + 32 * i + 4 * kg;
          const uint2 lo = *reinterpret_cast<const uint2 *>(pr);
          const uint2 hi = *reinterpret_cast<const uint2 *>(pr + 16);
          pa = __builtin_bit_cast(f16x8, v4(lo.x, lo.y, hi.x, hi.y));
        }
        // SiLU of the pre-activations of token blocks (2 i, 2 i + 1), hidden
        // block fb, as the fp16 B operand
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
          const float bias = B1s[16 * fb + l16];
          f16x8 hb;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            hb[v] = (_Float16)silu_scaled(acc[2 * i][fb][v] + bias);
            hb[4 + v] = (_Float16)silu_scaled(acc[2 * i + 1][fb][v] + bias);
          }
          accH[fb] = mfma(pa, hb, accH[fb]);
        }
      }
    }
    // ---- residual rows of the round (vector ALUs): accV[g][vd] += p delta ----
    {
#pragma unroll
      for (int gi = 0; gi < GQ; ++gi) accV[gi] *= st[2 * GQ + gi];
      for (int k0 = 0; k0 < n_rows; k0 += NW * RB) {
        if (k0 > 0) res_load(k0);
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          if (k0 + rg + NW * u < n_rows) {
            const f32x4 p4 = *reinterpret_cast<const f32x4 *>(Ps + (rcode[u] & 0xFF) * GQ);
            const float x = rx[u] * rsv;
#pragma unroll
            for (int gi = 0; gi < GQ; ++gi) accV[gi] = fmaf(p4[gi], x, accV[gi]);
          }
        }
      }
    }
    // the next round's residual list (its first 64 index entries prefetched)
    list_res(row0, xn, e0n, e1n, (rd + 1) & 1);
    __syncthreads();   // round's LDS (logits, p, residual lists) free again
  }

  // ---- partial rows -------------------------------------------------------------
  const int n_prow = (1 + NTQ) * a.n_split;   // per (b, h): chunk rows, then NTQ tail rows per split
  float *part = a.part + (bhs * n_prow + s) * g * a.PW;
  // hidden sums of the four waves (their slices) of every unit of the quarter
  float *ahm = reinterpret_cast<float *>(sm + S::AHM);
  if (kg == 0) {
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
      *reinterpret_cast<f32x4 *>(ahm + ((w * FQ) + 16 * fb + l16) * GQ) = accH[fb];
  }
  __syncthreads();
  for (int i = tid; i < FQ * GQ; i += NTH) {   // (unit of the quarter, head)
    const int f = i / GQ, gi = i % GQ;
    const float x = (ahm[(0 * FQ + f) * GQ + gi] + ahm[(1 * FQ + f) * GQ + gi]) +
                    (ahm[(2 * FQ + f) * GQ + gi] + ahm[(3 * FQ + f) * GQ + gi]);
    if (gi < g) part[(long)gi * a.PW + 4 + fq * FQ + f] = x * NEG_LN2;
  }
  {  // value sums of this quarter's head dims: the four row groups in order
    float *rvr = reinterpret_cast<float *>(sm + S::RVR);
#pragma unroll
    for (int gi = 0; gi < GQ; ++gi) rvr[(rg * GQ + gi) * DQ + lane] = accV[gi];
    __syncthreads();
    if (vg < g) {
      const float x = (rvr[(0 * GQ + vg) * DQ + lane] + rvr[(1 * GQ + vg) * DQ + lane]) +
                      (rvr[(2 * GQ + vg) * DQ + lane] + rvr[(3 * GQ + vg) * DQ + lane]);
      part[(long)vg * a.PW + 4 + FF + fq * DQ + lane] = x;
    }
  }
  if (fq == 0) {
    if (tid < g) {
      part[(long)tid * a.PW + 0] = st[tid];
      part[(long)tid * a.PW + 1] = st[GQ + tid];
      part[(long)tid * a.PW + 2] = st[GQ + tid];
      part[(long)tid * a.PW + 3] = 0.f;
    }
    return;
  }

  // ---- quarters 1..3: a third each of this split's share of the tail -----------
  // Chunks of up to TCH tokens: V rows staged in the (now free) A area; the
  // logits of 16-token tile w on the matrix cores (K rows as the A operand
  // straight from memory, bf16 q as the B operand, fp32 sums); an online
  // softmax per query head over the chunks; p . V on the vector ALUs.
  const int t0s = min(a.T, s * a.tail_per_split), t1s = min(a.T, t0s + a.tail_per_split);
  const int tq = (t1s - t0s + NTQ - 1) / NTQ;
  const int tb = min(t1s, t0s + (fq - 1) * tq), te = min(t1s, tb + tq);
  const long tail_base = (bh * a.T) * DH;
  const uint16_t *kt = reinterpret_cast<const uint16_t *>(a.k_tail) + tail_base;
  const uint16_t *vt = reinterpret_cast<const uint16_t *>(a.v_tail) + tail_base;
  uint16_t *tvs = reinterpret_cast<uint16_t *>(sm + S::TVS);
  float *tp = Ps;   // [TCH][GQ] logits, then p, of the chunk
  __syncthreads();   // the merge area is read
  if (tid < GQ) {
    st[tid] = -INFINITY;
    st[GQ + tid] = 0.f;
  }
  // q of head l16 (< g) as bf16 B operands, dims 32 ks + 8 kg .. + 8
  constexpr int NKD = DH / 32;
  u32x4 qfr[NKD];
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + ((long)b * a.Hq + (long)h * g + (l16 < g ? l16 : 0)) * DH + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) qfr[ks] = l16 < g ? gld16(qb + 32 * ks) : v4(0, 0, 0, 0);
  }
  float tv[4] = {0.f, 0.f, 0.f, 0.f};   // (vg, dims 4 lane .. 4 lane + 3)
  constexpr int TPC = TCH * DH / 8 / NTH;   // 16-byte pieces per thread of V
  for (int c0 = tb; c0 < te; c0 += TCH) {
    const int nt = min(TCH, te - c0);
    u32x4 vp[TPC], kf[NKD];
#pragma unroll
    for (int i = 0; i < TPC; ++i) {
      const int pc = tid + NTH * i, t = pc / (DH / 8), part8 = pc % (DH / 8);
      vp[i] = gld16(vt + (long)(c0 + min(t, nt - 1)) * DH + 8 * part8);
    }
    {
      const uint16_t *kr = kt + (long)(c0 + min(16 * w + l16, nt - 1)) * DH + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) kf[ks] = gld16(kr + 32 * ks);
    }
#pragma unroll
    for (int i = 0; i < TPC; ++i) lst16(tvs + 8 * (tid + NTH * i), vp[i]);
    {  // logits of tokens 16 w .. 16 w + 15 (lane: head l16, tokens 4 kg + v)
      f32x4 la = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[ks]),
                                                     __builtin_bit_cast(bf16x8, qfr[ks]), la, 0, 0, 0);
      if (l16 < GQ)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * w + 4 * kg + v;
          tp[t * GQ + l16] = (t < nt && l16 < g) ? la[v] * a.scale_log2 : -INFINITY;
        }
    }
    __syncthreads();
    if (w < GQ) {   // online softmax of head w over the chunk's nt <= TCH tokens
      const float x = lane < nt ? tp[lane * GQ + w] : -INFINITY;
      const float m_old = st[w], m_new = fmaxf(m_old, wave_max(x));
      const float p = x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x - m_new);
      if (lane < nt) tp[lane * GQ + w] = p;
      const float ps = wave_sum(p);
      if (lane == 0) {
        const float alpha = (m_old == -INFINITY || m_new == -INFINITY) ? (m_old == m_new ? 1.f : 0.f)
                                                                       : __builtin_amdgcn_exp2f(m_old - m_new);
        st[2 * GQ + w] = alpha;
        st[GQ + w] = st[GQ + w] * alpha + ps;
        st[w] = m_new;
      }
    }
    __syncthreads();
    if (vg < g) {   // p . V: thread (vg, dims 4 lane .. 4 lane + 3)
      const float alpha = st[2 * GQ + vg];
#pragma unroll
      for (int i = 0; i < 4; ++i) tv[i] *= alpha;
      for (int t = 0; t < nt; ++t) {
        const float p = tp[t * GQ + vg];
        const uint2 v2 = *reinterpret_cast<const uint2 *>(tvs + t * DH + 4 * lane);
        tv[0] = fmaf(p, bf16_bits_to_f32(v2.x & 0xFFFFu), tv[0]);
        tv[1] = fmaf(p, bf16_bits_to_f32(v2.x >> 16), tv[1]);
        tv[2] = fmaf(p, bf16_bits_to_f32(v2.y & 0xFFFFu), tv[2]);
        tv[3] = fmaf(p, bf16_bits_to_f32(v2.y >> 16), tv[3]);
      }
    }
    __syncthreads();   // the chunk's staging and p are free again
  }
  float *tpart = a.part + (bhs * n_prow + a.n_split + s * NTQ + (fq - 1)) * g * a.PW;
  if (tid < g) {
    tpart[(long)tid * a.PW + 0] = st[tid];
    tpart[(long)tid * a.PW + 1] = st[GQ + tid];
    tpart[(long)tid * a.PW + 2] = 0.f;
    tpart[(long)tid * a.PW + 3] = 0.f;
  }
  if (vg < g)
#pragma unroll
    for (int i = 0; i < 4; ++i) tpart[(long)vg * a.PW + 4 + FF + 4 * lane + i] = tv[i];
}

template <typename TC, int NK>
static hipError_t go(const AttendArgs &a, hipStream_t st) {
  const size_t smem = Smem<NK * KS>::BYTES;
  static const bool lds_ok = (allow_dynamic_lds(k_attend_absorb<TC, NK>, smem), true);
  (void)lds_ok;
  if (a.tps % NW != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_attend_absorb<TC, NK>), dim3(a.B * a.Hkv * a.n_split * NQ), dim3(NTH), smem, st, a);
  return hipGetLastError();
}

}  // namespace absorb

bool absorb_supported(int act, int coeff, int resid, int dh, int F, int r, int C, int g, int k_eff) {
  return act == LOWRAM_BF16 && coeff == resid && (coeff == LOWRAM_BF16 || coeff == LOWRAM_I8) &&
         dh == absorb::DH && F == absorb::FF && (r == 384 || r == 512) && C % absorb::TT == 0 &&
         g <= absorb::GQ && k_eff >= 1 && k_eff <= absorb::MAXSEL;
}

// Splits per (b, h): about one workgroup per CU over the four quarters, at
// least one round (four slices) per split, at most 16 splits (64 partial rows
// with the tail's three per split); tps = 64-token slices per split (a
// multiple of four); tail tokens per split; partial rows per (b, h).
void absorb_plan(int B, int Hkv, int k_eff, int C, int T, int &n_split, int &tps, int &tail_per_split,
                 int &n_part) {
  const int n_slices = k_eff * (C / absorb::TT);
  int want = (256 + absorb::NQ * B * Hkv - 1) / (absorb::NQ * B * Hkv);
  const int max_split = (n_slices + absorb::NW - 1) / absorb::NW;
  if (want > max_split) want = max_split;
  if (want > 16) want = 16;
  if (want < 1) want = 1;
  tps = (n_slices + want - 1) / want;
  tps = (tps + absorb::NW - 1) / absorb::NW * absorb::NW;
  n_split = (n_slices + tps - 1) / tps;
  tail_per_split = (T + n_split - 1) / n_split;
  n_part = (1 + absorb::NTQ) * n_split;
}

hipError_t launch_select_absorb(const AttendArgs &a, const float *landmark, double *part, long q_bstride,
                                hipStream_t st) {
  absorb::SelectAbsorbArgs x;
  x.landmark = landmark;
  x.part = part;
  x.q_bstride = q_bstride;
  x.n_sel = select_rank_blocks(a.r) * a.Hkv * a.B;
  const int n_tiles = (absorb::FF / absorb::AK) * (a.r / absorb::AK) * a.B * a.Hkv;
  hipLaunchKernelGGL(absorb::k_select_absorb, dim3(((x.n_sel + 7) & ~7) + n_tiles), dim3(256), 0, st, a, x);
  return hipGetLastError();
}

hipError_t launch_attend_absorb(int coeff, const AttendArgs &a, hipStream_t st) {
  const bool i8 = coeff == LOWRAM_I8;
  if (a.r == 384) return i8 ? absorb::go<int8_t, 12>(a, st) : absorb::go<bf16, 12>(a, st);
  if (a.r == 512) return i8 ? absorb::go<int8_t, 16>(a, st) : absorb::go<bf16, 16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lowram
