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
// k_absorb (run with the chunk selection, before the attend kernel) forms, per
// (sequence, kv head) of the layer, A = -log2(e) W1 U_{l,h} (rounded to fp16
// once; int8 caches fold the per-rank scale in) and q~_g = U_{l,h}^T q_g for
// the g query heads (fp32, split into an fp16 part and the fp16 rounding of
// the remainder).
//
// k_attend_absorb: one workgroup of 8 waves per (sequence b, kv head h, split
// s, half of F).  A split is a run of 64-token slices of the chunks selected
// for h; a round takes two of them (128 tokens).  Wave (tw, fw) owns slice tw
// of the round and hidden units [64 fw, 64 fw + 64) of the half.  Per round,
// over the rank in 32-wide k-steps:
//   H^T[t][f] += C[t][r] A^T[r][f] on fp16 MFMAs: coefficient fragments go
//     straight from global memory into registers and are converted to fp16
//     (bf16 coefficients are exact in fp16's range, int8 codes always); the A
//     slab of a k-step is shared by the 8 waves through LDS (double-buffered,
//     loaded two k-steps ahead, one barrier per k-step); fp16 A (11
//     significant bits) rather than bf16 keeps the hidden pre-activations at
//     the accuracy of an fp16 rebuilt key;
//   logits[t][g] += C[t][r] q~^T[r][g] with q~ as fp16 hi and lo parts, taken
//     in turn by the four waves of a slice (wave fw on k-steps ks = fw mod 4),
//     so each logit carries the fp32 q~ to about 2^-22 relative against exact
//     coefficients.
// Then, per round: the logits are summed over the four waves (fixed order),
// a workgroup-wide online softmax per query head (p in fp16), SiLU of the
// hidden pre-activations (held in -log2(e) units: one exp2, one reciprocal),
// accH^T[g][f] += p^T H^T on the matrix cores, and, in the first half, the
// residual rows of the round's tokens on the vector ALUs.
// Both halves compute the same logits bit for bit, so their softmax states
// agree; each writes its half of the hidden sums into the split's partial row
// and the first half writes (m, l, mass, accV).  The second half also attends
// its share of the uncompressed tail into a separate partial row (hidden sums
// zero), so the combine merges 2 n_split rows per (b, h).
//
// Method: keys as per-token coefficients on a group basis (zicq.com English
// summary, "Cross-Layer Low-Rank Key Compression"); values from the per-head
// predictor plus residuals of the worst tokens ("Core Mechanism"); only
// query-selected chunks are rebuilt (rit.work page, generation section);
// attention softmax(q K^T / sqrt(d_h)) V (OjaKV page, section 3).
#include <type_traits>

#include "attend_common.hpp"

namespace lowram {
namespace absorb {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int DH = 256;          // head dim handled here
constexpr int FF = 512;          // predictor hidden width handled here
constexpr int FH = FF / 2;       // hidden units per workgroup (one half)
constexpr int NW = 8;            // waves per workgroup
constexpr int NTH = NW * WAVE;
constexpr int TT = 64;           // tokens per wave slice
constexpr int RT = 2 * TT;       // tokens per round
constexpr int NTT = TT / 16;     // 16-token blocks of a slice
constexpr int FWV = FH / 4;      // hidden units per wave (64)
constexpr int NFB = FWV / 16;    // 16-wide hidden blocks per wave
constexpr int KS = 32;           // ranks per k-step
constexpr int ALD = KS + 8;      // A slab row stride, 16-bit elements (80 bytes)
constexpr int GQ = 4;            // query heads per kv head (at most)
// coefficient k-steps in registers (DC - 1 ahead; DC divides the k-step count):
// 3 at r = 384 (12 k-steps), 2 at r = 512, where four would not fit the
// register file
template <int NK> constexpr int dc_of() { return NK % 3 == 0 ? 3 : 2; }
constexpr int SLAB_P = FH * KS / 8 / NTH;   // 16-byte A slab pieces per thread and k-step (2)
constexpr int MAXSEL = 512;      // selected chunks staged per (b, h)
constexpr int MAXRES = TT;       // residual rows listed per slice and round
constexpr int RSTAGE = 32;       // residual rows of a round staged in LDS (more: read from global)
constexpr int TCH = 32;          // tail tokens per staged chunk
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
  __device__ static f16x8 get(raw v) {  // |code| <= 127 is exact in fp16
    const int8_t *b = reinterpret_cast<const int8_t *>(&v);
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)(float)b[i];
    return o;
  }
};
template <typename TR> struct ResRow;
template <> struct ResRow<bf16> {
  static constexpr int ES = 2;
  __device__ static void get(const void *rv, long e, int d, float s0, float s1, float &x0, float &x1) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(rv) + e * DH + d);
    x0 = bf16_bits_to_f32(v & 0xFFFFu);
    x1 = bf16_bits_to_f32(v >> 16);
  }
};
template <> struct ResRow<int8_t> {
  static constexpr int ES = 1;
  __device__ static void get(const void *rv, long e, int d, float s0, float s1, float &x0, float &x1) {
    const uint16_t v = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const int8_t *>(rv) + e * DH + d);
    x0 = (float)(int8_t)(v & 0xFFu) * s0;
    x1 = (float)(int8_t)(v >> 8) * s1;
  }
};

// ---------------------------------------------------------------------------
// A = -log2(e) W1 U_{l,h} (fp16) and q~_g = U_{l,h}^T q_g (fp16 hi, lo) for
// one 64 x 64 tile of (hidden unit, rank); grid (F / 64, r / 64, B Hkv), 256
// threads.  int8 caches: both carry the per-rank scale of the codes.
// All of a wave's W1 fragments are loaded first, under the staging of the
// U^T tile (dword LDS writes of two head dims, consecutive over the lanes);
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

__global__ __launch_bounds__(256) void k_absorb(const AttendArgs a) {
  __shared__ __align__(16) AbsorbSmem sm;
  const int ft = blockIdx.x, rt = blockIdx.y, bh = blockIdx.z;
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
  // U[2 dp + 1][8 oc ..] and writes eight dwords ut[8 oc + i][2 dp .. 2 dp + 1]
  constexpr int NIT = (DH / 2) * (AK / 8) / 256;   // items per thread (4)
  u32x4 ua[NIT], ub[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int it = tid + 256 * k, dp = it % (DH / 2), oc = it / (DH / 2);
    const uint16_t *up = U + (long)(2 * dp) * r + rt * AK + 8 * oc;
    ua[k] = gld16(up);
    ub[k] = gld16(up + r);
  }
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int it = tid + 256 * k, dp = it % (DH / 2), oc = it / (DH / 2);
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
  uint16_t *A = a.absA + (long)bh * FF * r + (long)(ft * AK) * r + rt * AK;
#pragma unroll
  for (int k = 0; k < AK * AK / 8 / 256; ++k) {
    const int pc = tid + 256 * k, row = pc / (AK / 8), part = pc % (AK / 8);
    *reinterpret_cast<u32x4 *>(A + (long)row * r + 8 * part) = *reinterpret_cast<const u32x4 *>(&sm.ot[row][8 * part]);
  }
}

// ---------------------------------------------------------------------------
// LDS of the attend kernel (bytes)
// ---------------------------------------------------------------------------
template <int R>
struct Smem {
  static constexpr int AS = 0;                            // 2 x [FH][ALD] bf16 A slabs
  static constexpr int QT = AS + 2 * FH * ALD * 2;        // [2][GQ][R] bf16 q~ hi, lo
  static constexpr int B1S = QT + 2 * GQ * R * 2;         // [FH] fp32 -log2(e) b1 of this half
  static constexpr int LGP = B1S + FH * 4;                // [4 fw][RT][GQ] fp32 logit parts
  static constexpr int PS = LGP + 4 * RT * GQ * 4;        // [RT][GQ] fp32 p of the round
  static constexpr int P16 = PS + RT * GQ * 4;            // [GQ][RT] fp16 p (MFMA operand)
  static constexpr int ST = P16 + GQ * RT * 2;            // [3][GQ] m, l, alpha
  static constexpr int RC = ST + 3 * GQ * 4;              // [2] residual row counts of the round's slices
  static constexpr int RL = RC + 4 * 4;                   // [2][MAXRES] residual rows (entry, token in round)
  static constexpr int SEL = RL + 2 * MAXRES * 4;         // [MAXSEL] selected chunks of (b, h)
  static constexpr int QF = SEL + MAXSEL * 4;             // [GQ][DH] fp32 q (tail)
  static constexpr int RS = QF + GQ * DH * 4;             // [RSTAGE][DH * ES] residual rows of the round
  static constexpr int BYTES = RS + RSTAGE * DH * 2;
  // the tail (second half, after the rounds) stages TCH tokens of K and V in the slab area
  static constexpr int TKS = 0, TVS = TKS + TCH * DH * 2;
  static_assert(TVS + TCH * DH * 2 <= QT, "tail staging does not fit");
  // end of the kernel: per-wave hidden sums [NW][FWV][GQ] over the A slabs
  static constexpr int AHM = 0;
  static_assert(AHM + NW * FWV * GQ * 4 <= QT, "merge area does not fit");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Block -> (b, h, split, half).  Workgroups are dispatched round-robin over
// the 8 XCDs; the linear id is remapped so that each XCD receives a contiguous
// run of (b, h, split, half): the two halves of a split share the coefficient
// tiles and the splits of a (b, h) share A in one L2.
__device__ __forceinline__ void coords(const AttendArgs &a, int &b, int &h, int &s, int &fh) {
  const int n = gridDim.x;
  int u = blockIdx.x;
  if (n % 8 == 0) u = (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8;
  fh = u & 1;
  s = (u >> 1) % a.n_split;
  const int bh = (u >> 1) / a.n_split;
  h = bh % a.Hkv;
  b = bh / a.Hkv;
}

template <typename TC, int NK>
__global__ __launch_bounds__(NTH, 1) void k_attend_absorb(const AttendArgs a) {
  constexpr int R = NK * KS;
  constexpr int DC = dc_of<NK>();
  using S = Smem<R>;
  using CT = Coef<TC>;
  extern __shared__ __align__(16) unsigned char sm[];
  uint16_t *As = reinterpret_cast<uint16_t *>(sm + S::AS);
  const uint16_t *Qt = reinterpret_cast<const uint16_t *>(sm + S::QT);
  float *B1s = reinterpret_cast<float *>(sm + S::B1S);
  float *Lgp = reinterpret_cast<float *>(sm + S::LGP);
  float *Ps = reinterpret_cast<float *>(sm + S::PS);
  uint16_t *P16 = reinterpret_cast<uint16_t *>(sm + S::P16);
  float *st = reinterpret_cast<float *>(sm + S::ST);   // m [GQ], l [GQ], alpha [GQ]
  int32_t *rc = reinterpret_cast<int32_t *>(sm + S::RC);
  int32_t *rl = reinterpret_cast<int32_t *>(sm + S::RL);
  int32_t *selS = reinterpret_cast<int32_t *>(sm + S::SEL);
  float *qf = reinterpret_cast<float *>(sm + S::QF);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tw = w & 1, fw = w >> 1;
  const int l16 = lane & 15, kg = lane >> 4;
  int b, h, s, fh;
  coords(a, b, h, s, fh);
  const int g = a.g, C = a.C;
  const long bh = ((long)b * a.G + a.layer) * a.Hkv + h;   // (b, layer, h)
  const long bhs = (long)b * a.Hkv + h;                      // (b, h)

  // ---- prologue ---------------------------------------------------------------
  const uint16_t *Aw = a.absA + bhs * (long)FF * R + (long)fh * FH * R;   // this half's rows of A
  const rsrc_t Ar = make_rsrc(Aw, (uint32_t)(FH * R * 2));
  // A slab pieces: thread loads 16 bytes of rows tid / 4 + 128 i, ranks 8 (tid % 4) + 32 ks
  const uint32_t a_voff = (uint32_t)(((tid >> 2) * R + 8 * (tid & 3)) * 2);
  auto slab_ld = [&](int ks, u32x4 *u) {
#pragma unroll
    for (int i = 0; i < SLAB_P; ++i)
      u[i] = __builtin_amdgcn_raw_buffer_load_b128(Ar, a_voff, (uint32_t)((ks * KS + i * (NTH / 4) * R) * 2), 0);
  };
  auto slab_st = [&](int buf, const u32x4 *u) {
#pragma unroll
    for (int i = 0; i < SLAB_P; ++i)
      lst16(As + buf * FH * ALD + ((tid >> 2) + i * (NTH / 4)) * ALD + 8 * (tid & 3), u[i]);
  };
  u32x4 ur[2][SLAB_P];
  slab_ld(0, ur[0]);
  slab_ld(1, ur[1]);

  const int k_eff = a.k_eff;
  const int32_t *selp = a.sel + bhs * k_eff;
  for (int i = tid; i < k_eff; i += NTH) selS[i] = selp[i];
  {  // q~ hi and lo rows of this (b, h)
    const uint16_t *Qg = a.absQ + bhs * 2 * GQ * R;
    for (int i = tid; i < 2 * GQ * R / 8; i += NTH)
      lst16(reinterpret_cast<uint16_t *>(sm + S::QT) + 8 * i, gld16(Qg + 8 * i));
  }
  const uint16_t *B1 = reinterpret_cast<const uint16_t *>(a.b1) + bh * FF + fh * FH;
  for (int i = tid; i < FH; i += NTH) B1s[i] = bf16_bits_to_f32(B1[i]) * NEG_LOG2E;
  if (tid < GQ) {
    st[tid] = -INFINITY;
    st[GQ + tid] = 0.f;
    st[2 * GQ + tid] = 0.f;
  }
  if (fh == 1) {  // the tail share needs q itself
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q) + ((long)b * a.Hq + (long)h * g) * DH;
    for (int i = tid; i < GQ * DH; i += NTH) qf[i] = (i / DH) < g ? bf16_bits_to_f32(qb[i]) : 0.f;
  }

  const int n_slices = k_eff * (C / TT);
  const int sl0 = s * a.tps, sl1 = min(n_slices, sl0 + a.tps);
  const int rounds = (a.tps + 1) / 2;
  const int r = R;
  const TC *cf = reinterpret_cast<const TC *>(a.coeff) + (long)b * a.N * r;
  const rsrc_t Cr = make_rsrc(cf, (uint32_t)((long)a.N * r * CT::ES));
  const uint32_t c_voff = (uint32_t)((l16 * r + 8 * kg) * CT::ES);   // + (row + 16 tt) r + 32 ks
  const int32_t *rptr = a.res_ptr + bh * (a.N / C + 1);
  const int32_t *ridx = a.res_idx + bh * a.n_res;
  // residual scales of this thread's two head dims (int8), residual-pass mapping:
  // thread (query head vg, dims 2 vd, 2 vd + 1)
  const int vg = tid >> 7, vd = 2 * (tid & 127);
  float rs0 = 1.f, rs1 = 1.f;
  if (sizeof(TC) == 1 && a.res_scale) {
    rs0 = f16_bits_to_f32(a.res_scale[bh * DH + vd]);
    rs1 = f16_bits_to_f32(a.res_scale[bh * DH + vd + 1]);
  }
  float accV0 = 0.f, accV1 = 0.f;   // first half: residual sums of (vg, vd), (vg, vd + 1)
  f32x4 accH[NFB];                  // hidden sums [16 g][16 f] per block (rows g < GQ live)
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) accH[fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // token row of slice sig for this wave (a slice past the split reads zeros)
  auto slice_row = [&](int sig) -> long {
    return sig < sl1 ? (long)selS[(sig * TT) / C] * C + (sig * TT) % C : (long)a.N;
  };
  auto c_soff = [&](long row, int tt, int ks) -> uint32_t {
    return (uint32_t)(((row + 16 * tt) * r + ks * KS) * CT::ES);
  };
  __syncthreads();
  slab_st(0, ur[0]);
  slab_ld(2, ur[0]);
  long row0 = slice_row(sl0 + tw);
  typename CT::raw cr[DC][NTT];   // coefficient ring: k-step ks in cr[ks % DC]
#pragma unroll
  for (int q = 0; q < DC - 1; ++q)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) cr[q][tt] = CT::ld(Cr, c_voff, c_soff(row0, tt, q));
  __syncthreads();

  static_assert(NK % DC == 0 && NK % 2 == 0 && NK >= 4, "ring sizes must divide the k-step count");
  for (int rd = 0; rd < rounds; ++rd) {
    const int sig = sl0 + 2 * rd + tw;
    const bool has = sig < sl1;
    const bool more = rd + 1 < rounds;
    const long row0n = more ? slice_row(sig + 2) : (long)a.N;
    // residual rows of this wave's slice (first half; waves fw == 0 list them)
    if (fh == 0 && fw == 0) {
      int cnt = 0;
      if (has) {
        const int jc = (int)(row0 / C), t0 = (int)(row0 % C);
        const int e0 = rptr[jc], e1 = rptr[jc + 1];
        for (int base = e0; base < e1; base += WAVE) {
          const int e = base + lane;
          const int t = e < e1 ? ridx[e] - jc * C - t0 : -1;
          const bool in = e < e1 && t >= 0 && t < TT;
          const uint64_t m = __ballot(in);
          const int pos = cnt + __popcll(m & lanemask_lt());
          if (in && pos < MAXRES) rl[tw * MAXRES + pos] = (e << 8) | (TT * tw + t);
          cnt += __popcll(m);
        }
      }
      if (lane == 0) rc[tw] = cnt;
    }
    // ---- k-loop: hidden pre-activations and logit parts ----------------------
    f32x4 acc[NTT][NFB];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) acc[tt][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 lg[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) lg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *a_rd = As + (FWV * fw + l16) * ALD + 8 * kg;   // + buf FH ALD + 16 fb ALD
    sfor<NK>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      constexpr int buf = ks & 1;
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
      // slab ks + 1 (of this round, or slab 0 of the next) -> the other buffer,
      // slab ks + 3 into the register ring; both buffers were last read before
      // the previous barrier
      if (ks + 1 < NK || more) {
        slab_st(buf ^ 1, ur[(ks + 1) & 1]);
        if (ks + 3 < NK || more) slab_ld((ks + 3) % NK, ur[(ks + 1) & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      f16x8 c8[NTT];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) c8[tt] = CT::get(cr[ks % DC][tt]);
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) {
        const f16x8 af = ldh8(a_rd + buf * FH * ALD + 16 * fb * ALD);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[tt][fb] = mfma(c8[tt], af, acc[tt][fb]);
      }
      if ((ks & 3) == fw) {  // this wave's turn at the logits: q~ hi, lo as B operands (head l16)
        const f16x8 z8 = __builtin_bit_cast(f16x8, v4(0, 0, 0, 0));
        const uint16_t *qr = Qt + l16 * r + ks * KS + 8 * kg;
        const f16x8 qh = l16 < GQ ? ldh8(qr) : z8, ql = l16 < GQ ? ldh8(qr + GQ * r) : z8;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          lg[tt] = mfma(c8[tt], qh, lg[tt]);
          lg[tt] = mfma(c8[tt], ql, lg[tt]);
        }
      }
      __syncthreads();
    });
    row0 = row0n;
    // residual rows of the round (first half): rows k < RSTAGE of the two
    // slices' lists, 16-byte pieces issued now and stored to LDS after SiLU
    constexpr int RPC = DH * (int)sizeof(TC) / 16;   // 16-byte pieces per row
    constexpr int RSP = RSTAGE * RPC / NTH;          // pieces per thread
    static_assert(RSTAGE * RPC % NTH == 0, "residual staging pieces");
    const TC *rval = reinterpret_cast<const TC *>(a.res_val) + bh * (long)a.n_res * DH;
    int n_r0 = 0, n_rows = 0;
    u32x4 rsv[RSP];
    if (fh == 0) {
      n_r0 = min(rc[0], MAXRES);
      n_rows = n_r0 + min(rc[1], MAXRES);
#pragma unroll
      for (int i = 0; i < RSP; ++i) {
        const int pc = tid + NTH * i, k = pc / RPC, part = pc % RPC;
        rsv[i] = v4(0, 0, 0, 0);
        if (k < n_rows) {
          const int code = k < n_r0 ? rl[k] : rl[MAXRES + k - n_r0];
          rsv[i] = gld16(reinterpret_cast<const unsigned char *>(rval) + ((long)(code >> 8) * DH * sizeof(TC)) + 16 * part);
        }
      }
    }
    // ---- logits of the round: parts of the four waves of each slice ---------
    // lg[tt] lane (l16 = head, kg): tokens 16 tt + 4 kg + v of the slice
    if (l16 < GQ) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) Lgp[(fw * RT + TT * tw + 16 * tt + 4 * kg + v) * GQ + l16] = lg[tt][v];
    }
    // SiLU of the pre-activations (independent of the softmax): hidden block fb,
    // token pair i of blocks (2 i, 2 i + 1) as the fp16 B operand of the p . H product
    f16x8 hb[NTT / 2][NFB];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
      const float bias = B1s[FWV * fw + 16 * fb + l16];
#pragma unroll
      for (int i = 0; i < NTT / 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hb[i][fb][v] = (_Float16)silu_scaled(acc[2 * i][fb][v] + bias);
          hb[i][fb][4 + v] = (_Float16)silu_scaled(acc[2 * i + 1][fb][v] + bias);
        }
    }
    if (fh == 0) {
      unsigned char *rs = sm + S::RS;
#pragma unroll
      for (int i = 0; i < RSP; ++i) {
        const int pc = tid + NTH * i;
        if (pc / RPC < n_rows) lst16(rs + 16 * pc, rsv[i]);
      }
    }
    __syncthreads();
    // ---- softmax of the round, workgroup-wide: waves 0..3 take head w --------
    if (w < GQ) {
      const int gi = w;
      float x[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = lane + WAVE * u;           // token of the round
        const int sl = sl0 + 2 * rd + u;         // its slice
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) v += Lgp[(k * RT + t) * GQ + gi];
        x[u] = (sl < sl1 && gi < g) ? v * a.scale_log2 : -INFINITY;
      }
      const float mx = wave_max(fmaxf(x[0], x[1]));
      const float m_old = st[gi], m_new = fmaxf(m_old, mx);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
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
      const f16x8 z8 = __builtin_bit_cast(f16x8, v4(0, 0, 0, 0));
#pragma unroll
      for (int i = 0; i < NTT / 2; ++i) {
        f16x8 pa = z8;
        if (l16 < GQ) {
          const uint16_t *pr = P16 + l16 * RT + TT * tw + 32 * i + 4 * kg;
          const uint2 lo = *reinterpret_cast<const uint2 *>(pr);
          const uint2 hi = *reinterpret_cast<const uint2 *>(pr + 16);
          pa = __builtin_bit_cast(f16x8, v4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) accH[fb] = mfma(pa, hb[i][fb], accH[fb]);
      }
    }
    // ---- residual rows of the round (first half, vector ALUs): thread
    // (head vg, dims vd, vd + 1); staged rows from LDS, any past RSTAGE from
    // global memory eight at a time ----------------------------------------------
    if (fh == 0) {
      const float alpha = st[2 * GQ + vg];
      accV0 *= alpha;
      accV1 *= alpha;
      if (vg < g) {
        const unsigned char *rs = sm + S::RS;
        const int ns = min(n_rows, RSTAGE);
        for (int k = 0; k < ns; ++k) {
          const int code = k < n_r0 ? rl[k] : rl[MAXRES + k - n_r0];
          const float p = Ps[(code & 0xFF) * GQ + vg];
          float x0, x1;
          ResRow<TC>::get(rs + (long)k * DH * sizeof(TC), 0, vd, rs0, rs1, x0, x1);
          accV0 = fmaf(p, x0, accV0);
          accV1 = fmaf(p, x1, accV1);
        }
        for (int k0 = RSTAGE; k0 < n_rows; k0 += 8) {
          float x0v[8], x1v[8], pv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int k = min(k0 + u, n_rows - 1);
            const int code = k < n_r0 ? rl[k] : rl[MAXRES + k - n_r0];
            pv[u] = k0 + u < n_rows ? Ps[(code & 0xFF) * GQ + vg] : 0.f;
            ResRow<TC>::get(rval, (long)(code >> 8), vd, rs0, rs1, x0v[u], x1v[u]);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            accV0 = fmaf(pv[u], x0v[u], accV0);
            accV1 = fmaf(pv[u], x1v[u], accV1);
          }
        }
      }
    }
    __syncthreads();   // round's LDS (logit parts, p, residual lists) free again
  }

  // ---- partial rows -------------------------------------------------------------
  const int n_prow = 2 * a.n_split;   // partial rows per (b, h): chunk rows, then tail rows
  float *part = a.part + (bhs * n_prow + s) * g * a.PW;
  // hidden sums of the two slices' waves of each block of 64 units
  float *ahm = reinterpret_cast<float *>(sm + S::AHM);
  if (kg == 0) {
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
      *reinterpret_cast<f32x4 *>(ahm + ((w * FWV) + 16 * fb + l16) * GQ) = accH[fb];
  }
  __syncthreads();
  for (int i = tid; i < FH * GQ; i += NTH) {   // (unit of the half, head)
    const int f = i / GQ, gi = i % GQ, fwi = f / FWV, fl = f % FWV;
    const float x = ahm[((2 * fwi) * FWV + fl) * GQ + gi] + ahm[((2 * fwi + 1) * FWV + fl) * GQ + gi];
    if (gi < g) part[(long)gi * a.PW + 4 + fh * FH + f] = x * NEG_LN2;
  }
  if (fh == 0) {
    if (tid < g) {
      part[(long)tid * a.PW + 0] = st[tid];
      part[(long)tid * a.PW + 1] = st[GQ + tid];
      part[(long)tid * a.PW + 2] = st[GQ + tid];
      part[(long)tid * a.PW + 3] = 0.f;
    }
    if (vg < g) {
      part[(long)vg * a.PW + 4 + FF + vd] = accV0;
      part[(long)vg * a.PW + 4 + FF + vd + 1] = accV1;
    }
    return;
  }

  // ---- second half: this split's share of the tail, its own partial row -----------
  // Chunks of TCH tokens: K and V rows staged in the (now free) slab area with
  // all loads in flight at once, logits per wave and token (lane: 4 head dims),
  // then an online softmax per query head over the chunks.
  const int tb = min(a.T, s * a.tail_per_split), te = min(a.T, tb + a.tail_per_split);
  const long tail_base = (bh * a.T) * DH;
  const uint16_t *kt = reinterpret_cast<const uint16_t *>(a.k_tail) + tail_base;
  const uint16_t *vt = reinterpret_cast<const uint16_t *>(a.v_tail) + tail_base;
  uint16_t *tks = reinterpret_cast<uint16_t *>(sm + S::TKS), *tvs = reinterpret_cast<uint16_t *>(sm + S::TVS);
  float *tp = Ps;   // [TCH][GQ] logits, then p, of the chunk
  if (tid < GQ) {
    st[tid] = -INFINITY;
    st[GQ + tid] = 0.f;
  }
  float tv0 = 0.f, tv1 = 0.f;   // (vg, vd), (vg, vd + 1)
  constexpr int TPC = TCH * DH / 8 / NTH;   // 16-byte pieces per thread of K (and of V)
  for (int c0 = tb; c0 < te; c0 += TCH) {
    const int nt = min(TCH, te - c0);
    u32x4 kp[TPC], vp[TPC];
#pragma unroll
    for (int i = 0; i < TPC; ++i) {
      const int pc = tid + NTH * i, t = pc / (DH / 8), part = pc % (DH / 8);
      const long off = (long)(c0 + min(t, nt - 1)) * DH + 8 * part;
      kp[i] = gld16(kt + off);
      vp[i] = gld16(vt + off);
    }
#pragma unroll
    for (int i = 0; i < TPC; ++i) {
      const int pc = tid + NTH * i;
      lst16(tks + 8 * pc, kp[i]);
      lst16(tvs + 8 * pc, vp[i]);
    }
    __syncthreads();
    for (int t = w; t < nt; t += NW) {
      const uint2 kr = *reinterpret_cast<const uint2 *>(tks + t * DH + 4 * lane);
      const float k4[4] = {bf16_bits_to_f32(kr.x & 0xFFFFu), bf16_bits_to_f32(kr.x >> 16),
                           bf16_bits_to_f32(kr.y & 0xFFFFu), bf16_bits_to_f32(kr.y >> 16)};
      float x[GQ];
#pragma unroll
      for (int gi = 0; gi < GQ; ++gi) {
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(qf + gi * DH + 4 * lane);
        x[gi] = fmaf(qv[0], k4[0], fmaf(qv[1], k4[1], fmaf(qv[2], k4[2], qv[3] * k4[3])));
      }
#pragma unroll
      for (int gi = 0; gi < GQ; ++gi) x[gi] = wave_sum(x[gi]);
      const float xl = lane == 0 ? x[0] : lane == 1 ? x[1] : lane == 2 ? x[2] : x[3];
      if (lane < GQ) tp[t * GQ + lane] = lane < g ? xl * a.scale_log2 : -INFINITY;
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
    if (vg < g) {
      const float alpha = st[2 * GQ + vg];
      tv0 *= alpha;
      tv1 *= alpha;
      for (int t = 0; t < nt; ++t) {
        const float p = tp[t * GQ + vg];
        const uint32_t v2 = *reinterpret_cast<const uint32_t *>(tvs + t * DH + vd);
        tv0 = fmaf(p, bf16_bits_to_f32(v2 & 0xFFFFu), tv0);
        tv1 = fmaf(p, bf16_bits_to_f32(v2 >> 16), tv1);
      }
    }
    __syncthreads();   // the chunk's staging and p are free again
  }
  float *tpart = a.part + (bhs * n_prow + a.n_split + s) * g * a.PW;
  if (tid < g) {
    tpart[(long)tid * a.PW + 0] = st[tid];
    tpart[(long)tid * a.PW + 1] = st[GQ + tid];
    tpart[(long)tid * a.PW + 2] = 0.f;
    tpart[(long)tid * a.PW + 3] = 0.f;
  }
  for (int i = tid; i < g * FF; i += NTH) tpart[(long)(i / FF) * a.PW + 4 + i % FF] = 0.f;
  if (vg < g) {
    tpart[(long)vg * a.PW + 4 + FF + vd] = tv0;
    tpart[(long)vg * a.PW + 4 + FF + vd + 1] = tv1;
  }
}

template <typename TC, int NK>
static hipError_t go(const AttendArgs &a, hipStream_t st) {
  const size_t smem = Smem<NK * KS>::BYTES;
  static const bool lds_ok = (allow_dynamic_lds(k_attend_absorb<TC, NK>, smem), true);
  (void)lds_ok;
  hipLaunchKernelGGL((k_attend_absorb<TC, NK>), dim3(a.B * a.Hkv * a.n_split * 2), dim3(NTH), smem, st, a);
  return hipGetLastError();
}

}  // namespace absorb

bool absorb_supported(int act, int coeff, int resid, int dh, int F, int r, int C, int g, int k_eff) {
  return act == LOWRAM_BF16 && coeff == resid && (coeff == LOWRAM_BF16 || coeff == LOWRAM_I8) &&
         dh == absorb::DH && F == absorb::FF && (r == 384 || r == 512) && C % absorb::TT == 0 &&
         g <= absorb::GQ && k_eff >= 1 && k_eff <= absorb::MAXSEL;
}

// Splits per (b, h): about one workgroup per CU over the two halves, at least
// one round (two slices) per split, at most 32 splits (64 partial rows with the
// tail's); tps = 64-token slices per split (even); tail tokens per split.
void absorb_plan(int B, int Hkv, int k_eff, int C, int T, int &n_split, int &tps, int &tail_per_split) {
  const int n_slices = k_eff * (C / absorb::TT);
  int want = (256 + 2 * B * Hkv - 1) / (2 * B * Hkv);
  const int max_split = (n_slices + 1) / 2;
  if (want > max_split) want = max_split;
  if (want > 32) want = 32;
  if (want < 1) want = 1;
  tps = (n_slices + want - 1) / want;
  tps += tps & 1;
  n_split = (n_slices + tps - 1) / tps;
  tail_per_split = (T + n_split - 1) / n_split;
  if (tail_per_split > absorb::RT) {  // the tail share must fit one round's p area
    n_split = (T + absorb::RT - 1) / absorb::RT;
    tps = (n_slices + n_split - 1) / n_split;
    tps += tps & 1;
    tail_per_split = (T + n_split - 1) / n_split;
  }
}

hipError_t launch_absorb(const AttendArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(absorb::k_absorb, dim3(absorb::FF / absorb::AK, a.r / absorb::AK, a.B * a.Hkv), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_attend_absorb(int coeff, const AttendArgs &a, hipStream_t st) {
  const bool i8 = coeff == LOWRAM_I8;
  if (a.r == 384) return i8 ? absorb::go<int8_t, 12>(a, st) : absorb::go<bf16, 12>(a, st);
  if (a.r == 512) return i8 ? absorb::go<int8_t, 16>(a, st) : absorb::go<bf16, 16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lowram
