// Internal declarations shared by the host layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lowram.h"

namespace lowram {

// Kernel-side view of one decode call (device pointers, sizes).
struct AttendArgs {
  const void *q;          // [B][Hq][dh] act
  const void *basis;      // [B][D][r] act
  const void *w1, *b1;    // [B][G][Hkv][F][dh], [B][G][Hkv][F] act
  const void *coeff;      // [B][N][r] coeff
  const uint16_t *coeff_scale;  // [B][r] f16 or null
  const int32_t *res_ptr;       // [B][G][Hkv][n_c+1]
  const int32_t *res_idx;       // [B][G][Hkv][n_res]
  const void *res_val;          // [B][G][Hkv][n_res][dh] resid
  const uint16_t *res_scale;    // [B][G][Hkv][dh] f16 or null
  const void *k_tail, *v_tail;  // [B][G][Hkv][T][dh] act
  const int32_t *sel;           // [B][Hkv][k_eff]
  const double *score_part;     // [B][Hkv][select_rank_blocks(r)][n_c] fp64 partial chunk scores
                                // when the attend kernel selects itself, else null
  int32_t *sel_out;             // [B][Hkv][k_eff] copy of the selection (in-kernel selection only) or null
  // reuse of rebuilt tiles across steps (register-chained kernel only); rtiles
  // null when reuse is off.  The slot table has two halves; the clock's parity
  // names the current one, the combine advances the clock.
  void *rtiles;                 // [B][G][Hkv][rslots][chain_tile_bytes(F)]: rebuilt keys
  int32_t *rt_chunk;            // [B][G][Hkv][2][rslots] chunk held by each slot, -1 if none
  int32_t *rt_stamp;            // [B][G][Hkv][2][rslots] use count of each slot's last use
  const int32_t *rclock;        // [B][G][Hkv] calls made on each head's table
  int32_t *rhits;               // [B][Hkv] chunks read back this step, or null
  int rslots;
  float *part;                  // [B][Hkv][n_split+1][g][PW]
  int B, G, Hq, Hkv, dh, r, F, N, C, T, k_eff, n_res, layer;
  int g, cps, n_split, PW;
  int path;                     // LOWRAM_PATH_* of these dims
  int tps, tail_per_split;      // chained / absorbed kernels: tiles (slices) and tail tokens per split
  int vsub;                     // vector kernel: token ranges per selected chunk (split = slot * vsub + range)
  float scale_log2;             // log2(e) / sqrt(dh)
  const float *qtg;             // chained kernel: [B][Hkv][QTG_G][r] float32 U_{l,h}^T q_g (select stage)
  const uint16_t *qfrag;        // per-chunk kernel: [B][Hkv][2][16][r] hi/lo operand columns (select stage)
  // absorbed kernel (head dim 256): workspace of the absorbed first layer
  uint16_t *absA;               // [B][Hkv][F][r] fp16: -log2(e) W1 U_{l,h} (int8: times the rank scales)
  uint16_t *absQ;               // [B][Hkv][2][4][r] fp16: U_{l,h}^T q_g, hi then lo parts
};

struct CombineArgs {
  const float *part;    // [B][Hkv][n_total][g][PW]
  int32_t *rclock;      // [B][G][Hkv] reuse clocks advanced once per (b, h), or null
  const void *w2, *b2;  // [B][G][Hkv][dh][F], [B][G][Hkv][dh] act (null when F == 0)
  void *out;            // [B][Hq][dh] act
  // rows [0, n_comp) of the n_total per (b, h) carry rebuilt chunks; the rows
  // after them hold tail tokens only, and their hidden sums (zero) are not read
  int B, G, Hq, Hkv, dh, F, layer, g, n_comp, n_total, PW;
};

// launchers (return hipSuccess or the launch error)
// Chunk scores (float64).  Partial scores per block of 64 ranks go to part
// [B][Hkv][select_rank_blocks(r)][n_c] (workspace); the score of a chunk is the
// sum of its partials in block order.  If scores is not null the sums are
// written to scores [B][Hkv][n_c], and if k_eff > 0 (scores required) the
// selection into sel and, optionally, a copy into sel_out.
inline int select_rank_blocks(int r) { return (r + 63) / 64; }
// Besides the scores, the partial-score kernel can write q~_g = U_{l,h}^T q_g
// of the query heads of every kv head, for the kernels that take logits in
// coefficient space:
//  qtg:   float32 [B][Hkv][QTG_G][r] (g <= QTG_G; rows past the group zero),
//         the chained kernel's form;
//  qfrag: 16-bit [B][Hkv][2][16][r] MFMA operand columns of hi/lo halves
//         (mode 1: bf16; mode 2: fp16 of q~ times the int8 rank scales
//         `scale` [B][r]), the per-chunk kernel's form (g <= 16).
constexpr int QTG_G = 4;
constexpr int QTG_MAX = 16;
struct QOut {
  float *qtg = nullptr;
  uint16_t *qfrag = nullptr;
  const uint16_t *scale = nullptr;
  int mode = 0;
};
hipError_t launch_select(int act, const void *q, long q_bstride, const void *basis,
                         const float *landmark, int B, int Hq, int Hkv, int dh, int r, int n_c,
                         int D, int layer, int k_eff, int32_t *sel, int32_t *sel_out,
                         double *part, double *scores, hipStream_t st, const QOut &qo = QOut(),
                         const AttendArgs *absorb = nullptr);
hipError_t launch_attend(int act, int coeff, int resid, const AttendArgs &a, hipStream_t st);
// True when the per-chunk MFMA kernel covers these shapes (else the VALU kernel)
bool mfma_supported(const AttendArgs &a, int act, int coeff, int resid);
// Register-chained rebuild-and-attend: the shapes it covers, its split plan
// (splits per (b, h), 64-token tiles per split, tail tokens per split) and the
// launcher.  Its partials fold the tail in: n_split of them per (b, h).
bool chain_supported(int act, int coeff, int resid, int dh, int F, int r, int C, int g, int k_eff);
// Largest chunk count for which the chained kernel ranks the fp64 chunk scores
// itself (each workgroup, in its prologue) instead of reading a selection.
constexpr int CHAIN_SELECT_MAX_NC = 512;
void chain_plan(int B, int Hkv, int k_eff, int C, int T, int &n_split, int &tps, int &tail_per_split);
hipError_t launch_attend_chain(int coeff, const AttendArgs &a, hipStream_t st);
// Largest chunk count for which the absorbed kernel ranks the chunk scores
// itself (one chunk per thread of its prologue).
constexpr int ABSORB_SELECT_MAX_NC = 256;
// Absorbed-first-layer rebuild-and-attend (head dim 256): shapes, split plan
// (splits per (b, h), 64-token slices per split, tail tokens per split), the
// per-call formation of A = W1 U_{l,h} and q~ (in the launch of the partial
// chunk scores) and the attend launcher.  1 + 3 partial rows per split: the
// split's chunks, then three shares of its part of the tail.
bool absorb_supported(int act, int coeff, int resid, int dh, int F, int r, int C, int g, int k_eff);
void absorb_plan(int B, int Hkv, int k_eff, int C, int T, int &n_split, int &tps, int &tail_per_split,
                 int &n_part);
hipError_t launch_attend_absorb(int coeff, const AttendArgs &a, hipStream_t st);
// The partial chunk scores (bf16, d_h = 256) and A, q~ into the workspace,
// in one launch.
hipError_t launch_select_absorb(const AttendArgs &a, const float *landmark, double *part, long q_bstride,
                                hipStream_t st);
constexpr int REUSE_HIT = 1 << 30;
size_t chain_tile_bytes(int F);  // bytes of one cached 128-token chunk (its rebuilt keys)
constexpr int REUSE_MAX_SLOTS = 256;
hipError_t launch_combine(int act, const CombineArgs &a, hipStream_t st);
hipError_t launch_dense(int act, const void *q, const void *k, const void *v, long batch_stride,
                        int B, int Hq, int Hkv, int dh, int n, int tps, int n_split, float *part,
                        int PW, hipStream_t st);

struct CompressArgs {
  const void *k, *v;            // [B][G][Hkv][N][dh] act
  const void *basis, *w1, *b1, *w2, *b2;
  void *coeff;                  // [B][N][r] coeff
  uint16_t *coeff_scale;        // [B][r]
  float *landmark;              // [B][n_c][r]
  int32_t *res_ptr, *res_idx;
  void *res_val;
  uint16_t *res_scale;
  double *c64;                  // workspace [B][N][r] (int8 coefficients only)
  double *err;                  // workspace [B][G][Hkv][N]
  double *d64;                  // workspace [B][G][Hkv][n_res][dh] (int8 residuals only)
  int B, G, Hq, Hkv, dh, r, F, N, C, n_res, act, coeff_dt, resid_dt;
};
hipError_t run_compress(const CompressArgs &a, hipStream_t st);
void compress_coefficients(const CompressArgs &a, hipStream_t st);  // C1 (+ Q1) only

struct FitArgs {
  const void *basis, *w1, *b1, *w2, *b2;  // initial weights (act)
  const void *k, *v;                       // [B][G][Hkv][N][dh] act
  void *o_w1, *o_b1, *o_w2, *o_b2;         // fitted weights (act); may alias the initial ones
  double *loss;                            // [B][G][Hkv][steps + 1] or null
  void *coeff; uint16_t *coeff_scale; double *c64;  // workspace: stored coefficients
  float *khat, *apre, *hid, *res;          // workspace: [z][N][dh], [z][N][F], [z][N][F], [z][N][dh]
  float *m_w1, *m_b1, *m_w2, *m_b2;        // workspace: float32 master weights
  double *part;                            // workspace: [z][64][max(F, dh)] partial sums
  int B, G, Hkv, dh, r, F, N, steps, act, coeff_dt;
  float lr;
};
hipError_t run_fit(const FitArgs &a, hipStream_t st);

struct BasisArgs {
  const void *k;                 // [B][G][Hkv][N][dh] act
  void *basis;                   // [B][D][r] act (output)
  float *gram;                   // workspace [B][D][D]
  float *yt, *qt;                // workspace [B][r][D] each
  float *cbuf;                   // workspace [B][32][r]
  float *cpart;                  // workspace [B][16][32][r]: sliced block dots
  double *nrm;                   // workspace [B][32]
  double *mpart;                 // workspace [B][ceil(D / 256)][32][32]: in-block Gram slices
  double *tri;                   // workspace [B][32][32]: inverse Cholesky factor of a block
  int32_t *dep;                  // workspace [B][32]: rows of a block replaced as dependent
  int B, G, Hkv, dh, r, N, iterations, act;
};
hipError_t run_basis(const BasisArgs &a, hipStream_t st);
int basis_max_dim();             // largest D the basis kernels take

struct EvictArgs {
  const void *basis;
  const void *obs_q;            // [n_obs][B][G][Hq][dh]
  int n_obs, keep;
  const void *coeff; const float *landmark;
  const int32_t *res_ptr, *res_idx; const void *res_val;
  void *d_coeff; float *d_landmark; int32_t *d_res_ptr, *d_res_idx; void *d_res_val;  // d_coeff null: count only
  int d_n_res;                  // residual rows per (b, l, h) that dst holds
  int32_t *keep_out;            // [B][keep]
  int32_t *live_out;            // [B][G][Hkv] residual rows of the kept chunks, or null
  double *spart;                // workspace [B][Hkv][select_rank_blocks(r)][n_c]
  double *scores;               // workspace [B][Hkv][n_c]
  double *acc;                  // workspace [B][n_c]
  int B, G, Hq, Hkv, dh, r, N, C, n_res, act, coeff_dt, resid_dt;
};
hipError_t run_evict(const EvictArgs &a, hipStream_t st);

struct RepackArgs {
  const void *basis, *w1, *b1, *w2, *b2;
  const void *k_tail, *v_tail;  // [B][G][Hkv][T][dh] act; tokens [0, C) are packed
  const void *coeff; const uint16_t *coeff_scale; const float *landmark;
  const int32_t *res_ptr, *res_idx; const void *res_val; const uint16_t *res_scale;
  void *d_coeff; uint16_t *d_coeff_scale; float *d_landmark;
  int32_t *d_res_ptr, *d_res_idx; void *d_res_val; uint16_t *d_res_scale;
  double *err;                  // workspace [B][G][Hkv][C]
  double *c64;                  // workspace [B][C][r] (int8 coefficients only)
  double *part;                 // workspace [S][B][C][r], S = project_splits(B, C, D, r) > 1
  int32_t *t_idx;               // workspace [B][G][Hkv][C]
  int32_t *t_ptr;               // workspace [B][G][Hkv][2]
  double *dall;                 // workspace [B][G][Hkv][C][dh]: float64 delta of every new token
  int B, G, Hq, Hkv, dh, r, F, N, C, T, n_res, m, act, coeff_dt, resid_dt;
};
hipError_t run_repack(const RepackArgs &a, hipStream_t st);

// Slices of the D-long reduction of a projection of N tokens: doubled while the
// launch stays within about 512 workgroups and each slice keeps >= 256 of D.
inline int project_splits(int B, int N, int D, int r) {
  const long tiles = (long)((r + 63) / 64) * ((N + 63) / 64) * B;
  int S = 1;
  while (tiles * S * 2 <= 512 && D / (S * 2) >= 256) S *= 2;
  return S;
}

// Kernels with more than 64 KiB of dynamic LDS declare it once per instantiation.
template <typename K>
inline void allow_dynamic_lds(K kernel, size_t bytes) {
  if (bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

inline int dtype_bytes(int dt) {
  return dt == LOWRAM_F32 ? 4 : (dt == LOWRAM_I8 ? 1 : 2);
}

}  // namespace lowram
