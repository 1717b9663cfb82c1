/*
 * lowram.h -- C ABI of the MI355X (gfx950) compressed-KV decode-attention library.
 *
 * The method (LowRAM: "Low-Rank Keys and Amortised Values for Composable KV
 * Cache Compression at Test-Time", abstract on mlinfo.pages.dev; summaries on
 * zicq.com and rit.work) stores
 *   - keys of a group of adjacent layers as per-token coefficients on a shared
 *     low-rank basis (zicq.com English summary, "Cross-Layer Low-Rank Key
 *     Compression"; xKV on the rit.work page),
 *   - values as a per-head predictor V_hat = f(K) plus residuals
 *     delta = V - V_hat for the tokens it reconstructs worst (zicq.com English
 *     summary, "Core Mechanism"; abstract),
 * and at each decode step rebuilds only the query-selected context chunks,
 * while tokens produced after prefill stay uncompressed (rit.work page,
 * generation section).  Attention is softmax(q K^T / sqrt(d_h)) V (OjaKV page,
 * section 3).
 *
 * Conventions for every entry point
 *   Ownership   The caller owns every buffer.  All tensor pointers are DEVICE
 *               pointers unless a comment says "host".  The library never
 *               allocates or frees memory, keeps no pointer after return and
 *               never synchronises the stream.
 *   Ordering    Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *               stream) in call order; outputs are valid once that work ends.
 *   Errors      Arguments are validated on the host before anything is
 *               enqueued; on error nothing is enqueued and a status is
 *               returned.  LOWRAM_E_HIP means a launch failed (the stream may
 *               then hold part of the work).  lowram_last_error() returns a
 *               thread-local message for the last failing call on the thread.
 *   Alignment   Every tensor pointer must be 16-byte aligned; the workspace
 *               256-byte aligned.
 *   Threads     Functions are re-entrant; calls that share output buffers or a
 *               workspace must not overlap.
 *   Layouts     Row-major, innermost index last.  D = layers * heads_kv *
 *               head_dim, ordered (layer, kv head, dim).  n_c = n_ctx / chunk.
 *               GQA: query head g reads kv head (g * heads_kv) / heads_q.
 *   Dtypes      act = F32: everything float32.  act = BF16: q, out, K, V, tail,
 *               basis and predictor in bfloat16; coeff and resid BF16 or I8
 *               (int8 with float16 per-channel scales).  Landmarks are always
 *               float32, indices int32.
 */
#ifndef LOWRAM_H
#define LOWRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOWRAM_OK = 0,
  LOWRAM_E_INVALID = 1,      /* bad sizes, pointers, alignment or layer index    */
  LOWRAM_E_UNSUPPORTED = 2,  /* valid request outside what the kernels implement */
  LOWRAM_E_WORKSPACE = 3,    /* workspace too small                               */
  LOWRAM_E_HIP = 4           /* a HIP launch failed                               */
} lowram_status;

typedef enum { LOWRAM_F32 = 0, LOWRAM_BF16 = 1, LOWRAM_F16 = 2, LOWRAM_I8 = 3 } lowram_dtype;

typedef enum {
  LOWRAM_OP_COMPRESS = 0,
  LOWRAM_OP_DECODE = 1,
  LOWRAM_OP_EVICT = 2,
  LOWRAM_OP_DENSE = 3,
  LOWRAM_OP_REPACK = 4,
  LOWRAM_OP_FIT = 5,
  LOWRAM_OP_BASIS = 6
} lowram_op;

/* Sizes of one xKV group over a batch.  All counts are per sequence. */
typedef struct {
  int32_t batch;      /* B: sequences                                      */
  int32_t layers;     /* G: layers in the group                            */
  int32_t heads_q;    /* H_q                                               */
  int32_t heads_kv;   /* H_kv, divides H_q, H_q / H_kv <= 16               */
  int32_t head_dim;   /* d_h, multiple of 8, <= 256                        */
  int32_t rank;       /* r, multiple of 8, <= D                            */
  int32_t hidden;     /* F: predictor hidden width, multiple of 8          */
  int32_t n_ctx;      /* N: compressed tokens, multiple of chunk (may be 0)*/
  int32_t chunk;      /* C: tokens per chunk                               */
  int32_t top_k;      /* chunks selected per kv head; clamped to n_c       */
  int32_t n_tail;     /* T: uncompressed tail tokens (may be 0)            */
  int32_t n_res;      /* residual capacity per (b, layer, kv head), <= N   */
  int32_t act;        /* lowram_dtype of q/out/K/V/tail/basis/predictor    */
  int32_t coeff;      /* lowram_dtype of the coefficients                  */
  int32_t resid;      /* lowram_dtype of the residual rows                 */
} lowram_dims;

/* Per-context state that is not per token: the group basis and the per-head
 * value predictor f(k) = W2 SiLU(W1 k + b1) + b2 (act dtype). */
typedef struct {
  const void *basis;  /* [B][D][r]          */
  const void *w1;     /* [B][G][Hkv][F][dh] */
  const void *b1;     /* [B][G][Hkv][F]     */
  const void *w2;     /* [B][G][Hkv][dh][F] */
  const void *b2;     /* [B][G][Hkv][dh]    */
} lowram_model;

/* The compressed cache of one group. */
typedef struct {
  void *coeff;        /* [B][N][r] coeff dtype: per-token coefficients shared by the group */
  void *coeff_scale;  /* [B][r] float16 when coeff is I8, else NULL                        */
  float *landmark;    /* [B][n_c][r] float32: mean dequantised coefficient of each chunk   */
  int32_t *res_ptr;   /* [B][G][Hkv][n_c+1]: residual rows of chunk j are [ptr[j], ptr[j+1]) */
  int32_t *res_idx;   /* [B][G][Hkv][n_res]: token index of each residual row, ascending   */
  void *res_val;      /* [B][G][Hkv][n_res][dh] resid dtype: delta = v - v_hat              */
  void *res_scale;    /* [B][G][Hkv][dh] float16 when resid is I8, else NULL                */
} lowram_cache;

/* Predictor weights written by lowram_fit_predictor (act dtype, shapes as in
 * lowram_model). */
typedef struct {
  void *w1;           /* [B][G][Hkv][F][dh] */
  void *b1;           /* [B][G][Hkv][F]     */
  void *w2;           /* [B][G][Hkv][dh][F] */
  void *b2;           /* [B][G][Hkv][dh]    */
} lowram_predictor;

/* Workspace bytes `op` needs for these dims (host only, enqueues nothing). */
lowram_status lowram_workspace_bytes(const lowram_dims *dims, int32_t op, size_t *bytes);

/* Which rebuild-and-attend kernel decode calls with these dims run (host only,
 * enqueues nothing).  *path is one of:
 *   LOWRAM_PATH_CHAIN  register-chained kernel (d_h = 128, C = 128, g <= 4,
 *                      compiled (r, F, dtype) shapes); with n_c <= 512 it also
 *                      ranks the chunk scores in its prologue;
 *   LOWRAM_PATH_ABSORB head dim 256 (F = 512, r = 384 or 512, g <= 4): the
 *                      first predictor layer absorbed into the basis
 *                      (A = W1 U_{l,h}, formed per call in the workspace) and
 *                      logits taken in coefficient space, on the matrix cores;
 *                      with n_c <= 256 it also ranks the chunk scores in its
 *                      prologue;
 *   LOWRAM_PATH_MFMA   one workgroup per selected chunk on the matrix cores
 *                      (other bf16 shapes compiled for it, g <= 16), logits in
 *                      coefficient space;
 *   LOWRAM_PATH_VALU   vector-ALU kernel (float32 and every other shape);
 *   LOWRAM_PATH_NONE   no chunk is selected (top_k = 0): only the tail.
 * The choice depends on the dims alone; results agree with the oracle on
 * every path. */
enum { LOWRAM_PATH_NONE = 0, LOWRAM_PATH_CHAIN = 1, LOWRAM_PATH_MFMA = 2, LOWRAM_PATH_VALU = 3,
       LOWRAM_PATH_ABSORB = 4 };
lowram_status lowram_decode_kernel(const lowram_dims *dims, int32_t *path);

/* Storage accounting (host only).  *dense = M_KV = 2 L H_kv d_h N s for the
 * group with s = 2 (bf16) or 4 (f32 act) -- the M_KV formula of the zicq.com
 * English summary, "Core Mechanism" -- and *compressed = coefficients + basis
 * + predictor + residual rows with int32 indices (n_res of them) + CSR
 * pointers + float32 landmarks + fp16 scales, per sequence.  The tail is
 * identical on both sides and counted in neither.  Either pointer may be NULL. */
lowram_status lowram_cache_bytes(const lowram_dims *dims, uint64_t *compressed, uint64_t *dense);

/* Compress a prefill of N tokens (zicq.com "Core Mechanism" and "Cross-Layer
 * Low-Rank Key Compression"; abstract).  For each sequence:
 *   c_t = U^T k_t^cat, stored rounded to coeff dtype (I8: per-channel scales
 *   over the N tokens, s = fp16(max|c|/127), q = clamp(rne(c/s), +-127));
 *   e_t = ||v_t - f_{l,h}(U_{l,h} deq(c_t))||^2 in float64 per (layer, head);
 *   the n_res tokens with the largest e (lowest index wins ties) keep
 *   delta = v - v_hat rounded to resid dtype (I8: per-dim scales over those
 *   rows), stored in ascending token order with chunk CSR pointers;
 *   landmark_j = mean of deq(c_t) over chunk j, float64 rounded to float32.
 * k, v: [B][G][Hkv][N][dh] act dtype.  out: every cache pointer the dtypes
 * need.  Workspace: lowram_workspace_bytes(LOWRAM_OP_COMPRESS). */
lowram_status lowram_compress(const lowram_dims *dims, const lowram_model *model, const void *k,
                              const void *v, const lowram_cache *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* One decode step of attention at `layer` of the group for one new query per
 * sequence (rit.work generation section; OjaKV section 3).  For each (b, kv
 * head h):
 *   q~ = U_{l,h}^T sum_{g in group(h)} q_g and s_j = q~ . landmark_j in
 *   float64; the top min(top_k, n_c) chunks by (s desc, j asc) are selected;
 *   their keys U_{l,h} deq(c_t) and values f(k_hat) + delta (residual rows)
 *   are rebuilt in registers/LDS; each query head attends over them plus the
 *   layer's T tail tokens with scale 1/sqrt(d_h).
 * q: [B][Hq][dh]; k_tail, v_tail: [B][G][Hkv][T][dh] (the whole group; the
 * layer is selected here); out: [B][Hq][dh], act dtype.  sel_out: optional
 * [B][Hkv][min(top_k, n_c)] int32, chunk indices ascending.  Error if no chunk
 * is selected and T = 0.  Workspace: lowram_workspace_bytes(LOWRAM_OP_DECODE). */
lowram_status lowram_decode_attn(const lowram_dims *dims, int32_t layer, const lowram_model *model,
                                 const lowram_cache *cache, const void *q, const void *k_tail,
                                 const void *v_tail, void *out, int32_t *sel_out, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* The three stages lowram_decode_attn runs, for callers that schedule or time
 * them separately.  They communicate through the workspace, which must be the
 * same buffer with the same dims and layer for all three.
 *   select:  chunk scores and top-k (writes the selection into the workspace
 *            and, if sel_out != NULL, into sel_out); also U_{l,h}^T q_g of
 *            every query head of this call into the workspace on the CHAIN,
 *            MFMA and ABSORB paths, and W1 U_{l,h} on LOWRAM_PATH_ABSORB;
 *   attend:  rebuild-and-attend over the selected chunks and the tail, writing
 *            per-split softmax partials into the workspace (a kernel that
 *            ranks the chunk scores itself takes the same selection again);
 *   combine: merges the partials and applies the hoisted second predictor
 *            layer, writing out. */
lowram_status lowram_decode_select(const lowram_dims *dims, int32_t layer, const lowram_model *model,
                                   const lowram_cache *cache, const void *q, int32_t *sel_out,
                                   void *workspace, size_t workspace_bytes, void *stream);
lowram_status lowram_decode_attend(const lowram_dims *dims, int32_t layer, const lowram_model *model,
                                   const lowram_cache *cache, const void *q, const void *k_tail,
                                   const void *v_tail, void *workspace, size_t workspace_bytes,
                                   void *stream);
lowram_status lowram_decode_combine(const lowram_dims *dims, int32_t layer, const lowram_model *model,
                                    void *out, void *workspace, size_t workspace_bytes, void *stream);

/* lowram_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array of
 * LOWRAM_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends; this call allocates nothing.  Same
 * arguments, kernels and results as lowram_decode_attn (same bits).
 * Errors: LOWRAM_E_WORKSPACE when lowram_workspace_bytes(LOWRAM_OP_DECODE)
 * exceeds the array; LOWRAM_E_INVALID when `stream` belongs to another device
 * than the current one.  Every call on one GPU uses that GPU's array: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The kernels write every workspace byte they read,
 * so the array's contents from an earlier call do not matter. */
#define LOWRAM_NOALLOC_SCRATCH_BYTES (32u << 20)
lowram_status lowram_decode_attn_noalloc(const lowram_dims *dims, int32_t layer, const lowram_model *model,
                                         const lowram_cache *cache, const void *q, const void *k_tail,
                                         const void *v_tail, void *out, int32_t *sel_out, void *stream);

/* Reuse of rebuilt chunks across decode steps (rit.work generation section: the
 * context is split into chunks, those suited to the current query are picked,
 * and data already rebuilt is reused).  A table of `slots` slots per (sequence,
 * layer, kv head) keeps the rebuilt keys U_{l,h} deq(c~) of recently selected
 * chunks, as fp16, in a layout private to the library
 * (lowram_reuse_tile_bytes per slot).  Each call maps the selected chunks to
 * slots inside the attend kernel: a chunk already held is a hit; the others,
 * in ascending chunk order, take the least recently used slots that no hit of
 * this step holds (older use first, then lower slot) and are stored there once
 * rebuilt; when slots run out a chunk is rebuilt and not stored.  A wave
 * whose tile hits reads its keys back instead of multiplying the coefficients
 * by the basis (the coefficients are still read: the logits are taken from
 * them); the keys read back are the bits the kernel would compute, so the
 * output equals lowram_decode_attn's bit for bit.
 * The slot bookkeeping has two halves: clock's parity names the current one,
 * each call writes the updated table into the other half and advances clock.
 * The caller allocates the table and, before its first use, fills slot_chunk
 * (both halves) with -1 and slot_stamp and clock with 0.  It must reset the
 * table when the cache's chunks change meaning (eviction renumbers them) or
 * the model's basis changes; a re-pack only appends chunks and keeps it
 * valid.  Calls that share a table must not overlap. */
typedef struct {
  void *tiles;          /* [B][G][Hkv][slots][tile bytes]                            */
  int32_t *slot_chunk;  /* [B][G][Hkv][2][slots] chunk held by each slot, -1 if none */
  int32_t *slot_stamp;  /* [B][G][Hkv][2][slots] use count of each slot's last use   */
  int32_t *clock;       /* [B][G][Hkv] calls made on each head's table               */
  int32_t slots;        /* slots per (b, layer, kv head), 1 .. 256                   */
} lowram_reuse;

/* Bytes of one slot for these dims (host only).  LOWRAM_E_UNSUPPORTED unless
 * lowram_decode_kernel reports LOWRAM_PATH_CHAIN. */
lowram_status lowram_reuse_tile_bytes(const lowram_dims *dims, size_t *bytes);

/* lowram_decode_attn with the reuse table above (same arguments, plus reuse and
 * hits_out: optional [B][Hkv] int32, the number of selected chunks found in the
 * table).  Same kernels as lowram_decode_attn.  Needs the register-chained
 * kernel; LOWRAM_E_UNSUPPORTED otherwise.  Workspace: LOWRAM_OP_DECODE. */
lowram_status lowram_decode_attn_reuse(const lowram_dims *dims, int32_t layer, const lowram_model *model,
                                       const lowram_cache *cache, const void *q, const void *k_tail,
                                       const void *v_tail, void *out, int32_t *sel_out,
                                       const lowram_reuse *reuse, int32_t *hits_out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Eviction composed on top of the compressed cache (zicq.com Chinese summary,
 * composition with quantisation and eviction).  acc_j = sum over the n_obs
 * observation queries, the G layers and the Hkv heads of the chunk score s_j
 * (as in decode) in float64; the keep_chunks chunks with the largest acc
 * (lowest index wins ties) are copied to dst in ascending chunk order:
 * coefficients, landmarks and residual rows, with residual token indices
 * renumbered to the new positions.  dst has n_ctx' = keep_chunks * chunk and
 * dst_n_res residual rows per (b, layer, kv head), 0 <= dst_n_res <= n_res;
 * dst res_ptr[n_c'] rows are live.  Scales are unchanged (dst coeff_scale /
 * res_scale may alias src's).
 * Sizing: the kept chunks of a head hold some number of residual rows, known
 * only once the chunks are chosen.  With dst = NULL nothing is copied and only
 * keep_out and live_out are written; a caller that wants a cache sized to its
 * rows runs that first and then calls again with dst_n_res = max(live_out).
 * A head whose kept rows exceed dst_n_res keeps its first dst_n_res rows (its
 * pointers are clamped, so decode never reads a row dst lacks); live_out shows
 * the count before that clamp.
 * obs_q: [n_obs][B][G][Hq][dh] act dtype.  keep_out: optional [B][keep_chunks]
 * int32 kept source chunk indices.  live_out: optional [B][G][Hkv] int32.
 * Workspace: LOWRAM_OP_EVICT. */
lowram_status lowram_evict(const lowram_dims *dims, const lowram_model *model,
                           const lowram_cache *src, const void *obs_q, int32_t n_obs,
                           int32_t keep_chunks, int32_t dst_n_res, const lowram_cache *dst,
                           int32_t *keep_out, int32_t *live_out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Tail growth: move the oldest `chunk` tokens of the uncompressed tail into
 * the compressed cache as one new chunk.  The rit.work page (generation
 * section) keeps post-prefill tokens uncompressed and leaves open what happens
 * as that tail grows; the reading implemented here compresses each full chunk
 * of it the way the prefill was compressed (zicq.com "Core Mechanism" and
 * "Cross-Layer Low-Rank Key Compression"), against the existing basis,
 * predictor and int8 scales:
 *   c_t = U^T k_t^cat for tail tokens t = 0..C-1, stored rounded to coeff
 *   dtype (I8: q = clamp(rne(c/s), +-127) with src's coeff_scale, unchanged);
 *   landmark_{n_c} = mean of deq(c_t), float64 rounded to float32;
 *   per (layer, head): e_t = ||v_t - f(U_{l,h} deq(c_t))||^2 in float64 and
 *   the n_new_res tokens with the largest e (lowest index wins ties) keep
 *   delta = v - v_hat rounded to resid dtype (I8: src's res_scale, unchanged);
 *   the residual sets of the existing chunks are kept as they are.
 * dims describe src: n_ctx = N (may be 0 for float caches; >= chunk for
 * int8), n_res = src's residual capacity, n_tail = T >= chunk.  k_tail,
 * v_tail: [B][G][Hkv][T][dh] act dtype, tokens [0, chunk) are packed (the
 * caller then drops them from its tail).  dst: a cache for n_ctx' = N + chunk
 * and capacity n_res' = n_res + n_new_res, 0 <= n_new_res <= chunk: coeff
 * rows 0..N-1 and landmarks 0..n_c-1 are copied from src; dst res_ptr has
 * n_c + 2 entries, equal to src's for j <= n_c, and the new rows (tokens
 * N + t, ascending) follow src's res_ptr[n_c] live rows; the rest of the
 * capacity is zeroed.  Scales: dst coeff_scale / res_scale receive src's (they
 * may alias src's).  src and dst must not share any other storage.
 * Workspace: LOWRAM_OP_REPACK. */
lowram_status lowram_repack(const lowram_dims *dims, const lowram_model *model,
                            const lowram_cache *src, const void *k_tail, const void *v_tail,
                            int32_t n_new_res, const lowram_cache *dst, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Test-time fitting of the value predictor (abstract: a lightweight per-head
 * predictor fitted at test time, from scratch or from a meta-learned start
 * that needs fewer steps; rit.work values section: trained during prefill on
 * the context's keys).  Reading implemented: `steps` steps of full-batch
 * gradient descent with step size lr on
 *   L = (1/N) sum_t ||v_t - f(k_hat_t)||^2,  f(k) = W2 SiLU(W1 k + b1) + b2,
 * per (sequence, layer, kv head), starting from model's weights, with
 * k_hat = U_{l,h} deq(c~) from the coefficients lowram_compress would store
 * for these keys (same rounding; int8 scales over the N tokens).  Gradients
 * and master weights are float32 (sums over tokens in a fixed order); the
 * weights are rounded to act dtype once, into out (which may alias model's
 * weight arrays).  k, v: [B][G][Hkv][N][dh] act dtype.  loss: optional
 * [B][G][Hkv][steps + 1] float64, L before each step and after the last.
 * Call it before lowram_compress, which then uses the fitted weights.
 * Workspace: LOWRAM_OP_FIT (float32 activations of all N tokens:
 * about 4 B (G Hkv N (2 F + 2 dh)) bytes). */
lowram_status lowram_fit_predictor(const lowram_dims *dims, const lowram_model *model,
                                   const void *k, const void *v, int32_t steps, float lr,
                                   const lowram_predictor *out, double *loss, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* The group key basis at prefill (rit.work keys section: xKV finds a few
 * principal directions of the keys; zicq.com "Cross-Layer Low-Rank Key
 * Compression": one basis shared by adjacent layers).  Per sequence: the
 * float32 Gram matrix G = K_cat^T K_cat of the N prefill keys (K_cat: N x D,
 * dims ordered (layer, kv head, dim)), then `iterations` steps of subspace
 * iteration Q <- orth(G Q) from a fixed counter-hash start, orth = blocks of
 * 32 rows projected off the finished rows and orthonormalised by a float64
 * Cholesky factorisation of their 32 x 32 Gram matrix, each block twice
 * (numerically dependent rows replaced by pseudo-random ones in the first
 * pass).  basis (out): [B][D][r] act dtype, orthonormal
 * columns spanning the dominant r-dimensional subspace of G; unlike an
 * eigensolver's output they are not rotated to individual eigenvectors, which
 * changes no reconstruction U U^T k.  Deterministic.  k: [B][G][Hkv][N][dh]
 * act dtype (N = n_ctx >= 1).  D <= 8192.  Workspace: LOWRAM_OP_BASIS
 * (4 B (D^2 + 2 r D) bytes and a little more). */
lowram_status lowram_key_basis(const lowram_dims *dims, const void *k, int32_t iterations, void *basis,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Uncompressed decode attention, the comparator for the compressed path:
 * out[b][g] = softmax(k_b,h q_g / sqrt(d_h)) v_b,h over n_tokens tokens
 * (OjaKV section 3).  Uses batch, heads_q, heads_kv, head_dim and act of dims.
 * q: [B][Hq][dh]; k, v: element (b, h, t, d) at b*batch_stride +
 * (h*n_tokens + t)*dh + d (so one layer of a [B][G][Hkv][n][dh] cache can be
 * passed with batch_stride = G*Hkv*n*dh); out: [B][Hq][dh].
 * Workspace: LOWRAM_OP_DENSE with dims.n_ctx = n_tokens. */
lowram_status lowram_dense_decode_attn(const lowram_dims *dims, const void *q, const void *k,
                                       const void *v, int32_t n_tokens, int64_t batch_stride,
                                       void *out, void *workspace, size_t workspace_bytes,
                                       void *stream);

const char *lowram_status_string(lowram_status status);
const char *lowram_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LOWRAM_H */
