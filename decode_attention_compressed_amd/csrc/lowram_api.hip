// Host side of the C ABI: argument validation, workspace plans and launch
// sequencing on the caller's stream.  Nothing here allocates device memory or
// synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "internal.hpp"

using namespace lowram;

// Device memory of lowram_decode_attn_noalloc: its decode workspace (chunk
// selection, partial scores, split partials).  Every GPU the library runs on
// holds one copy, at an address of its own, until the process ends.  Host code
// never passes this name to a kernel or a copy: it takes the device address
// from hipGetSymbolAddress once per device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[LOWRAM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

lowram_status fail(lowram_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lowram_status hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return LOWRAM_OK;
  return fail(LOWRAM_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t WS_ALIGN = 256;
size_t align_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int n_chunks(const lowram_dims *d) { return d->chunk > 0 ? d->n_ctx / d->chunk : 0; }

lowram_status check_dims(const lowram_dims *d) {
  if (!d) return fail(LOWRAM_E_INVALID, "dims is NULL");
  if (d->batch < 1 || d->layers < 1 || d->heads_kv < 1 || d->heads_q < 1)
    return fail(LOWRAM_E_INVALID, "batch, layers, heads_q and heads_kv must be >= 1");
  if (d->heads_q % d->heads_kv != 0)
    return fail(LOWRAM_E_INVALID, "heads_q (%d) must be a multiple of heads_kv (%d)", d->heads_q, d->heads_kv);
  if (d->heads_q / d->heads_kv > 16)
    return fail(LOWRAM_E_UNSUPPORTED, "at most 16 query heads per kv head");
  if (d->heads_kv > 16) return fail(LOWRAM_E_UNSUPPORTED, "at most 16 kv heads per layer");
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(LOWRAM_E_UNSUPPORTED, "head_dim %d: supported 64, 128, 256", d->head_dim);
  const long D = (long)d->layers * d->heads_kv * d->head_dim;
  if (d->rank < 16 || d->rank % 16 != 0 || d->rank > 2048)
    return fail(LOWRAM_E_UNSUPPORTED, "rank %d: must be a multiple of 16 in [16, 2048]", d->rank);
  if (d->rank > D) return fail(LOWRAM_E_INVALID, "rank %d exceeds the group key dim %ld", d->rank, D);
  if (d->hidden < 64 || d->hidden % 64 != 0)
    return fail(LOWRAM_E_UNSUPPORTED, "hidden %d: must be a positive multiple of 64", d->hidden);
  if (d->chunk < 1) return fail(LOWRAM_E_INVALID, "chunk must be >= 1");
  if (d->n_ctx < 0 || d->n_ctx % d->chunk != 0)
    return fail(LOWRAM_E_INVALID, "n_ctx %d must be a non-negative multiple of chunk %d", d->n_ctx, d->chunk);
  if (d->n_ctx > (1 << 22)) return fail(LOWRAM_E_UNSUPPORTED, "n_ctx above 4M tokens");
  if (n_chunks(d) > 8192) return fail(LOWRAM_E_UNSUPPORTED, "more than 8192 chunks");
  if (d->top_k < 0 || d->n_tail < 0) return fail(LOWRAM_E_INVALID, "top_k and n_tail must be >= 0");
  if (d->n_res < 0 || d->n_res > d->n_ctx)
    return fail(LOWRAM_E_INVALID, "n_res %d must lie in [0, n_ctx]", d->n_res);
  if (d->act == LOWRAM_F32) {
    if (d->coeff != LOWRAM_F32 || d->resid != LOWRAM_F32)
      return fail(LOWRAM_E_UNSUPPORTED, "float32 caches store coefficients and residuals in float32");
  } else if (d->act == LOWRAM_BF16) {
    if ((d->coeff != LOWRAM_BF16 && d->coeff != LOWRAM_I8) || (d->resid != LOWRAM_BF16 && d->resid != LOWRAM_I8))
      return fail(LOWRAM_E_UNSUPPORTED, "bfloat16 caches store coefficients/residuals in bf16 or int8");
  } else {
    return fail(LOWRAM_E_UNSUPPORTED, "act dtype must be F32 or BF16");
  }
  return LOWRAM_OK;
}

// Decode workspace plan.  The register-chained and matrix-core attend kernels
// fold the tail into their n_split partials per (b, h); the vector kernel
// writes one partial per selected chunk plus one for the tail.
struct DecodePlan {
  int path;  // LOWRAM_PATH_*
  int k_eff, cps, n_split, n_part, PW, tps, tail_per_split;
  int vsub;  // vector kernel: token ranges per selected chunk, one workgroup each
  size_t sel_off, sp_off, sc_off, part_off, absA_off, absQ_off, qtg_off, bytes;
};

// bytes of the select stage's U^T q_g for the kernels that take logits in
// coefficient space: float32 rows (chained kernel) or hi/lo operand columns
// (per-chunk matrix-core kernel)
size_t qtilde_bytes(const lowram_dims *d, int path) {
  const size_t bh = (size_t)d->batch * d->heads_kv;
  if (path == LOWRAM_PATH_CHAIN) return 4 * bh * QTG_G * d->rank;
  if (path == LOWRAM_PATH_MFMA) return 2 * bh * 2 * 16 * d->rank;
  return 0;
}

DecodePlan decode_plan(const lowram_dims *d) {
  DecodePlan p;
  const int n_c = n_chunks(d);
  const int g = d->heads_q / d->heads_kv;
  p.k_eff = d->top_k < n_c ? d->top_k : n_c;
  p.cps = 1;
  p.tps = 0;
  p.tail_per_split = 0;
  p.vsub = 1;
  p.path = LOWRAM_PATH_NONE;
  if (chain_supported(d->act, d->coeff, d->resid, d->head_dim, d->hidden, d->rank, d->chunk, g, p.k_eff)) {
    chain_plan(d->batch, d->heads_kv, p.k_eff, d->chunk, d->n_tail, p.n_split, p.tps, p.tail_per_split);
    p.n_part = p.n_split;
    p.path = LOWRAM_PATH_CHAIN;
  } else if (absorb_supported(d->act, d->coeff, d->resid, d->head_dim, d->hidden, d->rank, d->chunk, g, p.k_eff) &&
             (long)d->n_ctx * d->rank * 2 < (1L << 31)) {
    absorb_plan(d->batch, d->heads_kv, p.k_eff, d->chunk, d->n_tail, p.n_split, p.tps, p.tail_per_split, p.n_part);
    p.path = LOWRAM_PATH_ABSORB;
  } else {
    p.n_split = p.k_eff > 0 ? (p.k_eff + p.cps - 1) / p.cps : 0;
    // the matrix-core kernel folds the tail into its splits (one tail partial
    // when nothing is selected); the vector kernel writes it separately
    AttendArgs t;
    memset(&t, 0, sizeof t);
    t.C = d->chunk; t.g = g; t.dh = d->head_dim; t.F = d->hidden; t.r = d->rank;
    if (mfma_supported(t, d->act, d->coeff, d->resid)) {
      p.n_part = p.n_split > 0 ? p.n_split : 1;
      p.path = LOWRAM_PATH_MFMA;
    } else {
      // few (b, h, chunk) units: each chunk's tokens are split into up to 8
      // ranges of at least 16 tokens, one workgroup each, toward 256 workgroups
      const long units = (long)d->batch * d->heads_kv * p.k_eff;
      while (p.vsub < 8 && units * p.vsub < 256 && d->chunk % (2 * p.vsub) == 0 && d->chunk / (2 * p.vsub) >= 16)
        p.vsub *= 2;
      p.n_split = p.k_eff * p.vsub;
      p.n_part = p.n_split + 1;
      p.path = LOWRAM_PATH_VALU;
    }
  }
  if (p.k_eff == 0) p.path = LOWRAM_PATH_NONE;
  p.PW = 4 + d->hidden + d->head_dim;
  p.sel_off = 0;
  p.sp_off = align_up(sizeof(int32_t) * (size_t)d->batch * d->heads_kv * (p.k_eff > 0 ? p.k_eff : 1));
  p.sc_off = p.sp_off + align_up(sizeof(double) * (size_t)d->batch * d->heads_kv * select_rank_blocks(d->rank) *
                                 (n_c > 0 ? n_c : 1));
  p.part_off = p.sc_off + align_up(sizeof(double) * (size_t)d->batch * d->heads_kv * (n_c > 0 ? n_c : 1));
  p.absA_off = p.part_off + align_up(sizeof(float) * (size_t)d->batch * d->heads_kv * p.n_part * g * p.PW);
  const bool absorbed = p.path == LOWRAM_PATH_ABSORB;
  p.absQ_off = p.absA_off + (absorbed ? align_up(2 * (size_t)d->batch * d->heads_kv * d->hidden * d->rank) : 0);
  p.qtg_off = p.absQ_off + (absorbed ? align_up(2 * (size_t)d->batch * d->heads_kv * 2 * 4 * d->rank) : 0);
  p.bytes = p.qtg_off + align_up(qtilde_bytes(d, p.path));
  return p;
}

struct CompressPlan {
  size_t err_off, c64_off, d64_off, bytes;
};

CompressPlan compress_plan(const lowram_dims *d) {
  CompressPlan p;
  const size_t bl = (size_t)d->batch * d->layers * d->heads_kv;
  p.err_off = 0;
  p.c64_off = align_up(sizeof(double) * bl * d->n_ctx);
  p.d64_off = p.c64_off + (d->coeff == LOWRAM_I8 ? align_up(sizeof(double) * (size_t)d->batch * d->n_ctx * d->rank) : 0);
  p.bytes = p.d64_off + (d->resid == LOWRAM_I8 ? align_up(sizeof(double) * bl * d->n_res * d->head_dim) : 0);
  return p;
}

struct EvictPlan {
  size_t scores_off, spart_off, acc_off, keep_off, bytes;
};

EvictPlan evict_plan(const lowram_dims *d) {
  EvictPlan p;
  const size_t n_c = (size_t)(n_chunks(d) > 0 ? n_chunks(d) : 1);
  p.scores_off = 0;
  p.spart_off = align_up(sizeof(double) * d->batch * d->heads_kv * n_c);
  p.acc_off = p.spart_off + align_up(sizeof(double) * d->batch * d->heads_kv * select_rank_blocks(d->rank) * n_c);
  p.keep_off = p.acc_off + align_up(sizeof(double) * d->batch * n_c);
  p.bytes = p.keep_off + align_up(sizeof(int32_t) * d->batch * n_c);
  return p;
}

// Re-pack workspace: sized for m = C (the most a C-token chunk can keep).
struct RepackPlan {
  size_t err_off, c64_off, part_off, idx_off, ptr_off, dall_off, bytes;
};

RepackPlan repack_plan(const lowram_dims *d) {
  RepackPlan p;
  const size_t bl = (size_t)d->batch * d->layers * d->heads_kv, C = (size_t)d->chunk;
  const int D = d->layers * d->heads_kv * d->head_dim;
  const int S = project_splits(d->batch, d->chunk, D, d->rank);
  p.err_off = 0;
  p.c64_off = align_up(sizeof(double) * bl * C);
  p.part_off = p.c64_off + (d->coeff == LOWRAM_I8 ? align_up(sizeof(double) * (size_t)d->batch * C * d->rank) : 0);
  p.idx_off = p.part_off + (S > 1 ? align_up(sizeof(double) * (size_t)S * d->batch * C * d->rank) : 0);
  p.ptr_off = p.idx_off + align_up(sizeof(int32_t) * bl * C);
  p.dall_off = p.ptr_off + align_up(sizeof(int32_t) * bl * 2);
  p.bytes = p.dall_off + align_up(sizeof(double) * bl * C * d->head_dim);
  return p;
}

// Predictor-fit workspace: the stored coefficients (+ int8 staging), float32
// k_hat, pre-activations (later their gradient), hidden activations,
// residuals, and the float32 master weights.
struct FitPlan {
  size_t coeff_off, cscale_off, c64_off, khat_off, apre_off, hid_off, res_off, master_off, part_off, bytes;
};

FitPlan fit_plan(const lowram_dims *d) {
  FitPlan p;
  const size_t B = d->batch, N = d->n_ctx, r = d->rank, F = d->hidden, dh = d->head_dim;
  const size_t Z = B * d->layers * d->heads_kv;
  const size_t cb = d->coeff == LOWRAM_I8 ? 1 : (d->coeff == LOWRAM_F32 ? 4 : 2);
  p.coeff_off = 0;
  p.cscale_off = align_up(B * N * r * cb);
  p.c64_off = p.cscale_off + align_up(B * r * 2);
  p.khat_off = p.c64_off + (d->coeff == LOWRAM_I8 ? align_up(sizeof(double) * B * N * r) : 0);
  p.apre_off = p.khat_off + align_up(4 * Z * N * dh);
  p.hid_off = p.apre_off + align_up(4 * Z * N * F);
  p.res_off = p.hid_off + align_up(4 * Z * N * F);
  p.master_off = p.res_off + align_up(4 * Z * N * dh);
  p.part_off = p.master_off + align_up(4 * Z * (2 * F * dh + F + dh));
  p.bytes = p.part_off + align_up(sizeof(double) * Z * 64 * (F > dh ? F : dh));
  return p;
}

// Key-basis workspace: the D x D Gram matrix, two r x D row sets, the block
// products and row norms (float32 / float64).
struct BasisPlan {
  size_t gram_off, yt_off, qt_off, c_off, cpart_off, nrm_off, mpart_off, tri_off, dep_off, bytes;
};

BasisPlan basis_plan(const lowram_dims *d) {
  BasisPlan p;
  const size_t B = d->batch, r = d->rank, D = (size_t)d->layers * d->heads_kv * d->head_dim;
  p.gram_off = 0;
  p.yt_off = align_up(4 * B * D * D);
  p.qt_off = p.yt_off + align_up(4 * B * r * D);
  p.c_off = p.qt_off + align_up(4 * B * r * D);
  p.cpart_off = p.c_off + align_up(4 * B * 32 * r);
  p.nrm_off = p.cpart_off + align_up(4 * B * 16 * 32 * r);
  p.mpart_off = p.nrm_off + align_up(8 * B * 32);
  p.tri_off = p.mpart_off + align_up(8 * B * ((D + 255) / 256) * 32 * 32);
  p.dep_off = p.tri_off + align_up(8 * B * 32 * 32);
  p.bytes = p.dep_off + align_up(4 * B * 32);
  return p;
}

struct DensePlan {
  int tps, n_split, PW;
  size_t bytes;
};

DensePlan dense_plan(const lowram_dims *d, int n_tokens) {
  DensePlan p;
  const long work = (long)n_tokens * d->batch * d->heads_kv;
  long tps = (work + 2047) / 2048;
  tps = ((tps + 63) / 64) * 64;
  if (tps < 64) tps = 64;
  p.tps = (int)tps;
  p.n_split = n_tokens > 0 ? (int)((n_tokens + tps - 1) / tps) : 1;
  p.PW = 4 + d->head_dim;
  p.bytes = align_up(sizeof(float) * (size_t)d->batch * d->heads_kv * p.n_split *
                     (d->heads_q / d->heads_kv) * p.PW);
  return p;
}

// The dense comparator only reads batch, heads, head_dim and act.
lowram_status check_dense_dims(const lowram_dims *d) {
  if (!d) return fail(LOWRAM_E_INVALID, "dims is NULL");
  if (d->batch < 1 || d->heads_kv < 1 || d->heads_q < 1 || d->heads_q % d->heads_kv != 0)
    return fail(LOWRAM_E_INVALID, "bad batch or head counts");
  if (d->heads_q / d->heads_kv > 16) return fail(LOWRAM_E_UNSUPPORTED, "at most 16 query heads per kv head");
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(LOWRAM_E_UNSUPPORTED, "head_dim %d: supported 64, 128, 256", d->head_dim);
  if (d->act != LOWRAM_F32 && d->act != LOWRAM_BF16) return fail(LOWRAM_E_UNSUPPORTED, "act must be F32 or BF16");
  if (d->n_ctx < 0) return fail(LOWRAM_E_INVALID, "n_ctx must be >= 0");
  return LOWRAM_OK;
}

lowram_status check_ws(void *ws, size_t have, size_t need) {
  if (need > have) return fail(LOWRAM_E_WORKSPACE, "workspace of %zu bytes, %zu needed", have, need);
  if (need && !ws) return fail(LOWRAM_E_INVALID, "workspace is NULL");
  if (((uintptr_t)ws & (WS_ALIGN - 1)) != 0) return fail(LOWRAM_E_INVALID, "workspace must be 256-byte aligned");
  return LOWRAM_OK;
}

#define REQUIRE_PTR(p)                                                             \
  do {                                                                             \
    if (!(p)) return fail(LOWRAM_E_INVALID, "%s is NULL", #p);                     \
    if (!aligned16(p)) return fail(LOWRAM_E_INVALID, "%s is not 16-byte aligned", #p); \
  } while (0)
#define OPTIONAL_PTR(p)                                                            \
  do {                                                                             \
    if ((p) && !aligned16(p)) return fail(LOWRAM_E_INVALID, "%s is not 16-byte aligned", #p); \
  } while (0)

lowram_status check_decode_inputs(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                  const lowram_cache *c, const DecodePlan &p) {
  if (layer < 0 || layer >= d->layers)
    return fail(LOWRAM_E_INVALID, "layer %d outside [0, %d)", layer, d->layers);
  if (p.k_eff == 0 && d->n_tail == 0)
    return fail(LOWRAM_E_INVALID, "nothing to attend: no chunk selected and no tail");
  if (!m) return fail(LOWRAM_E_INVALID, "model is NULL");
  if (p.k_eff > 0) {
    if (!c) return fail(LOWRAM_E_INVALID, "cache is NULL");
    REQUIRE_PTR(m->basis); REQUIRE_PTR(m->w1); REQUIRE_PTR(m->b1);
    REQUIRE_PTR(c->coeff); REQUIRE_PTR(c->landmark); REQUIRE_PTR(c->res_ptr);
    if (d->n_res > 0) { REQUIRE_PTR(c->res_idx); REQUIRE_PTR(c->res_val); }
    if (d->coeff == LOWRAM_I8) REQUIRE_PTR(c->coeff_scale);
    if (d->resid == LOWRAM_I8 && d->n_res > 0) REQUIRE_PTR(c->res_scale);
  }
  return LOWRAM_OK;
}

// True when the attend kernel ranks the chunk scores itself.
bool attend_selects(const lowram_dims *d, const DecodePlan &p) {
  return (p.path == LOWRAM_PATH_CHAIN && n_chunks(d) <= CHAIN_SELECT_MAX_NC) ||
         (p.path == LOWRAM_PATH_ABSORB && n_chunks(d) <= ABSORB_SELECT_MAX_NC);
}

AttendArgs make_attend(const lowram_dims *d, int32_t layer, const lowram_model *m,
                       const lowram_cache *c, const void *q, const void *kt, const void *vt,
                       void *ws, const DecodePlan &p, int32_t *sel_out) {
  AttendArgs a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k_tail = kt; a.v_tail = vt;
  if (m) { a.basis = m->basis; a.w1 = m->w1; a.b1 = m->b1; }
  if (c) {
    a.coeff = c->coeff; a.coeff_scale = (const uint16_t *)c->coeff_scale;
    a.res_ptr = c->res_ptr; a.res_idx = c->res_idx; a.res_val = c->res_val;
    a.res_scale = (const uint16_t *)c->res_scale;
  }
  a.sel = reinterpret_cast<const int32_t *>((char *)ws + p.sel_off);
  a.score_part = attend_selects(d, p) ? reinterpret_cast<const double *>((char *)ws + p.sp_off) : nullptr;
  a.sel_out = attend_selects(d, p) ? sel_out : nullptr;
  a.part = reinterpret_cast<float *>((char *)ws + p.part_off);
  a.B = d->batch; a.G = d->layers; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.dh = d->head_dim;
  a.r = d->rank; a.F = d->hidden; a.N = d->n_ctx; a.C = d->chunk; a.T = d->n_tail;
  a.k_eff = p.k_eff; a.n_res = d->n_res; a.layer = layer;
  a.g = d->heads_q / d->heads_kv; a.cps = p.cps; a.n_split = p.n_split; a.PW = p.PW;
  a.path = p.path; a.tps = p.tps; a.tail_per_split = p.tail_per_split; a.vsub = p.vsub;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)d->head_dim);
  if (p.path == LOWRAM_PATH_CHAIN && ws) a.qtg = reinterpret_cast<const float *>((char *)ws + p.qtg_off);
  if (p.path == LOWRAM_PATH_MFMA && ws) a.qfrag = reinterpret_cast<const uint16_t *>((char *)ws + p.qtg_off);
  if (p.path == LOWRAM_PATH_ABSORB && ws) {
    a.absA = reinterpret_cast<uint16_t *>((char *)ws + p.absA_off);
    a.absQ = reinterpret_cast<uint16_t *>((char *)ws + p.absQ_off);
  }
  return a;
}

}  // namespace

extern "C" {

const char *lowram_status_string(lowram_status s) {
  switch (s) {
    case LOWRAM_OK: return "ok";
    case LOWRAM_E_INVALID: return "invalid argument";
    case LOWRAM_E_UNSUPPORTED: return "unsupported";
    case LOWRAM_E_WORKSPACE: return "workspace too small";
    case LOWRAM_E_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *lowram_last_error(void) { return g_err.c_str(); }

lowram_status lowram_workspace_bytes(const lowram_dims *d, int32_t op, size_t *bytes) {
  lowram_status st = op == LOWRAM_OP_DENSE ? check_dense_dims(d) : check_dims(d);
  if (st != LOWRAM_OK) return st;
  if (!bytes) return fail(LOWRAM_E_INVALID, "bytes is NULL");
  switch (op) {
    case LOWRAM_OP_COMPRESS: *bytes = compress_plan(d).bytes; return LOWRAM_OK;
    case LOWRAM_OP_DECODE: *bytes = decode_plan(d).bytes; return LOWRAM_OK;
    case LOWRAM_OP_EVICT: *bytes = evict_plan(d).bytes; return LOWRAM_OK;
    case LOWRAM_OP_DENSE: *bytes = dense_plan(d, d->n_ctx).bytes; return LOWRAM_OK;
    case LOWRAM_OP_REPACK: *bytes = repack_plan(d).bytes; return LOWRAM_OK;
    case LOWRAM_OP_FIT: *bytes = fit_plan(d).bytes; return LOWRAM_OK;
    case LOWRAM_OP_BASIS: *bytes = basis_plan(d).bytes; return LOWRAM_OK;
  }
  return fail(LOWRAM_E_INVALID, "unknown op %d", op);
}

lowram_status lowram_decode_kernel(const lowram_dims *d, int32_t *path) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  if (!path) return fail(LOWRAM_E_INVALID, "path is NULL");
  *path = decode_plan(d).path;
  return LOWRAM_OK;
}

lowram_status lowram_cache_bytes(const lowram_dims *d, uint64_t *compressed, uint64_t *dense) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const uint64_t G = d->layers, H = d->heads_kv, dh = d->head_dim, N = d->n_ctx, r = d->rank;
  const uint64_t F = d->hidden, n_c = (uint64_t)n_chunks(d), D = G * H * dh;
  const uint64_t s = dtype_bytes(d->act), sc = dtype_bytes(d->coeff), sr = dtype_bytes(d->resid);
  if (dense) *dense = 2 * G * H * dh * N * s;
  if (compressed) {
    uint64_t t = N * r * sc + D * r * s + G * H * (2 * F * dh + F + dh) * s;
    t += G * H * (uint64_t)d->n_res * (dh * sr + 4) + G * H * (n_c + 1) * 4 + n_c * r * 4;
    if (d->coeff == LOWRAM_I8) t += r * 2;
    if (d->resid == LOWRAM_I8) t += G * H * dh * 2;
    *compressed = t;
  }
  return LOWRAM_OK;
}

lowram_status lowram_compress(const lowram_dims *d, const lowram_model *m, const void *k,
                              const void *v, const lowram_cache *out, void *ws, size_t ws_bytes,
                              void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  if (d->n_ctx < d->chunk) return fail(LOWRAM_E_INVALID, "compress needs at least one chunk");
  if (!m || !out) return fail(LOWRAM_E_INVALID, "model and out must not be NULL");
  REQUIRE_PTR(k); REQUIRE_PTR(v);
  REQUIRE_PTR(m->basis); REQUIRE_PTR(m->w1); REQUIRE_PTR(m->b1); REQUIRE_PTR(m->w2); REQUIRE_PTR(m->b2);
  REQUIRE_PTR(out->coeff); REQUIRE_PTR(out->landmark); REQUIRE_PTR(out->res_ptr);
  if (d->n_res > 0) { REQUIRE_PTR(out->res_idx); REQUIRE_PTR(out->res_val); }
  if (d->coeff == LOWRAM_I8) REQUIRE_PTR(out->coeff_scale);
  if (d->resid == LOWRAM_I8) REQUIRE_PTR(out->res_scale);
  const CompressPlan p = compress_plan(d);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  CompressArgs a;
  memset(&a, 0, sizeof a);
  a.k = k; a.v = v; a.basis = m->basis; a.w1 = m->w1; a.b1 = m->b1; a.w2 = m->w2; a.b2 = m->b2;
  a.coeff = out->coeff; a.coeff_scale = (uint16_t *)out->coeff_scale; a.landmark = out->landmark;
  a.res_ptr = out->res_ptr; a.res_idx = out->res_idx; a.res_val = out->res_val;
  a.res_scale = (uint16_t *)out->res_scale;
  a.err = reinterpret_cast<double *>((char *)ws + p.err_off);
  a.c64 = reinterpret_cast<double *>((char *)ws + p.c64_off);
  a.d64 = reinterpret_cast<double *>((char *)ws + p.d64_off);
  a.B = d->batch; a.G = d->layers; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.dh = d->head_dim;
  a.r = d->rank; a.F = d->hidden; a.N = d->n_ctx; a.C = d->chunk; a.n_res = d->n_res;
  a.act = d->act; a.coeff_dt = d->coeff; a.resid_dt = d->resid;
  return hip_status(run_compress(a, (hipStream_t)stream), "lowram_compress");
}

}  // extern "C"

namespace {

// Partial chunk scores, and the summed scores and the selection itself unless
// the attend kernel will rank the scores (with_topk false); arguments already
// validated.
// The combine stage; with rclock it also advances the reuse clock of every
// (b, layer, h) once, after the attend kernel has read it.
lowram_status run_combine(const lowram_dims *d, int32_t layer, const lowram_model *m, void *out, void *ws,
                          const DecodePlan &p, int32_t *rclock, void *stream) {
  CombineArgs a;
  memset(&a, 0, sizeof a);
  a.part = reinterpret_cast<const float *>((char *)ws + p.part_off);
  a.rclock = rclock;
  a.w2 = m ? m->w2 : nullptr; a.b2 = m ? m->b2 : nullptr; a.out = out;
  a.B = d->batch; a.G = d->layers; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.dh = d->head_dim;
  a.F = d->hidden; a.layer = layer; a.g = d->heads_q / d->heads_kv;
  a.n_comp = p.k_eff > 0 ? p.n_split : 0; a.n_total = p.n_part; a.PW = p.PW;
  return hip_status(launch_combine(d->act, a, (hipStream_t)stream), "lowram_decode_combine");
}

lowram_status run_select(const lowram_dims *d, int32_t layer, const lowram_model *m,
                         const lowram_cache *c, const void *q, int32_t *sel_out, void *ws,
                         const DecodePlan &p, bool with_topk, void *stream) {
  if (p.k_eff == 0) return LOWRAM_OK;
  const long D = (long)d->layers * d->heads_kv * d->head_dim;
  int32_t *sel = reinterpret_cast<int32_t *>((char *)ws + p.sel_off);
  double *sp = reinterpret_cast<double *>((char *)ws + p.sp_off);
  double *sc = reinterpret_cast<double *>((char *)ws + p.sc_off);
  QOut qo;
  if (p.path == LOWRAM_PATH_CHAIN) qo.qtg = reinterpret_cast<float *>((char *)ws + p.qtg_off);
  if (p.path == LOWRAM_PATH_MFMA) {
    qo.qfrag = reinterpret_cast<uint16_t *>((char *)ws + p.qtg_off);
    qo.mode = d->coeff == LOWRAM_I8 ? 2 : 1;
    qo.scale = reinterpret_cast<const uint16_t *>(c->coeff_scale);
  }
  // absorbed path: A = W1 U_{l,h} and q~ for this call, in the launch of the
  // partial scores
  AttendArgs ab;
  if (p.path == LOWRAM_PATH_ABSORB) ab = make_attend(d, layer, m, c, q, nullptr, nullptr, ws, p, nullptr);
  return hip_status(launch_select(d->act, q, (long)d->heads_q * d->head_dim, m->basis, c->landmark,
                                  d->batch, d->heads_q, d->heads_kv, d->head_dim, d->rank,
                                  n_chunks(d), (int)D, layer, with_topk ? p.k_eff : 0, sel, sel_out,
                                  sp, with_topk ? sc : nullptr, (hipStream_t)stream, qo,
                                  p.path == LOWRAM_PATH_ABSORB ? &ab : nullptr),
                    "lowram_decode_select");
}

}  // namespace

extern "C" {

lowram_status lowram_decode_select(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                   const lowram_cache *c, const void *q, int32_t *sel_out,
                                   void *ws, size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const DecodePlan p = decode_plan(d);
  if ((st = check_decode_inputs(d, layer, m, c, p)) != LOWRAM_OK) return st;
  REQUIRE_PTR(q);
  OPTIONAL_PTR(sel_out);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  return run_select(d, layer, m, c, q, sel_out, ws, p, true, stream);
}

lowram_status lowram_decode_attend(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                   const lowram_cache *c, const void *q, const void *k_tail,
                                   const void *v_tail, void *ws, size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const DecodePlan p = decode_plan(d);
  if ((st = check_decode_inputs(d, layer, m, c, p)) != LOWRAM_OK) return st;
  REQUIRE_PTR(q);
  if (d->n_tail > 0) { REQUIRE_PTR(k_tail); REQUIRE_PTR(v_tail); }
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  const AttendArgs a = make_attend(d, layer, m, c, q, k_tail, v_tail, ws, p, nullptr);
  return hip_status(launch_attend(d->act, d->coeff, d->resid, a, (hipStream_t)stream),
                    "lowram_decode_attend");
}

lowram_status lowram_decode_combine(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                    void *out, void *ws, size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const DecodePlan p = decode_plan(d);
  if (layer < 0 || layer >= d->layers)
    return fail(LOWRAM_E_INVALID, "layer %d outside [0, %d)", layer, d->layers);
  if (p.k_eff == 0 && d->n_tail == 0)
    return fail(LOWRAM_E_INVALID, "nothing to attend: no chunk selected and no tail");
  REQUIRE_PTR(out);
  if (p.k_eff > 0) {
    if (!m) return fail(LOWRAM_E_INVALID, "model is NULL");
    REQUIRE_PTR(m->w2); REQUIRE_PTR(m->b2);
  }
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  return run_combine(d, layer, m, out, ws, p, nullptr, stream);
}

lowram_status lowram_decode_attn(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                 const lowram_cache *c, const void *q, const void *k_tail,
                                 const void *v_tail, void *out, int32_t *sel_out, void *ws,
                                 size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const DecodePlan p = decode_plan(d);
  if ((st = check_decode_inputs(d, layer, m, c, p)) != LOWRAM_OK) return st;
  REQUIRE_PTR(q); REQUIRE_PTR(out); OPTIONAL_PTR(sel_out);
  if (d->n_tail > 0) { REQUIRE_PTR(k_tail); REQUIRE_PTR(v_tail); }
  if (p.k_eff > 0) { REQUIRE_PTR(m->w2); REQUIRE_PTR(m->b2); }
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  // When the attend kernel ranks the scores itself, the top-k kernel is skipped
  // and the attend kernel writes sel_out; the results are the same bits.
  const bool in_attend = attend_selects(d, p);
  if ((st = run_select(d, layer, m, c, q, in_attend ? nullptr : sel_out, ws, p, !in_attend, stream)) != LOWRAM_OK)
    return st;
  const AttendArgs a = make_attend(d, layer, m, c, q, k_tail, v_tail, ws, p, sel_out);
  if ((st = hip_status(launch_attend(d->act, d->coeff, d->resid, a, (hipStream_t)stream), "lowram_decode_attend")) != LOWRAM_OK)
    return st;
  return lowram_decode_combine(d, layer, m, out, ws, ws_bytes, stream);
}

lowram_status lowram_reuse_tile_bytes(const lowram_dims *d, size_t *bytes) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  if (!bytes) return fail(LOWRAM_E_INVALID, "bytes is NULL");
  const DecodePlan p = decode_plan(d);
  if (p.path != LOWRAM_PATH_CHAIN)
    return fail(LOWRAM_E_UNSUPPORTED, "reuse needs the register-chained attend kernel (see lowram_decode_kernel)");
  *bytes = chain_tile_bytes(d->hidden);
  return LOWRAM_OK;
}

lowram_status lowram_decode_attn_reuse(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                       const lowram_cache *c, const void *q, const void *k_tail,
                                       const void *v_tail, void *out, int32_t *sel_out,
                                       const lowram_reuse *reuse, int32_t *hits_out, void *ws,
                                       size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const DecodePlan p = decode_plan(d);
  if ((st = check_decode_inputs(d, layer, m, c, p)) != LOWRAM_OK) return st;
  if (p.path != LOWRAM_PATH_CHAIN)
    return fail(LOWRAM_E_UNSUPPORTED, "reuse needs the register-chained attend kernel and a selected chunk");
  if (p.k_eff > CHAIN_SELECT_MAX_NC)
    return fail(LOWRAM_E_UNSUPPORTED, "reuse assigns slots to at most %d selected chunks (top_k %d)",
                CHAIN_SELECT_MAX_NC, p.k_eff);
  REQUIRE_PTR(q); REQUIRE_PTR(out); OPTIONAL_PTR(sel_out); OPTIONAL_PTR(hits_out);
  if (d->n_tail > 0) { REQUIRE_PTR(k_tail); REQUIRE_PTR(v_tail); }
  REQUIRE_PTR(m->w2); REQUIRE_PTR(m->b2);
  if (!reuse) return fail(LOWRAM_E_INVALID, "reuse is NULL");
  if (reuse->slots < 1 || reuse->slots > REUSE_MAX_SLOTS)
    return fail(LOWRAM_E_INVALID, "reuse slots %d outside [1, %d]", reuse->slots, REUSE_MAX_SLOTS);
  REQUIRE_PTR(reuse->tiles); REQUIRE_PTR(reuse->slot_chunk); REQUIRE_PTR(reuse->slot_stamp);
  REQUIRE_PTR(reuse->clock);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  const bool in_attend = attend_selects(d, p);
  if ((st = run_select(d, layer, m, c, q, in_attend ? nullptr : sel_out, ws, p, !in_attend, stream)) != LOWRAM_OK)
    return st;
  AttendArgs a = make_attend(d, layer, m, c, q, k_tail, v_tail, ws, p, sel_out);
  a.rtiles = reuse->tiles;
  a.rt_chunk = reuse->slot_chunk;
  a.rt_stamp = reuse->slot_stamp;
  a.rclock = reuse->clock;
  a.rhits = hits_out;
  a.rslots = reuse->slots;
  if ((st = hip_status(launch_attend(d->act, d->coeff, d->resid, a, (hipStream_t)stream), "lowram_decode_attn_reuse")) != LOWRAM_OK)
    return st;
  return run_combine(d, layer, m, out, ws, p, reuse->clock, stream);
}

lowram_status lowram_evict(const lowram_dims *d, const lowram_model *m, const lowram_cache *src,
                           const void *obs_q, int32_t n_obs, int32_t keep_chunks, int32_t dst_n_res,
                           const lowram_cache *dst, int32_t *keep_out, int32_t *live_out, void *ws,
                           size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const int n_c = n_chunks(d);
  if (n_c < 1) return fail(LOWRAM_E_INVALID, "evict needs at least one chunk");
  if (keep_chunks < 1 || keep_chunks > n_c)
    return fail(LOWRAM_E_INVALID, "keep_chunks %d outside [1, %d]", keep_chunks, n_c);
  if (n_obs < 0) return fail(LOWRAM_E_INVALID, "n_obs must be >= 0");
  if (!m || !src) return fail(LOWRAM_E_INVALID, "model and src must not be NULL");
  if (!dst && !keep_out && !live_out)
    return fail(LOWRAM_E_INVALID, "nothing to write: dst, keep_out and live_out are all NULL");
  if (n_obs > 0) REQUIRE_PTR(obs_q);
  REQUIRE_PTR(m->basis);
  REQUIRE_PTR(src->coeff); REQUIRE_PTR(src->landmark); REQUIRE_PTR(src->res_ptr);
  if (d->n_res > 0) { REQUIRE_PTR(src->res_idx); REQUIRE_PTR(src->res_val); }
  OPTIONAL_PTR(keep_out); OPTIONAL_PTR(live_out);
  if (dst) {
    if (dst_n_res < 0 || dst_n_res > d->n_res)
      return fail(LOWRAM_E_INVALID, "dst_n_res %d outside [0, n_res %d]", dst_n_res, d->n_res);
    REQUIRE_PTR(dst->coeff); REQUIRE_PTR(dst->landmark); REQUIRE_PTR(dst->res_ptr);
    if (dst_n_res > 0) { REQUIRE_PTR(dst->res_idx); REQUIRE_PTR(dst->res_val); }
    if (src->coeff == dst->coeff || src->res_ptr == dst->res_ptr ||
        (dst_n_res > 0 && src->res_val == dst->res_val))
      return fail(LOWRAM_E_INVALID, "src and dst must not share coefficient or residual storage");
  }
  const EvictPlan p = evict_plan(d);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  EvictArgs a;
  memset(&a, 0, sizeof a);
  a.basis = m->basis; a.obs_q = obs_q; a.n_obs = n_obs; a.keep = keep_chunks;
  a.coeff = src->coeff; a.landmark = src->landmark; a.res_ptr = src->res_ptr;
  a.res_idx = src->res_idx; a.res_val = src->res_val;
  if (dst) {
    a.d_coeff = dst->coeff; a.d_landmark = dst->landmark; a.d_res_ptr = dst->res_ptr;
    a.d_res_idx = dst->res_idx; a.d_res_val = dst->res_val; a.d_n_res = dst_n_res;
  }
  a.keep_out = keep_out ? keep_out : reinterpret_cast<int32_t *>((char *)ws + p.keep_off);
  a.live_out = live_out;
  a.scores = reinterpret_cast<double *>((char *)ws + p.scores_off);
  a.spart = reinterpret_cast<double *>((char *)ws + p.spart_off);
  a.acc = reinterpret_cast<double *>((char *)ws + p.acc_off);
  a.B = d->batch; a.G = d->layers; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.dh = d->head_dim;
  a.r = d->rank; a.N = d->n_ctx; a.C = d->chunk; a.n_res = d->n_res;
  a.act = d->act; a.coeff_dt = d->coeff; a.resid_dt = d->resid;
  return hip_status(run_evict(a, (hipStream_t)stream), "lowram_evict");
}

lowram_status lowram_repack(const lowram_dims *d, const lowram_model *m, const lowram_cache *src,
                            const void *k_tail, const void *v_tail, int32_t n_new_res,
                            const lowram_cache *dst, void *ws, size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  if (d->n_tail < d->chunk)
    return fail(LOWRAM_E_INVALID, "re-pack needs a full chunk in the tail (n_tail %d < chunk %d)",
                d->n_tail, d->chunk);
  if (n_new_res < 0 || n_new_res > d->chunk)
    return fail(LOWRAM_E_INVALID, "n_new_res %d outside [0, chunk %d]", n_new_res, d->chunk);
  if ((d->coeff == LOWRAM_I8 || d->resid == LOWRAM_I8) && d->n_ctx < d->chunk)
    return fail(LOWRAM_E_INVALID, "int8 re-pack needs the scales of a compressed prefill (n_ctx >= chunk)");
  lowram_dims d2 = *d;
  d2.n_ctx = d->n_ctx + d->chunk;
  d2.n_res = d->n_res + n_new_res;
  if ((st = check_dims(&d2)) != LOWRAM_OK) return st;
  if (!m || !src || !dst) return fail(LOWRAM_E_INVALID, "model, src and dst must not be NULL");
  REQUIRE_PTR(k_tail); REQUIRE_PTR(v_tail);
  REQUIRE_PTR(m->basis); REQUIRE_PTR(m->w1); REQUIRE_PTR(m->b1); REQUIRE_PTR(m->w2); REQUIRE_PTR(m->b2);
  REQUIRE_PTR(src->res_ptr);
  if (d->n_ctx > 0) { REQUIRE_PTR(src->coeff); REQUIRE_PTR(src->landmark); }
  if (d->n_res > 0) { REQUIRE_PTR(src->res_idx); REQUIRE_PTR(src->res_val); }
  REQUIRE_PTR(dst->coeff); REQUIRE_PTR(dst->landmark); REQUIRE_PTR(dst->res_ptr);
  if (d2.n_res > 0) { REQUIRE_PTR(dst->res_idx); REQUIRE_PTR(dst->res_val); }
  if (d->coeff == LOWRAM_I8) { REQUIRE_PTR(src->coeff_scale); REQUIRE_PTR(dst->coeff_scale); }
  if (d->resid == LOWRAM_I8) { REQUIRE_PTR(src->res_scale); REQUIRE_PTR(dst->res_scale); }
  if (src->coeff == dst->coeff || src->landmark == dst->landmark || src->res_ptr == dst->res_ptr ||
      (d->n_res > 0 && (src->res_idx == dst->res_idx || src->res_val == dst->res_val)))
    return fail(LOWRAM_E_INVALID, "src and dst must not share coefficient, landmark or residual storage");
  const RepackPlan p = repack_plan(d);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  RepackArgs a;
  memset(&a, 0, sizeof a);
  a.basis = m->basis; a.w1 = m->w1; a.b1 = m->b1; a.w2 = m->w2; a.b2 = m->b2;
  a.k_tail = k_tail; a.v_tail = v_tail;
  a.coeff = src->coeff; a.coeff_scale = (const uint16_t *)src->coeff_scale; a.landmark = src->landmark;
  a.res_ptr = src->res_ptr; a.res_idx = src->res_idx; a.res_val = src->res_val;
  a.res_scale = (const uint16_t *)src->res_scale;
  a.d_coeff = dst->coeff; a.d_coeff_scale = (uint16_t *)dst->coeff_scale; a.d_landmark = dst->landmark;
  a.d_res_ptr = dst->res_ptr; a.d_res_idx = dst->res_idx; a.d_res_val = dst->res_val;
  a.d_res_scale = (uint16_t *)dst->res_scale;
  a.err = reinterpret_cast<double *>((char *)ws + p.err_off);
  a.c64 = reinterpret_cast<double *>((char *)ws + p.c64_off);
  a.part = reinterpret_cast<double *>((char *)ws + p.part_off);
  a.t_idx = reinterpret_cast<int32_t *>((char *)ws + p.idx_off);
  a.t_ptr = reinterpret_cast<int32_t *>((char *)ws + p.ptr_off);
  a.dall = reinterpret_cast<double *>((char *)ws + p.dall_off);
  a.B = d->batch; a.G = d->layers; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.dh = d->head_dim;
  a.r = d->rank; a.F = d->hidden; a.N = d->n_ctx; a.C = d->chunk; a.T = d->n_tail;
  a.n_res = d->n_res; a.m = n_new_res;
  a.act = d->act; a.coeff_dt = d->coeff; a.resid_dt = d->resid;
  return hip_status(run_repack(a, (hipStream_t)stream), "lowram_repack");
}

lowram_status lowram_fit_predictor(const lowram_dims *d, const lowram_model *m, const void *k,
                                   const void *v, int32_t steps, float lr,
                                   const lowram_predictor *out, double *loss, void *ws,
                                   size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  if (d->n_ctx < d->chunk) return fail(LOWRAM_E_INVALID, "fitting needs at least one chunk of tokens");
  if (steps < 0 || steps > 100000) return fail(LOWRAM_E_INVALID, "steps %d outside [0, 100000]", steps);
  if (!(lr >= 0.f) || lr > 1e6f) return fail(LOWRAM_E_INVALID, "lr must be a finite value >= 0");
  if (!m || !out) return fail(LOWRAM_E_INVALID, "model and out must not be NULL");
  REQUIRE_PTR(k); REQUIRE_PTR(v);
  REQUIRE_PTR(m->basis); REQUIRE_PTR(m->w1); REQUIRE_PTR(m->b1); REQUIRE_PTR(m->w2); REQUIRE_PTR(m->b2);
  REQUIRE_PTR(out->w1); REQUIRE_PTR(out->b1); REQUIRE_PTR(out->w2); REQUIRE_PTR(out->b2);
  OPTIONAL_PTR(loss);
  const FitPlan p = fit_plan(d);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  const size_t Z = (size_t)d->batch * d->layers * d->heads_kv, F = d->hidden, dh = d->head_dim;
  char *w = (char *)ws;
  FitArgs a;
  memset(&a, 0, sizeof a);
  a.basis = m->basis; a.w1 = m->w1; a.b1 = m->b1; a.w2 = m->w2; a.b2 = m->b2;
  a.k = k; a.v = v;
  a.o_w1 = out->w1; a.o_b1 = out->b1; a.o_w2 = out->w2; a.o_b2 = out->b2;
  a.loss = loss;
  a.coeff = w + p.coeff_off;
  a.coeff_scale = reinterpret_cast<uint16_t *>(w + p.cscale_off);
  a.c64 = reinterpret_cast<double *>(w + p.c64_off);
  a.khat = reinterpret_cast<float *>(w + p.khat_off);
  a.apre = reinterpret_cast<float *>(w + p.apre_off);
  a.hid = reinterpret_cast<float *>(w + p.hid_off);
  a.res = reinterpret_cast<float *>(w + p.res_off);
  a.m_w1 = reinterpret_cast<float *>(w + p.master_off);
  a.m_b1 = a.m_w1 + Z * F * dh;
  a.m_w2 = a.m_b1 + Z * F;
  a.m_b2 = a.m_w2 + Z * dh * F;
  a.part = reinterpret_cast<double *>(w + p.part_off);
  a.B = d->batch; a.G = d->layers; a.Hkv = d->heads_kv; a.dh = d->head_dim; a.r = d->rank;
  a.F = d->hidden; a.N = d->n_ctx; a.steps = steps; a.act = d->act; a.coeff_dt = d->coeff;
  a.lr = lr;
  return hip_status(run_fit(a, (hipStream_t)stream), "lowram_fit_predictor");
}

lowram_status lowram_key_basis(const lowram_dims *d, const void *k, int32_t iterations, void *basis,
                               void *ws, size_t ws_bytes, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const int D = d->layers * d->heads_kv * d->head_dim;
  if (d->n_ctx < 1) return fail(LOWRAM_E_INVALID, "the basis needs at least one token (n_ctx >= 1)");
  if (D > basis_max_dim())
    return fail(LOWRAM_E_UNSUPPORTED, "group key dim %d above %d for the basis kernels", D, basis_max_dim());
  if (iterations < 0 || iterations > 1000) return fail(LOWRAM_E_INVALID, "iterations %d outside [0, 1000]", iterations);
  REQUIRE_PTR(k); REQUIRE_PTR(basis);
  const BasisPlan p = basis_plan(d);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  char *w = (char *)ws;
  BasisArgs a;
  memset(&a, 0, sizeof a);
  a.k = k; a.basis = basis;
  a.gram = reinterpret_cast<float *>(w + p.gram_off);
  a.yt = reinterpret_cast<float *>(w + p.yt_off);
  a.qt = reinterpret_cast<float *>(w + p.qt_off);
  a.cbuf = reinterpret_cast<float *>(w + p.c_off);
  a.cpart = reinterpret_cast<float *>(w + p.cpart_off);
  a.nrm = reinterpret_cast<double *>(w + p.nrm_off);
  a.mpart = reinterpret_cast<double *>(w + p.mpart_off);
  a.tri = reinterpret_cast<double *>(w + p.tri_off);
  a.dep = reinterpret_cast<int32_t *>(w + p.dep_off);
  a.B = d->batch; a.G = d->layers; a.Hkv = d->heads_kv; a.dh = d->head_dim; a.r = d->rank;
  a.N = d->n_ctx; a.iterations = iterations; a.act = d->act;
  return hip_status(run_basis(a, (hipStream_t)stream), "lowram_key_basis");
}

lowram_status lowram_dense_decode_attn(const lowram_dims *d, const void *q, const void *k,
                                       const void *v, int32_t n_tokens, int64_t batch_stride,
                                       void *out, void *ws, size_t ws_bytes, void *stream) {
  lowram_status st = check_dense_dims(d);
  if (st != LOWRAM_OK) return st;
  if (n_tokens < 1) return fail(LOWRAM_E_INVALID, "n_tokens must be >= 1");
  if (batch_stride < (int64_t)d->heads_kv * n_tokens * d->head_dim && d->batch > 1)
    return fail(LOWRAM_E_INVALID, "batch_stride smaller than one sequence's keys");
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(out);
  const DensePlan p = dense_plan(d, n_tokens);
  if ((st = check_ws(ws, ws_bytes, p.bytes)) != LOWRAM_OK) return st;
  float *part = reinterpret_cast<float *>(ws);
  hipError_t e = launch_dense(d->act, q, k, v, (long)batch_stride, d->batch, d->heads_q,
                              d->heads_kv, d->head_dim, n_tokens, p.tps, p.n_split, part, p.PW,
                              (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "lowram_dense_decode_attn");
  CombineArgs a;
  memset(&a, 0, sizeof a);
  a.part = part; a.out = out;
  a.B = d->batch; a.G = 1; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.dh = d->head_dim;
  a.F = 0; a.layer = 0; a.g = d->heads_q / d->heads_kv; a.n_comp = 0; a.n_total = p.n_split; a.PW = p.PW;
  return hip_status(launch_combine(d->act, a, (hipStream_t)stream), "lowram_dense_decode_attn");
}

}  // extern "C"

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_noalloc_mu;
void *g_noalloc_ptr[NOALLOC_MAX_DEVICES];  // device address of `scratch`, per device

// The current device's copy of the scratch array: looked up once per device,
// with that device current, and kept.
lowram_status noalloc_scratch(void *stream, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(LOWRAM_E_UNSUPPORTED, "device %d: at most %d devices", dev, NOALLOC_MAX_DEVICES);
  if (stream) {
    hipDevice_t sdev = -1;
    if ((e = hipStreamGetDevice((hipStream_t)stream, &sdev)) != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(LOWRAM_E_INVALID, "stream belongs to device %d, the current device is %d", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LOWRAM_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return LOWRAM_OK;
}

}  // namespace

extern "C" {

lowram_status lowram_decode_attn_noalloc(const lowram_dims *d, int32_t layer, const lowram_model *m,
                                         const lowram_cache *c, const void *q, const void *k_tail,
                                         const void *v_tail, void *out, int32_t *sel_out, void *stream) {
  lowram_status st = check_dims(d);
  if (st != LOWRAM_OK) return st;
  const size_t need = decode_plan(d).bytes;
  if (need > (size_t)LOWRAM_NOALLOC_SCRATCH_BYTES)
    return fail(LOWRAM_E_WORKSPACE, "decode needs %zu bytes of workspace, the static scratch holds %zu",
                need, (size_t)LOWRAM_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((st = noalloc_scratch(stream, &ws)) != LOWRAM_OK) return st;
  return lowram_decode_attn(d, layer, m, c, q, k_tail, v_tail, out, sel_out, ws,
                            (size_t)LOWRAM_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
