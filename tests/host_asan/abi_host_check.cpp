// Host-side check of the C ABI under AddressSanitizer: the sizing queries,
// the kernel choice and the argument checks of every entry point, called with
// valid dims and with invalid ones.  Nothing here reaches the GPU: each call
// either answers from the dims alone or is rejected before any HIP call.
// Prints "ok" and exits 0 when every expectation holds.
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "lowram.h"

static int failures = 0;

#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n",   \
                   __FILE__, __LINE__, #cond, lowram_last_error());               \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

static lowram_dims dims(int B, int G, int Hq, int Hkv, int dh, int r, int F, int N, int C, int k,
                        int T, int n_res, int act, int coeff, int resid) {
  lowram_dims d;
  std::memset(&d, 0, sizeof d);
  d.batch = B; d.layers = G; d.heads_q = Hq; d.heads_kv = Hkv; d.head_dim = dh; d.rank = r;
  d.hidden = F; d.n_ctx = N; d.chunk = C; d.top_k = k; d.n_tail = T; d.n_res = n_res;
  d.act = act; d.coeff = coeff; d.resid = resid;
  return d;
}

// The sizing queries answer for valid dims, with sizes that grow with the batch.
static void check_valid(const lowram_dims &d, int32_t want_path) {
  size_t ws = 0, ws2 = 0;
  EXPECT(lowram_workspace_bytes(&d, LOWRAM_OP_DECODE, &ws) == LOWRAM_OK);
  EXPECT(ws > 0);
  int32_t path = -1;
  EXPECT(lowram_decode_kernel(&d, &path) == LOWRAM_OK);
  EXPECT(path == want_path);
  uint64_t comp = 0, dense = 0;
  EXPECT(lowram_cache_bytes(&d, &comp, &dense) == LOWRAM_OK);
  EXPECT(comp > 0 && dense > comp);
  lowram_dims d2 = d;
  d2.batch = 2 * d.batch;
  EXPECT(lowram_workspace_bytes(&d2, LOWRAM_OP_DECODE, &ws2) == LOWRAM_OK);
  EXPECT(ws2 > ws);
  for (int32_t op = 0; op < 8; ++op) {  // every op code, valid or not, answers without a fault
    size_t b = 0;
    (void)lowram_workspace_bytes(&d, op, &b);
  }
}

// Invalid dims are rejected by every entry point before any device work.
static void check_rejected(const lowram_dims &d) {
  size_t ws = 0;
  EXPECT(lowram_workspace_bytes(&d, LOWRAM_OP_DECODE, &ws) != LOWRAM_OK);
  int32_t path = -1;
  EXPECT(lowram_decode_kernel(&d, &path) != LOWRAM_OK);
  uint64_t comp = 0, dense = 0;
  EXPECT(lowram_cache_bytes(&d, &comp, &dense) != LOWRAM_OK);
  lowram_model m;
  std::memset(&m, 0, sizeof m);
  lowram_cache c;
  std::memset(&c, 0, sizeof c);
  char buf[64];
  EXPECT(lowram_decode_attn(&d, 0, &m, &c, buf, buf, buf, buf, nullptr, buf, sizeof buf, nullptr) != LOWRAM_OK);
  EXPECT(lowram_decode_attn_noalloc(&d, 0, &m, &c, buf, buf, buf, buf, nullptr, nullptr) != LOWRAM_OK);
  EXPECT(lowram_decode_select(&d, 0, &m, &c, buf, nullptr, buf, sizeof buf, nullptr) != LOWRAM_OK);
  EXPECT(lowram_decode_attend(&d, 0, &m, &c, buf, buf, buf, buf, sizeof buf, nullptr) != LOWRAM_OK);
  EXPECT(lowram_decode_combine(&d, 0, &m, buf, buf, sizeof buf, nullptr) != LOWRAM_OK);
  EXPECT(lowram_compress(&d, &m, buf, buf, &c, buf, sizeof buf, nullptr) != LOWRAM_OK);
  EXPECT(lowram_dense_decode_attn(&d, buf, buf, buf, 16, 0, buf, buf, sizeof buf, nullptr) != LOWRAM_OK);
  const char *msg = lowram_last_error();
  EXPECT(msg != nullptr && std::strlen(msg) > 0);
}

int main() {
  for (int s = -2; s < 16; ++s) EXPECT(lowram_status_string((lowram_status)s) != nullptr);

  // the measured shapes: llama8b-32k, qwen4b-64k, composed int8, tiny fp32
  const lowram_dims llama = dims(4, 4, 32, 8, 128, 512, 256, 32768, 128, 32, 128, 4096,
                                 LOWRAM_BF16, LOWRAM_BF16, LOWRAM_BF16);
  const lowram_dims qwen = dims(4, 2, 16, 4, 256, 384, 512, 65536, 256, 16, 256, 6554,
                                LOWRAM_BF16, LOWRAM_BF16, LOWRAM_BF16);
  const lowram_dims comp = dims(2, 4, 32, 8, 128, 256, 256, 32768, 128, 64, 128, 2048,
                                LOWRAM_BF16, LOWRAM_I8, LOWRAM_I8);
  const lowram_dims tiny = dims(1, 2, 4, 2, 64, 32, 128, 1024, 64, 4, 16, 256,
                                LOWRAM_F32, LOWRAM_F32, LOWRAM_F32);
  check_valid(llama, LOWRAM_PATH_CHAIN);
  check_valid(qwen, LOWRAM_PATH_ABSORB);
  check_valid(comp, LOWRAM_PATH_CHAIN);
  check_valid(tiny, LOWRAM_PATH_VALU);

  // malformed dims: each one field out of range
  lowram_dims bad[12];
  for (auto &b : bad) b = llama;
  bad[0].batch = 0;
  bad[1].heads_q = 30;            // not a multiple of heads_kv
  bad[2].head_dim = 100;          // not a multiple of 8
  bad[3].head_dim = 512;          // above 256
  bad[4].rank = 0;
  bad[5].n_ctx = 1000;            // not a multiple of the chunk
  bad[6].chunk = 0;
  bad[7].n_res = 40000;           // above N
  bad[8].act = 99;
  bad[9].coeff = 99;
  bad[10].heads_kv = 0;
  bad[11].layers = -1;
  for (const auto &b : bad) check_rejected(b);

  // null output pointers of the sizing queries
  EXPECT(lowram_workspace_bytes(&llama, LOWRAM_OP_DECODE, nullptr) != LOWRAM_OK);
  EXPECT(lowram_decode_kernel(&llama, nullptr) != LOWRAM_OK);
  EXPECT(lowram_workspace_bytes(nullptr, LOWRAM_OP_DECODE, nullptr) != LOWRAM_OK);

  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
