// Host-side driver for the sanitizer build of the library (AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code only; no GPU).  It calls
// the size queries over many random configurations and every compute entry
// point with arguments that the host validation must reject, so that no call
// reaches a kernel launch.  Each result is checked against the documented
// behaviour: a status code from the header's list, workspace sizes that are
// multiples of 256 bytes and repeatable, and the exact status of each
// rejected call.  Prints "host_sanitize OK <checks>" and exits 0, or names
// the first failed check and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "mla.h"

static long g_checks = 0;

#define CHECK(cond, ...)                                  \
  do {                                                    \
    ++g_checks;                                           \
    if (!(cond)) {                                        \
      fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                       \
      fprintf(stderr, "\n");                              \
      exit(1);                                            \
    }                                                     \
  } while (0)

// xorshift64*: deterministic test inputs
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 0x2545F4914F6CDD1Dull;
}
static int rand_int(int lo, int hi) {  // inclusive
  return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1));
}

static mla_dims_t v2_dims(int kv_dtype, int precision) {
  mla_dims_t d;
  memset(&d, 0, sizeof(d));
  d.n_heads = 128;
  d.d_head = 128;
  d.d_latent = 512;
  d.d_rope = 64;
  d.page_size = 64;
  d.kv_dtype = kv_dtype;
  d.q_dtype = MLA_BF16;
  d.precision = precision;
  d.yarn_alpha = 1.0f;
  d.yarn_beta = 32.0f;
  d.yarn_orig_len = 4096;
  return d;
}

static bool known_status(int32_t s) { return s <= 0 && s >= MLA_ERR_ARG; }

// Workspace sizes over random batches, lengths, query counts, split
// requests, cache formats, head counts and precision modes.
static void sweep_workspace_sizes() {
  const int kv_types[] = {MLA_F32, MLA_BF16, MLA_FP8_E4M3, MLA_FP6_E2M3};
  const int heads[] = {1, 4, 16, 32, 128, 256};
  for (int it = 0; it < 4000; ++it) {
    mla_dims_t d = v2_dims(kv_types[rand_int(0, 3)], rand_int(0, 3));
    d.n_heads = heads[rand_int(0, 5)];
    if (rand_int(0, 9) == 0) d.q_dtype = MLA_F32;
    const int batch = rand_int(1, 300);
    const int T = (rand_int(0, 3) == 0) ? rand_int(1, 16) : 1 << rand_int(0, 3);
    std::vector<int32_t> lens(batch);
    const int max_len = rand_int(0, 1) ? 4096 : 200000;
    for (int b = 0; b < batch; ++b) lens[b] = rand_int(T, max_len);
    if (rand_int(0, 49) == 0) lens[rand_int(0, batch - 1)] = T - 1;   // invalid length
    int splits = rand_int(0, 3) ? 0 : rand_int(1, 64);
    if (rand_int(0, 99) == 0) splits = -1;
    if (rand_int(0, 99) == 0) splits = 5000;
    size_t bytes = 12345, bytes2 = 54321;
    const int32_t s1 = mla_decode_workspace_size(&d, lens.data(), batch, T, splits, &bytes);
    const int32_t s2 = mla_decode_workspace_size(&d, lens.data(), batch, T, splits, &bytes2);
    CHECK(known_status(s1), "unknown status %d", s1);
    CHECK(s1 == s2, "status not repeatable: %d then %d", s1, s2);
    if (s1 == MLA_OK) {
      CHECK(bytes == bytes2, "size not repeatable: %zu then %zu", bytes, bytes2);
      CHECK(bytes % 256 == 0, "size %zu not a multiple of 256", bytes);
    }
    if (splits < 0 || splits > 4096) CHECK(s1 == MLA_ERR_ARG, "split request %d gave %d", splits, s1);
    // one chunk per sequence and no recomputation flags: no workspace
    if (s1 == MLA_OK && splits == 1 && d.precision == MLA_PREC_BF16)
      CHECK(bytes == 0, "unsplit BF16 plan asked for %zu bytes", bytes);
  }
  // a NULL result pointer or NULL lengths are refused
  mla_dims_t d = v2_dims(MLA_BF16, MLA_PREC_AUTO);
  int32_t one = 16;
  size_t bytes = 0;
  CHECK(mla_decode_workspace_size(&d, &one, 1, 1, 0, nullptr) == MLA_ERR_NULL, "NULL bytes");
  CHECK(mla_decode_workspace_size(&d, nullptr, 1, 1, 0, &bytes) == MLA_ERR_NULL, "NULL lengths");
  CHECK(mla_decode_workspace_size(nullptr, &one, 1, 1, 0, &bytes) == MLA_ERR_NULL, "NULL dims");
  CHECK(mla_decode_workspace_size(&d, &one, 0, 1, 0, &bytes) != MLA_OK, "batch 0");
}

static void sweep_other_sizes() {
  for (int it = 0; it < 2000; ++it) {
    mla_dims_t d = v2_dims(rand_int(0, 1) ? MLA_BF16 : MLA_FP8_E4M3, MLA_PREC_AUTO);
    if (rand_int(0, 4) == 0) d.n_heads = rand_int(1, 300);
    const int d_model = rand_int(0, 3) ? 5120 : rand_int(-5, 20000);
    const int n = rand_int(-2, 5000);
    size_t a = 1, b = 2, c = 3, e = 4;
    const int32_t s1 = mla_kv_produce_workspace_size(&d, d_model, n, &a);
    const int32_t s2 = mla_kv_produce_workspace_size(&d, d_model, n, &b);
    CHECK(known_status(s1) && s1 == s2, "kv_produce status %d / %d", s1, s2);
    if (s1 == MLA_OK) CHECK(a == b, "kv_produce size not repeatable");
    const int o_dtype = rand_int(0, 1) ? MLA_BF16 : MLA_F32;
    const int32_t s3 = mla_out_proj_workspace_size(&d, d_model, n, o_dtype, &c);
    const int32_t s4 = mla_out_proj_workspace_size(&d, d_model, n, o_dtype, &e);
    CHECK(known_status(s3) && s3 == s4, "out_proj status %d / %d", s3, s4);
    if (s3 == MLA_OK) CHECK(c == e, "out_proj size not repeatable");
    if (n < 1) CHECK(s1 != MLA_OK && s3 != MLA_OK, "n = %d accepted", n);
  }
}

// Compute entry points with arguments the host validation must reject (no
// kernel may be launched: there is no GPU here).
static void rejected_calls() {
  alignas(256) static uint8_t buf[1 << 16];   // host bytes standing in for device pointers
  void* p = buf;
  void* odd = buf + 8;                        // not 16-byte aligned
  mla_dims_t d = v2_dims(MLA_BF16, MLA_PREC_AUTO);
  int32_t lens[2] = {64, 64};
  float* f = (float*)buf;

  CHECK(mla_absorb_q(nullptr, p, p, p, nullptr, p, 1, nullptr) == MLA_ERR_NULL, "absorb NULL dims");
  CHECK(mla_absorb_q(&d, nullptr, p, p, nullptr, p, 1, nullptr) == MLA_ERR_NULL, "absorb NULL q");
  CHECK(mla_absorb_q(&d, p, p, p, nullptr, p, 0, nullptr) != MLA_OK, "absorb 0 tokens");
  {
    mla_dims_t bad = d;
    bad.q_dtype = 7;
    CHECK(mla_absorb_q(&bad, p, p, p, nullptr, p, 1, nullptr) == MLA_ERR_DTYPE, "absorb dtype");
    bad = d;
    bad.d_latent = 0;
    CHECK(mla_absorb_q(&bad, p, p, p, nullptr, p, 1, nullptr) == MLA_ERR_DIMS, "absorb dims");
  }

  CHECK(mla_decode_attn(nullptr, p, p, nullptr, nullptr, 0, 64, (int32_t*)p, lens, 2, 1, 0,
                        p, sizeof(buf), f, f, nullptr) == MLA_ERR_NULL, "decode NULL dims");
  CHECK(mla_decode_attn(&d, nullptr, p, nullptr, nullptr, 0, 64, (int32_t*)p, lens, 2, 1, 0,
                        p, sizeof(buf), f, f, nullptr) == MLA_ERR_NULL, "decode NULL q");
  CHECK(mla_decode_attn(&d, odd, p, nullptr, nullptr, 0, 64, (int32_t*)p, lens, 2, 1, 0, p,
                        sizeof(buf), f, f, nullptr) == MLA_ERR_ALIGN, "decode misaligned q");
  {
    int32_t short_lens[2] = {64, 0};
    CHECK(mla_decode_attn(&d, p, p, nullptr, nullptr, 0, 64, (int32_t*)p, short_lens, 2, 1, 0,
                          p, sizeof(buf), f, f, nullptr) == MLA_ERR_SEQLEN, "decode L = 0");
    int32_t long_lens[2] = {64, 65};
    CHECK(mla_decode_attn(&d, p, p, nullptr, nullptr, 0, 64, (int32_t*)p, long_lens, 2, 1, 0,
                          p, sizeof(buf), f, f, nullptr) == MLA_ERR_SEQLEN, "decode L > capacity");
  }
  {
    int32_t big[1] = {8192};
    size_t need = 0;
    CHECK(mla_decode_workspace_size(&d, big, 1, 1, 8, &need) == MLA_OK && need > 0, "need");
    CHECK(mla_decode_attn(&d, p, p, nullptr, nullptr, 0, 8192, (int32_t*)p, big, 1, 1, 8, p,
                          need - 256, f, f, nullptr) == MLA_ERR_WORKSPACE, "decode small workspace");
    CHECK(mla_decode_attn(&d, p, p, nullptr, nullptr, 0, 8192, (int32_t*)p, big, 1, 1, 8,
                          nullptr, need, f, f, nullptr) == MLA_ERR_WORKSPACE, "decode no workspace");
  }
  {
    mla_dims_t fp8 = v2_dims(MLA_FP8_E4M3, MLA_PREC_AUTO);
    CHECK(mla_decode_attn(&fp8, p, p, nullptr, nullptr, 0, 64, (int32_t*)p, lens, 2, 1, 0, p,
                          sizeof(buf), f, f, nullptr) == MLA_ERR_NULL, "fp8 cache without scales");
    mla_dims_t x2 = v2_dims(MLA_FP8_E4M3, MLA_PREC_BF16X2);
    CHECK(mla_decode_attn(&x2, p, p, f, nullptr, 0, 64, (int32_t*)p, lens, 2, 1, 0, p,
                          sizeof(buf), f, f, nullptr) == MLA_ERR_UNSUPPORTED, "BF16X2 on fp8");
  }
  CHECK(mla_decode_attn_noalloc(nullptr, p, p, nullptr, nullptr, 0, 64, (int32_t*)p, lens, 2, 1,
                                0, f, f, nullptr) == MLA_ERR_NULL, "noalloc NULL dims");

  {
    int32_t seq[1] = {0}, pos[1] = {0};
    CHECK(mla_cache_append(&d, nullptr, p, seq, pos, nullptr, 1, 0, 64, 64, 0, p, nullptr, 1,
                           nullptr) == MLA_ERR_NULL, "append NULL rows");
    CHECK(mla_cache_append(&d, p, p, seq, pos, nullptr, 1, 0, 64, 64, 0, odd, nullptr, 1,
                           nullptr) == MLA_ERR_ALIGN, "append misaligned cache");
    CHECK(mla_cache_append(&d, p, p, seq, pos, nullptr, 1, 0, 64, 64, 0, p, nullptr, 0,
                           nullptr) != MLA_OK, "append 0 rows");
  }

  CHECK(mla_up_proj_v(&d, nullptr, p, p, MLA_F32, 1, nullptr) == MLA_ERR_NULL, "up_proj NULL");
  CHECK(mla_up_proj_v(&d, f, p, p, 9, 1, nullptr) == MLA_ERR_DTYPE, "up_proj dtype");
  CHECK(mla_up_proj_v(&d, f, p, p, MLA_F32, 0, nullptr) != MLA_OK, "up_proj 0 tokens");

  CHECK(mla_out_proj(&d, nullptr, MLA_BF16, p, 5120, p, MLA_F32, 1, p, sizeof(buf), nullptr) ==
            MLA_ERR_NULL, "out_proj NULL o");
  CHECK(mla_out_proj(&d, p, MLA_BF16, p, 5120, p, MLA_F32, 1, nullptr, 0, nullptr) ==
            MLA_ERR_WORKSPACE, "out_proj no workspace");
  CHECK(mla_out_proj_pack(&d, nullptr, 5120, p, nullptr) == MLA_ERR_NULL, "pack NULL");
  CHECK(mla_out_proj_packed(&d, p, p, 5120, p, MLA_F32, 1, nullptr, 0, nullptr) ==
            MLA_ERR_WORKSPACE, "packed no workspace");

  {
    int32_t seq[1] = {0}, pos[1] = {0};
    float gain[512];
    CHECK(mla_kv_produce(&d, nullptr, 5120, p, gain, 1e-6f, seq, pos, nullptr, 1, 0, 64, 64, 0,
                         p, nullptr, 1, p, sizeof(buf), nullptr) == MLA_ERR_NULL, "produce NULL h");
    CHECK(mla_kv_produce(&d, p, 5120, p, gain, 1e-6f, seq, pos, nullptr, 1, 0, 64, 64, 0, p,
                         nullptr, 1, nullptr, 0, nullptr) == MLA_ERR_WORKSPACE,
          "produce no workspace");
  }

  {
    int32_t* ip = (int32_t*)buf;
    CHECK(mla_check_page_table(&d, nullptr, 8, ip, 4, 100, ip, nullptr) == MLA_ERR_NULL, "check NULL table");
    CHECK(mla_check_page_table(&d, ip, 8, nullptr, 4, 100, ip, nullptr) == MLA_ERR_NULL, "check NULL lens");
    CHECK(mla_check_page_table(&d, ip, 8, ip, 4, 100, nullptr, nullptr) == MLA_ERR_NULL, "check NULL result");
    CHECK(mla_check_page_table(&d, ip, 0, ip, 4, 100, ip, nullptr) == MLA_ERR_ARG, "check 0 pages");
    CHECK(mla_check_page_table(&d, ip, 8, ip, 4, 0, ip, nullptr) == MLA_ERR_ARG, "check 0 cache pages");
    CHECK(mla_check_page_table(&d, ip, 1 << 16, ip, 1 << 16, 100, ip, nullptr) == MLA_ERR_ARG,
          "check table too large");
  }

  {
    int32_t* ip = (int32_t*)buf;
    CHECK(mla_absorb_append(nullptr, p, p, p, nullptr, p, 4, p, p, ip, ip, nullptr, 2, 0, 64, 128,
                            0, p, nullptr, 4, nullptr) == MLA_ERR_NULL, "absorb_append NULL dims");
    CHECK(mla_absorb_append(&d, p, p, p, nullptr, p, 0, p, p, ip, ip, nullptr, 2, 0, 64, 128, 0,
                            p, nullptr, 4, nullptr) == MLA_ERR_ARG, "absorb_append 0 tokens");
    CHECK(mla_absorb_append(&d, p, p, p, nullptr, p, 4, p, p, ip, ip, nullptr, 2, 0, 64, 128, 0,
                            odd, nullptr, 4, nullptr) == MLA_ERR_ALIGN, "absorb_append cache");
    CHECK(mla_absorb_append(&d, p, p, p, nullptr, p, 4, p, p, ip, ip, nullptr, 2, 0, 64, 100, 0,
                            p, nullptr, 4, nullptr) == MLA_ERR_ARG, "absorb_append capacity");
  }

  for (int32_t s = 5; s >= -12; --s) {
    const char* t = mla_status_string(s);
    CHECK(t != nullptr && strlen(t) > 0, "status string %d", s);
  }
  CHECK(mla_version() > 0, "version");
}

int main() {
  sweep_workspace_sizes();
  sweep_other_sizes();
  rejected_calls();
  printf("host_sanitize OK %ld\n", g_checks);
  return 0;
}
