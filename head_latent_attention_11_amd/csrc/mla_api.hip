// C ABI of the MLA decode library: argument validation, split planning and
// kernel launches.  Every check runs on the host before the first HIP call,
// so invalid arguments never touch the device.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "mla_common.hpp"

namespace mla {
hipError_t launch_absorb(const mla_dims_t&, bool, const void*, const void*, const void*,
                         const int32_t*, void*, int, RopeFreq, hipStream_t);
hipError_t launch_append(const mla_dims_t&, const void*, const void*, const int32_t*,
                         const int32_t*, const int32_t*, int, int, int, long long, int,
                         void*, float*, int, RopeFreq, hipStream_t, bool, int, int, const float*,
                         float);
hipError_t launch_combine(const DecodeArgs&, hipStream_t);
size_t gemm_xwt_workspace(int, int, int, int, int);
hipError_t launch_gemm_xwt(const void*, int, const void*, int, void*, bool, int, int, int, void*,
                           hipStream_t);
hipError_t launch_up_proj(const mla_dims_t&, bool, const float*, const void*, void*, bool,
                          int, hipStream_t);
hipError_t launch_decode_mfma(const DecodeArgs&, const ItemTable&, hipStream_t);
static_assert(sizeof(DecodeArgs) + sizeof(ItemTable) <= 4096,
              "the attention kernel's arguments must stay within 4 KB");
hipError_t launch_decode_general(const DecodeArgs&, hipStream_t);
hipError_t launch_decode_small(const DecodeArgs&, const ItemTable&, int rows_wg, hipStream_t);
}  // namespace mla

using namespace mla;

namespace {

constexpr int32_t kVersion = 10000;   // 1.0.0
constexpr int64_t kRowsPerWorkgroup = 128;  // query rows per attention workgroup (fast path)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Dimension and dtype checks shared by every entry point.
int32_t check_dims(const mla_dims_t* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->n_heads < 1 || d->n_heads > 4096) return MLA_ERR_DIMS;
  if (d->d_head < 1 || d->d_head > 256) return MLA_ERR_DIMS;
  if (d->d_latent < 4 || d->d_latent > 512 || (d->d_latent & 3)) return MLA_ERR_DIMS;
  if (d->d_rope < 0 || d->d_rope > 128 || (d->d_rope & 1)) return MLA_ERR_DIMS;
  if (d->page_size != kPage) return MLA_ERR_DIMS;
  if (d->q_dtype != MLA_F32 && d->q_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d->kv_dtype != MLA_F32 && d->kv_dtype != MLA_BF16 && d->kv_dtype != MLA_FP8_E4M3)
    return MLA_ERR_DTYPE;
  if (!(d->softmax_scale >= 0.f) || !isfinite(d->softmax_scale)) return MLA_ERR_ARG;
  if (!(d->rope_base >= 0.f) || !isfinite(d->rope_base)) return MLA_ERR_ARG;
  if (d->precision != MLA_PREC_BF16 && d->precision != MLA_PREC_FP32) return MLA_ERR_ARG;
  if (!isfinite(d->yarn_factor) || d->yarn_factor < 0.f) return MLA_ERR_ARG;
  if (d->yarn_factor > 1.f) {                        // context extension in use
    if (!(d->yarn_alpha > 0.f) || !(d->yarn_beta > d->yarn_alpha) || !isfinite(d->yarn_beta))
      return MLA_ERR_ARG;
    if (d->yarn_orig_len < 1) return MLA_ERR_ARG;
    if (!(d->yarn_coef >= 0.f) || !isfinite(d->yarn_coef)) return MLA_ERR_ARG;
  }
  return MLA_OK;
}

// The matrix-core path: DeepSeek-V2 / V3 / V2-Lite MLA shapes with bf16
// operands (absorption and up-projection run one head per workgroup).
bool fast_shape(const mla_dims_t* d) {
  return d->d_head == 128 && d->d_latent == 512 && d->d_rope == 64 && d->q_dtype == MLA_BF16;
}

// Attention in blocks of 128 rows: 32 heads of one query token per wave.
bool fast_decode(const mla_dims_t* d, int T) {
  return fast_shape(d) && d->precision == MLA_PREC_BF16 &&
         (d->kv_dtype == MLA_BF16 || d->kv_dtype == MLA_FP8_E4M3) && d->n_heads % 32 == 0 &&
         ((int64_t)d->n_heads * T) % kRowsPerWorkgroup == 0;
}

// Attention in blocks of 16 or 32 rows (16 heads of one query token per
// row sub-block) for the other head counts that are multiples of 16, bf16
// or fp8 cache.  Returns the rows per block, or 0.
int small_decode_rows(const mla_dims_t* d, int T) {
  if (!fast_shape(d) || d->precision != MLA_PREC_BF16 ||
      (d->kv_dtype != MLA_BF16 && d->kv_dtype != MLA_FP8_E4M3) || d->n_heads % 16 != 0 ||
      fast_decode(d, T))
    return 0;
  const int64_t rows = (int64_t)d->n_heads * T;
  return rows % 32 == 0 ? 32 : 16;
}

// Format of the absorbed query.
int32_t qabs_dtype(const mla_dims_t* d) {
  return d->precision == MLA_PREC_FP32 ? MLA_F32 : d->q_dtype;
}

RopeFreq rope_of(const mla_dims_t* d) {
  RopeFreq r;
  r.base = d->rope_base > 0.f ? d->rope_base : 10000.f;
  r.factor = d->yarn_factor > 1.f ? d->yarn_factor : 1.f;
  r.alpha = d->yarn_alpha;
  r.beta = d->yarn_beta;
  r.orig_len = (float)d->yarn_orig_len;
  return r;
}

// 1/sqrt(d_h + d_h^R), times the YaRN logit factor (c ln s + 1)^2 when
// context extension is on; an explicit softmax_scale replaces both.
float softmax_scale_of(const mla_dims_t* d) {
  if (d->softmax_scale > 0.f) return d->softmax_scale;
  double sc = 1.0 / sqrt((double)(d->d_head + d->d_rope));
  if (d->yarn_factor > 1.f) {
    const double m = (double)d->yarn_coef * log((double)d->yarn_factor) + 1.0;
    sc *= m * m;
  }
  return (float)sc;
}

int32_t status_of(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

struct Plan {
  int num_splits;   // > 0: per-sequence equal splits
  int chunk;        // global chunk when num_splits == 0
  int n_items;
  int row_blocks;
  bool any_split;
  bool part_bf16;
  size_t ws_bytes;
};

// Split-KV plan.  num_splits > 0 cuts each sequence into at most that many
// chunks of equal size (multiple of 64 tokens).  num_splits == 0 picks one
// chunk length for all sequences so that the work items fill the GPU about
// once: chunk = ceil(total tokens * row blocks / 256 CUs), rounded up to 64
// and at least 256 tokens.
int32_t make_plan(const mla_dims_t* d, const int32_t* lens, int B, int T,
                  int num_splits, Plan* p) {
  if (B < 1 || T < 1 || T > 1024) return MLA_ERR_ARG;
  if (num_splits < 0 || num_splits > 4096) return MLA_ERR_ARG;
  const int small = small_decode_rows(d, T);
  const bool fast = fast_decode(d, T) || small > 0;   // matrix-core kernels
  const int64_t rows = (int64_t)d->n_heads * T;
  const int64_t rb = small > 0 ? rows / small : fast ? rows / kRowsPerWorkgroup : rows;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < 1 || lens[b] < T) return MLA_ERR_SEQLEN;
    total += lens[b];
  }
  p->num_splits = num_splits;
  p->row_blocks = (int)rb;
  p->chunk = 0;
  if (num_splits == 0) {
    const int64_t target_items = std::max<int64_t>(1, (kNumCU + rb - 1) / rb);
    int64_t c = (total + target_items - 1) / target_items;
    c = ((c + kPage - 1) / kPage) * kPage;
    c = std::max<int64_t>(c, kMinChunk);
    c = std::min<int64_t>(c, 1 << 30);
    p->chunk = (int)c;
  }
  int64_t items = 0;
  bool any = false;
  for (int b = 0; b < B; ++b) {
    const int ns = splits_of(lens[b], p->num_splits, p->chunk);
    items += ns;
    any = any || ns > 1;
  }
  if (items * rb > INT32_MAX / 2) return MLA_ERR_ARG;
  p->n_items = (int)items;
  p->any_split = any;
  // partials: fp32 LSE per (item, row), then the latent partials (bf16 on
  // the matrix-core path, fp32 on the general path)
  const size_t part_elem = fast ? 2 : 4;
  const size_t lse_bytes = ((size_t)items * rows * sizeof(float) + 255) / 256 * 256;
  p->part_bf16 = fast;
  p->ws_bytes = any ? lse_bytes + (size_t)items * rows * d->d_latent * part_elem : 0;
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_version(void) { return kVersion; }

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_DIMS: return "dimension fields inconsistent or out of range";
    case MLA_ERR_DTYPE: return "unknown or unsupported dtype combination";
    case MLA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MLA_ERR_SEQLEN: return "a sequence length is < 1, < T, or beyond the cache capacity";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_UNSUPPORTED: return "request not supported by this build";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_ARG: return "invalid count, size or flag argument";
    default: return "unknown status";
  }
}

int32_t mla_absorb_q(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                     const void* w_uk, const int32_t* q_pos, void* q_abs,
                     int32_t n_tokens, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!q_nope || !w_uk || !q_abs || (dims->d_rope > 0 && !q_rope)) return MLA_ERR_NULL;
  if (n_tokens < 1) return MLA_ERR_ARG;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_abs) ||
      (q_rope && !aligned16(q_rope)))
    return MLA_ERR_ALIGN;
  const bool fast = fast_shape(dims);
  return status_of(launch_absorb(*dims, fast, q_nope, q_rope, w_uk, q_pos, q_abs, n_tokens,
                                 rope_of(dims), (hipStream_t)stream));
}

int32_t mla_cache_append(const mla_dims_t* dims, const void* new_c, const void* new_kr,
                         const int32_t* seq_idx, const int32_t* pos,
                         const int32_t* page_table, int32_t batch, int32_t max_pages,
                         int32_t max_len, int64_t cache_rows, int32_t apply_rope,
                         void* cache, float* kv_scale, int32_t n_rows, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!new_c || !seq_idx || !pos || !cache || (dims->d_rope > 0 && !new_kr))
    return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_FP8_E4M3) {
    if (!kv_scale) return MLA_ERR_NULL;
  } else if (kv_scale) {
    return MLA_ERR_ARG;
  }
  if (n_rows < 1 || batch < 1 || cache_rows < 1) return MLA_ERR_ARG;
  if (apply_rope != 0 && apply_rope != 1) return MLA_ERR_ARG;
  if (page_table) {
    if (max_pages < 1) return MLA_ERR_ARG;
  } else {
    if (max_len < 1) return MLA_ERR_ARG;
    if ((int64_t)batch * max_len > cache_rows) return MLA_ERR_ARG;
  }
  if (dims->d_latent + dims->d_rope > 640) return MLA_ERR_DIMS;
  if (!aligned16(new_c) || !aligned16(cache) || (new_kr && !aligned16(new_kr)))
    return MLA_ERR_ALIGN;
  return status_of(launch_append(*dims, new_c, new_kr, seq_idx, pos, page_table, batch,
                                 max_pages, max_len, cache_rows, apply_rope, cache,
                                 kv_scale, n_rows, rope_of(dims), (hipStream_t)stream,
                                 dims->kv_dtype == MLA_F32, dims->d_latent, dims->d_rope,
                                 nullptr, 0.f));
}

// Checks shared by the cache writers (mla_cache_append, mla_kv_produce).
static int32_t check_append(const mla_dims_t* dims, const int32_t* seq_idx, const int32_t* pos,
                            const int32_t* page_table, int32_t batch, int32_t max_pages,
                            int32_t max_len, int64_t cache_rows, int32_t apply_rope,
                            const void* cache, const float* kv_scale, int32_t n_rows) {
  if (!seq_idx || !pos || !cache) return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_FP8_E4M3) {
    if (!kv_scale) return MLA_ERR_NULL;
  } else if (kv_scale) {
    return MLA_ERR_ARG;
  }
  if (n_rows < 1 || batch < 1 || cache_rows < 1) return MLA_ERR_ARG;
  if (apply_rope != 0 && apply_rope != 1) return MLA_ERR_ARG;
  if (page_table) {
    if (max_pages < 1) return MLA_ERR_ARG;
  } else {
    if (max_len < 1) return MLA_ERR_ARG;
    if ((int64_t)batch * max_len > cache_rows) return MLA_ERR_ARG;
  }
  if (dims->d_latent + dims->d_rope > 640) return MLA_ERR_DIMS;
  if (!aligned16(cache)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

static size_t produce_rows_bytes(const mla_dims_t* d, int32_t n_rows) {
  return ((size_t)n_rows * (d->d_latent + d->d_rope) * sizeof(float) + 255) / 256 * 256;
}

int32_t mla_kv_produce_workspace_size(const mla_dims_t* dims, int32_t d_model, int32_t n_rows,
                                      size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL;
  if (d_model < 1 || n_rows < 1) return MLA_ERR_ARG;
  const int D = dims->d_latent + dims->d_rope;
  *bytes = produce_rows_bytes(dims, n_rows) +
           gemm_xwt_workspace(D, d_model, n_rows, dims->q_dtype, dims->q_dtype);
  return MLA_OK;
}

int32_t mla_kv_produce(const mla_dims_t* dims, const void* h, int32_t d_model,
                       const void* w_dkv_kr, const float* norm_gain, float norm_eps,
                       const int32_t* seq_idx, const int32_t* pos, const int32_t* page_table,
                       int32_t batch, int32_t max_pages, int32_t max_len, int64_t cache_rows,
                       int32_t apply_rope, void* cache, float* kv_scale, int32_t n_rows,
                       void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!h || !w_dkv_kr) return MLA_ERR_NULL;
  st = check_append(dims, seq_idx, pos, page_table, batch, max_pages, max_len, cache_rows,
                    apply_rope, cache, kv_scale, n_rows);
  if (st != MLA_OK) return st;
  if (d_model < 1) return MLA_ERR_ARG;
  if (!(norm_eps >= 0.f) || !isfinite(norm_eps)) return MLA_ERR_ARG;
  if (!aligned16(h) || !aligned16(w_dkv_kr) || (norm_gain && !aligned16(norm_gain)) ||
      (workspace && !aligned16(workspace)))
    return MLA_ERR_ALIGN;
  const int D = dims->d_latent + dims->d_rope;
  const size_t rows_b = produce_rows_bytes(dims, n_rows);
  const size_t need = rows_b + gemm_xwt_workspace(D, d_model, n_rows, dims->q_dtype,
                                                  dims->q_dtype);
  if (!workspace || ws_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  float* rows = (float*)workspace;
  hipError_t e = launch_gemm_xwt(h, dims->q_dtype, w_dkv_kr, dims->q_dtype, rows, true, n_rows,
                                 D, d_model, (char*)workspace + rows_b, s);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  return status_of(launch_append(*dims, rows, rows + dims->d_latent, seq_idx, pos, page_table,
                                 batch, max_pages, max_len, cache_rows, apply_rope, cache,
                                 kv_scale, n_rows, rope_of(dims), s, true, D, D, norm_gain,
                                 norm_eps));
}

int32_t mla_decode_workspace_size(const mla_dims_t* dims, const int32_t* seq_lens_host,
                                  int32_t batch, int32_t q_tokens, int32_t num_splits,
                                  size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!seq_lens_host || !bytes) return MLA_ERR_NULL;
  Plan p;
  st = make_plan(dims, seq_lens_host, batch, q_tokens, num_splits, &p);
  if (st != MLA_OK) return st;
  *bytes = p.ws_bytes;
  return MLA_OK;
}

int32_t mla_decode_attn(const mla_dims_t* dims, const void* q_abs, const void* cache,
                        const float* kv_scale, const int32_t* page_table, int32_t max_pages,
                        int32_t max_len, const int32_t* seq_lens,
                        const int32_t* seq_lens_host, int32_t batch, int32_t q_tokens,
                        int32_t num_splits, void* workspace, size_t ws_bytes,
                        float* out_latent, float* out_lse, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!q_abs || !cache || !seq_lens || !seq_lens_host || !out_latent || !out_lse)
    return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_FP8_E4M3 && !kv_scale) return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(cache) || !aligned16(out_latent) ||
      !aligned16(out_lse) || (workspace && !aligned16(workspace)))
    return MLA_ERR_ALIGN;
  Plan p;
  st = make_plan(dims, seq_lens_host, batch, q_tokens, num_splits, &p);
  if (st != MLA_OK) return st;
  const int64_t cap = page_table ? (int64_t)max_pages * kPage : (int64_t)max_len;
  if (page_table ? max_pages < 1 : max_len < 1) return MLA_ERR_ARG;
  for (int b = 0; b < batch; ++b)
    if (seq_lens_host[b] > cap) return MLA_ERR_SEQLEN;
  if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes)) return MLA_ERR_WORKSPACE;

  DecodeArgs a = {};
  a.q_abs = q_abs;
  a.cache = cache;
  a.kv_scale = kv_scale;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  const int64_t rows = (int64_t)dims->n_heads * q_tokens;
  const size_t lse_bytes = ((size_t)p.n_items * rows * sizeof(float) + 255) / 256 * 256;
  a.part_lse = p.any_split ? (float*)workspace : nullptr;
  a.part_o = p.any_split ? (void*)((char*)workspace + lse_bytes) : nullptr;
  a.part_bf16 = p.part_bf16 ? 1 : 0;
  a.out_latent = out_latent;
  a.out_lse = out_lse;
  a.B = batch;
  a.T = q_tokens;
  a.n_h = dims->n_heads;
  a.d_c = dims->d_latent;
  a.d_r = dims->d_rope;
  a.max_pages = page_table ? max_pages : 0;
  a.max_len = page_table ? 0 : max_len;
  a.num_splits = p.num_splits;
  a.chunk = p.chunk;
  a.n_items = p.n_items;
  a.row_blocks = p.row_blocks;
  a.q_dtype = qabs_dtype(dims);
  a.kv_dtype = dims->kv_dtype;
  a.scale_log2 = softmax_scale_of(dims) * 1.4426950408889634f;
  {
    bool uniform = seq_lens_host[0] > 0;
    for (int b = 1; b < batch && uniform; ++b) uniform = seq_lens_host[b] == seq_lens_host[0];
    if (uniform &&
        (int64_t)batch * splits_of(seq_lens_host[0], p.num_splits, p.chunk) == p.n_items)
      a.uniform_len = seq_lens_host[0];
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const int small_rows = small_decode_rows(dims, q_tokens);
  if (fast_decode(dims, q_tokens) || small_rows > 0) {
    ItemTable tab;
    tab.n = 0;
    tab.uniform_len = a.uniform_len;
    if (a.uniform_len > 0) {
    } else if (p.n_items <= kItemTable && batch < (1 << 20)) {
      // items in sequence order with their token counts, then largest first
      struct It { uint32_t key; int32_t id; int32_t size; };
      std::vector<It> its;
      its.reserve(p.n_items);
      for (int b = 0; b < batch; ++b) {
        const int L = seq_lens_host[b];
        const int c = chunk_of(L, p.num_splits, p.chunk);
        const int ns = splits_of(L, p.num_splits, p.chunk);
        for (int sp = 0; sp < ns && sp < 4096; ++sp)
          its.push_back({uint32_t(b) | (uint32_t(sp) << 20), (int32_t)its.size(),
                         std::min(c, L - sp * c)});
      }
      if ((int64_t)its.size() == p.n_items) {
        std::stable_sort(its.begin(), its.end(),
                         [](const It& x, const It& y) { return x.size > y.size; });
        // Workgroup g runs table entry xcd_logical_index(g, G) / row_blocks:
        // the entries are filled with the largest items in the order in
        // which workgroups first reach them.
        const int n = (int)its.size(), G = n * p.row_blocks;
        std::vector<char> done(n, 0);
        int next = 0;
        for (int g = 0; g < G && next < n; ++g) {
          const int i = xcd_logical_index(g, G) / p.row_blocks;
          if (done[i]) continue;
          done[i] = 1;
          tab.seq_split[i] = its[next].key;
          tab.item_id[i] = its[next].id;
          ++next;
        }
        tab.n = (next == n) ? n : 0;
      }
    }
    e = small_rows > 0 ? launch_decode_small(a, tab, small_rows, s) : launch_decode_mfma(a, tab, s);
  } else {
    e = launch_decode_general(a, s);
  }
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  if (p.any_split) {
    e = launch_combine(a, s);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

int32_t mla_out_proj_workspace_size(const mla_dims_t* dims, int32_t d_model, int32_t n_tokens,
                                    int32_t o_dtype, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL;
  if (o_dtype != MLA_F32 && o_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d_model < 1 || n_tokens < 1) return MLA_ERR_ARG;
  *bytes = gemm_xwt_workspace(d_model, dims->n_heads * dims->d_head, n_tokens, o_dtype,
                              dims->q_dtype);
  return MLA_OK;
}

int32_t mla_out_proj(const mla_dims_t* dims, const void* o, int32_t o_dtype, const void* w_o,
                     int32_t d_model, void* u, int32_t u_dtype, int32_t n_tokens,
                     void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!o || !w_o || !u) return MLA_ERR_NULL;
  if (o_dtype != MLA_F32 && o_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (u_dtype != MLA_F32 && u_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d_model < 1 || n_tokens < 1) return MLA_ERR_ARG;
  if (!aligned16(o) || !aligned16(w_o) || !aligned16(u) || (workspace && !aligned16(workspace)))
    return MLA_ERR_ALIGN;
  const int K = dims->n_heads * dims->d_head;
  const size_t need = gemm_xwt_workspace(d_model, K, n_tokens, o_dtype, dims->q_dtype);
  if (need > 0 && (!workspace || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  return status_of(launch_gemm_xwt(o, o_dtype, w_o, dims->q_dtype, u, u_dtype == MLA_F32,
                                   n_tokens, d_model, K, workspace, (hipStream_t)stream));
}

int32_t mla_up_proj_v(const mla_dims_t* dims, const float* latent, const void* w_uv,
                      void* out, int32_t out_dtype, int32_t n_tokens, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!latent || !w_uv || !out) return MLA_ERR_NULL;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (n_tokens < 1) return MLA_ERR_ARG;
  if (!aligned16(latent) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  return status_of(launch_up_proj(*dims, fast_shape(dims), latent, w_uv, out,
                                  out_dtype == MLA_F32, n_tokens, (hipStream_t)stream));
}

}  // extern "C"
