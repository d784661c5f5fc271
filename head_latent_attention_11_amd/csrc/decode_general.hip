// Attention over the latent cache, general path (any dimensions, every
// q / kv number format).  One workgroup per (work item, query row).
//
// Absorbed form of the attention-output equation ("DeepSeek-V3 Technical
// Report" notes, MLA section; absorption per "DeepSeek-V2: Strong,
// Economical, Efficient", Appendix C):
//   s_j = scale * q_abs . [c_j ; k^R_j],  latent = sum_j softmax(s)_j c_j.
// Tokens are processed in chunks of 256 with an online softmax (running max
// m and sum l, both in the log2 domain).
#include <math.h>

#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

template <int KV> __device__ inline float kv_elem(const void* cache, size_t i);
template <> __device__ inline float kv_elem<MLA_F32>(const void* c, size_t i) {
  return ((const float*)c)[i];
}
template <> __device__ inline float kv_elem<MLA_BF16>(const void* c, size_t i) {
  return bf16_bits_to_f32(((const uint16_t*)c)[i]);
}
template <> __device__ inline float kv_elem<MLA_FP8_E4M3>(const void* c, size_t i) {
  return e4m3_to_f32(((const uint8_t*)c)[i]);
}

template <int QD, int KV>
__global__ __launch_bounds__(256) void decode_general_kernel(DecodeArgs a) {
  constexpr int NT = 256;
  __shared__ float s_q[1024];
  __shared__ float s_p[NT];
  __shared__ long long s_row[NT];
  __shared__ float s_red[NT / 64];
  const int tid = threadIdx.x;
  const int rows = a.n_h * a.T;
  const int D = a.d_c + a.d_r;
  const int g = blockIdx.x;
  const int item = g / rows, row = g % rows;
  const ItemLoc loc = locate_item(a.seq_lens, a.B, a.num_splits, a.chunk, item);
  if (loc.b < 0) return;
  const int b = loc.b;
  const int L = a.seq_lens[b];
  const int c = chunk_of(L, a.num_splits, a.chunk);
  const int t0 = loc.s * c;
  const int tau = row / a.n_h, head = row % a.n_h;
  const int limit = L - a.T + tau;                     // last visible position
  const int t1 = min(min(L, t0 + c), limit + 1);
  const int nq = b * a.T + tau;

  for (int e = tid; e < D; e += NT) {
    const size_t qi = ((size_t)nq * a.n_h + head) * D + e;
    s_q[e] = (QD == MLA_F32) ? ((const float*)a.q_abs)[qi]
                             : bf16_bits_to_f32(((const uint16_t*)a.q_abs)[qi]);
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;   // log2-domain running max, sum
  float acc0 = 0.f, acc1 = 0.f;          // latent dims tid, tid + 256
  for (int base = t0; base < t1; base += NT) {
    const int j = base + tid;
    float s = -INFINITY;
    long long crow = -1;
    if (j < t1) {
      if (a.page_table)
        crow = (long long)a.page_table[(size_t)b * a.max_pages + j / kPage] * kPage + j % kPage;
      else
        crow = (long long)b * a.max_len + j;
      float dot = 0.f;
      for (int e = 0; e < D; ++e) dot = fmaf(s_q[e], kv_elem<KV>(a.cache, (size_t)crow * D + e), dot);
      if (KV == MLA_FP8_E4M3) dot *= a.kv_scale[crow];
      s = dot * a.scale_log2;
    }
    s_row[tid] = crow;
    // chunk max
    float mx = s;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if ((tid & 63) == 0) s_red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float p = exp2f(s - m_use);
    s_p[tid] = p;
    float ps = p;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off, 64);
    if ((tid & 63) == 0) s_red[tid >> 6] = ps;
    __syncthreads();
    ps = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    l_run = l_run * alpha + ps;
    m_run = m_new;
    acc0 *= alpha;
    acc1 *= alpha;
    const int n = min(NT, t1 - base);
    for (int jj = 0; jj < n; ++jj) {
      const float pj = s_p[jj];
      const long long cr = s_row[jj];
      float w = pj;
      if (KV == MLA_FP8_E4M3) w *= a.kv_scale[cr];
      if (tid < a.d_c) acc0 = fmaf(w, kv_elem<KV>(a.cache, (size_t)cr * D + tid), acc0);
      if (tid + NT < a.d_c) acc1 = fmaf(w, kv_elem<KV>(a.cache, (size_t)cr * D + tid + NT), acc1);
    }
    __syncthreads();
  }

  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  const float lse = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  float* dst;
  float* dlse;
  if (loc.ns == 1) {
    dst = a.out_latent + ((size_t)nq * a.n_h + head) * a.d_c;
    dlse = a.out_lse + (size_t)nq * a.n_h + head;
  } else {
    dst = (float*)a.part_o + ((size_t)item * rows + row) * a.d_c;
    dlse = a.part_lse + (size_t)item * rows + row;
  }
  if (tid < a.d_c) dst[tid] = acc0 * inv;
  if (tid + NT < a.d_c) dst[tid + NT] = acc1 * inv;
  if (tid == 0) *dlse = lse;
}

hipError_t launch_decode_general(const DecodeArgs& a, hipStream_t st) {
  const int grid = a.n_items * a.n_h * a.T;
#define MLA_GEN(QD, KV)                                                        \
  if (a.q_dtype == QD && a.kv_dtype == KV) {                                   \
    hipLaunchKernelGGL((decode_general_kernel<QD, KV>), dim3(grid), dim3(256), \
                       0, st, a);                                              \
    return hipGetLastError();                                                  \
  }
  MLA_GEN(MLA_F32, MLA_F32)
  MLA_GEN(MLA_F32, MLA_BF16)
  MLA_GEN(MLA_F32, MLA_FP8_E4M3)
  MLA_GEN(MLA_BF16, MLA_F32)
  MLA_GEN(MLA_BF16, MLA_BF16)
  MLA_GEN(MLA_BF16, MLA_FP8_E4M3)
#undef MLA_GEN
  return hipErrorInvalidValue;
}

}  // namespace mla
