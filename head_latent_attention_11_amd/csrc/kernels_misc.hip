// Query absorption, cache append, split combine and value up-projection.
//
// Sources: "DeepSeek-V2: Strong, Economical, Efficient", section 2.1.2 and
// Appendix C (W^UK absorbed into the query side, W^UV applied after the
// latent sum), section 2.1.3 (decoupled RoPE, cached shared k^R);
// "DeepSeek-V3 Technical Report" notes, MLA section (head-block layout of
// W^UK / W^UV; attention-output equation whose sum over tokens is what the
// split combine re-associates).
#include <math.h>

#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

// ============================================================ RoPE helper
// Interleaved pairs (2k, 2k+1) rotated by pos * theta_k (rope_theta, with
// or without context extension); angle and rotation in double precision.
__device__ inline void rope_rot(float x0, float x1, int pos, double theta, float* y0, float* y1) {
  double ang = (double)pos * theta;
  double s, c;
  sincos(ang, &s, &c);
  *y0 = (float)((double)x0 * c - (double)x1 * s);
  *y1 = (float)((double)x0 * s + (double)x1 * c);
}
__device__ inline void rope_pair(float x0, float x1, int pos, int k, int d,
                                 const RopeFreq& rf, float* y0, float* y1) {
  rope_rot(x0, x1, pos, rope_theta(k, d, rf), y0, y1);
}

template <typename T> __device__ inline float load_f(const T* p, size_t i);
template <> __device__ inline float load_f<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float load_f<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}
template <typename T> __device__ inline void store_f(T* p, size_t i, float v);
template <> __device__ inline void store_f<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ inline void store_f<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

// ====================================================== absorb: MFMA path
// q_abs[n, i, 0:512] = W^UK_i^T q_nope[n, i, :], d_h = 128.  One workgroup
// per (head i, block of 128 latent columns); wave w owns 32 columns and
// computes D^T[cols x tokens] = W^T q^T for blocks of 32 tokens.  Every
// global access is coalesced (16-byte chunks, consecutive lanes on
// consecutive addresses): a lane-per-row pattern would cost the address
// unit one cycle per lane.  The 128 x 128 W^UK_i block and each query block
// are staged row-major in LDS; W^UK is read back column-wise with the gfx950
// transposing LDS read (within each group of 16 lanes, ds_read_b64_tr_b16
// hands lane i element i%4 of the 8-byte chunks addressed by lanes 4k + i/4,
// k = 0..3, so four rows of 16 elements come back as 16 columns of 4), and
// the results go back through LDS so that each token's 128 columns are
// written as one contiguous run.
constexpr int kAbsCols = 128, kAbsDh = 128, kAbsLdsRow = kAbsCols + 8;
constexpr int kAbsOutRow = 528;       // bytes per token row of the output staging

typedef short shortx4 __attribute__((ext_vector_type(4)));

// two floats -> packed bf16 pair (hardware round to nearest even)
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

__device__ inline shortx4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (shortx4 __attribute__((address_space(3)))*)(p));
}

template <typename OutT>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ q_pos,
    OutT* __restrict__ q_abs, int n_tok, int n_h, RopeFreq rope) {
  constexpr int DC = 512, DR = 64, D = DC + DR;
  __shared__ __attribute__((aligned(16))) uint16_t ws[kAbsDh * kAbsLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t qs[32 * kAbsLdsRow];
  __shared__ __attribute__((aligned(16))) unsigned char os[32 * kAbsOutRow];
  const int head = blockIdx.x >> 2, cb = blockIdx.x & 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, j = lane & 15;

  // blockIdx.y splits the tokens when there are few heads: group y takes
  // the blocks of 32 tokens t0 = 32 (y + k gridDim.y).
  // The RoPE part q_abs[..., 512:576] is shared out over the head's
  // workgroups: pair p = 256 cb + tid + 1024 (y + u gridDim.y) (token p / 32,
  // pair k = p % 32 = tid % 32 for every u).  The first pair's inputs are
  // loaded before the W^UK block (loads complete in order) and rotated while
  // it is in flight.
  const int n_pairs = n_tok * (DR / 2), rk = tid & 31;
  const int p_first = 1024 * blockIdx.y + cb * 256 + tid, p_step = 1024 * gridDim.y;
  const int t_first = 32 * blockIdx.y, t_step = 32 * gridDim.y;
  float rx0 = 0.f, rx1 = 0.f;
  int rpos = 0;
  if (p_first < n_pairs) {
    const uint16_t* src = q_rope + ((size_t)(p_first >> 5) * n_h + head) * DR + 2 * rk;
    rx0 = bf16_bits_to_f32(src[0]);
    rx1 = bf16_bits_to_f32(src[1]);
    if (q_pos) rpos = q_pos[p_first >> 5];
  }

  // query block loader: 32 tokens x 128 d_h = 512 chunks of 16 bytes
  auto load_q = [&](int t0, u32x4* qv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i, t = ch >> 4, c8 = (ch & 15) * 8;
      qv[i] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + t < n_tok) qv[i] = *(const u32x4*)(q_nope + ((size_t)(t0 + t) * n_h + head) * kAbsDh + c8);
    }
  };
  auto store_q = [&](const u32x4* qv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i, t = ch >> 4, c8 = (ch & 15) * 8;
      *(u32x4*)(qs + t * kAbsLdsRow + c8) = qv[i];
    }
  };
  u32x4 qv[2];
  load_q(t_first, qv);
  // W^UK[head][r][cb*128 : cb*128 + 128], row-major 16-byte chunks
  const uint16_t* wsrc = w_uk + (size_t)head * kAbsDh * DC + cb * kAbsCols;
  u32x4 stg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + 256 * i, r = ch >> 4, c8 = (ch & 15) * 8;
    stg[i] = *(const u32x4*)(wsrc + (size_t)r * DC + c8);
  }
  const double theta = q_pos ? rope_theta(rk, DR, rope) : 0.0;
  for (int p = p_first; p < n_pairs; p += p_step) {
    const int tok = p >> 5;
    float x0 = rx0, x1 = rx1;
    int pos = rpos;
    if (p != p_first) {
      const uint16_t* src = q_rope + ((size_t)tok * n_h + head) * DR + 2 * rk;
      x0 = bf16_bits_to_f32(src[0]);
      x1 = bf16_bits_to_f32(src[1]);
      if (q_pos) pos = q_pos[tok];
    }
    if (q_pos) rope_rot(x0, x1, pos, theta, &x0, &x1);
    OutT* dst = q_abs + ((size_t)tok * n_h + head) * D + DC + 2 * rk;
    if constexpr (sizeof(OutT) == 4) {
      *(float2*)dst = float2{x0, x1};
    } else {
      *(uint32_t*)dst = pack_bf16x2(x0, x1);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + 256 * i, r = ch >> 4, c8 = (ch & 15) * 8;
    *(u32x4*)(ws + r * kAbsLdsRow + c8) = stg[i];
  }
  store_q(qv);
  __syncthreads();

  // A operand (W^T, lane: column 32*wave + l32, d_h values 16k + 8h + e)
  bf16x8 af[kAbsDh / 16];
  const int colbase = wave * 32 + 16 * (g & 1) + 4 * (j & 3);
#pragma unroll
  for (int k = 0; k < kAbsDh / 16; ++k) {
    const int r0 = 16 * k + 8 * h;
    const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(ws + (r0 + (j >> 2)) * kAbsLdsRow + colbase));
    const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(ws + (r0 + 4 + (j >> 2)) * kAbsLdsRow + colbase));
    af[k] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  }

  for (int t0 = t_first; t0 < n_tok; t0 += t_step) {
    if (t0 > t_first) {                // next query block (loaded during the last one)
      __syncthreads();                 // the last block's operand reads and copy-out are done
      store_q(qv);
      __syncthreads();
    }
    if (t0 + t_step < n_tok) load_q(t0 + t_step, qv);   // in flight during this block
    floatx16 acc = {};
#pragma unroll
    for (int k = 0; k < kAbsDh / 16; ++k) {
      const bf16x8 bq = *(const bf16x8*)(qs + l32 * kAbsLdsRow + 16 * k + 8 * h);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[k], bq, acc, 0, 0, 0);
    }
    // acc[r]: column-in-block 8(r/4) + 4h + r%4 of wave's 32, token l32
    OutT* orow = (OutT*)(os + l32 * kAbsOutRow) + wave * 32;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if constexpr (sizeof(OutT) == 4)
        *(floatx4*)(orow + 8 * jj + 4 * h) =
            floatx4{acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]};
      else
        *(u32x2*)(orow + 8 * jj + 4 * h) = u32x2{pack_bf16x2(acc[4 * jj], acc[4 * jj + 1]),
                                                pack_bf16x2(acc[4 * jj + 2], acc[4 * jj + 3])};
    }
    __syncthreads();
    // 32 tokens x 128 columns, 16-byte chunks, each token's run contiguous
    constexpr int per_row = kAbsCols * (int)sizeof(OutT) / 16;
#pragma unroll
    for (int i = 0; i < 32 * per_row / 256; ++i) {
      const int ch = tid + 256 * i, t = ch / per_row, c = ch % per_row;
      if (t0 + t < n_tok)
        *(u32x4*)((unsigned char*)(q_abs + ((size_t)(t0 + t) * n_h + head) * D + cb * kAbsCols) + 16 * c) =
            *(const u32x4*)(os + t * kAbsOutRow + 16 * c);
    }
  }
}

// =================================================== absorb: general path
template <typename T, typename OutT>
__global__ __launch_bounds__(256) void absorb_general_kernel(
    const T* __restrict__ q_nope, const T* __restrict__ q_rope,
    const T* __restrict__ w_uk, const int32_t* __restrict__ q_pos,
    OutT* __restrict__ q_abs, int n_tok, int n_h, int d_h, int d_c, int d_r,
    RopeFreq rope) {
  const int D = d_c + d_r;
  const size_t total = (size_t)n_tok * n_h * D;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int e = int(idx % D);
    const size_t row = idx / D;            // tok * n_h + head
    const int head = int(row % n_h), tok = int(row / n_h);
    float v;
    if (e < d_c) {
      float acc = 0.f;
      const T* q = q_nope + row * d_h;
      const T* w = w_uk + (size_t)head * d_h * d_c + e;
      for (int r = 0; r < d_h; ++r) acc = fmaf(load_f(q, r), load_f(w, (size_t)r * d_c), acc);
      v = acc;
    } else {
      const int k = (e - d_c) >> 1;
      const T* q = q_rope + row * d_r;
      float x0 = load_f(q, 2 * k), x1 = load_f(q, 2 * k + 1);
      if (q_pos) rope_pair(x0, x1, q_pos[tok], k, d_r, rope, &x0, &x1);
      v = ((e - d_c) & 1) ? x1 : x0;
    }
    store_f(q_abs, idx, v);
  }
}

// ================================================================ append
// One wave per new row.  Source rows are F32 or BF16, row r of new_c at
// r * c_stride (elements), of new_kr at r * kr_stride.  With norm_gain, the
// c^KV part is RMS-normalised first: c_i * g_i / sqrt(mean(c^2) + eps).
template <typename SrcT, int KV>
__global__ __launch_bounds__(256) void append_kernel(
    const SrcT* __restrict__ new_c, const SrcT* __restrict__ new_kr,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int B, int max_pages, int max_len,
    long long cache_rows, int apply_rope, void* __restrict__ cache,
    float* __restrict__ kv_scale, int n_rows, int d_c, int d_r, RopeFreq rope,
    int c_stride, int kr_stride, const float* __restrict__ norm_gain, float norm_eps) {
  const int lane = threadIdx.x & 63;
  const int D = d_c + d_r;
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < n_rows; r += gridDim.x * 4) {
    const int sq = seq_idx[r], p = pos[r];
    if (sq < 0 || sq >= B || p < 0) continue;
    long long row;
    if (page_table) {
      if (p / kPage >= max_pages) continue;
      const int page = page_table[(size_t)sq * max_pages + p / kPage];
      if (page < 0) continue;
      row = (long long)page * kPage + p % kPage;
    } else {
      if (p >= max_len) continue;
      row = (long long)sq * max_len + p;
    }
    if (row >= cache_rows) continue;

    // gather this lane's elements (at most 10 per lane: D <= 640)
    float v[10];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 10; ++k) {
      const int e = lane + 64 * k;
      float x = 0.f;
      if (e < d_c) {
        x = load_f(new_c, (size_t)r * c_stride + e);
      } else if (e < D) {
        const int q = e - d_c;
        if (apply_rope) {
          const int kp = q >> 1;
          float x0 = load_f(new_kr, (size_t)r * kr_stride + 2 * kp);
          float x1 = load_f(new_kr, (size_t)r * kr_stride + 2 * kp + 1);
          float y0, y1;
          rope_pair(x0, x1, p, kp, d_r, rope, &y0, &y1);
          x = (q & 1) ? y1 : y0;
        } else {
          x = load_f(new_kr, (size_t)r * kr_stride + q);
        }
      }
      v[k] = x;
    }
    if (norm_gain) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 10; ++k)
        if (lane + 64 * k < d_c) ss = fmaf(v[k], v[k], ss);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
      const float inv = 1.0f / sqrtf(ss / float(d_c) + norm_eps);
#pragma unroll
      for (int k = 0; k < 10; ++k)
        if (lane + 64 * k < d_c) v[k] = v[k] * inv * norm_gain[lane + 64 * k];
    }
#pragma unroll
    for (int k = 0; k < 10; ++k) amax = fmaxf(amax, fabsf(v[k]));
    if (KV == MLA_F32) {
      float* dst = (float*)cache + row * D;
#pragma unroll
      for (int k = 0; k < 10; ++k) if (lane + 64 * k < D) dst[lane + 64 * k] = v[k];
    } else if (KV == MLA_BF16) {
      uint16_t* dst = (uint16_t*)cache + row * D;
#pragma unroll
      for (int k = 0; k < 10; ++k) if (lane + 64 * k < D) dst[lane + 64 * k] = f32_to_bf16_bits(v[k]);
    } else {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const float s = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
      uint8_t* dst = (uint8_t*)cache + row * D;
#pragma unroll
      for (int k = 0; k < 10; ++k)
        if (lane + 64 * k < D) dst[lane + 64 * k] = uint8_t(f32_to_e4m3(__fdiv_rn(v[k], s)));
      if (lane == 0) kv_scale[row] = s;
    }
  }
}

// =============================================================== combine
// LSE combine of the split partials of one (query token, head) row:
// lse = ln sum_s e^{lse_s};  latent = sum_s e^{lse_s - lse} latent_s.
// Exact re-association of the sum in the attention-output equation.
// One wave per row, four rows per workgroup.  The split LSEs are read lane-
// parallel and reduced with cross-lane operations; each lane then owns 8
// latent dims and streams the partials with several loads in flight.
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int R = blockIdx.x * 4 + (threadIdx.x >> 6);      // global row (nq * n_h + head)
  const int rows = a.n_h * a.T;
  if (R >= a.B * rows) return;
  const int b = R / rows, row = R % rows;
  int ns, first;
  if (a.uniform_len > 0) {                                // same length everywhere
    ns = splits_of(a.uniform_len, a.num_splits, a.chunk);
    first = b * ns;
  } else {
    ns = splits_of(a.seq_lens[b], a.num_splits, a.chunk);
    // first work item of sequence b: splits of the sequences before it
    first = 0;
    for (int b0 = 0; b0 < b; b0 += 64) {
      const int bb = b0 + lane;
      first += (bb < b) ? splits_of(a.seq_lens[bb], a.num_splits, a.chunk) : 0;
    }
    first = wave_sum_i(first);
  }
  if (ns <= 1) return;                                    // written by the attention kernel
  const float* lse_p = a.part_lse + (size_t)first * rows + row;
  float* out = a.out_latent + (size_t)R * a.d_c;
  const int d0 = 8 * lane;                                // this lane's 8 dims
  const size_t pstride = (size_t)rows * a.d_c;            // elements between splits
  if (a.part_bf16 && ns <= 16) {
    // Few splits: every load (LSEs and partials) is issued before any of
    // them is used, so the row costs one memory latency.
    const float lse_l = (lane < ns) ? lse_p[(size_t)lane * rows] : -INFINITY;
    const uint16_t* src = (const uint16_t*)a.part_o + ((size_t)first * rows + row) * a.d_c + d0;
    u32x4 v[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < ns) v[s] = *(const u32x4*)(src + (size_t)s * pstride);
    const float mx = wave_max(lse_l);
    if (mx == -INFINITY) {                                // no visible token at all
      *(floatx4*)(out + d0) = floatx4{0.f, 0.f, 0.f, 0.f};
      *(floatx4*)(out + d0 + 4) = floatx4{0.f, 0.f, 0.f, 0.f};
      if (lane == 0) a.out_lse[R] = -INFINITY;
      return;
    }
    const float e_l = (lane < ns) ? expf(lse_l - mx) : 0.f;
    const float wsum = wave_sum(e_l);
    const float w_l = e_l * (1.0f / wsum);
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < ns) {
        const float w = __shfl(w_l, s, 64);
        acc0 += w * floatx4{__builtin_bit_cast(float, v[s][0] << 16), __builtin_bit_cast(float, v[s][0] & 0xFFFF0000u),
                            __builtin_bit_cast(float, v[s][1] << 16), __builtin_bit_cast(float, v[s][1] & 0xFFFF0000u)};
        acc1 += w * floatx4{__builtin_bit_cast(float, v[s][2] << 16), __builtin_bit_cast(float, v[s][2] & 0xFFFF0000u),
                            __builtin_bit_cast(float, v[s][3] << 16), __builtin_bit_cast(float, v[s][3] & 0xFFFF0000u)};
      }
    }
    *(floatx4*)(out + d0) = acc0;
    *(floatx4*)(out + d0 + 4) = acc1;
    if (lane == 0) a.out_lse[R] = mx + logf(wsum);
    return;
  }
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lse_p[(size_t)s * rows]);
  mx = wave_max(mx);
  if (mx == -INFINITY) {                                  // no visible token at all
    for (int d = d0; d < min(d0 + 8, a.d_c); d += 4) *(floatx4*)(out + d) = floatx4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0) a.out_lse[R] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int s = lane; s < ns; s += 64) wsum += expf(lse_p[(size_t)s * rows] - mx);
  wsum = wave_sum(wsum);
  const float inv = 1.0f / wsum;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (a.part_bf16) {                                      // fast path: d_c = 512
    const uint16_t* src = (const uint16_t*)a.part_o + ((size_t)first * rows + row) * a.d_c + d0;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int n = min(64, ns - s0);
      const float w_l = (lane < n) ? expf(lse_p[(size_t)(s0 + lane) * rows] - mx) * inv : 0.f;
      int s = 0;
      for (; s + 4 <= n; s += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const u32x4*)(src + (size_t)(s0 + s + u) * pstride);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = __shfl(w_l, s + u, 64);
          acc0 += w * floatx4{__builtin_bit_cast(float, v[u][0] << 16), __builtin_bit_cast(float, v[u][0] & 0xFFFF0000u),
                              __builtin_bit_cast(float, v[u][1] << 16), __builtin_bit_cast(float, v[u][1] & 0xFFFF0000u)};
          acc1 += w * floatx4{__builtin_bit_cast(float, v[u][2] << 16), __builtin_bit_cast(float, v[u][2] & 0xFFFF0000u),
                              __builtin_bit_cast(float, v[u][3] << 16), __builtin_bit_cast(float, v[u][3] & 0xFFFF0000u)};
        }
      }
      for (; s < n; ++s) {
        const u32x4 v = *(const u32x4*)(src + (size_t)(s0 + s) * pstride);
        const float w = __shfl(w_l, s, 64);
        acc0 += w * floatx4{__builtin_bit_cast(float, v[0] << 16), __builtin_bit_cast(float, v[0] & 0xFFFF0000u),
                            __builtin_bit_cast(float, v[1] << 16), __builtin_bit_cast(float, v[1] & 0xFFFF0000u)};
        acc1 += w * floatx4{__builtin_bit_cast(float, v[2] << 16), __builtin_bit_cast(float, v[2] & 0xFFFF0000u),
                            __builtin_bit_cast(float, v[3] << 16), __builtin_bit_cast(float, v[3] & 0xFFFF0000u)};
      }
    }
    *(floatx4*)(out + d0) = acc0;
    *(floatx4*)(out + d0 + 4) = acc1;
  } else {                                                // general path: fp32, d_c % 4 == 0
    const float* src = (const float*)a.part_o + ((size_t)first * rows + row) * a.d_c;
    const bool has0 = d0 < a.d_c, has1 = d0 + 4 < a.d_c;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int n = min(64, ns - s0);
      const float w_l = (lane < n) ? expf(lse_p[(size_t)(s0 + lane) * rows] - mx) * inv : 0.f;
      for (int s = 0; s < n; ++s) {
        const float w = __shfl(w_l, s, 64);
        const float* ps = src + (size_t)(s0 + s) * pstride;
        if (has0) acc0 += w * *(const floatx4*)(ps + d0);
        if (has1) acc1 += w * *(const floatx4*)(ps + d0 + 4);
      }
    }
    if (has0) *(floatx4*)(out + d0) = acc0;
    if (has1) *(floatx4*)(out + d0 + 4) = acc1;
  }
  if (lane == 0) a.out_lse[R] = mx + logf(wsum);
}

// ===================================================== up-projection: MFMA
// out[n, i, :] = W^UV_i latent[n, i, :], d_h = 128, d_c = 512.  One
// workgroup of 8 waves per (head i, half of the d_h rows): 2 n_h
// workgroups, grouped so that both halves of a head run on one XCD and share
// its L2 copy of the head's latent rows.  All global loads are coalesced
// (16-byte chunks on consecutive lanes): the 64 x 512 W^UV block is staged
// in LDS as is, and each block of 32 latent rows (fp32) is staged as bf16
// hi + lo parts (x = hi + lo + O(2^-17 x)), so the bf16 products keep nearly
// fp32 accuracy with W^UV exact in bf16.  Wave (mi, ni) computes the 16 x 16
// output block d_h rows 16 mi .. of the half, tokens 16 ni .. of the block
// with v_mfma_f32_16x16x32_bf16.
__device__ inline int xcd_grouped(int i, int n) {
  // workgroups are dispatched round-robin over the 8 XCDs
  return (n & 7) ? i : (i & 7) * (n >> 3) + (i >> 3);
}

constexpr int kUpRow = 520;           // bf16 elements per LDS row (1040 bytes)

template <typename OutT>
__global__ __launch_bounds__(512) void up_proj_mfma_kernel(
    const float* __restrict__ latent, const uint16_t* __restrict__ w_uv,
    OutT* __restrict__ out, int n_tok, int n_h) {
  constexpr int DC = 512, DH = 128;
  __shared__ __attribute__((aligned(16))) uint16_t sw[64 * kUpRow];
  __shared__ __attribute__((aligned(16))) uint16_t sh[32 * kUpRow];
  __shared__ __attribute__((aligned(16))) uint16_t sl[32 * kUpRow];
  const int L = xcd_grouped(blockIdx.x, gridDim.x);
  const int head = L >> 1, half = L & 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mi = wave & 3, ni = wave >> 2;
  const int r16 = lane & 15, g = lane >> 4;

  const uint16_t* wsrc = w_uv + ((size_t)head * DH + 64 * half) * DC;
  u32x4 wv[8];                         // 64 rows x 64 chunks
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + 512 * i, r = ch >> 6, c8 = (ch & 63) * 8;
    wv[i] = *(const u32x4*)(wsrc + (size_t)r * DC + c8);
  }
  floatx4 v[8];                        // 32 rows x 128 chunks of 4 floats
  auto load_latent = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = tid + 512 * i, t = ch >> 7, c4 = (ch & 127) * 4;
      v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (t0 + t < n_tok) v[i] = *(const floatx4*)(latent + ((size_t)(t0 + t) * n_h + head) * DC + c4);
    }
  };
  // blockIdx.y splits the tokens when there are few heads: group y takes
  // the blocks of 32 tokens t0 = 32 (y + k gridDim.y)
  const int t_first = 32 * blockIdx.y, t_step = 32 * gridDim.y;
  load_latent(t_first);
  for (int t0 = t_first; t0 < n_tok; t0 += t_step) {
    if (t0 == t_first) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = tid + 512 * i, r = ch >> 6, c8 = (ch & 63) * 8;
        *(u32x4*)(sw + r * kUpRow + c8) = wv[i];
      }
    } else {
      __syncthreads();                 // the previous block's reads are done
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = tid + 512 * i, t = ch >> 7, c4 = (ch & 127) * 4;
      u32x2 hi, lo;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x0 = v[i][2 * e], x1 = v[i][2 * e + 1];
        const bf16x2 hb = bf16x2{(__bf16)x0, (__bf16)x1};
        hi[e] = __builtin_bit_cast(uint32_t, hb);
        lo[e] = pack_bf16x2(x0 - (float)hb[0], x1 - (float)hb[1]);
      }
      *(u32x2*)(sh + t * kUpRow + c4) = hi;
      *(u32x2*)(sl + t * kUpRow + c4) = lo;
    }
    if (t0 + t_step < n_tok) load_latent(t0 + t_step);   // in flight during this block
    __syncthreads();

    floatx4 acc_hi = {0.f, 0.f, 0.f, 0.f}, acc_lo = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* pa = sw + (16 * mi + r16) * kUpRow + 8 * g;
    const int bo = (16 * ni + r16) * kUpRow + 8 * g;
#pragma unroll
    for (int s = 0; s < DC / 32; ++s) {
      const bf16x8 a = *(const bf16x8*)(pa + 32 * s);
      const bf16x8 bh = *(const bf16x8*)(sh + bo + 32 * s);
      const bf16x8 bl = *(const bf16x8*)(sl + bo + 32 * s);
      acc_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc_hi, 0, 0, 0);
      acc_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc_lo, 0, 0, 0);
    }
    // acc[e]: d_h row 64 half + 16 mi + 4 g + e, token t0 + 16 ni + r16
    const int tok = t0 + 16 * ni + r16;
    if (tok < n_tok) {
      const floatx4 r = acc_hi + acc_lo;
      OutT* dst = out + ((size_t)tok * n_h + head) * DH + 64 * half + 16 * mi + 4 * g;
      if constexpr (sizeof(OutT) == 4)
        *(floatx4*)dst = r;
      else
        *(u32x2*)dst = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    }
  }
}

// =========================================== up-projection: general path
template <typename T, typename OutT>
__global__ __launch_bounds__(256) void up_proj_general_kernel(
    const float* __restrict__ latent, const T* __restrict__ w_uv,
    OutT* __restrict__ out, int n_tok, int n_h, int d_h, int d_c) {
  const size_t total = (size_t)n_tok * n_h * d_h;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int r = int(idx % d_h);
    const size_t row = idx / d_h;         // tok * n_h + head
    const int head = int(row % n_h);
    const float* x = latent + row * d_c;
    const T* w = w_uv + ((size_t)head * d_h + r) * d_c;
    float acc = 0.f;
    for (int c = 0; c < d_c; ++c) acc = fmaf(load_f(w, c), x[c], acc);
    store_f(out, idx, acc);
  }
}

// ================================================================ launchers
hipError_t launch_absorb(const mla_dims_t& d, bool fast, const void* q_nope,
                         const void* q_rope, const void* w_uk,
                         const int32_t* q_pos, void* q_abs, int n_tok,
                         RopeFreq rope, hipStream_t st) {
  const bool out_f32 = d.q_dtype == MLA_F32 || d.precision == MLA_PREC_FP32;
  if (fast) {
    // four workgroups per head; with few heads the tokens are split over up
    // to 256 workgroups in all
    const int groups = std::max(1, std::min((n_tok + 31) / 32, kNumCU / (4 * d.n_heads)));
    const dim3 grid(d.n_heads * 4, groups);
    if (out_f32)
      hipLaunchKernelGGL(absorb_mfma_kernel<float>, grid, dim3(256), 0, st,
                         (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (float*)q_abs, n_tok,
                         d.n_heads, rope);
    else
      hipLaunchKernelGGL(absorb_mfma_kernel<uint16_t>, grid, dim3(256), 0, st,
                         (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (uint16_t*)q_abs, n_tok,
                         d.n_heads, rope);
  } else {
    const size_t total = (size_t)n_tok * d.n_heads * (d.d_latent + d.d_rope);
    const int grid = (int)std::min<size_t>((total + 255) / 256, 65535);
    if (d.q_dtype == MLA_F32)
      hipLaunchKernelGGL((absorb_general_kernel<float, float>), dim3(grid), dim3(256), 0, st,
                         (const float*)q_nope, (const float*)q_rope, (const float*)w_uk,
                         q_pos, (float*)q_abs, n_tok, d.n_heads, d.d_head,
                         d.d_latent, d.d_rope, rope);
    else if (out_f32)
      hipLaunchKernelGGL((absorb_general_kernel<uint16_t, float>), dim3(grid), dim3(256), 0,
                         st, (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (float*)q_abs, n_tok, d.n_heads,
                         d.d_head, d.d_latent, d.d_rope, rope);
    else
      hipLaunchKernelGGL((absorb_general_kernel<uint16_t, uint16_t>), dim3(grid), dim3(256),
                         0, st, (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (uint16_t*)q_abs, n_tok, d.n_heads,
                         d.d_head, d.d_latent, d.d_rope, rope);
  }
  return hipGetLastError();
}

hipError_t launch_append(const mla_dims_t& d, const void* new_c, const void* new_kr,
                         const int32_t* seq_idx, const int32_t* pos,
                         const int32_t* page_table, int B, int max_pages,
                         int max_len, long long cache_rows, int apply_rope,
                         void* cache, float* kv_scale, int n_rows,
                         RopeFreq rope, hipStream_t st, bool src_f32, int c_stride,
                         int kr_stride, const float* norm_gain, float norm_eps) {
  const int grid = std::min((n_rows + 3) / 4, 16384);
#define MLA_APPEND(ST, KV)                                                                   \
  hipLaunchKernelGGL((append_kernel<ST, KV>), dim3(grid), dim3(256), 0, st,                  \
                     (const ST*)new_c, (const ST*)new_kr, seq_idx, pos, page_table, B,       \
                     max_pages, max_len, cache_rows, apply_rope, cache, kv_scale, n_rows,    \
                     d.d_latent, d.d_rope, rope, c_stride, kr_stride, norm_gain, norm_eps)
  if (d.kv_dtype == MLA_F32) MLA_APPEND(float, MLA_F32);
  else if (d.kv_dtype == MLA_BF16 && !src_f32) MLA_APPEND(uint16_t, MLA_BF16);
  else if (d.kv_dtype == MLA_BF16) MLA_APPEND(float, MLA_BF16);
  else if (!src_f32) MLA_APPEND(uint16_t, MLA_FP8_E4M3);
  else MLA_APPEND(float, MLA_FP8_E4M3);
#undef MLA_APPEND
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3((a.B * a.T * a.n_h + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_up_proj(const mla_dims_t& d, bool fast, const float* latent,
                          const void* w_uv, void* out, bool out_f32, int n_tok,
                          hipStream_t st) {
  if (fast) {
    // two workgroups per head; with few heads the tokens are split over up
    // to 256 workgroups in all
    const int tok_blocks = (n_tok + 31) / 32;
    const int groups = std::max(1, std::min(tok_blocks, kNumCU / (2 * d.n_heads)));
    const dim3 grid(d.n_heads * 2, groups);
    if (out_f32)
      hipLaunchKernelGGL(up_proj_mfma_kernel<float>, grid, dim3(512), 0, st,
                         latent, (const uint16_t*)w_uv, (float*)out, n_tok, d.n_heads);
    else
      hipLaunchKernelGGL(up_proj_mfma_kernel<uint16_t>, grid, dim3(512), 0, st,
                         latent, (const uint16_t*)w_uv, (uint16_t*)out, n_tok, d.n_heads);
  } else {
    const size_t total = (size_t)n_tok * d.n_heads * d.d_head;
    const int grid = (int)std::min<size_t>((total + 255) / 256, 65535);
#define MLA_UP(WT, OT)                                                              \
    hipLaunchKernelGGL((up_proj_general_kernel<WT, OT>), dim3(grid), dim3(256), 0, st, \
                       latent, (const WT*)w_uv, (OT*)out, n_tok, d.n_heads, d.d_head,  \
                       d.d_latent)
    if (d.q_dtype == MLA_F32) {
      if (out_f32) MLA_UP(float, float); else MLA_UP(float, uint16_t);
    } else {
      if (out_f32) MLA_UP(uint16_t, float); else MLA_UP(uint16_t, uint16_t);
    }
#undef MLA_UP
  }
  return hipGetLastError();
}

}  // namespace mla
