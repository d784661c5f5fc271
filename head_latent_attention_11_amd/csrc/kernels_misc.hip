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
// Interleaved pairs (2k, 2k+1) rotated by pos * base^(-2k/d); angle and
// rotation in double precision.
__device__ inline void rope_pair(float x0, float x1, int pos, int k, int d,
                                 float base, float* y0, float* y1) {
  double theta = pow((double)base, -2.0 * (double)k / (double)d);
  double ang = (double)pos * theta;
  double s, c;
  sincos(ang, &s, &c);
  *y0 = (float)((double)x0 * c - (double)x1 * s);
  *y1 = (float)((double)x0 * s + (double)x1 * c);
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
// computes D^T[cols x tokens] = W^T q^T.  The 128 x 128 W^UK_i block is
// staged row-major in LDS with 16-byte writes and read back column-wise
// with the gfx950 transposing LDS read: within each group of 16 lanes,
// ds_read_b64_tr_b16 hands lane i element i%4 of the 8-byte chunks
// addressed by lanes 4k + i/4 (k = 0..3), so four rows of 16 elements come
// back as 16 columns of 4.
constexpr int kAbsCols = 128, kAbsDh = 128, kAbsLdsRow = kAbsCols + 8;

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
    OutT* __restrict__ q_abs, int n_tok, int n_h, float rope_base) {
  constexpr int DC = 512, DR = 64, D = DC + DR;
  __shared__ __attribute__((aligned(16))) uint16_t ws[kAbsDh * kAbsLdsRow];
  const int head = blockIdx.x >> 2, cb = blockIdx.x & 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, j = lane & 15;

  // first token block's query operands, issued before the W^UK staging
  bf16x8 bq0[kAbsDh / 16];
#pragma unroll
  for (int k = 0; k < kAbsDh / 16; ++k) {
    bq0[k] = bf16x8{};
    if (l32 < n_tok)
      bq0[k] = *(const bf16x8*)(q_nope + ((size_t)l32 * n_h + head) * kAbsDh + 16 * k + 8 * h);
  }
  // stage W^UK[head][r][cb*128 : cb*128 + 128] row-major (16-byte chunks)
  const uint16_t* wsrc = w_uk + (size_t)head * kAbsDh * DC + cb * kAbsCols;
  u32x4 stg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + 256 * i, r = ch >> 4, c8 = (ch & 15) * 8;
    stg[i] = *(const u32x4*)(wsrc + (size_t)r * DC + c8);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + 256 * i, r = ch >> 4, c8 = (ch & 15) * 8;
    *(u32x4*)(ws + r * kAbsLdsRow + c8) = stg[i];
  }
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

  for (int t0 = 0; t0 < n_tok; t0 += 32) {
    const int tok = t0 + l32;         // B-operand column
    bf16x8 bq[kAbsDh / 16];
#pragma unroll
    for (int k = 0; k < kAbsDh / 16; ++k) {
      bq[k] = bq0[k];
      if (t0 > 0) {
        bq[k] = bf16x8{};
        if (tok < n_tok)
          bq[k] = *(const bf16x8*)(q_nope + ((size_t)tok * n_h + head) * kAbsDh + 16 * k + 8 * h);
      }
    }
    floatx16 acc = {};
#pragma unroll
    for (int k = 0; k < kAbsDh / 16; ++k)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[k], bq[k], acc, 0, 0, 0);
    // acc[r]: column-in-block 8(r/4) + 4h + r%4 of wave's 32, token l32
    if (tok < n_tok) {
      OutT* dst = q_abs + ((size_t)tok * n_h + head) * D + cb * kAbsCols + wave * 32;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if constexpr (sizeof(OutT) == 4)
          *(floatx4*)(dst + 8 * jj + 4 * h) =
              floatx4{acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]};
        else
          *(u32x2*)(dst + 8 * jj + 4 * h) = u32x2{pack_bf16x2(acc[4 * jj], acc[4 * jj + 1]),
                                                 pack_bf16x2(acc[4 * jj + 2], acc[4 * jj + 3])};
      }
    }
  }

  // the RoPE part q_abs[..., 512:576] is written by the cb == 0 workgroups
  if (cb == 0) {
    for (int idx = tid; idx < n_tok * (DR / 2); idx += 256) {
      const int tok = idx / (DR / 2), k = idx % (DR / 2);
      const uint16_t* src = q_rope + ((size_t)tok * n_h + head) * DR + 2 * k;
      float x0 = bf16_bits_to_f32(src[0]), x1 = bf16_bits_to_f32(src[1]);
      if (q_pos) rope_pair(x0, x1, q_pos[tok], k, DR, rope_base, &x0, &x1);
      OutT* dst = q_abs + ((size_t)tok * n_h + head) * D + DC + 2 * k;
      if constexpr (sizeof(OutT) == 4) {
        dst[0] = x0;
        dst[1] = x1;
      } else {
        dst[0] = f32_to_bf16_bits(x0);
        dst[1] = f32_to_bf16_bits(x1);
      }
    }
  }
}

// =================================================== absorb: general path
template <typename T, typename OutT>
__global__ __launch_bounds__(256) void absorb_general_kernel(
    const T* __restrict__ q_nope, const T* __restrict__ q_rope,
    const T* __restrict__ w_uk, const int32_t* __restrict__ q_pos,
    OutT* __restrict__ q_abs, int n_tok, int n_h, int d_h, int d_c, int d_r,
    float rope_base) {
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
      if (q_pos) rope_pair(x0, x1, q_pos[tok], k, d_r, rope_base, &x0, &x1);
      v = ((e - d_c) & 1) ? x1 : x0;
    }
    store_f(q_abs, idx, v);
  }
}

// ================================================================ append
// One wave per new row.  Source rows are F32 (F32 cache) or BF16.
template <typename SrcT, int KV>
__global__ __launch_bounds__(256) void append_kernel(
    const SrcT* __restrict__ new_c, const SrcT* __restrict__ new_kr,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int B, int max_pages, int max_len,
    long long cache_rows, int apply_rope, void* __restrict__ cache,
    float* __restrict__ kv_scale, int n_rows, int d_c, int d_r, float rope_base) {
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
        x = load_f(new_c, (size_t)r * d_c + e);
      } else if (e < D) {
        const int q = e - d_c;
        if (apply_rope) {
          const int kp = q >> 1;
          float x0 = load_f(new_kr, (size_t)r * d_r + 2 * kp);
          float x1 = load_f(new_kr, (size_t)r * d_r + 2 * kp + 1);
          float y0, y1;
          rope_pair(x0, x1, p, kp, d_r, rope_base, &y0, &y1);
          x = (q & 1) ? y1 : y0;
        } else {
          x = load_f(new_kr, (size_t)r * d_r + q);
        }
      }
      v[k] = x;
      amax = fmaxf(amax, fabsf(x));
    }
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
  const int L = a.seq_lens[b];
  const int ns = splits_of(L, a.num_splits, a.chunk);
  if (ns <= 1) return;                                    // written by the attention kernel
  // first work item of sequence b: splits of the sequences before it
  int first = 0;
  for (int b0 = 0; b0 < b; b0 += 64) {
    const int bb = b0 + lane;
    first += (bb < b) ? splits_of(a.seq_lens[bb], a.num_splits, a.chunk) : 0;
  }
  first = wave_sum_i(first);
  const float* lse_p = a.part_lse + (size_t)first * rows + row;
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lse_p[(size_t)s * rows]);
  mx = wave_max(mx);
  float* out = a.out_latent + (size_t)R * a.d_c;
  const int d0 = 8 * lane;                                // this lane's 8 dims
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
  const size_t pstride = (size_t)rows * a.d_c;            // elements between splits
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
// workgroup of 4 waves per (head i, block of 32 tokens); wave w owns d_h
// rows 32w .. 32w+31.  All global loads are issued first: each lane's 32
// W^UV operands (the workgroup streams W^UV_i once) and its share of the
// latent block (32 tokens x 512 fp32), which is then staged in LDS as bf16
// hi + lo parts (x = hi + lo + O(2^-17 x)), so the bf16 MFMA keeps nearly
// fp32 accuracy with W^UV exact in bf16.
constexpr int kUpLds = 512 + 8;       // padded bf16 row of the latent block

template <typename OutT>
__global__ __launch_bounds__(256) void up_proj_mfma_kernel(
    const float* __restrict__ latent, const uint16_t* __restrict__ w_uv,
    OutT* __restrict__ out, int n_tok, int n_h) {
  constexpr int DC = 512, DH = 128;
  __shared__ __attribute__((aligned(16))) uint16_t s_hi[32 * kUpLds];
  __shared__ __attribute__((aligned(16))) uint16_t s_lo[32 * kUpLds];
  const int head = blockIdx.x, t0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int m = wave * 32 + l32;                    // d_h row (A-operand row)
  const uint16_t* wrow = w_uv + ((size_t)head * DH + m) * DC;

  bf16x8 wa[DC / 16];
#pragma unroll
  for (int k = 0; k < DC / 16; ++k) wa[k] = *(const bf16x8*)(wrow + 16 * k + 8 * h);
  // latent block: 4096 chunks of 4 floats, 16 per thread
  floatx4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ch = tid + 256 * i, t = ch >> 7, c4 = (ch & 127) * 4;
    v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (t0 + t < n_tok) v[i] = *(const floatx4*)(latent + ((size_t)(t0 + t) * n_h + head) * DC + c4);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ch = tid + 256 * i, t = ch >> 7, c4 = (ch & 127) * 4;
    u32x2 hi, lo;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x0 = v[i][2 * e], x1 = v[i][2 * e + 1];
      const bf16x2 hb = bf16x2{(__bf16)x0, (__bf16)x1};
      hi[e] = __builtin_bit_cast(uint32_t, hb);
      lo[e] = pack_bf16x2(x0 - (float)hb[0], x1 - (float)hb[1]);
    }
    *(u32x2*)(s_hi + t * kUpLds + c4) = hi;
    *(u32x2*)(s_lo + t * kUpLds + c4) = lo;
  }
  __syncthreads();

  floatx16 acc_hi = {}, acc_lo = {};
#pragma unroll
  for (int k = 0; k < DC / 16; ++k) {
    const bf16x8 bh = *(const bf16x8*)(s_hi + l32 * kUpLds + 16 * k + 8 * h);
    const bf16x8 bl = *(const bf16x8*)(s_lo + l32 * kUpLds + 16 * k + 8 * h);
    acc_hi = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[k], bh, acc_hi, 0, 0, 0);
    acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[k], bl, acc_lo, 0, 0, 0);
  }
  const int tok = t0 + l32;
  if (tok < n_tok) {
    OutT* dst = out + ((size_t)tok * n_h + head) * DH + wave * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 r = {acc_hi[4 * j] + acc_lo[4 * j], acc_hi[4 * j + 1] + acc_lo[4 * j + 1],
                         acc_hi[4 * j + 2] + acc_lo[4 * j + 2], acc_hi[4 * j + 3] + acc_lo[4 * j + 3]};
      if constexpr (sizeof(OutT) == 4) {
        *(floatx4*)(dst + 8 * j + 4 * h) = r;
      } else {
        *(u32x2*)(dst + 8 * j + 4 * h) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      }
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
                         float rope_base, hipStream_t st) {
  const bool out_f32 = d.q_dtype == MLA_F32 || d.precision == MLA_PREC_FP32;
  if (fast) {
    if (out_f32)
      hipLaunchKernelGGL(absorb_mfma_kernel<float>, dim3(d.n_heads * 4), dim3(256), 0, st,
                         (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (float*)q_abs, n_tok,
                         d.n_heads, rope_base);
    else
      hipLaunchKernelGGL(absorb_mfma_kernel<uint16_t>, dim3(d.n_heads * 4), dim3(256), 0, st,
                         (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (uint16_t*)q_abs, n_tok,
                         d.n_heads, rope_base);
  } else {
    const size_t total = (size_t)n_tok * d.n_heads * (d.d_latent + d.d_rope);
    const int grid = (int)std::min<size_t>((total + 255) / 256, 65535);
    if (d.q_dtype == MLA_F32)
      hipLaunchKernelGGL((absorb_general_kernel<float, float>), dim3(grid), dim3(256), 0, st,
                         (const float*)q_nope, (const float*)q_rope, (const float*)w_uk,
                         q_pos, (float*)q_abs, n_tok, d.n_heads, d.d_head,
                         d.d_latent, d.d_rope, rope_base);
    else if (out_f32)
      hipLaunchKernelGGL((absorb_general_kernel<uint16_t, float>), dim3(grid), dim3(256), 0,
                         st, (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (float*)q_abs, n_tok, d.n_heads,
                         d.d_head, d.d_latent, d.d_rope, rope_base);
    else
      hipLaunchKernelGGL((absorb_general_kernel<uint16_t, uint16_t>), dim3(grid), dim3(256),
                         0, st, (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (uint16_t*)q_abs, n_tok, d.n_heads,
                         d.d_head, d.d_latent, d.d_rope, rope_base);
  }
  return hipGetLastError();
}

hipError_t launch_append(const mla_dims_t& d, const void* new_c, const void* new_kr,
                         const int32_t* seq_idx, const int32_t* pos,
                         const int32_t* page_table, int B, int max_pages,
                         int max_len, long long cache_rows, int apply_rope,
                         void* cache, float* kv_scale, int n_rows,
                         float rope_base, hipStream_t st) {
  const int grid = std::min((n_rows + 3) / 4, 16384);
  if (d.kv_dtype == MLA_F32)
    hipLaunchKernelGGL((append_kernel<float, MLA_F32>), dim3(grid), dim3(256), 0, st,
                       (const float*)new_c, (const float*)new_kr, seq_idx, pos,
                       page_table, B, max_pages, max_len, cache_rows, apply_rope,
                       cache, kv_scale, n_rows, d.d_latent, d.d_rope, rope_base);
  else if (d.kv_dtype == MLA_BF16)
    hipLaunchKernelGGL((append_kernel<uint16_t, MLA_BF16>), dim3(grid), dim3(256), 0, st,
                       (const uint16_t*)new_c, (const uint16_t*)new_kr, seq_idx, pos,
                       page_table, B, max_pages, max_len, cache_rows, apply_rope,
                       cache, kv_scale, n_rows, d.d_latent, d.d_rope, rope_base);
  else
    hipLaunchKernelGGL((append_kernel<uint16_t, MLA_FP8_E4M3>), dim3(grid), dim3(256), 0, st,
                       (const uint16_t*)new_c, (const uint16_t*)new_kr, seq_idx, pos,
                       page_table, B, max_pages, max_len, cache_rows, apply_rope,
                       cache, kv_scale, n_rows, d.d_latent, d.d_rope, rope_base);
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
    const dim3 grid(d.n_heads, (n_tok + 31) / 32);
    if (out_f32)
      hipLaunchKernelGGL(up_proj_mfma_kernel<float>, grid, dim3(256), 0, st,
                         latent, (const uint16_t*)w_uv, (float*)out, n_tok, d.n_heads);
    else
      hipLaunchKernelGGL(up_proj_mfma_kernel<uint16_t>, grid, dim3(256), 0, st,
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
