// Query absorption, cache append, split combine and value up-projection.
//
// Sources: "DeepSeek-V2: Strong, Economical, Efficient", section 2.1.2 and
// Appendix C (W^UK absorbed into the query side, W^UV applied after the
// latent sum), section 2.1.3 (decoupled RoPE, cached shared k^R);
// "DeepSeek-V3 Technical Report" notes, MLA section (head-block layout of
// W^UK / W^UV; attention-output equation whose sum over tokens is what the
// split combine re-associates).
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

// ============================================================ RoPE helper
// Interleaved pairs (2k, 2k+1) rotated by pos * theta_k (rope_theta, with
// or without context extension); angle and rotation in double precision.
// The angle pos * theta is formed and reduced to [-pi, pi] in double
// (positions up to 2^17 times frequencies near 1 need that: an fp32 angle of
// 1e5 rad has a unit roundoff of ~0.008 rad); sine, cosine and the rotation
// then run in fp32 (relative error ~1e-7).  Double-precision sine and cosine
// per pair made the rotations a large part of the absorption.
__device__ inline void rope_rot(float x0, float x1, int pos, double theta, float* y0, float* y1) {
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0.15915494309189535);            // turns: ang / (2 pi)
  const float r = (float)fma(-k, 6.283185307179586, ang);      // in [-pi, pi]
  float s, c;
  sincosf(r, &s, &c);
  *y0 = x0 * c - x1 * s;
  *y1 = x0 * s + x1 * c;
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
constexpr int kAbsRopeBatch = 8;      // RoPE pairs of a thread whose loads fly together

typedef short shortx4 __attribute__((ext_vector_type(4)));

// two floats -> packed bf16 pair (hardware round to nearest even)
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

__device__ inline shortx4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (shortx4 __attribute__((address_space(3)))*)(p));
}

// PAIRS (bf16 output only): each row is written as the pair hi = bf16(q),
// lo = bf16(q - hi), hi in elements [0, D) and lo in [D, 2D) of a 2D row.
// One workgroup's share (bx: head * 4 + column block; by of gy: token
// group), as a function so that the absorption can also run inside the
// combined absorption + append launch.
template <typename OutT, bool PAIRS>
__device__ __forceinline__ void absorb_mfma_block(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ q_pos,
    OutT* __restrict__ q_abs, int n_tok, int n_h, const RopeFreq& rope, int bx, int by,
    int gy) {
  constexpr int DC = 512, DR = 64, D = DC + DR;
  constexpr int QROW = PAIRS ? 2 * D : D;     // elements per q_abs row
  static_assert(!PAIRS || sizeof(OutT) == 2, "query pairs are bf16");
  __shared__ __attribute__((aligned(16))) uint16_t ws[kAbsDh * kAbsLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t qs[32 * kAbsLdsRow];
  __shared__ __attribute__((aligned(16))) unsigned char os[32 * kAbsOutRow];
  const int head = bx >> 2, cb = bx & 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, j = lane & 15;

  // blockIdx.y splits the tokens when there are few heads: group y takes
  // the blocks of 32 tokens t0 = 32 (y + k gridDim.y).
  // The RoPE part q_abs[..., 512:576] is shared out over the head's
  // workgroups: pair p = 256 cb + tid + 1024 (y + u gridDim.y) (token p / 32,
  // pair k = p % 32 = tid % 32 for every u), kAbsRopeBatch pairs of a thread
  // at a time.  A batch's inputs are loaded at clamped indices, with no
  // branch around the loads (so that they are in flight together), the
  // first batch before the W^UK block; its rotations run while that block
  // is in flight.
  const int n_pairs = n_tok * (DR / 2), rk = tid & 31;
  const int p_first = 1024 * by + cb * 256 + tid, p_step = 1024 * gy;
  const int t_first = 32 * by, t_step = 32 * gy;
  uint32_t rxy[kAbsRopeBatch];         // the pair's two bf16 inputs
  int rpos[kAbsRopeBatch];
  auto load_pairs = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kAbsRopeBatch; ++u) {
      const int tok = min(p0 + u * p_step, n_pairs - 1) >> 5;
      rxy[u] = *(const uint32_t*)(q_rope + ((size_t)tok * n_h + head) * DR + 2 * rk);
      rpos[u] = q_pos ? q_pos[tok] : 0;
    }
  };
  load_pairs(p_first);

  // query block loader: 32 tokens x 128 d_h = 512 chunks of 16 bytes.
  // Tokens past n_tok load the last token again (never stored), so no branch
  // surrounds the loads.
  auto load_q = [&](int t0, u32x4* qv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i, c8 = (ch & 15) * 8;
      const int t = min(t0 + (ch >> 4), n_tok - 1);
      qv[i] = *(const u32x4*)(q_nope + ((size_t)t * n_h + head) * kAbsDh + c8);
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
  for (int p0 = p_first; p0 < n_pairs; p0 += kAbsRopeBatch * p_step) {
    if (p0 != p_first) load_pairs(p0);
#pragma unroll
    for (int u = 0; u < kAbsRopeBatch; ++u) {
      const int p = p0 + u * p_step;
      float x0 = bf16_bits_to_f32(uint16_t(rxy[u])), x1 = bf16_bits_to_f32(uint16_t(rxy[u] >> 16));
      if (q_pos) rope_rot(x0, x1, rpos[u], theta, &x0, &x1);
      if (p < n_pairs) {
        OutT* dst = q_abs + ((size_t)(p >> 5) * n_h + head) * QROW + DC + 2 * rk;
        if constexpr (sizeof(OutT) == 4) {
          *(float2*)dst = float2{x0, x1};
        } else {
          const uint32_t hi = pack_bf16x2(x0, x1);
          *(uint32_t*)dst = hi;
          if constexpr (PAIRS)
            *(uint32_t*)(dst + D) = pack_bf16x2(x0 - __builtin_bit_cast(float, hi << 16),
                                                x1 - __builtin_bit_cast(float, hi & 0xFFFF0000u));
        }
      }
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

  // One block of 32 tokens.  FULL blocks (all 32 tokens exist) store their
  // rows with no per-lane test: stores share the memory counter with loads,
  // and stores under a per-lane branch make the compiler wait for every
  // store in flight (the previous block's copy-out) before it stages the
  // next query block.  Only the last, partial block tests its tokens.
  auto block = [&](int t0, auto full) {
    constexpr bool FULL = decltype(full)::value;
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
      if constexpr (sizeof(OutT) == 4) {
        *(floatx4*)(orow + 8 * jj + 4 * h) =
            floatx4{acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]};
      } else {
        const u32x2 hi = u32x2{pack_bf16x2(acc[4 * jj], acc[4 * jj + 1]),
                               pack_bf16x2(acc[4 * jj + 2], acc[4 * jj + 3])};
        *(u32x2*)(orow + 8 * jj + 4 * h) = hi;
        if constexpr (PAIRS)          // lo parts: columns 128.. of the staging row
          *(u32x2*)(orow + kAbsCols + 8 * jj + 4 * h) = u32x2{
              pack_bf16x2(acc[4 * jj] - __builtin_bit_cast(float, hi[0] << 16),
                          acc[4 * jj + 1] - __builtin_bit_cast(float, hi[0] & 0xFFFF0000u)),
              pack_bf16x2(acc[4 * jj + 2] - __builtin_bit_cast(float, hi[1] << 16),
                          acc[4 * jj + 3] - __builtin_bit_cast(float, hi[1] & 0xFFFF0000u))};
      }
    }
    __syncthreads();
    // 32 tokens x 128 columns, 16-byte chunks, each token's run contiguous
    // (pairs: the hi run, then the lo run D elements further)
    constexpr int run = kAbsCols * (int)sizeof(OutT) / 16;   // chunks per run
    constexpr int per_row = PAIRS ? 2 * run : run;
#pragma unroll
    for (int i = 0; i < 32 * per_row / 256; ++i) {
      const int ch = tid + 256 * i, t = ch / per_row, c = ch % per_row;
      const int part = PAIRS ? c / run : 0, cc = PAIRS ? c % run : c;
      if (FULL || t0 + t < n_tok)
        *(u32x4*)((unsigned char*)(q_abs + ((size_t)(t0 + t) * n_h + head) * QROW + part * D +
                                   cb * kAbsCols) + 16 * cc) =
            *(const u32x4*)(os + t * kAbsOutRow + 16 * c);
    }
  };
  int t0 = t_first;
  for (; t0 + 32 <= n_tok; t0 += t_step) block(t0, std::true_type{});
  if (t0 < n_tok) block(t0, std::false_type{});
}

template <typename OutT, bool PAIRS = false>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ q_pos,
    OutT* __restrict__ q_abs, int n_tok, int n_h, RopeFreq rope) {
  absorb_mfma_block<OutT, PAIRS>(q_nope, q_rope, w_uk, q_pos, q_abs, n_tok, n_h, rope,
                                 blockIdx.x, blockIdx.y, gridDim.y);
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
// Cache slot of new row r (sequence seq_idx[r], position pos[r]), or -1 when
// the row is skipped (sequence or position out of range, unmapped page, slot
// past the cache).
__device__ inline long long append_slot(const int32_t* __restrict__ seq_idx,
                                        const int32_t* __restrict__ pos,
                                        const int32_t* __restrict__ page_table, int B,
                                        int max_pages, int max_len, long long cache_rows, int r) {
  const int sq = seq_idx[r], p = pos[r];
  if (sq < 0 || sq >= B || p < 0) return -1;
  long long row;
  if (page_table) {
    if (p / kPage >= max_pages) return -1;
    const int page = page_table[(size_t)sq * max_pages + p / kPage];
    if (page < 0) return -1;
    row = (long long)page * kPage + p % kPage;
  } else {
    if (p >= max_len) return -1;
    row = (long long)sq * max_len + p;
  }
  return row < cache_rows ? row : -1;
}

// One wave writes cache slot `row` from a new row whose element e of c^KV is
// ld_c(e) and element q of k^R is ld_kr(q): optional RoPE of k^R at position
// p, optional RMS norm of the c^KV part (c_i * g_i / sqrt(mean(c^2) + eps)),
// then the cache format (fp32, bf16, 6-bit blocks, or fp8 with a row scale).
// Every load of the row (and of the norm gains) is issued before the first
// is used, at clamped indices, and the lane's elements are selected after:
// loads inside per-element branches would each wait for the previous one.
template <int KV, typename LdC, typename LdKr>
__device__ inline void append_row(LdC ld_c, LdKr ld_kr, int lane, long long row, int p,
                                  int apply_rope, void* __restrict__ cache,
                                  float* __restrict__ kv_scale, int d_c, int d_r, RopeFreq rope,
                                  const float* __restrict__ norm_gain, float norm_eps) {
  const int D = d_c + d_r;
  // element lane + 64 k (at most 10 per lane: D <= 640)
  float xc[10], xa[10], xb[10], gn[10];
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const int e = lane + 64 * k;
    const int q = min(max(e - d_c, 0), d_r - 1);
    xc[k] = ld_c(min(e, d_c - 1));
    xa[k] = ld_kr(apply_rope ? (q & ~1) : q);          // the pair's first element, or q
    xb[k] = ld_kr(apply_rope ? (q | 1) : q);           // the pair's second element
    gn[k] = norm_gain ? norm_gain[min(e, d_c - 1)] : 1.f;
  }
  float v[10];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const int e = lane + 64 * k;
    float x = 0.f;
    if (64 * k < D && 64 * k + 63 >= d_c) {           // the wave holds k^R elements here
      const int q = min(max(e - d_c, 0), d_r - 1);
      float y = xa[k];
      if (apply_rope) {
        float y0, y1;
        rope_pair(xa[k], xb[k], p, q >> 1, d_r, rope, &y0, &y1);
        y = (q & 1) ? y1 : y0;
      }
      x = (e >= d_c && e < D) ? y : 0.f;
    }
    v[k] = (e < d_c) ? xc[k] : x;
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
      if (lane + 64 * k < d_c) v[k] = v[k] * inv * gn[k];
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
  } else if (KV == MLA_FP6_E2M3) {
    // D = 576: element lane + 64 k is element lane % 32 of block 2 k +
    // lane / 32, so each block is one half-wave at one k
    uint8_t* dst = (uint8_t*)cache + row * kMxRowBytes;
    const int i = lane & 31;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      float am = fabsf(v[k]);
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
      const int ex = mx_block_exponent(am);
      const uint32_t c = f32_to_e2m3(ldexpf(v[k], -ex));   // exact scaling
      const uint32_t c1 = __shfl_down(c, 1, 64), c2 = __shfl_down(c, 2, 64);
      const uint32_t c3 = __shfl_down(c, 3, 64);
      const int blk = 2 * k + (lane >> 5);
      if ((i & 3) == 0) {                  // codes i .. i+3: 24 bits, 3 bytes
        const uint32_t w = c | (c1 << 6) | (c2 << 12) | (c3 << 18);
        uint8_t* q = dst + 24 * blk + 3 * (i >> 2);
        q[0] = uint8_t(w);
        q[1] = uint8_t(w >> 8);
        q[2] = uint8_t(w >> 16);
      }
      if (i == 0) dst[432 + blk] = uint8_t(ex + 127);
    }
    if (lane == 0) { dst[450] = 0; dst[451] = 0; }
  } else {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float sc = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
    uint8_t* dst = (uint8_t*)cache + row * D;
#pragma unroll
    for (int k = 0; k < 10; ++k)
      if (lane + 64 * k < D) dst[lane + 64 * k] = uint8_t(f32_to_e4m3(__fdiv_rn(v[k], sc)));
    if (lane == 0) kv_scale[row] = sc;
  }
}

// One wave per new row.  Source rows are F32 or BF16, row r of new_c at
// r * c_stride (elements), of new_kr at r * kr_stride.
// Rows block * 4 + wave, + nblocks * 4, ... (one row per wave at a time).
template <typename SrcT, int KV>
__device__ __forceinline__ void append_rows(
    const SrcT* __restrict__ new_c, const SrcT* __restrict__ new_kr,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int B, int max_pages, int max_len,
    long long cache_rows, int apply_rope, void* __restrict__ cache,
    float* __restrict__ kv_scale, int n_rows, int d_c, int d_r, const RopeFreq& rope,
    int c_stride, int kr_stride, const float* __restrict__ norm_gain, float norm_eps,
    int block, int nblocks) {
  const int lane = threadIdx.x & 63;
  for (int r = block * 4 + (threadIdx.x >> 6); r < n_rows; r += nblocks * 4) {
    const long long row = append_slot(seq_idx, pos, page_table, B, max_pages, max_len,
                                      cache_rows, r);
    if (row < 0) continue;
    const SrcT* c = new_c + (size_t)r * c_stride;
    const SrcT* kr = new_kr + (size_t)r * kr_stride;
    append_row<KV>([&](int e) { return load_f(c, e); }, [&](int q) { return load_f(kr, q); },
                   lane, row, pos[r], apply_rope, cache, kv_scale, d_c, d_r, rope, norm_gain,
                   norm_eps);
  }
}

template <typename SrcT, int KV>
__global__ __launch_bounds__(256) void append_kernel(
    const SrcT* __restrict__ new_c, const SrcT* __restrict__ new_kr,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int B, int max_pages, int max_len,
    long long cache_rows, int apply_rope, void* __restrict__ cache,
    float* __restrict__ kv_scale, int n_rows, int d_c, int d_r, RopeFreq rope,
    int c_stride, int kr_stride, const float* __restrict__ norm_gain, float norm_eps) {
  append_rows<SrcT, KV>(new_c, new_kr, seq_idx, pos, page_table, B, max_pages, max_len,
                        cache_rows, apply_rope, cache, kv_scale, n_rows, d_c, d_r, rope,
                        c_stride, kr_stride, norm_gain, norm_eps, blockIdx.x, gridDim.x);
}

// The step's absorption and cache append in one launch (they read and write
// disjoint buffers).  Every workgroup runs one (column block, token group)
// share of the absorption; before it, workgroup b's four waves append rows
// 4b .. 4b + 3 (and 4 (b + k * workgroups) .. for more rows), so the append
// takes no workgroup slots of its own: the absorption's LDS allows two
// workgroups per CU, and extra append workgroups would push absorption
// workgroups into a second round.  bf16 query and rows, bf16 absorbed query
// (or query pairs), bf16 / fp8 / 6-bit cache.
template <bool PAIRS, int KV>
__global__ __launch_bounds__(256) void absorb_append_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ q_pos,
    uint16_t* __restrict__ q_abs, int n_tok, int n_h, int abs_x, int abs_y,
    const uint16_t* __restrict__ new_c, const uint16_t* __restrict__ new_kr,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int B, int max_pages, int max_len,
    long long cache_rows, int apply_rope, void* __restrict__ cache,
    float* __restrict__ kv_scale, int n_rows, RopeFreq rope) {
  append_rows<uint16_t, KV>(new_c, new_kr, seq_idx, pos, page_table, B, max_pages, max_len,
                            cache_rows, apply_rope, cache, kv_scale, n_rows, 512, 64, rope, 512,
                            64, nullptr, 0.f, blockIdx.x, gridDim.x);
  absorb_mfma_block<uint16_t, PAIRS>(q_nope, q_rope, w_uk, q_pos, q_abs, n_tok, n_h, rope,
                                     blockIdx.x % abs_x, blockIdx.x / abs_x, abs_y);
}

// The cache producer's second half: one workgroup per new row sums the
// projection's K-block partials of the row (part [nkb, n_rows, D] fp32, in
// K-block order) into LDS, then wave 0 appends the row as append_kernel does.
template <int KV>
__global__ __launch_bounds__(192) void produce_append_kernel(
    const float* __restrict__ part, int nkb, const int32_t* __restrict__ seq_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ page_table, int B,
    int max_pages, int max_len, long long cache_rows, int apply_rope,
    void* __restrict__ cache, float* __restrict__ kv_scale, int n_rows, int d_c, int d_r,
    RopeFreq rope, const float* __restrict__ norm_gain, float norm_eps) {
  __shared__ __attribute__((aligned(16))) float srow[640];
  const int r = blockIdx.x, tid = threadIdx.x;
  const long long row = append_slot(seq_idx, pos, page_table, B, max_pages, max_len,
                                    cache_rows, r);
  if (row < 0) return;                 // uniform over the workgroup
  const int D = d_c + d_r;             // D % 4 == 0
  const size_t kstride = (size_t)n_rows * D;
  if (4 * tid < D) {
    // every K block's partial is loaded before any is added (at most 16 in
    // flight), then summed in K-block order
    const float* src = part + (size_t)r * D + 4 * tid;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nkb; k0 += 16) {
      floatx4 v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k0 + k < nkb) v[k] = *(const floatx4*)(src + (k0 + k) * kstride);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k0 + k < nkb) acc += v[k];
    }
    *(floatx4*)(srow + 4 * tid) = acc;
  }
  __syncthreads();
  if (tid < 64)
    append_row<KV>([&](int e) { return srow[e]; }, [&](int q) { return srow[d_c + q]; }, tid,
                   row, pos[r], apply_rope, cache, kv_scale, d_c, d_r, rope, norm_gain,
                   norm_eps);
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
  // global row (nq * n_h + head), one per wave
  const int R = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
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
  const uint8_t* pbase = (const uint8_t*)a.part_o + ((size_t)first * rows + row) * a.part_row_bytes;
  const size_t pstride = (size_t)rows * a.part_row_bytes; // bytes between splits
  // format of split s's partial: fp32 on the general path and for items
  // recomputed with split operands (flag set), else bf16
  const int32_t* flags = a.esc_flags ? a.esc_flags + (size_t)first * a.fast_rb + row / 128
                                     : nullptr;
  auto bf16_lo = [](uint32_t x) { return __builtin_bit_cast(float, x << 16); };
  auto bf16_hi = [](uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); };
  if (a.part_bf16 && ns <= 16) {
    // Few splits: every load (LSEs and partials) is issued before any of
    // them is used, so the row costs one memory latency.  Bit s of fmask:
    // split s holds fp32 (the item was recomputed with split operands), in
    // a slot of fp32 size; the mask is the same for the whole wave, so the
    // format choices are scalar branches outside the loads.
    const float lse_l = (lane < ns) ? lse_p[(size_t)lane * rows] : -INFINITY;
    const uint64_t fmask = flags ? __ballot(lane < ns && flags[(size_t)lane * a.fast_rb] != 0) : 0;
    u32x4 v0[16], v1[16];
    if (fmask == 0) {
#pragma unroll
      for (int sp = 0; sp < 16; ++sp)
        if (sp < ns) v0[sp] = *(const u32x4*)(pbase + (size_t)sp * pstride + 2 * d0);
    } else {
      // bf16 entries read 16 bytes past their 16 (inside the fp32-size slot)
#pragma unroll
      for (int sp = 0; sp < 16; ++sp)
        if (sp < ns) {
          const uint8_t* src = pbase + (size_t)sp * pstride + (((fmask >> sp) & 1) ? 4 * d0 : 2 * d0);
          v0[sp] = *(const u32x4*)src;
          v1[sp] = *(const u32x4*)(src + 16);
        }
    }
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
    for (int sp = 0; sp < 16; ++sp) {
      if (sp < ns) {
        const float w = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), sp));
        if ((fmask >> sp) & 1) {
          acc0 += w * __builtin_bit_cast(floatx4, v0[sp]);
          acc1 += w * __builtin_bit_cast(floatx4, v1[sp]);
        } else {
          acc0 += w * floatx4{bf16_lo(v0[sp][0]), bf16_hi(v0[sp][0]), bf16_lo(v0[sp][1]), bf16_hi(v0[sp][1])};
          acc1 += w * floatx4{bf16_lo(v0[sp][2]), bf16_hi(v0[sp][2]), bf16_lo(v0[sp][3]), bf16_hi(v0[sp][3])};
        }
      }
    }
    *(floatx4*)(out + d0) = acc0;
    *(floatx4*)(out + d0 + 4) = acc1;
    if (lane == 0) a.out_lse[R] = mx + logf(wsum);
    return;
  }
  float mx = -INFINITY;
  for (int sp = lane; sp < ns; sp += 64) mx = fmaxf(mx, lse_p[(size_t)sp * rows]);
  mx = wave_max(mx);
  if (mx == -INFINITY) {                                  // no visible token at all
    for (int d = d0; d < min(d0 + 8, a.d_c); d += 4) *(floatx4*)(out + d) = floatx4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0) a.out_lse[R] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int sp = lane; sp < ns; sp += 64) wsum += expf(lse_p[(size_t)sp * rows] - mx);
  wsum = wave_sum(wsum);
  const float inv = 1.0f / wsum;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // general path: d_c % 4 == 0; lanes past d_c read the row's first bytes
  // (in bounds) and never store
  const bool has0 = d0 < a.d_c, has1 = d0 + 4 < a.d_c;
  const int off0 = has0 ? 4 * d0 : 0, off1 = has1 ? 4 * d0 + 16 : 0;
  // Splits in batches of 16: every partial load of a batch is issued before
  // any of them is used.  A split's format (bit s of fmask: fp32, else bf16
  // with d_c = 512) only selects its addresses, so the loads carry no branch;
  // a bf16 entry loads its 16 bytes twice.  Slots past the batch's n splits
  // read its last split again (same format) with weight 0.
  for (int s0 = 0; s0 < ns; s0 += 16) {
    const int n = min(16, ns - s0);
    const float w_l = (lane < n) ? expf(lse_p[(size_t)(s0 + lane) * rows] - mx) * inv : 0.f;
    const uint64_t fmask = !a.part_bf16 ? ~0ull
                           : flags ? __ballot(lane < n && flags[(size_t)(s0 + lane) * a.fast_rb] != 0)
                                   : 0ull;
    u32x4 v0[16], v1[16];
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) {
      const int sc = min(sp, n - 1);
      const uint8_t* src = pbase + (size_t)(s0 + sc) * pstride;
      const bool f32 = (fmask >> sc) & 1;
      v0[sp] = *(const u32x4*)(src + (f32 ? off0 : 2 * d0));
      v1[sp] = *(const u32x4*)(src + (f32 ? off1 : 2 * d0));
    }
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) {
      const float w = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), sp));
      if ((fmask >> min(sp, n - 1)) & 1) {
        acc0 += w * __builtin_bit_cast(floatx4, v0[sp]);
        acc1 += w * __builtin_bit_cast(floatx4, v1[sp]);
      } else {
        acc0 += w * floatx4{bf16_lo(v0[sp][0]), bf16_hi(v0[sp][0]), bf16_lo(v0[sp][1]), bf16_hi(v0[sp][1])};
        acc1 += w * floatx4{bf16_lo(v0[sp][2]), bf16_hi(v0[sp][2]), bf16_lo(v0[sp][3]), bf16_hi(v0[sp][3])};
      }
    }
  }
  if (has0) *(floatx4*)(out + d0) = acc0;
  if (has1) *(floatx4*)(out + d0 + 4) = acc1;
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
  // 32 rows x 128 chunks of 4 floats.  Rows past the end read the last
  // token's row (their outputs are not stored), with no branch around the
  // loads, so that the block in flight is not waited for early.
  floatx4 v[8];
  auto load_latent = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = tid + 512 * i, t = min(t0 + (ch >> 7), n_tok - 1), c4 = (ch & 127) * 4;
      v[i] = *(const floatx4*)(latent + ((size_t)t * n_h + head) * DC + c4);
    }
  };
  // blockIdx.y splits the tokens when there are few heads: group y takes
  // the blocks of 32 tokens t0 = 32 (y + k gridDim.y)
  const int t_first = 32 * blockIdx.y, t_step = 32 * gridDim.y;
  load_latent(t_first);
  // W^UV into LDS, then each wave's A operands (its 16 d_h rows, all 512
  // latent dims: 64 VGPRs) into registers once: they are the same for every
  // token block, and reading them from LDS per block was a third of the
  // block's LDS traffic
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + 512 * i, r = ch >> 6, c8 = (ch & 63) * 8;
    *(u32x4*)(sw + r * kUpRow + c8) = wv[i];
  }
  __syncthreads();
  bf16x8 af[DC / 32];
  {
    const uint16_t* pa = sw + (16 * mi + r16) * kUpRow + 8 * g;
#pragma unroll
    for (int s = 0; s < DC / 32; ++s) af[s] = *(const bf16x8*)(pa + 32 * s);
  }
  for (int t0 = t_first; t0 < n_tok; t0 += t_step) {
    if (t0 != t_first) __syncthreads();   // the previous block's reads are done
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
    const int bo = (16 * ni + r16) * kUpRow + 8 * g;
#pragma unroll
    for (int s = 0; s < DC / 32; ++s) {
      const bf16x8 bh = *(const bf16x8*)(sh + bo + 32 * s);
      const bf16x8 bl = *(const bf16x8*)(sl + bo + 32 * s);
      acc_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bh, acc_hi, 0, 0, 0);
      acc_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bl, acc_lo, 0, 0, 0);
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
hipError_t launch_absorb(const mla_dims_t& d, bool fast, bool pairs, const void* q_nope,
                         const void* q_rope, const void* w_uk,
                         const int32_t* q_pos, void* q_abs, int n_tok,
                         RopeFreq rope, hipStream_t st) {
  const bool out_f32 = d.q_dtype == MLA_F32 || d.precision == MLA_PREC_FP32;
  if (fast) {
    // four workgroups per head; with few heads the tokens are split over up
    // to 256 workgroups in all
    const int groups = std::max(1, std::min((n_tok + 31) / 32, kNumCU / (4 * d.n_heads)));
    const dim3 grid(d.n_heads * 4, groups);
    if (pairs)
      hipLaunchKernelGGL((absorb_mfma_kernel<uint16_t, true>), grid, dim3(256), 0, st,
                         (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                         (const uint16_t*)w_uk, q_pos, (uint16_t*)q_abs, n_tok,
                         d.n_heads, rope);
    else if (out_f32)
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
  else if (d.kv_dtype == MLA_FP6_E2M3 && !src_f32) MLA_APPEND(uint16_t, MLA_FP6_E2M3);
  else if (d.kv_dtype == MLA_FP6_E2M3) MLA_APPEND(float, MLA_FP6_E2M3);
  else if (!src_f32) MLA_APPEND(uint16_t, MLA_FP8_E4M3);
  else MLA_APPEND(float, MLA_FP8_E4M3);
#undef MLA_APPEND
  return hipGetLastError();
}

// One launch for the absorption and the append when both take their fast
// paths (see absorb_append_kernel); returns hipErrorInvalidValue otherwise.
hipError_t launch_absorb_append(const mla_dims_t& d, bool pairs, const void* q_nope,
                                const void* q_rope, const void* w_uk, const int32_t* q_pos,
                                void* q_abs, int n_tok, const void* new_c, const void* new_kr,
                                const int32_t* seq_idx, const int32_t* pos,
                                const int32_t* page_table, int B, int max_pages, int max_len,
                                long long cache_rows, int apply_rope, void* cache,
                                float* kv_scale, int n_rows, RopeFreq rope, hipStream_t st) {
  const int abs_y = std::max(1, std::min((n_tok + 31) / 32, kNumCU / (4 * d.n_heads)));
  const int abs_x = 4 * d.n_heads;
  const long long total = (long long)abs_x * abs_y;
  if (total > INT_MAX) return hipErrorInvalidValue;
#define MLA_AA(P, KV)                                                                         \
  hipLaunchKernelGGL((absorb_append_kernel<P, KV>), dim3((unsigned)total), dim3(256), 0, st,  \
                     (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk, \
                     q_pos, (uint16_t*)q_abs, n_tok, d.n_heads, abs_x, abs_y,                 \
                     (const uint16_t*)new_c, (const uint16_t*)new_kr, seq_idx, pos,           \
                     page_table, B, max_pages, max_len, cache_rows, apply_rope, cache,        \
                     kv_scale, n_rows, rope)
  if (d.kv_dtype == MLA_BF16) {
    if (pairs) MLA_AA(true, MLA_BF16); else MLA_AA(false, MLA_BF16);
  } else if (d.kv_dtype == MLA_FP8_E4M3) {
    if (pairs) MLA_AA(true, MLA_FP8_E4M3); else MLA_AA(false, MLA_FP8_E4M3);
  } else if (d.kv_dtype == MLA_FP6_E2M3) {
    if (pairs) MLA_AA(true, MLA_FP6_E2M3); else MLA_AA(false, MLA_FP6_E2M3);
  } else {
    return hipErrorInvalidValue;
  }
#undef MLA_AA
  return hipGetLastError();
}

hipError_t launch_produce_append(const mla_dims_t& d, const float* part, int nkb,
                                 const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* page_table, int B, int max_pages, int max_len,
                                 long long cache_rows, int apply_rope, void* cache,
                                 float* kv_scale, int n_rows, RopeFreq rope, hipStream_t st,
                                 const float* norm_gain, float norm_eps) {
#define MLA_PRODUCE(KV)                                                                       \
  hipLaunchKernelGGL((produce_append_kernel<KV>), dim3(n_rows), dim3(192), 0, st, part, nkb,  \
                     seq_idx, pos, page_table, B, max_pages, max_len, cache_rows, apply_rope, \
                     cache, kv_scale, n_rows, d.d_latent, d.d_rope, rope, norm_gain, norm_eps)
  if (d.kv_dtype == MLA_F32) MLA_PRODUCE(MLA_F32);
  else if (d.kv_dtype == MLA_BF16) MLA_PRODUCE(MLA_BF16);
  else if (d.kv_dtype == MLA_FP6_E2M3) MLA_PRODUCE(MLA_FP6_E2M3);
  else MLA_PRODUCE(MLA_FP8_E4M3);
#undef MLA_PRODUCE
  return hipGetLastError();
}

// ============================================================ page-table check
// Debug aid: every page id that a sequence's length makes the kernels read
// (entries p < ceil(L_b / page) of row b) must lie in [0, n_pages).  One
// workgroup walks the table (a debug path: no speed needed, and a single
// workgroup can set its own result without a clearing launch).
// result: [0] out-of-range entries, [1] flat index b * max_pages + p of the
// first (-1 if none), [2] its value (0 if none), [3] sequences whose length
// is < 0 or > max_pages * page (their whole row is checked).
__global__ __launch_bounds__(1024) void page_table_check_kernel(
    const int32_t* __restrict__ pt, int max_pages, const int32_t* __restrict__ lens, int batch,
    long long n_pages, int32_t* __restrict__ result) {
  __shared__ int s_count, s_first, s_badlen;
  if (threadIdx.x == 0) {
    s_count = 0;
    s_first = INT_MAX;
    s_badlen = 0;
  }
  __syncthreads();
  int count = 0, first = INT_MAX, badlen = 0;
  const long long total = (long long)batch * max_pages;
  for (long long i = threadIdx.x; i < total; i += blockDim.x) {
    const int b = (int)(i / max_pages), p = (int)(i - (long long)b * max_pages);
    const int L = lens[b];
    const bool len_ok = L >= 0 && (long long)L <= (long long)max_pages * kPage;
    if (p == 0 && !len_ok) ++badlen;
    const int used = len_ok ? (L + kPage - 1) / kPage : max_pages;
    if (p < used) {
      const int v = pt[i];
      if (v < 0 || (long long)v >= n_pages) {
        ++count;
        first = min(first, (int)i);
      }
    }
  }
  if (count) {
    atomicAdd(&s_count, count);
    atomicMin(&s_first, first);
  }
  if (badlen) atomicAdd(&s_badlen, badlen);
  __syncthreads();
  if (threadIdx.x == 0) {
    result[0] = s_count;
    result[1] = s_count ? s_first : -1;
    result[2] = s_count ? pt[s_first] : 0;
    result[3] = s_badlen;
  }
}

hipError_t launch_page_table_check(const int32_t* pt, int max_pages, const int32_t* lens,
                                   int batch, long long n_pages, int32_t* result,
                                   hipStream_t st) {
  hipLaunchKernelGGL(page_table_check_kernel, dim3(1), dim3(1024), 0, st, pt, max_pages, lens,
                     batch, n_pages, result);
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
