// Shared definitions of the MLA decode library (device and host side).
//
// Number formats: bfloat16 is the top half of an IEEE binary32; the fp8
// cache uses OCP FP8 E4M3 ("e4m3fn": bias 7, 3 mantissa bits, max 448,
// no infinities).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 64;            // tokens per page of a paged cache
constexpr int kNumCU = 256;          // MI355X compute units
constexpr int kNumXCD = 8;           // accelerator complex dies (own L2 each)
constexpr int kMinChunk = 256;       // smallest automatic KV chunk (tokens)
// s_waitcnt immediate that waits for every vector-memory load and nothing
// else (gfx9 encoding: vmcnt in bits 3:0 and 15:14 = 0, expcnt 6:4 = 7,
// lgkmcnt 11:8 = 15)
constexpr int kWaitVm0 = 0x0F70;

// ---------------------------------------------------------------- formats
__host__ __device__ inline float bf16_bits_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = uint32_t(b) << 16;
  return v.f;
}

// float -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__host__ __device__ inline uint16_t f32_to_bf16_bits(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  uint32_t u = v.u;
  if ((u & 0x7F800000u) == 0x7F800000u) return uint16_t((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// E4M3 code -> float (exact).  Codes 0x7F / 0xFF (NaN) never occur in a
// cache written by the append kernel.
__host__ __device__ inline float e4m3_to_f32(uint32_t code) {
  uint32_t em = code & 0x7Fu;
  float mag;
  if (em >= 8) {
    union { uint32_t u; float f; } v;
    v.u = ((em >> 3) + 120u) << 23 | (em & 7u) << 20;
    mag = v.f;
  } else {
    mag = float(em) * 0.001953125f;   // m * 2^-9 (subnormal)
  }
  return (code & 0x80u) ? -mag : mag;
}

// float -> nearest E4M3 code, ties to even mantissa, |x| >= 448 saturates.
__host__ __device__ inline uint32_t f32_to_e4m3(float x) {
  union { uint32_t u; float f; } v;
  v.f = x;
  uint32_t sign = (v.u >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7E;
  } else if (a < 0.015625f) {                // below 2^-6: subnormal grid
    code = uint32_t(rintf(a * 512.0f));      // exact scaling; ties to even
  } else {
    union { uint32_t u; float f; } w;
    w.f = a;
    uint32_t e = (w.u >> 23) - 127u + 7u;    // biased E4M3 exponent, 1..15
    uint32_t mant = w.u & 0x7FFFFFu;
    uint32_t q = mant >> 20, rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    if (q == 8) { q = 0; ++e; }
    code = (e << 3) | q;                     // a < 448 keeps this <= 0x7E
  }
  return code | sign;
}

// float -> nearest E2M3 code (ties to the even code), magnitudes from 7.5
// up saturating to 7.5; the sign bit of x becomes bit 5.  |x| < 8 in use.
__host__ __device__ inline uint32_t f32_to_e2m3(float x) {
  union { uint32_t u; float f; } v;
  v.f = x;
  const uint32_t sign = (v.u >> 26) & 0x20u;
  const float a = fabsf(x);
  uint32_t code;
  if (!(a < 7.5f)) {
    code = 0x1F;
  } else if (a < 1.0f) {                     // subnormal grid m/8 (m = 8 is 1.0)
    code = uint32_t(rintf(a * 8.0f));
  } else {
    union { uint32_t u; float f; } w;
    w.f = a;
    const int E = int((w.u >> 23) & 0xFF) - 127;   // 0, 1 or 2
    uint32_t e = uint32_t(E + 1);
    uint32_t q = uint32_t(rintf((ldexpf(a, -E) - 1.0f) * 8.0f));
    if (q == 8) { q = 0; ++e; }
    code = (e << 3) | q;                     // a < 7.5 keeps this <= 0x1F
  }
  return code | sign;
}

// Shared exponent of a block of 32 elements of the 6-bit cache:
// floor(log2 amax) - 2 kept in [-126, 127] (-126 for amax = 0).
__host__ __device__ inline int mx_block_exponent(float amax) {
  union { uint32_t u; float f; } v;
  v.f = amax;
  const int e = int((v.u >> 23) & 0xFF) - 127 - 2;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}
constexpr int kMxRowBytes = 452;     // 6-bit cache row: 432 code bytes, 18 exponents, 2 pad

// ------------------------------------------------------------------ RoPE
// Frequencies of the interleaved pairs (2k, 2k+1): theta_k = base^(-2k/d),
// and with context extension (factor > 1, YaRN's NTK-by-parts rule) pair k,
// which turns r_k = orig_len theta_k / (2 pi) times over the original
// context, takes (1 - g) theta_k / factor + g theta_k with g = clamp((r_k -
// alpha) / (beta - alpha), 0, 1).  Computed in double precision on the host,
// once per call, and handed to the kernels as a table (a power in double
// precision per rotated pair would dominate the append of a decode step).
constexpr int kMaxRopePairs = 64;     // d_rope <= 128
struct RopeFreq {
  double theta[kMaxRopePairs];
};

inline double rope_theta_host(int k, int d, double base, double factor, double alpha,
                              double beta, double orig_len) {
  const double theta = pow(base, -2.0 * (double)k / (double)d);
  if (!(factor > 1.0)) return theta;
  const double turns = orig_len * theta / 6.283185307179586;
  double g = (turns - alpha) / (beta - alpha);
  g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
  return (1.0 - g) * theta / factor + g * theta;
}

__host__ __device__ inline double rope_theta(int k, int /*d*/, const RopeFreq& rf) {
  return rf.theta[k];
}

// ------------------------------------------------------------ split planner
// Tokens per KV chunk of sequence b.  num_splits > 0: each sequence is cut
// into at most num_splits chunks of equal size rounded up to the page size;
// otherwise every sequence uses the global chunk `chunk`.
__host__ __device__ inline int chunk_of(int L, int num_splits, int chunk) {
  if (num_splits > 0) {
    int c = (L + num_splits - 1) / num_splits;
    return ((c + kPage - 1) / kPage) * kPage;
  }
  return chunk;
}

__host__ __device__ inline int splits_of(int L, int num_splits, int chunk) {
  int c = chunk_of(L, num_splits, chunk);
  return (L + c - 1) / c;
}

// Logical work index of a workgroup so that consecutive logical indices run
// on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
__host__ __device__ inline int xcd_logical_index(int g, int G) {
  int q = G / kNumXCD, r = G % kNumXCD;
  int x = g % kNumXCD;
  return x * q + (x < r ? x : r) + g / kNumXCD;
}

// Arguments of the attention kernels (passed by value).
struct DecodeArgs {
  const void* q_abs;          // [B*T, n_h, D] bf16 (fast) / q_dtype (general);
                              // query pairs: [B*T, n_h, 2, D] bf16 (hi, lo)
  const void* cache;          // contiguous [B, max_len, D] or paged
  const float* kv_scale;      // fp8: one float per cache row
  const int32_t* page_table;  // [B, max_pages] or nullptr
  const int32_t* seq_lens;    // [B]
  void* part_o;               // [n_items, rows] partial latent outputs of d_c
                              // elements, part_row_bytes apart (bf16 when
                              // part_bf16 and the item is not escalated, else fp32)
  float* part_lse;            // [n_items, rows]
  int32_t* esc_flags;         // [n_items, rows / 128] or nullptr: 1 = the item's
                              // 128-row block is recomputed with split operands
  int32_t part_bf16;
  int32_t part_row_bytes;     // bytes between consecutive partial rows
  int32_t q_row_bytes;        // bytes between consecutive q_abs rows
  int32_t fast_rb;            // 128-row blocks per item (flag index stride)
  float esc_log2;             // escalation threshold on scaled scores (log2 units)
  float* out_latent;          // [B*T, n_h, d_c]
  float* out_lse;             // [B*T, n_h]
  int32_t B, T, n_h, d_c, d_r;
  int32_t max_pages, max_len;
  int32_t num_splits, chunk, n_items, row_blocks;
  int32_t q_dtype, kv_dtype;
  float scale_log2;           // softmax scale * log2(e)
  int32_t uniform_len;        // > 0: every sequence has this length
};

// Work items of a plan (passed by value).  uniform_len > 0: every sequence
// has this length and item = b * splits + s.  Else the host lists the items
// when there are at most kItemTable of them, largest first in the order the
// workgroups are dealt out (round-robin over the XCDs, each item's row blocks
// on one XCD), so the long items start first and spread over all XCDs; n = 0: the
// kernel locates them in sequence order.  Partials are stored at the item's
// index in sequence order (item_id), where the combine looks for them.
constexpr int kItemTable = 448;     // keeps the kernel arguments under 4 KB
struct ItemTable {
  int32_t uniform_len;
  int32_t n;
  uint32_t seq_split[kItemTable];   // sequence | split << 20
  int32_t item_id[kItemTable];      // index in sequence order
};

}  // namespace mla
