// Pieces shared by the 128-row attention kernels (decode_mfma.hip for bf16
// and 6-bit tiles, decode_fp8.hip for fp8 tiles): the token order of the
// score registers and the write-back of a work item's rows.
//
// Absorbed MLA decode ("DeepSeek-V2: Strong, Economical, Efficient", section
// 2.1.2 and Appendix C; attention-output equation of the "DeepSeek-V3
// Technical Report" notes, MLA section).  A workgroup of 4 waves owns 128
// query rows of one work item; after the tile loop wave w holds O^T for
// latent dims 128 w .. 128 w + 127 of all 128 rows in 16 accumulator blocks
// of 32 x 32 (block 4 db + rb: dims 128 w + 32 db + 8 (r/4) + 4 h + r%4 in
// register r of a lane in half h, row 32 rb + l%32), and the softmax sums of
// the rows 32 w .. 32 w + 31 (one partial per lane half).
#pragma once

#include <math.h>

#include "mla_common.hpp"

namespace mla {

// Score-row order inside a tile.  MFMA row m of the scores (the K operand
// row read by lane m % 32) is tile row tile_row(m) = 16 (m/16) + (m/4)%4 +
// 4 (m%4).  Score register r of a lane in half h (row m = 8(r/4) + 4h +
// r%4) holds token tile_row(m).  The permutation keeps the operand reads of
// the kernels free of LDS bank conflicts (each kernel states how).
__device__ __forceinline__ int tile_row(int m) {
  return 16 * (m >> 4) + ((m >> 2) & 3) + 4 * (m & 3);
}
__device__ __forceinline__ int reg_token(int r, int h) {
  return tile_row(8 * (r >> 2) + 4 * h + (r & 3));
}

// Normalise and write a work item's 128 rows: the final output (fp32 rows
// and the LSE) when the item is a whole sequence, else this split's partial
// (normalised, bf16) and its LSE.  l_run: this lane's partial softmax sum of
// row 32 wave + l%32; m_ref: that row's reference (log2 domain).  stage:
// LDS of at least 139,264 bytes that no wave reads any more once every
// wave's loads have landed (the kernel's tile ring); s_inv: 128 floats of
// LDS.  Called by every thread of the workgroup (it holds a barrier).
__device__ __forceinline__ void store_rows(const DecodeArgs& a, const floatx16 (&o)[16],
                                           float l_run, float m_ref, uint8_t* stage,
                                           float* s_inv, int b, int rb, int item_id, int ns,
                                           int rows, int tid) {
  const int lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  if (a.esc_flags && tid == 0) a.esc_flags[(size_t)item_id * a.fast_rb + rb] = 0;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  const float lse = (l_tot > 0.f) ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  if (h == 0) s_inv[32 * wave + l32] = inv;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile loads past the end still write LDS
  __syncthreads();                                   // the ring is free; s_inv is in
  float inv_rb[4];
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) inv_rb[r4] = s_inv[32 * r4 + l32];
  constexpr int DC = 512;
  const int row0 = rb * 128;                         // first row of the workgroup
  const int own0 = row0 + 32 * wave;                 // first row this wave owns
  if (ns == 1) {
    // fp32 rows: 512 bytes per row from this wave, two passes of 64 rows
    constexpr int SROW = 528;
    uint8_t* stg = stage + wave * (64 * SROW);
    const size_t g0 = (size_t)b * rows + row0;
    uint8_t* dst = (uint8_t*)(a.out_latent + g0 * DC) + 512 * wave;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const int r4 = 2 * p + r2;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const floatx16& ob = o[4 * db + r4];
            const floatx4 v = {ob[4 * jj], ob[4 * jj + 1], ob[4 * jj + 2], ob[4 * jj + 3]};
            *(floatx4*)(stg + (32 * r2 + l32) * SROW + 4 * (32 * db + 8 * jj + 4 * h)) =
                v * inv_rb[r4];
          }
        }
      }
      // 64 rows x 512 bytes: one store covers two rows
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        const int r = 2 * n + (lane >> 5);
        *(floatx4*)(dst + (size_t)(64 * p + r) * (4 * DC) + 16 * (lane & 31)) =
            *(const floatx4*)(stg + r * SROW + 16 * (lane & 31));
      }
    }
    if (h == 0) a.out_lse[(size_t)b * rows + own0 + l32] = lse;
  } else {
    // split partial, normalised, stored as bf16 (combined in fp32): 256
    // bytes per row from this wave, all 128 rows at once
    constexpr int SROW = 272;
    uint8_t* stg = stage + wave * (128 * SROW);
    const size_t g0 = (size_t)item_id * rows + row0;
    uint8_t* dst = (uint8_t*)a.part_o + g0 * a.part_row_bytes + 256 * wave;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const floatx16& ob = o[4 * db + r4];
          const float w = inv_rb[r4];
          const bf16x2 p01 = {(__bf16)(ob[4 * jj] * w), (__bf16)(ob[4 * jj + 1] * w)};
          const bf16x2 p23 = {(__bf16)(ob[4 * jj + 2] * w), (__bf16)(ob[4 * jj + 3] * w)};
          *(u32x2*)(stg + (32 * r4 + l32) * SROW + 2 * (32 * db + 8 * jj + 4 * h)) =
              u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
        }
      }
    }
    // 128 rows x 256 bytes: one store covers four rows
#pragma unroll
    for (int n = 0; n < 32; ++n) {
      const int r = 4 * n + (lane >> 4);
      *(u32x4*)(dst + (size_t)r * a.part_row_bytes + 16 * (lane & 15)) =
          *(const u32x4*)(stg + r * SROW + 16 * (lane & 15));
    }
    if (h == 0) a.part_lse[(size_t)item_id * rows + own0 + l32] = lse;
  }
}

}  // namespace mla
