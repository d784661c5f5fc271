// Attention over the latent cache with split bf16 operands on gfx950 matrix
// cores: the precise counterpart of the bf16 attention kernel.
//
// Same step as the bf16 kernel ("DeepSeek-V3 Technical Report" notes, MLA
// section, attention-output equation, in absorbed form: "DeepSeek-V2:
// Strong, Economical, Efficient", section 2.1.2 and Appendix C), with every
// rounded operand carried as a pair of bf16 numbers:
//   * the absorbed query as (hi, lo) = (bf16(q), bf16(q - hi)), stored that
//     way by the absorption, so a score is K.q_hi + K.q_lo (the cache rows
//     are exact in bf16): relative error ~2^-17 instead of 2^-9;
//   * the softmax weights as (hi, lo) in the P.C product, the normaliser the
//     fp32 sum of the weights;
//   * split partials in fp32.
// The bf16 rounding of the query moves a score by ~2^-9 of |q||k|; when a
// few cache rows of large norm take most of the softmax weight, that shows
// in the output.  The bf16 kernel flags such work items (largest scaled
// score past a threshold) and this kernel recomputes them; it also runs
// every item when split operands are asked for.
//
// Work decomposition: one workgroup of 4 waves per (work item, 64 query
// rows).  Wave w owns rows 16w .. 16w+15 for the scores (S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16, tokens as M, rows as N; the (hi, lo) query of
// its 16 rows stays in 144 VGPRs) and latent dims 128w .. 128w+127 of all
// 64 rows for O^T += C^T P^T (v_mfma_f32_32x32x16_bf16, accumulators in the
// matrix registers).  Weights go through an 8 KB LDS buffer.  Tiles of 32
// tokens go through a 4-slot LDS ring (rows padded to 1168 bytes), loaded
// HBM -> LDS by LDS-writing buffer loads, three tiles in flight.
//
// Token order.  Tile row r is token r of the tile.  In the scores, M index
// m of token block tb is tile row 16 tb + 4 (m%4) + m/4, so a lane (row j,
// g = lane/16) holds tokens 16 tb + 4 i + g, i = 0..3.  In the PV product,
// K slot 8 h + 4 c + k of half ks is token 4 (k + 4 h) + 2 ks + c: a lane's
// four weights of one token block land in one 8-byte piece of a B operand,
// and each transposed C^T read covers tile rows {4 j + const}, whose 64-byte
// runs fall on each LDS bank exactly twice at the 1168-byte pitch.
//
// Softmax in the log2 domain against a per-row reference m_ref (the row max
// of the first tile it sees), weights 2^(s - m_ref) accumulated without
// rescaling; a score more than 64 above m_ref restarts the item with m_ref
// raised (exact for any reference: LSE = m_ref + log2(sum)).
#include <math.h>

#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

namespace {
constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int XROWS = 64;                // query rows per workgroup
constexpr int TILE = 32;                 // tokens per staged tile
constexpr int LROW = 1168;               // LDS bytes per token row (1152 + 16 pad)
constexpr int NBUF = 4;                  // LDS ring of tiles
constexpr int NLOADS = 37;               // direct loads of 64 x 16 B per tile
constexpr int TILE_BYTES = NLOADS * 1024;
constexpr int NCH = 72;                  // 16-byte chunks per bf16 row
constexpr uint32_t kOOB = 0x40000000u;   // buffer offset past any valid range
constexpr float kNegInf = -INFINITY;

typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ inline u32x2 x2_tr16(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (shortx4 __attribute__((address_space(3)))*)(p)));
}

// LDS granule u (16 bytes) of a ring slot holds granule u % 73 of tile row
// u / 73 (u / 73 = (449 u) >> 15 for u < 2368); the pad granule of each row
// and granules past the 32 rows take an out-of-range offset (zero-filled).
__device__ inline uint32_t x2_src_offset(int u) {
  const int tk = (u * 449) >> 15;
  return (u - 73 * tk == NCH || tk >= TILE) ? kOOB : uint32_t(16 * (u - tk));
}

__device__ inline uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}
__device__ inline float lo16(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ inline float hi16(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }

template <int N>
__device__ __forceinline__ void x2_wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }
}  // namespace

// Software-pipelined step bodies (gen_decode_asm.py): the split-operand
// score sequence, MLA_ASM_QKX2_TILE.
#include "decode_mfma_asm.inc"

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_x2_kernel(DecodeArgs a, ItemTable tab, int row_blocks) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv[NBUF][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[8 * 1024];   // P^T (hi, lo) fragments
  __shared__ float s_inv[XROWS];
  __shared__ int s_restart;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int gi = xcd_logical_index(blockIdx.x, gridDim.x);
  const int item = gi / row_blocks, ph = gi % row_blocks;
  int b, s_idx, L, item_id = item;
  if (tab.uniform_len > 0) {
    L = tab.uniform_len;
    const int nsu = splits_of(L, a.num_splits, a.chunk);
    b = item / nsu;
    s_idx = item - b * nsu;
  } else if (tab.n > 0) {
    const uint32_t e = tab.seq_split[item];
    b = e & 0xFFFFF;
    s_idx = e >> 20;
    item_id = tab.item_id[item];
    L = a.seq_lens[b];
  } else {
    const ItemLoc loc = locate_item(a.seq_lens, a.B, a.num_splits, a.chunk, item);
    if (loc.b < 0) return;
    b = loc.b;
    s_idx = loc.s;
    L = a.seq_lens[loc.b];
  }
  b = __builtin_amdgcn_readfirstlane(b);
  L = __builtin_amdgcn_readfirstlane(L);
  item_id = __builtin_amdgcn_readfirstlane(item_id);
  const int row0 = ph * XROWS;                            // first row of the workgroup
  // recompute only what the bf16 kernel flagged (all items without flags)
  if (a.esc_flags && a.esc_flags[(size_t)item_id * a.fast_rb + row0 / 128] == 0) return;

  const int ns = splits_of(L, a.num_splits, a.chunk);
  const int c = chunk_of(L, a.num_splits, a.chunk);
  const int t0 = __builtin_amdgcn_readfirstlane(s_idx) * c;
  const int t_end = min(L, t0 + c);
  const int rows = a.n_h * a.T;
  const int qrow = row0 + 16 * wave + j;                  // this lane's score row
  const int tau = qrow / a.n_h;                           // the wave's 16 rows share it
  const int lim = __builtin_amdgcn_readfirstlane(min(t_end - 1, L - a.T + tau));
  const int tau_max = (row0 + XROWS - 1) / a.n_h;
  const int t_stage = __builtin_amdgcn_readfirstlane(min(t_end, L - a.T + tau_max + 1));
  const int ntiles = (t_stage > t0) ? (t_stage - t0 + TILE - 1) / TILE : 0;

  // ---- (hi, lo) query of this lane's row: B operands of the score MFMAs
  // (lane: row j of the wave's 16, dims 32 ks + 8 g .. + 7)
  bf16x8 qh[D / 32], ql[D / 32];
  {
    const uint8_t* qsrc = (const uint8_t*)a.q_abs + ((size_t)b * rows + qrow) * a.q_row_bytes + 16 * g;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qh[ks] = *(const bf16x8*)(qsrc + 64 * ks);
      ql[ks] = *(const bf16x8*)(qsrc + 2 * D + 64 * ks);
    }
    // landed here, before any tile load: the compiler does not count the
    // assembly loads, and its first use of a fragment (the score sequence,
    // inside the step loop) would otherwise wait for every load in flight
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }

  const uint32_t lds_ring = (uint32_t)(uintptr_t)&s_kv[0][0];
  const uint8_t* cache = (const uint8_t*)a.cache;
  const int seq_row0 = b * a.max_len;
  const int32_t* ptab = a.page_table ? a.page_table + (size_t)b * a.max_pages : nullptr;
  uint32_t voff[10];
#pragma unroll
  for (int n = 0; n < 10; ++n) voff[n] = x2_src_offset(64 * (wave + 4 * n) + lane);

  // loads of tile `tile` of the item into ring slot `buf` (wave-uniform)
  auto issue = [&](int tile, int buf) {
    const int ts = t0 + tile * TILE;
    const int nv = max(0, min(TILE, t_stage - ts));
    int r0 = 0;
    if (nv > 0) r0 = ptab ? ptab[ts / kPage] * kPage + (ts % kPage) : seq_row0 + ts;
    r0 = __builtin_amdgcn_readfirstlane(r0);
    const uint64_t ad = (uint64_t)(cache + (size_t)r0 * (2 * D));
    const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad),
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32)) & 0xFFFFu,
                      (uint32_t)__builtin_amdgcn_readfirstlane(nv * 2 * D), 0x00020000u};
    const uint32_t lb = lds_ring + buf * TILE_BYTES + 1024 * wave;
#pragma unroll
    for (int n = 0; n < 9; ++n)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(lb + 4096 * n), "v"(voff[n]), "s"(rs) : "memory");
    if (wave == 0)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(lds_ring + buf * TILE_BYTES + 1024 * 36), "v"(voff[9]), "s"(rs)
                   : "memory");
  };

  // per-lane LDS offsets
  const int qk_off = 4 * (j & 3) + (j >> 2);              // + 16 tb: tile row of M index j
  // transposed C^T reads: token 4 (k + 4 (G/2)) + 2 ks + c with G = lane/16,
  // k = (lane%16)/4; dims 128 wave + 32 db + 16 (G%2) + 4 (lane%4)
  const int pv_row = 4 * (((lane & 15) >> 2) + 4 * (lane >> 5));
  const int pv_col = 2 * (128 * wave + 16 * (g & 1) + 4 * (lane & 3));
  // P writes: fragment (rb = wave/2, ks = g/2, hl), lane 16 (wave%2) + j + 32 tb,
  // bytes 8 (g%2) .. +7
  const int pw_off = 1024 * (4 * (wave >> 1) + 2 * (g >> 1)) + 16 * (16 * (wave & 1) + j) + 8 * (g & 1);

  floatx16 o[8];                                          // [db * 2 + rb]
  float m_ref = kNegInf, m_seen = kNegInf, l_run = 0.f;
  if (tid == 0) s_restart = 0;
  __syncthreads();
  for (;;) {                                              // attempts (a restart is rare)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = floatx16{};
    l_run = 0.f;
    int restart = 0;
    for (int t = 0; t < 3; ++t)
      if (t < ntiles) issue(t, t);
    for (int it = 0; it < ntiles; ++it) {
      // tile it landed: this wave's loads of the (at most two) later tiles may fly
      const int later = min(2, ntiles - 1 - it);
      if (later == 2) {
        if (wave == 0) x2_wait_vm<20>(); else x2_wait_vm<18>();
      } else if (later == 1) {
        if (wave == 0) x2_wait_vm<10>(); else x2_wait_vm<9>();
      } else {
        x2_wait_vm<0>();
      }
      __syncthreads();          // every wave's share of tile it is in; PV of it-1 done
      if (it + 3 < ntiles) issue(it + 3, (it + 3) & 3);
      const uint8_t* slot = &s_kv[it & 3][0];
      const int ts = t0 + it * TILE;

      // ---- scores S^T = K (Q_hi + Q_lo)^T for the wave's 16 rows
      // (a generated sequence: five operand reads stay in flight, where the
      // compiler waited for each read before its two MFMAs; the hi query
      // fragments and the first nine lo ones are read from accumulation
      // registers, which hold them next to O (236 of 256), the other lo ones
      // from vector registers)
      floatx4 sh[2], sl[2];
      {
        const uint32_t ad = (uint32_t)(uintptr_t)(slot + qk_off * LROW + 16 * g);
        asm volatile(MLA_ASM_QKX2_TILE
                     : "=&v"(sh[0]), "=&v"(sh[1]), "=&v"(sl[0]), "=&v"(sl[1])
                     : "v"(ad), "a"(qh[0]), "a"(qh[1]), "a"(qh[2]), "a"(qh[3]), "a"(qh[4]),
                       "a"(qh[5]), "a"(qh[6]), "a"(qh[7]), "a"(qh[8]), "a"(qh[9]), "a"(qh[10]),
                       "a"(qh[11]), "a"(qh[12]), "a"(qh[13]), "a"(qh[14]), "a"(qh[15]),
                       "a"(qh[16]), "a"(qh[17]), "a"(ql[0]), "a"(ql[1]), "a"(ql[2]), "a"(ql[3]),
                       "a"(ql[4]), "a"(ql[5]), "a"(ql[6]), "a"(ql[7]), "a"(ql[8]), "v"(ql[9]),
                       "v"(ql[10]), "v"(ql[11]), "v"(ql[12]), "v"(ql[13]), "v"(ql[14]),
                       "v"(ql[15]), "v"(ql[16]), "v"(ql[17])
                     : "memory", MLA_ASM_QKX2_CLOBBERS);
      }
      // score (tb, i): token ts + 16 tb + 4 i + g of row qrow
      float x[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sv = (sh[tb][i] + sl[tb][i]) * a.scale_log2;
          x[4 * tb + i] = (ts + 16 * tb + 4 * i + g > lim) ? kNegInf : sv;
        }
      float mt = x[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) mt = fmaxf(mt, x[r]);
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));             // row max of the tile
      if (m_ref == kNegInf) m_ref = mt;                    // first tile the row sees
      const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
      uint32_t ph2[2][2], pl2[2][2];                       // [tb][pair]
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = exp2f(x[4 * tb + i] + neg_m);
          l_run += p[i];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t hi = pack2(p[2 * e], p[2 * e + 1]);
          ph2[tb][e] = hi;
          pl2[tb][e] = pack2(p[2 * e] - lo16(hi), p[2 * e + 1] - hi16(hi));
        }
      }
      m_seen = fmaxf(m_seen, mt);
      if (mt > m_ref + 64.0f) s_restart = 1;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        *(u32x2*)(s_p + pw_off + 512 * tb) = u32x2{ph2[tb][0], ph2[tb][1]};
        *(u32x2*)(s_p + pw_off + 1024 + 512 * tb) = u32x2{pl2[tb][0], pl2[tb][1]};
      }
      __syncthreads();                                     // every row's weights are in
      restart = __builtin_amdgcn_readfirstlane(s_restart);
      if (restart) break;

      // ---- O^T[wave's 128 dims, 64 rows] += C^T (P_hi + P_lo)^T
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 bp[2][2];                                   // [rb][hl]
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
            bp[rb][hl] = *(const bf16x8*)(s_p + 1024 * ((rb * 2 + ks) * 2 + hl) + 16 * lane);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint8_t* va = slot + (pv_row + 2 * ks) * LROW + pv_col + 64 * db;
          const u32x2 c0 = x2_tr16(va), c1 = x2_tr16(va + LROW);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{c0[0], c0[1], c1[0], c1[1]});
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            o[2 * db + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bp[rb][0], o[2 * db + rb], 0, 0, 0);
            o[2 * db + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bp[rb][1], o[2 * db + rb], 0, 0, 0);
          }
        }
      }
    }
    if (!restart) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load of this attempt in flight
    __syncthreads();                                   // everyone has read the flag and the ring
    if (tid == 0) s_restart = 0;
    m_ref = m_seen;                                    // row-uniform: the tile maxima are
    __syncthreads();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- normalise and write (the final output, or this split's fp32 partial)
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  const float lse = (l_tot > 0.f) ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : kNegInf;
  if (g == 0) s_inv[16 * wave + j] = inv;
  __syncthreads();
  const int h = lane >> 5, l32 = lane & 31;
  float* dst_base;
  size_t rstride;                                          // floats between rows
  if (ns == 1) {
    dst_base = a.out_latent + ((size_t)b * rows + row0) * DC;
    rstride = DC;
    if (g == 0) a.out_lse[(size_t)b * rows + qrow] = lse;
  } else {
    dst_base = (float*)((uint8_t*)a.part_o + ((size_t)item_id * rows + row0) * a.part_row_bytes);
    rstride = a.part_row_bytes / 4;
    if (g == 0) a.part_lse[(size_t)item_id * rows + qrow] = lse;
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float w = s_inv[32 * rb + l32];
    float* drow = dst_base + (size_t)(32 * rb + l32) * rstride + 128 * wave + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const floatx16& ob = o[2 * db + rb];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(floatx4*)(drow + 32 * db + 8 * q) =
            floatx4{ob[4 * q], ob[4 * q + 1], ob[4 * q + 2], ob[4 * q + 3]} * w;
    }
  }
}

hipError_t launch_decode_x2(const DecodeArgs& a, const ItemTable& tab, int row_blocks,
                            hipStream_t st) {
  const int grid = a.n_items * row_blocks;
  hipLaunchKernelGGL(decode_x2_kernel, dim3(grid), dim3(256), 0, st, a, tab, row_blocks);
  return hipGetLastError();
}

}  // namespace mla
