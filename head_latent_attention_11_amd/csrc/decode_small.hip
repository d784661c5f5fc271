// Attention over the latent cache on gfx950 matrix cores for small blocks of
// query rows: 16 or 32 rows per workgroup.  This covers head counts that
// are a multiple of 16 but give no multiple of 128 rows per sequence, e.g.
// the 16 heads of DeepSeek-V2-Lite ("DeepSeek-V2: Strong, Economical,
// Efficient", Appendix B) with one to four query tokens.
//
// Same contractions as the 128-row kernel (absorbed MLA decode, section
// 2.1.2 and Appendix C of the DeepSeek-V2 paper): per sequence
//   S^T = K Q_abs^T   (tokens x rows, K-dim 576)
//   O^T = C^T P^T     (512 x rows,    K-dim tokens)
// With 16 rows a cache row of 1152 bytes carries only ~35 kFLOP of work, so
// the kernel is bound by streaming the cache, not by the matrix cores; the
// design keeps three tiles in flight per workgroup and splits the matrix
// work of a tile over the four waves without duplicating any of it.
//
// Work decomposition
//   * A work item is (sequence b, KV chunk) x one block of RB = 16 NR query
//     rows (row = tau * n_h + head); a workgroup of 4 waves handles it.  Row
//     blocks of one item run on the same XCD (they share its L2 copy).
//   * KV tiles of 32 tokens move HBM -> LDS with buffer loads that write LDS
//     directly, through a 4-slot ring (rows padded to 1168 bytes); three
//     tiles stream in while one is used.  A load range that ends at the last
//     staged token writes zeros for the rest of the tile.  An fp8 tile's raw
//     rows land in the upper part of the slot with the 32 token scales
//     behind them, and are decoded in place to bf16 rows (exact: every E4M3
//     value is a bf16 value) once the tile is there; the scales multiply the
//     scores and the PV weights.  The query block is staged the same way
//     (into the last slot) before the loop and kept in VGPRs.
//   * Scores (v_mfma_f32_16x16x32_bf16; A = 16 tokens x 32 dims of K, B =
//     32 dims x 16 rows of Q^T): wave w takes token block tb = w % 2 and
//       NR = 1: the 16 rows over dims 288 (w / 2) .. +287 (the two halves
//               are added when the pieces are gathered),
//       NR = 2: row sub-block w / 2 over all 576 dims.
//     (64 rows run as two blocks of 32: holding four sub-blocks' queries
//     leaves too few registers to keep the operand reads ahead.)
//     The 16 x 16 pieces go through a small LDS buffer so that every wave
//     then holds all scores of the tile: lane (g, j) = (lane / 16, lane %
//     16) holds row j's scores of tokens tok_row(tb, 4 g + i), i = 0..3,
//     for both token blocks.
//   * Softmax per row in the log2 domain against a reference m_ref (the
//     first max the row sees, raised only when a later max exceeds it by
//     more than 8, with an exact rescaling of the row's accumulators and
//     sum).  Every wave computes the same weights.
//   * PV: wave w owns latent dims 128 w .. 128 w + 127 of all rows:
//     O^T[dim, row] += C^T[dim, tok] P^T[tok, row] (v_mfma_f32_16x16x32_bf16).
//     The B operand is the lane's own 8 weights (row j, the 8 tokens above:
//     the token order inside the K dimension is chosen to match), the A
//     operand comes from two transposing LDS reads (ds_read_b64_tr_b16:
//     within 16 lanes, lane i gets dim i of the four token rows addressed by
//     lanes 4k + i/4).  The accumulator lane (g, j) holds dims 4 g .. 4 g + 3
//     of row j, so each row's rescaling factor is the lane's own.
//   * Token order of a tile: MFMA row m of token block tb reads tile row
//     tok_row(tb, m) = 16 tb + 2 (m % 8) + m / 8.  The score-operand reads
//     of 16 lanes (16 rows 16 tb .. 16 tb + 15) and the transposing reads of
//     a half wave (eight rows of one parity, 32 bytes each) then fall on
//     distinct LDS banks at the 1168-byte pitch.
#include <math.h>

#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));

constexpr int kDim = 576;                  // cache row: 512 latent + 64 rope dims
constexpr int kLatent = 512;
constexpr int kRowBytes = 2 * kDim;        // bf16 cache row
constexpr int kTile = 32;                  // tokens per tile
constexpr int kPitch = 1168;               // LDS bytes per staged row (73 chunks of 16)
constexpr int kSlots = 4;                  // LDS ring
constexpr int kLoads = 37;                 // 1 KB direct loads per tile
constexpr int kSlotBytes = kLoads * 1024;
constexpr int kChunks = kRowBytes / 16;    // 72 chunks of 16 bytes per row
constexpr uint32_t kPastEnd = 0x40000000u; // buffer offset past any valid range
// fp8 cache: a tile's raw rows (32 x 576 codes, contiguous) land at kRawOff
// of its slot and are decoded in place into the bf16 row layout; its 32
// token scales land at kScaleOff, past the decoded rows.
constexpr int kRawOff = 18944;
constexpr int kScaleOff = kTile * kPitch;  // 37376
constexpr int kRawLoads = kTile * kDim / 1024;   // 18 loads of 1 KB
static_assert(kRawOff + kTile * kDim == kScaleOff, "raw rows end where the scales start");
static_assert(kScaleOff + 256 <= kSlotBytes, "the scale load writes 64 x 4 bytes");

// LDS chunk u of a slot holds chunk u % 73 of staged row u / 73, or nothing
// (the row's padding chunk, or past the 32 rows): then the source offset
// lies past the buffer's range and the load writes zeros.
// u / 73 = (449 u) >> 15 for u < 2368.
__device__ inline uint32_t staged_src_offset(int u) {
  const int r = (u * 449) >> 15;
  return (u - 73 * r == kChunks || r >= kTile) ? kPastEnd : uint32_t(16 * (u - r));
}

__device__ __forceinline__ int tok_row(int tb, int m) { return 16 * tb + 2 * (m & 7) + (m >> 3); }

// One 1 KB load (64 lanes x 16 bytes) from the buffer rs into LDS at lds.
__device__ __forceinline__ void dma_1k(uint32_t lds, uint32_t voff, u32x4 rs) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory");
}

// Wait until at most n of this wave's loads are in flight (n wave-uniform;
// counts that do not occur wait for all).
__device__ __forceinline__ void wait_loads(int n) {
  switch (n) {
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t ad = (uint64_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32)) & 0xFFFFu,
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

__device__ __forceinline__ shortx4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((shortx4 __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 E4M3 codes -> 8 bf16 values (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true));
  return r;
}

// x[l ^ 16] and x[l ^ 32] in lane l, without LDS.  v_permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second (v_permlane32_swap: the upper half with the lower half); with x
// in both, one operand comes back holding x[l] and the other x[l ^ 16] (or
// x[l ^ 32]), in an order that depends on the lane.  Written as assembly:
// the compiler's builtins take the two results as equal when the two inputs
// are, which they are not.
__device__ __forceinline__ void swap16(float& lo, float& hi) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ void swap32(float& lo, float& hi) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
}
// max / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// that hold one row's tokens)
__device__ __forceinline__ float group_max4(float x) {
  float lo = x, hi = x;
  swap16(lo, hi);
  x = fmaxf(lo, hi);
  lo = x; hi = x;
  swap32(lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float group_sum4(float x) {
  float lo = x, hi = x;
  swap16(lo, hi);
  x = lo + hi;
  lo = x; hi = x;
  swap32(lo, hi);
  return lo + hi;
}

}  // namespace

template <int NR, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_small_kernel(DecodeArgs a, ItemTable tab) {
  constexpr int RB = 16 * NR;                    // query rows per workgroup
  constexpr int KS = NR == 1 ? 9 : 18;           // 32-dim steps of a wave's scores
  static_assert(NR == 1 || NR == 2, "16 or 32 rows");
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kSlots][kSlotBytes];
  __shared__ __attribute__((aligned(16))) floatx4 s_x[4][64];   // score pieces

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int gi = xcd_logical_index(blockIdx.x, gridDim.x);
  const int item = gi / a.row_blocks, rb = gi % a.row_blocks;
  // work item -> (sequence, split, length), as for the 128-row kernel
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
  const int ns = splits_of(L, a.num_splits, a.chunk);
  const int c = chunk_of(L, a.num_splits, a.chunk);
  const int t0 = __builtin_amdgcn_readfirstlane(s_idx) * c;
  const int t_end = min(L, t0 + c);
  const int rows = a.n_h * a.T;
  const int row0 = rb * RB;
  // last visible token of each 16-row sub-block (its rows share one query
  // token: n_h is a multiple of 16)
  int lim[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr)
    lim[nr] = __builtin_amdgcn_readfirstlane(min(t_end - 1, L - a.T + (row0 + 16 * nr) / a.n_h));
  const int tau_max = (row0 + RB - 1) / a.n_h;
  const int t_stage = __builtin_amdgcn_readfirstlane(min(t_end, L - a.T + tau_max + 1));
  const int ntiles = (t_stage > t0) ? (t_stage - t0 + kTile - 1) / kTile : 0;

  const uint8_t* cache = (const uint8_t*)a.cache;
  const int seq_row0 = b * a.max_len;
  typedef __attribute__((address_space(4))) const int32_t* ConstI32;
  const ConstI32 ptab = a.page_table ? (ConstI32)(a.page_table + (size_t)b * a.max_pages) : nullptr;
  // Paged cache: the item's page ids (up to 128) are loaded once, one per
  // lane, and each tile takes its page from a lane with v_readlane; longer
  // items read the table per tile.  Items start on a page boundary.
  const int pg_first = t0 / kPage;
  const int pg_n = (ntiles > 0) ? (t_stage - t0 + kPage - 1) / kPage : 0;
  const bool pg_regs = ptab && pg_n <= 128;
  int pg_lo = 0, pg_hi = 0;
  if (pg_regs) {
    if (lane < pg_n) pg_lo = a.page_table[(size_t)b * a.max_pages + pg_first + lane];
    if (64 + lane < pg_n) pg_hi = a.page_table[(size_t)b * a.max_pages + pg_first + 64 + lane];
  }
  // buffer of the tile starting at token ts (a tile never crosses a page)
  constexpr int ROWB = FP8 ? kDim : kRowBytes;    // bytes per cache row
  // first cache row of the tile starting at token ts, and its valid rows
  auto tile_row0 = [&](int ts, int& nv) -> int {
    nv = max(0, min(kTile, t_stage - ts));
    int r0 = 0;
    if (nv > 0) {
      if (ptab) {
        const int k = ts / kPage - pg_first;
        const int pg = pg_regs ? __builtin_amdgcn_readlane(k < 64 ? pg_lo : pg_hi, k & 63)
                               : ptab[ts / kPage];
        r0 = pg * kPage + (ts % kPage);
      } else {
        r0 = seq_row0 + ts;
      }
    }
    return __builtin_amdgcn_readfirstlane(r0);
  };
  // bf16 rows (and the query block): wave w issues loads n = w + 4k of the
  // 37 that fill a slot (wave 0: 10 loads, others 9).  fp8: wave w issues
  // raw loads n = w + 4k of 18, wave 3 also the scales (waves 0, 1 and 3:
  // 5 loads, wave 2: 4).
  const int nld_q = wave == 0 ? 10 : 9;
  const int nld = FP8 ? (wave == 2 ? 4 : 5) : nld_q;
  uint32_t voff[10];
#pragma unroll
  for (int n = 0; n < 10; ++n) voff[n] = staged_src_offset(64 * (wave + 4 * n) + lane);
  const uint32_t ring = (uint32_t)(uintptr_t)&s_ring[0][0];
  auto issue = [&](const u32x4 rs, int slot) {
    const uint32_t lb = ring + slot * kSlotBytes + 1024 * wave;
#pragma unroll
    for (int n = 0; n < 9; ++n) dma_1k(lb + 4096 * n, voff[n], rs);
    if (wave == 0) dma_1k(lb + 4096 * 9, voff[9], rs);
  };
  auto issue_tile = [&](int ts, int slot) {
    int nv;
    const int r0 = tile_row0(ts, nv);
    if constexpr (!FP8) {
      issue(buffer_rsrc(cache + (size_t)r0 * kRowBytes, nv * kRowBytes), slot);
    } else {
      const u32x4 rs = buffer_rsrc(cache + (size_t)r0 * kDim, nv * kDim);
      const uint32_t lb = ring + slot * kSlotBytes + kRawOff;
#pragma unroll
      for (int k = 0; k < (kRawLoads + 3) / 4; ++k)
        if (wave + 4 * k < kRawLoads)
          dma_1k(lb + 1024 * (wave + 4 * k), uint32_t(1024 * (wave + 4 * k) + 16 * lane), rs);
      if (wave == 3) {
        const u32x4 ss = buffer_rsrc(a.kv_scale + r0, nv * 4);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :: "s"(ring + slot * kSlotBytes + kScaleOff),
                        "v"(uint32_t(lane < kTile ? 4 * lane : kPastEnd)), "s"(ss) : "memory");
      }
    }
  };

  // ---- query block -> VGPRs (B operands of the scores: lane (g, j) holds
  // row 16 nq + j, dims 32 ks + 8 g .. + 7).  The block's rows are staged
  // in the last ring slot; tiles 0, 1 and 2 go out right behind them.
  const uint8_t* qblk = (const uint8_t*)a.q_abs + ((size_t)b * rows + row0) * kRowBytes;
  issue(buffer_rsrc(qblk, RB * kRowBytes), kSlots - 1);
#pragma unroll
  for (int t = 0; t < kSlots - 1; ++t)
    if (t < ntiles) issue_tile(t0 + t * kTile, t);
  wait_loads(min(ntiles, kSlots - 1) * nld);     // the query loads have landed
  __syncthreads();
  const int tb = wave & 1;                       // token block of this wave's scores
  const int ks0 = NR == 1 ? 9 * (wave >> 1) : 0; // first 32-dim step
  const int nq = NR == 1 ? 0 : wave >> 1;        // row sub-block
  bf16x8 qf[KS];
  {
    const uint8_t* src = s_ring[kSlots - 1] + (16 * nq + j) * kPitch + 64 * ks0 + 16 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(src + 64 * ks);
  }

  // ---- per-lane LDS offsets of the operands
  const int k_off = tok_row(tb, j) * kPitch + 64 * ks0 + 16 * g;               // + 64 ks
  const int kq = (lane >> 2) & 3, m4 = lane & 3;
  const int v_off0 = tok_row(0, 4 * g + kq) * kPitch + 256 * wave + 8 * m4;     // + 32 cb
  const int v_off1 = tok_row(1, 4 * g + kq) * kPitch + 256 * wave + 8 * m4;

  floatx4 o[NR][8];
  float m_ref[NR], l_run[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    m_ref[nr] = -INFINITY;
    l_run[nr] = 0.f;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) o[nr][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  for (int it = 0; it < ntiles; ++it) {
    // tile it has landed (tiles it+1, it+2 may still be in flight), and
    // every wave is done with tile it-1 and with the score pieces
    wait_loads((min(ntiles, it + kSlots - 1) - it - 1) * nld);
    __syncthreads();
    if (it + kSlots - 1 < ntiles) issue_tile(t0 + (it + kSlots - 1) * kTile, (it + kSlots - 1) & 3);
    const uint8_t* kt = s_ring[it & 3];
    if constexpr (FP8) {
      // decode the raw tile in place: every thread reads its 9 chunks of 8
      // codes, then (after a barrier) writes them as bf16 rows
      u32x2 raw[kTile * kDim / 8 / 256];
#pragma unroll
      for (int i = 0; i < kTile * kDim / 8 / 256; ++i)
        raw[i] = *(const u32x2*)(kt + kRawOff + 8 * (tid + 256 * i));
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kTile * kDim / 8 / 256; ++i) {
        const int ci = tid + 256 * i;             // row ci / 72, codes 8 (ci % 72) ..
        *(u32x4*)(s_ring[it & 3] + 16 * ci + 16 * (ci / kChunks)) = e4m3x8_to_bf16x8(raw[i]);
      }
      __syncthreads();
    }

    // scores: this wave's piece.  All operand reads go out first (one LDS
    // latency per tile), then the products, in two chains.
    {
      bf16x8 kv[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[ks] = *(const bf16x8*)(kt + k_off + 64 * ks);
      floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[ks], qf[ks], s0, 0, 0, 0);
        if (ks + 1 < KS) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[ks + 1], qf[ks + 1], s1, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);   // the LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);   // then the products
      s_x[wave][lane] = s0 + s1;
    }
    __syncthreads();

    const int ts = t0 + it * kTile;
    // fp8: this lane's 8 token scales (scores and weights are multiplied by
    // them, so the codes enter the matrix products exactly)
    float sc[8];
    if constexpr (FP8) {
      const float* sp = (const float*)(kt + kScaleOff);
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = sp[tok_row(e >> 2, 4 * g + (e & 3))];
    }
    bf16x8 pk[NR];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      float x[8];                                // raw scores of row j
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const floatx4 v = NR == 1 ? s_x[t][lane] + s_x[t + 2][lane] : s_x[t + 2 * nr][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * t + i] = v[i];
      }
      if constexpr (FP8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= sc[e];
      }
      if (ts + kTile - 1 > lim[nr]) {            // the tile crosses the visibility limit
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (ts + tok_row(e >> 2, 4 * g + (e & 3)) > lim[nr]) x[e] = -INFINITY;
      }
      float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mt = group_max4(mt) * a.scale_log2;                        // the row's max over the tile (log2 domain)
      // The weights are taken against a reference m_ref that only moves
      // when the max exceeds it by more than 8 (weights up to 2^8): the
      // accumulators are rescaled rarely, and exactly.
      const bool raise = m_ref[nr] != -INFINITY && mt > m_ref[nr] + 8.0f;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? exp2_hw(m_ref[nr] - mt) : 1.0f;
        l_run[nr] *= alpha;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o[nr][cb] *= alpha;
      }
      if (raise || m_ref[nr] == -INFINITY) m_ref[nr] = mt;
      const float neg = (m_ref[nr] == -INFINITY) ? 0.f : -m_ref[nr];
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = exp2_hw(fmaf(x[e], a.scale_log2, neg));
      // the normaliser sums the weights as rounded to bf16 (unscaled), the
      // weights that enter the product (times the token scale for fp8)
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = (float)(__bf16)p[e];
      l_run[nr] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[nr][e] = (__bf16)(FP8 ? p[e] * sc[e] : pr[e]);
    }

    // PV: this wave's 128 latent dims of every row (reads first, then the
    // products)
    {
      shortx4 v0[8], v1[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        v0[cb] = lds_tr16(kt + v_off0 + 32 * cb);
        v1[cb] = lds_tr16(kt + v_off1 + 32 * cb);
      }
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0[cb], v1[cb], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nr = 0; nr < NR; ++nr)
          o[nr][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pk[nr], o[nr][cb], 0, 0, 0);
      }
    }
  }

  // ---- normalise and write: lane (g, j) holds dims 128 w + 16 cb + 4 g ..
  // + 3 of row 16 nr + j.  The final output in fp32, or this split's
  // partial in bf16 (combined in fp32).
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const float l_tot = group_sum4(l_run[nr]);
    const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    const float lse = (l_tot > 0.f) ? (m_ref[nr] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    const int row = row0 + 16 * nr + j;
    if (ns == 1) {
      const size_t gr = (size_t)b * rows + row;
      float* dst = a.out_latent + gr * kLatent + 128 * wave + 4 * g;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) *(floatx4*)(dst + 16 * cb) = o[nr][cb] * inv;
      if (wave == 0 && g == 0) a.out_lse[gr] = lse;
    } else {
      const size_t pr = (size_t)item_id * rows + row;
      uint8_t* dst = (uint8_t*)a.part_o + pr * a.part_row_bytes + (128 * wave + 4 * g) * 2;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const floatx4 v = o[nr][cb] * inv;
        const bf16x2 p01 = {(__bf16)v[0], (__bf16)v[1]};
        const bf16x2 p23 = {(__bf16)v[2], (__bf16)v[3]};
        *(u32x2*)(dst + 32 * cb) = u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
      }
      if (wave == 0 && g == 0) a.part_lse[pr] = lse;
    }
  }
}

// rows_wg: query rows per workgroup (16 or 32); a.row_blocks counts blocks
// of that many rows.
hipError_t launch_decode_small(const DecodeArgs& a, const ItemTable& tab, int rows_wg,
                               hipStream_t st) {
  const int grid = a.n_items * a.row_blocks;
  const bool fp8 = a.kv_dtype == MLA_FP8_E4M3;
  if (rows_wg == 16 && !fp8)
    hipLaunchKernelGGL((decode_small_kernel<1, false>), dim3(grid), dim3(256), 0, st, a, tab);
  else if (rows_wg == 16)
    hipLaunchKernelGGL((decode_small_kernel<1, true>), dim3(grid), dim3(256), 0, st, a, tab);
  else if (rows_wg == 32 && !fp8)
    hipLaunchKernelGGL((decode_small_kernel<2, false>), dim3(grid), dim3(256), 0, st, a, tab);
  else if (rows_wg == 32)
    hipLaunchKernelGGL((decode_small_kernel<2, true>), dim3(grid), dim3(256), 0, st, a, tab);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
