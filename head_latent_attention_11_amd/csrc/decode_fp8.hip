// Attention over an fp8 latent cache on gfx950 matrix cores.
//
// Absorbed MLA decode ("DeepSeek-V2: Strong, Economical, Efficient",
// section 2.1.2 and Appendix C; attention-output equation of the
// "DeepSeek-V3 Technical Report" notes, MLA section) over cache rows stored
// as 576 E4M3 codes with one fp32 scale per token (the cache format of
// mla_cache_append): per sequence the step is two dense contractions with
// the query rows as one matrix dimension,
//   S = Q_abs K^T   (rows x tokens, K-dim 576)
//   O = P C         (rows x 512,    K-dim tokens)
// with each token's scale applied to its scores and to its PV weights, so
// the codes enter the bf16 MFMA unscaled.
//
// Work decomposition (as in the bf16 kernel, decode_mfma.hip)
//   * One workgroup of 4 waves per (work item, 128 query rows); row blocks
//     of an item share an XCD (its L2).  For the scores wave w owns rows
//     32w .. 32w+31 (their absorbed queries stay in VGPRs); for the PV
//     product it owns latent dims 128w .. 128w+127 of all 128 rows (O^T in
//     the 256 accumulation registers).
//
// What differs from the bf16 kernel
//   * Tiles of 32 tokens stay raw in LDS (rows of 576 codes at a pitch of
//     592 bytes, copied HBM -> LDS by buffer loads that write LDS directly)
//     and the MFMA operands are converted in registers with
//     v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value is a bf16 value):
//     no decode pass through LDS, and the score operand reads move half the
//     bytes of bf16 tiles.
//       - Scores: lane l reads 16 codes of token row tile_row(l%32) at dims
//         32kk + 16(l/32) and converts them into the A operands of two
//         MFMAs (dims {32kk + 0..7, 32kk + 16..23} and the other eight);
//         the query fragments follow the same dim order.  At the 592-byte
//         pitch a token row starts 20t mod 64 banks further, so the 16 rows
//         of distinct residues mod 16 that 16 lanes read fill all 64 banks.
//       - PV: ds_read_b64_tr_b8 gives each lane one latent dim of 8 tokens
//         (C^T fragment); the 8 token rows of a 16-lane group are 2 apart
//         in tile_row order, i.e. 40 banks apart, which keeps the groups'
//         16-byte pieces in distinct banks.
//   * The 32 token scales of a tile are loaded straight into score-register
//     order (each lane of the scale load fetches the scale its LDS word
//     holds), and each lane reads its 16 with four 16-byte reads.
//   * A 7-slot ring: tile it+5 is loaded during step it, the softmax
//     weights are double-buffered, and each step ends with one barrier.
//     Step it: scores of tile it (slot it%7), then the PV product of tile
//     it-1 (slot (it-1)%7, weights buffer (it-1)%2) with the softmax of tile
//     it interleaved, weights of tile it into buffer it%2; wait for this
//     wave's loads of tile it+1; barrier.  The loads of tile it+5 go to the
//     slot of tile it-2, whose last reader (PV in step it-1) every wave has
//     finished at the barrier that ended step it-1.
//   * Steps whose tile has no masked token, after the first, run the scores
//     and the PV product with the softmax as one inline-assembly sequence:
//     the PV product's first operand reads go out under the last score
//     MFMAs.  Step 0 and the masked tail keep two sequences with the masking
//     and reference code between them; the three parts run one after
//     another (no branch around a block that writes O).
//   * Softmax against a fixed per-row reference with rare restarts, as in
//     the bf16 kernel (exact for any reference: LSE = m_ref + log2 sum p).
#include <math.h>

#include <type_traits>

#include "decode_tile.hpp"
#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

namespace {
constexpr int DC = 512, D = 576;
constexpr int ROWS_WG = 128;              // query rows per workgroup
constexpr int TILE = 32;                  // tokens per tile
constexpr int LROW = 592;                 // LDS bytes per token row (576 codes + 16 pad)
constexpr int GRAN = LROW / 16;           // 16-byte granules per LDS row (37)
constexpr int NLD = (TILE * GRAN + 63) / 64;   // loads of 64 x 16 B per tile (19)
constexpr int SCL = NLD * 1024;           // token scales of the tile (score order)
constexpr int SLOT = SCL + 256;           // the scale load writes 64 x 4 bytes
constexpr int NB = 7;                     // ring slots
constexpr int AHEAD = NB - 2;             // tile it + AHEAD is loaded in step it
constexpr int LPT = 5;                    // loads per wave per tile
constexpr int PBUF = NB * SLOT;           // two weight buffers of 8 KB after the ring
constexpr int KVW = PBUF + 2 * 8192;      // per wave: the token scales of a masked tile
constexpr int LDS_BYTES = KVW + 4 * 128;
constexpr int QROW = 592;                 // LDS bytes per staged half query row
constexpr int QLOADS = ROWS_WG * (QROW / 16) / 64;   // 1 KB loads per staged half (74)
constexpr int QSTAGE = 2 * SLOT;          // staged halves go to slots 2 .. 5
constexpr uint32_t kOOB = 0x40000000u;    // buffer offset past any valid range
constexpr float kNegInf = -INFINITY;

static_assert(4 * (NLD / 4) + 3 == NLD, "waves 0..2 issue 5 tile loads, wave 3 four + scales");
static_assert(QSTAGE + QLOADS * 1024 <= NB * SLOT, "staged query half fits the ring");
static_assert(KVW >= 4 * 64 * 528 && KVW >= 4 * 128 * 272, "epilogue staging");
static_assert(LDS_BYTES + 4 * ROWS_WG + 16 <= 160 * 1024, "LDS");
}  // namespace

// Software-pipelined bodies of the tile steps (gen_decode_asm.py).
#include "decode_mfma_asm.inc"

// LDS granule u of a tile's slot holds granule u % 37 of token row u / 37;
// the row's padding granule and granules past the 32 rows get an
// out-of-range offset (the load writes zeros there).
__device__ inline uint32_t fp8_tile_offset(int u) {
  const int t = u / GRAN, c = u - GRAN * t;
  return (c == GRAN - 1 || t >= TILE) ? kOOB : uint32_t(D * t + 16 * c);
}

// Staged query halves: 16-byte unit u holds row u / 37, unit u % 37 of the
// half (unit 36 is the row padding).  Rows are q_row_bytes apart (a
// constant at the call, so the offsets fold).
__device__ inline uint32_t fp8_q_offset(int u, int half, int q_row_bytes) {
  const int r = u / (QROW / 16), c = u - (QROW / 16) * r;
  return c == QROW / 16 - 1 ? kOOB : uint32_t(r * q_row_bytes + half * D + 16 * c);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_fp8_kernel(DecodeArgs a, ItemTable tab) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[LDS_BYTES];
  __shared__ float s_inv[ROWS_WG];
  __shared__ int s_restart;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31, g = lane >> 4, j = lane & 15;
  const int gi = xcd_logical_index(blockIdx.x, gridDim.x);
  const int item = gi / a.row_blocks, rb = gi % a.row_blocks;
  // work item -> (sequence, split, length), as in the bf16 kernel
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
  const int row = rb * ROWS_WG + wave * 32 + l32;
  const int tau = row / a.n_h;
  // last visible token; the 32 rows of a wave share tau (n_h % 32 == 0)
  const int lim = __builtin_amdgcn_readfirstlane(min(t_end - 1, L - a.T + tau));
  const int tau_max = (rb * ROWS_WG + ROWS_WG - 1) / a.n_h;
  const int t_stage = __builtin_amdgcn_readfirstlane(min(t_end, L - a.T + tau_max + 1));
  const int ntiles = (t_stage > t0) ? (t_stage - t0 + TILE - 1) / TILE : 0;

  const uint32_t lds0 = (uint32_t)(uintptr_t)&s_lds[0];
  const uint8_t* cache = (const uint8_t*)a.cache;
  const int seq_row0 = b * a.max_len;
  typedef __attribute__((address_space(4))) const int32_t* ConstI32;
  const ConstI32 ptab = a.page_table ? (ConstI32)(a.page_table + (size_t)b * a.max_pages) : nullptr;
  // paged cache: up to 128 page ids of the item in two registers, one per
  // lane, read back with v_readlane (longer items read the table per tile)
  const int pg_first = t0 / kPage;
  const int pg_n = (t_stage > t0) ? (t_stage - t0 + kPage - 1) / kPage : 0;
  const bool pg_regs = ptab && pg_n <= 128;
  int pg_lo = 0, pg_hi = 0;
  if (pg_regs) {
    if (lane < pg_n) pg_lo = a.page_table[(size_t)b * a.max_pages + pg_first + lane];
    if (64 + lane < pg_n) pg_hi = a.page_table[(size_t)b * a.max_pages + pg_first + 64 + lane];
    // wait for them here, before the query and tile loads: the compiler
    // does not count the assembly loads and would otherwise wait for all of
    // them (vmcnt(0)) at the first use of a page id
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }
#define MLA_PAGE(ts_)                                                                      \
  (pg_regs ? __builtin_amdgcn_readlane(((ts_) / kPage - pg_first) < 64 ? pg_lo : pg_hi,   \
                                       ((ts_) / kPage - pg_first) & 63)                  \
           : ptab[(ts_) / kPage])

  // Buffer descriptors of the tile starting at token ts (codes and scales):
  // the range ends at the tile's last valid token, so later tokens read as
  // zeros.  A tile never crosses a page (pages hold 64 tokens).
#define MLA_TILE_RSRC(ts_, rs_, rss_)                                                      \
  u32x4 rs_, rss_;                                                                       \
  {                                                                                      \
    const int ts__ = (ts_);                                                              \
    const int nv__ = max(0, min(TILE, t_stage - ts__));                                  \
    int r0__ = 0;                                                                        \
    if (nv__ > 0)                                                                        \
      r0__ = ptab ? MLA_PAGE(ts__) * kPage + (ts__ % kPage) : seq_row0 + ts__;          \
    r0__ = __builtin_amdgcn_readfirstlane(r0__);                                         \
    const uint64_t ad__ = (uint64_t)(cache + (size_t)r0__ * D);                          \
    rs_ = u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad__),                \
                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad__ >> 32)) & 0xFFFFu, \
                (uint32_t)__builtin_amdgcn_readfirstlane(nv__ * D), 0x00020000u};        \
    const uint64_t sa__ = (uint64_t)(a.kv_scale + r0__);                                 \
    rss_ = u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sa__),               \
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sa__ >> 32)) & 0xFFFFu, \
                 (uint32_t)__builtin_amdgcn_readfirstlane(nv__ * 4), 0x00020000u};       \
  }

  // Load n = wave + 4k (k = 0..4) of a tile fills LDS granules 64n .. 64n+63
  // of its slot; wave 3's fifth load is the tile's 32 token scales, lane i <
  // 32 fetching the scale of token reg_token(i % 16, i / 16).
  uint32_t voff[LPT];
#pragma unroll
  for (int k = 0; k < LPT; ++k) voff[k] = fp8_tile_offset(64 * (wave + 4 * k) + lane);
  if (wave == 3) voff[LPT - 1] = lane < TILE ? uint32_t(4 * reg_token(lane & 15, lane >> 4)) : kOOB;

  // the fifth load of a tile (the four others are issued by the score
  // sequence of a step, or by MLA_ISSUE_TILE)
#define MLA_ISSUE_FIFTH(slot_, rs_, rss_)                                                  \
  do {                                                                                   \
    if (wave < 3)                                                                        \
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"          \
                   :: "s"(lds0 + (slot_) * SLOT + 1024 * (wave + 4 * (LPT - 1))),       \
                      "v"(voff[LPT - 1]), "s"(rs_) : "memory");                          \
    else                                                                                 \
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"            \
                   :: "s"(lds0 + (slot_) * SLOT + SCL), "v"(voff[LPT - 1]), "s"(rss_)    \
                   : "memory");                                                          \
  } while (0)
#define MLA_ISSUE_TILE(ts_, slot_)                                                         \
  do {                                                                                   \
    MLA_TILE_RSRC(ts_, rs__, rss__);                                                     \
    _Pragma("unroll") for (int n__ = 0; n__ < LPT - 1; ++n__)                            \
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"          \
                   :: "s"(lds0 + (slot_) * SLOT + 1024 * (wave + 4 * n__)), "v"(voff[n__]), \
                      "s"(rs__) : "memory");                                             \
    MLA_ISSUE_FIFTH(slot_, rs__, rss__);                                                 \
  } while (0)

  // weight buffer 1 holds the weights of "tile -1" in step 0: zeros
#define MLA_ZERO_PBUF1()                                                                   \
  do {                                                                                   \
    *(u32x4*)(s_lds + PBUF + 8192 + 32 * tid) = u32x4{0u, 0u, 0u, 0u};                   \
    *(u32x4*)(s_lds + PBUF + 8192 + 32 * tid + 16) = u32x4{0u, 0u, 0u, 0u};              \
  } while (0)

  // ---- per-lane LDS offsets of the MFMA operands
  const int qk_off = tile_row(l32) * LROW + 16 * h;              // + 32 kk
  // transposed reads: lane j of 16-lane group g supplies 8 codes of token
  // row tile_row(8 (j/8) + 4 (g/2) + (j/2) % 4) at dims 128 w + 16 (g%2) +
  // 8 (j%2) (+ 16 rows per token half, + 32 dims per dim block); lane i of
  // the group receives dim 16 (g%2) + i of those 8 tokens
  const int pv_off = tile_row(8 * (j >> 3) + 4 * (g >> 1) + ((j >> 1) & 3)) * LROW +
                     128 * wave + 16 * (g & 1) + 8 * (j & 1);

  // ---- absorbed query rows -> MFMA B operands.  Fragment 2kk + e of lane
  // l: row 32 w + l%32, dims 32kk + 16 (l/32) + 8e .. +7.  The workgroup's
  // 128 rows are contiguous in memory; they are staged in two halves of 288
  // dims through ring slots 2..5 while tiles 0 and 1 load into slots 0, 1.
  bf16x8 qf[D / 16];
  const uint64_t qa = (uint64_t)((const uint8_t*)a.q_abs +
                                 ((size_t)b * rows + rb * ROWS_WG) * (2 * D));
  const u32x4 qrs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)qa),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(qa >> 32)) & 0xFFFFu,
                     uint32_t(ROWS_WG * (2 * D)), 0x00020000u};
#define MLA_Q_ISSUE(p_)                                                                    \
  do {                                                                                   \
    _Pragma("unroll") for (int n__ = 0; n__ < (QLOADS + 3) / 4; ++n__)                   \
      if (wave + 4 * n__ < QLOADS)                                                       \
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"        \
                     :: "s"(lds0 + QSTAGE + 1024 * (wave + 4 * n__)),                    \
                        "v"(fp8_q_offset(64 * (wave + 4 * n__) + lane, (p_), (2 * D))), \
                        "s"(qrs)                                                         \
                     : "memory");                                                        \
  } while (0)
#define MLA_Q_READ(p_)                                                                     \
  do {                                                                                   \
    const uint8_t* qsrc__ = s_lds + QSTAGE + (32 * wave + l32) * QROW + 32 * h;          \
    _Pragma("unroll") for (int n__ = 0; n__ < D / 64; ++n__) {                           \
      qf[(D / 32) * (p_) + 2 * n__] = *(const bf16x8*)(qsrc__ + 64 * n__);               \
      qf[(D / 32) * (p_) + 2 * n__ + 1] = *(const bf16x8*)(qsrc__ + 64 * n__ + 16);      \
    }                                                                                    \
  } while (0)

  if (tid == 0) s_restart = 0;
  MLA_Q_ISSUE(0);
  MLA_ISSUE_TILE(t0, 0);
  MLA_ISSUE_TILE(t0 + TILE, 1);
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LPT) : "memory");   // query half 0 landed
  __syncthreads();
  MLA_Q_READ(0);
  __syncthreads();                    // every wave has read half 0
  MLA_Q_ISSUE(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                    // half 1 and tiles 0, 1 landed
  MLA_Q_READ(1);
#pragma unroll
  for (int k = 0; k < D / 16; ++k) asm volatile("" ::"v"(qf[k]));
  MLA_ZERO_PBUF1();
  __syncthreads();                    // every wave has read half 1: slots 2.. are free
#pragma unroll
  for (int k = 2; k < AHEAD; ++k) MLA_ISSUE_TILE(t0 + k * TILE, k);
#undef MLA_Q_ISSUE
#undef MLA_Q_READ

  floatx16 o[DC / 32];
  float m_ref = kNegInf, m_seen = kNegInf, l_run = 0.f;
  const uint32_t pr = lds0 + PBUF + 16 * lane;   // this lane's weight fragments (+ 8 KB per buffer)

#pragma unroll
  for (int i = 0; i < DC / 32; ++i) o[i] = floatx16{};

  // Steps 0 .. ntiles of a pass over the item: step it takes the scores of
  // tile it and the PV product of tile it-1; the extra step ntiles takes the
  // PV product of the last tile (its own tile lies past every row's limit:
  // all scores masked, its softmax adds exact zeros).  The PV sequence of
  // step 0 zeroes O.  With CHECK, a score more than 64 above the row's
  // reference ends the pass early (returns true).
  auto run_steps = [&](auto check) __attribute__((always_inline)) -> bool {
    constexpr bool CHECK = decltype(check)::value;
    int sc = 0;                       // slot of tile it
    // One step as two sequences, with the masking and reference code
    // between them: the first step and tiles that reach past the wave's
    // visibility limit.
    auto step_split = [&](int it) __attribute__((always_inline)) {
      const int ts = t0 + it * TILE;
      const int si = (sc + AHEAD >= NB) ? sc + AHEAD - NB : sc + AHEAD;   // tile it + AHEAD
      const int sp = (sc == 0) ? NB - 1 : sc - 1;                         // tile it - 1
      MLA_TILE_RSRC(ts + AHEAD * TILE, rs_n, rss_n);
      const uint32_t lb_n = __builtin_amdgcn_readfirstlane(lds0 + si * SLOT + 1024 * wave);
      floatx16 s_cur;
      {
        const uint32_t ad = lds0 + sc * SLOT + qk_off;
        asm volatile(MLA_ASM_QK8_TILE
                     : "=&v"(s_cur)
                     : "v"(ad), "v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]),
                       "v"(qf[5]), "v"(qf[6]), "v"(qf[7]), "v"(qf[8]), "v"(qf[9]),
                       "v"(qf[10]), "v"(qf[11]), "v"(qf[12]), "v"(qf[13]), "v"(qf[14]),
                       "v"(qf[15]), "v"(qf[16]), "v"(qf[17]), "v"(qf[18]), "v"(qf[19]),
                       "v"(qf[20]), "v"(qf[21]), "v"(qf[22]), "v"(qf[23]), "v"(qf[24]),
                       "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]), "v"(qf[29]),
                       "v"(qf[30]), "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]),
                       "v"(qf[35]), "s"(rs_n), "s"(lb_n), "v"(voff[0]), "v"(voff[1]),
                       "v"(voff[2]), "v"(voff[3])
                     : "memory", MLA_ASM_QK8_CLOBBERS);
      }
      MLA_ISSUE_FIFTH(si, rs_n, rss_n);
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = s_cur[r];
      // this lane's 16 token scales (score-register order)
      uint32_t kva = lds0 + sc * SLOT + SCL + 64 * h;
      if (__builtin_expect(ts + TILE - 1 > lim, 0)) {
        // The tile holds tokens past the wave's visibility limit (register r
        // holds token reg_token(r, h)): their scores become -inf and their
        // scales 1 (zero-filled tokens past the end have scale 0), in a copy
        // of the scales for this wave, so that their weights are exact zeros.
        const float* kvp = (const float*)(s_lds + sc * SLOT + SCL) + 16 * h;
        float kv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          kv[r] = kvp[r];
          if (ts + reg_token(r, h) > lim) {
            sv[r] = kNegInf;
            kv[r] = 1.f;
          }
        }
        float* kw = (float*)(s_lds + KVW + 128 * wave) + 16 * h;
        if (l32 == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(floatx4*)(kw + 4 * q) = floatx4{kv[4 * q], kv[4 * q + 1], kv[4 * q + 2], kv[4 * q + 3]};
        }
        kva = lds0 + KVW + 128 * wave + 64 * h;
      }
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(m_ref == kNegInf) != 0, 0)) {
        // the first tile in which the row sees a token sets the reference
        const float* kvp = (const float*)(s_lds + (kva - lds0));
        float sc16[16], mt, tmp0;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc16[r] = sv[r] * kvp[r];   // as in the sequence
        asm volatile(MLA_ASM_SOFTMAX_MAX
                     : "=&v"(mt), "=&v"(tmp0)
                     : "v"(sc16[0]), "v"(sc16[1]), "v"(sc16[2]), "v"(sc16[3]), "v"(sc16[4]),
                       "v"(sc16[5]), "v"(sc16[6]), "v"(sc16[7]), "v"(sc16[8]), "v"(sc16[9]),
                       "v"(sc16[10]), "v"(sc16[11]), "v"(sc16[12]), "v"(sc16[13]),
                       "v"(sc16[14]), "v"(sc16[15]), "v"(a.scale_log2));
        if (m_ref == kNegInf) m_ref = mt;   // O and l are still zero here
      }
      const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
      // The PV product of tile it-1 with the softmax of tile it interleaved
      // (step 0: O is zeroed first, then tile 0 times the zeroed weight
      // buffer 1 adds exact zeros); the sequence writes this wave's weights
      // of tile it into P buffer it%2.
      const uint32_t vb = lds0 + (it == 0 ? 0 : sp * SLOT) + pv_off;
      const uint32_t pb = pr + 8192 * ((it + 1) & 1);
      const uint32_t pw = pr + 8192 * (it & 1) + 2048 * wave;   // this lane's weights of tile it
      float tmp;
      asm volatile(MLA_ASM_PV8_SOFTMAX_TILE
                   : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]),
                     "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]),
                     "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                     "+a"(o[15]), "+v"(sv[0]), "+v"(sv[1]), "+v"(sv[2]), "+v"(sv[3]),
                     "+v"(sv[4]), "+v"(sv[5]), "+v"(sv[6]), "+v"(sv[7]), "+v"(sv[8]),
                     "+v"(sv[9]), "+v"(sv[10]), "+v"(sv[11]), "+v"(sv[12]), "+v"(sv[13]),
                     "+v"(sv[14]), "+v"(sv[15]), "=&v"(tmp), "+v"(l_run)
                   : "v"(vb), "v"(pb), "v"(kva), "v"(neg_m), "v"(a.scale_log2),
                     "s"(__builtin_amdgcn_readfirstlane(it == 0 ? 1 : 0)), "v"(pw)
                   : "memory", MLA_ASM_PV8_SOFTMAX_CLOBBERS);
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"((AHEAD - 1) * LPT) : "memory");   // tile it+1 landed
      __syncthreads();
      sc = (sc + 1 == NB) ? 0 : sc + 1;
    };
    // One step of a tile none of whose tokens is masked, after the first
    // (every row's reference is set): scores, PV product and softmax in one
    // sequence, so the PV operand reads go out under the last score MFMAs.
    auto step_fused = [&](int it) __attribute__((always_inline)) {
      const int ts = t0 + it * TILE;
      const int si = (sc + AHEAD >= NB) ? sc + AHEAD - NB : sc + AHEAD;   // tile it + AHEAD
      const int sp = (sc == 0) ? NB - 1 : sc - 1;                         // tile it - 1
      MLA_TILE_RSRC(ts + AHEAD * TILE, rs_n, rss_n);
      const uint32_t lb_n = __builtin_amdgcn_readfirstlane(lds0 + si * SLOT + 1024 * wave);
      const uint32_t ad = lds0 + sc * SLOT + qk_off;
      const uint32_t vb = lds0 + sp * SLOT + pv_off;
      const uint32_t pb = pr + 8192 * ((it + 1) & 1);
      const uint32_t pw = pr + 8192 * (it & 1) + 2048 * wave;
      const uint32_t kva = lds0 + sc * SLOT + SCL + 64 * h;
      const float neg_m = -m_ref;
      float tmp;
      asm volatile(MLA_ASM_STEP8_TILE
                   : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]),
                     "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]),
                     "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                     "+a"(o[15]), "+v"(l_run), "=&v"(tmp)
                   : "v"(ad), "v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]),
                     "v"(qf[5]), "v"(qf[6]), "v"(qf[7]), "v"(qf[8]), "v"(qf[9]),
                     "v"(qf[10]), "v"(qf[11]), "v"(qf[12]), "v"(qf[13]), "v"(qf[14]),
                     "v"(qf[15]), "v"(qf[16]), "v"(qf[17]), "v"(qf[18]), "v"(qf[19]),
                     "v"(qf[20]), "v"(qf[21]), "v"(qf[22]), "v"(qf[23]), "v"(qf[24]),
                     "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]), "v"(qf[29]),
                     "v"(qf[30]), "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]),
                     "v"(qf[35]), "s"(rs_n), "s"(lb_n), "v"(voff[0]), "v"(voff[1]),
                     "v"(voff[2]), "v"(voff[3]), "v"(vb), "v"(pb), "v"(kva), "v"(neg_m),
                     "v"(a.scale_log2), "v"(pw)
                   : "memory", MLA_ASM_STEP8_CLOBBERS);
      MLA_ISSUE_FIFTH(si, rs_n, rss_n);
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"((AHEAD - 1) * LPT) : "memory");   // tile it+1 landed
      __syncthreads();
      sc = (sc + 1 == NB) ? 0 : sc + 1;
    };
    // tiles 0 .. nfull-1 hold no token past this wave's limit
    const int nfull = __builtin_amdgcn_readfirstlane(max(0, (lim - t0 + 1) / TILE));
    const int fused_end = min(nfull, ntiles + 1);
    step_split(0);
    int it = 1;
    for (; it < fused_end; ++it) step_fused(it);
    for (; it <= ntiles; ++it) step_split(it);
    if constexpr (CHECK) {
      // A weight above 2^64 (a score more than 64 above the row's
      // reference, the overflow risk) leaves a normaliser above 2^64: either
      // partial of a row above 2^63, or not finite, asks for a restart.
      if (__builtin_amdgcn_ballot_w64(!(l_run <= 0x1p63f)) != 0 && lane == 0) s_restart = 1;
      __syncthreads();
      const bool again = __builtin_amdgcn_readfirstlane(s_restart) != 0;
      return again;
    }
    return false;
  };

  // Reload tiles 0 .. AHEAD-1 after a pass ended early (its loads drained).
  auto reload = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                  // every wave is done with the ring
    if (tid == 0) s_restart = 0;
    MLA_ZERO_PBUF1();
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) MLA_ISSUE_TILE(t0 + k * TILE, k);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((AHEAD - 1) * LPT) : "memory");   // tile 0 landed
    __syncthreads();
  };

  if (__builtin_expect(run_steps(std::true_type{}), 0)) {
    // A restart (rare): the largest score of each row over the whole item
    // (a pass of the scores alone), then a pass with that reference, which
    // no score can exceed.
    reload();
    {
      int sc = 0;
      for (int it = 0; it < ntiles; ++it) {
        const int ts = t0 + it * TILE;
        const int si = (sc + AHEAD >= NB) ? sc + AHEAD - NB : sc + AHEAD;
        MLA_TILE_RSRC(ts + AHEAD * TILE, rs_n, rss_n);
        const uint32_t lb_n = __builtin_amdgcn_readfirstlane(lds0 + si * SLOT + 1024 * wave);
        floatx16 s_cur;
        const uint32_t ad = lds0 + sc * SLOT + qk_off;
        asm volatile(MLA_ASM_QK8_TILE
                     : "=&v"(s_cur)
                     : "v"(ad), "v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]),
                       "v"(qf[5]), "v"(qf[6]), "v"(qf[7]), "v"(qf[8]), "v"(qf[9]),
                       "v"(qf[10]), "v"(qf[11]), "v"(qf[12]), "v"(qf[13]), "v"(qf[14]),
                       "v"(qf[15]), "v"(qf[16]), "v"(qf[17]), "v"(qf[18]), "v"(qf[19]),
                       "v"(qf[20]), "v"(qf[21]), "v"(qf[22]), "v"(qf[23]), "v"(qf[24]),
                       "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]), "v"(qf[29]),
                       "v"(qf[30]), "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]),
                       "v"(qf[35]), "s"(rs_n), "s"(lb_n), "v"(voff[0]), "v"(voff[1]),
                       "v"(voff[2]), "v"(voff[3])
                     : "memory", MLA_ASM_QK8_CLOBBERS);
        MLA_ISSUE_FIFTH(si, rs_n, rss_n);
        const float* kvp = (const float*)(s_lds + sc * SLOT + SCL) + 16 * h;
        float sc16[16], mt, tmp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc16[r] = s_cur[r] * kvp[r];
          if (ts + reg_token(r, h) > lim) sc16[r] = kNegInf;
        }
        asm volatile(MLA_ASM_SOFTMAX_MAX
                     : "=&v"(mt), "=&v"(tmp)
                     : "v"(sc16[0]), "v"(sc16[1]), "v"(sc16[2]), "v"(sc16[3]), "v"(sc16[4]),
                       "v"(sc16[5]), "v"(sc16[6]), "v"(sc16[7]), "v"(sc16[8]), "v"(sc16[9]),
                       "v"(sc16[10]), "v"(sc16[11]), "v"(sc16[12]), "v"(sc16[13]),
                       "v"(sc16[14]), "v"(sc16[15]), "v"(a.scale_log2));
        m_seen = fmaxf(m_seen, mt);
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"((AHEAD - 1) * LPT) : "memory");
        __syncthreads();              // tile it+1 landed; slot of tile it-1 free
        sc = (sc + 1 == NB) ? 0 : sc + 1;
      }
    }
    reload();
    m_ref = m_seen;
    l_run = 0.f;
    run_steps(std::false_type{});
  }
#undef MLA_ISSUE_TILE
#undef MLA_ISSUE_FIFTH
#undef MLA_TILE_RSRC
#undef MLA_PAGE
#undef MLA_ZERO_PBUF1

  store_rows(a, o, l_run, m_ref, s_lds, s_inv, b, rb, item_id, ns, rows, tid);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, const ItemTable& tab, hipStream_t st) {
  // a.row_blocks counts blocks of 128 query rows
  const int grid = a.n_items * a.row_blocks;
  if (a.q_row_bytes != 2 * D) return hipErrorInvalidValue;   // plain bf16 query rows only
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(grid), dim3(256), 0, st, a, tab);
  return hipGetLastError();
}

}  // namespace mla
