// Attention over the latent cache on gfx950 matrix cores (the hot kernel).
//
// Absorbed MLA decode ("DeepSeek-V2: Strong, Economical, Efficient",
// section 2.1.2 and Appendix C; attention-output equation of the
// "DeepSeek-V3 Technical Report" notes, MLA section): all n_h heads of a
// query token share one cache row K_j = [c_j (512) ; k^R_j (64)], so per
// sequence the step is two dense contractions with the query rows as one
// matrix dimension:
//   S = Q_abs K^T   (rows x tokens, K-dim 576)
//   O = P C         (rows x 512,    K-dim tokens)
//
// Work decomposition
//   * A work item is (sequence b, KV chunk [t0, t0 + chunk)); one workgroup
//     of 4 waves handles 128 query rows (row = tau * n_h + head) of an item.
//     Row blocks of the same item are placed on the same XCD so that the
//     chunk is fetched from HBM once and re-read from that XCD's L2.
//   * For the scores, wave w owns rows 32w .. 32w+31: its absorbed queries
//     live in VGPRs for the whole item (36 MFMA operands of 8 bf16 = 144
//     VGPRs).  For the PV product, wave w owns latent dims 128w .. 128w+127
//     of all 128 rows: its accumulator O^T (128 x 128 fp32 = 256 registers)
//     stays in the matrix accumulators, and the softmax weights of every row
//     block reach it through an 8 KB LDS buffer.
//   * KV tiles of 32 tokens go through a 4-slot LDS ring (rows padded to
//     1168 bytes so the 16-byte operand reads of 16 token rows of distinct
//     residues mod 16 hit distinct banks).  Step i takes the scores of tile
//     i, then the PV product of tile i-1 interleaved with the softmax of
//     tile i, while tiles i+1 and i+2 stream in.
//     bf16 tiles move HBM -> LDS with buffer loads that write LDS directly
//     (no VGPR staging); a load range that ends at the last valid token makes
//     the hardware write zeros for masked tokens, so they enter the PV
//     product as exact zeros.  Raw 6-bit tiles are copied the same way into
//     the upper part of their slot and decoded in place to bf16 (exact) one
//     step before they are used.  fp8 tiles have a kernel of their own
//     (decode_fp8.hip) that converts its operands in registers.
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16) puts one row's 16 token scores
//     in each lane: the per-row max and sum need no cross-lane reduction
//     except with the partner lane (lane ^ 32).  The packed weights are then
//     already in the B-operand layout of O^T += C^T P^T (the token order
//     inside the K dimension is chosen to match the score layout), and the A
//     operand C^T comes from the transposing LDS read (ds_read_b64_tr_b16: in
//     each 16-lane group, lane i receives element i%4 of the 8-byte chunks
//     addressed by lanes 4k + i/4, k = 0..3, i.e. four token rows of 16
//     latent dims come back as 16 dims of 4 tokens).
//   * Softmax in the log2 domain against a per-row reference m_ref instead
//     of a running max: m_ref is the max of the first tile in which the row
//     sees a token, and p = 2^(s - m_ref) is accumulated without rescaling
//     (fp32 and bf16 share an 8-bit exponent, so p up to 2^64 is safe).  If
//     a later score exceeds m_ref by more than 64 the whole workgroup
//     restarts the work item with m_ref raised to the max seen so far; each
//     restart raises m_ref by more than 64, so restarts are rare and finite.
//     The result is exact for any reference: LSE = m_ref + log2(sum p).
#include <math.h>

#include "decode_tile.hpp"
#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

namespace {
constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int ROWS_WG = 128;             // query rows per workgroup (4 waves x 32)
constexpr int TILE = 32;                 // tokens per staged tile
constexpr int LROW = 1168;               // LDS bytes per token row (1152 + 16 pad)
constexpr int NBUF = 4;                  // LDS ring of tiles
constexpr int NLOADS = 37;               // direct loads of 64 x 16 B per tile
constexpr int TILE_BYTES = NLOADS * 1024;
constexpr int NLD = 10;                  // loads per wave per tile (wave 0: 10, others: 9)
constexpr int NCH = 72;                  // 16-byte chunks per bf16 row
constexpr int ROW6 = 452;                // fp6: bytes per cache row (432 codes, 18 exponents, pad)
constexpr int TILE6 = TILE * ROW6;       // fp6: raw tile (14464 bytes)
constexpr int NLD6 = (TILE6 + 1023) / 1024;   // fp6: 1 KB loads per raw tile (15)
constexpr int RAW6 = TILE_BYTES - NLD6 * 1024;  // fp6: raw tile at this offset of its slot
constexpr int NBLK6 = TILE * D / 32;     // fp6: blocks of 32 elements per tile (576)
constexpr int QROW = 592;                // LDS bytes per staged half query row (576 + 16 pad)
constexpr int QLOADS = ROWS_WG * (QROW / 16) / 64;   // 1 KB loads per staged half (74)
constexpr uint32_t kOOB = 0x40000000u;   // buffer offset past any valid range
constexpr float kNegInf = -INFINITY;
}  // namespace

typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ inline u32x2 lds_tr16(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (shortx4 __attribute__((address_space(3)))*)(p)));
}

// max(x[l], x[l ^ 32]) in every lane l.  v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; with x
// in both, one comes back as the lower halves and the other as the upper
// halves.  Written as assembly: the compiler's builtin for this instruction
// takes its two results as equal when its two inputs are, which they are not.
__device__ inline float pair_max32(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
  return fmaxf(lo, hi);
}

// One tile's S^T[token, head] for the wave's 32 heads (36 MFMAs over the
// 576 dims; kb is this lane's operand address: token l%32, dims 16k +
// 8(l/32)), and O^T[dim, head] += C^T[dim, tok] P^T[tok, head] (32 MFMAs;
// vb is this lane's transposed-read address).  Both are software-pipelined
// sequences (several LDS reads in flight ahead of the matrix pipe) written
// out by gen_decode_asm.py; they wait for all of their reads before they end.
#include "decode_mfma_asm.inc"

__device__ __forceinline__ floatx16 qk_tile(const uint8_t* kb, const bf16x8 (&q)[D / 16]) {
  floatx16 s;
  const uint32_t ad = (uint32_t)(uintptr_t)kb;
  asm volatile(MLA_ASM_QK_TILE
               : "=&v"(s)
               : "v"(ad), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]),
                 "v"(q[6]), "v"(q[7]), "v"(q[8]), "v"(q[9]), "v"(q[10]), "v"(q[11]), "v"(q[12]),
                 "v"(q[13]), "v"(q[14]), "v"(q[15]), "v"(q[16]), "v"(q[17]), "v"(q[18]),
                 "v"(q[19]), "v"(q[20]), "v"(q[21]), "v"(q[22]), "v"(q[23]), "v"(q[24]),
                 "v"(q[25]), "v"(q[26]), "v"(q[27]), "v"(q[28]), "v"(q[29]), "v"(q[30]),
                 "v"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35])
               : "memory", MLA_ASM_QK_CLOBBERS);
  return s;
}

// O^T[the wave's 128 dims, all 128 rows] += C^T P^T for one tile (vb: this
// lane's transposed-read address in the tile's slot, including the wave's
// dim offset; pb: this lane's address in the P^T fragment buffer).
__device__ __forceinline__ void pvd_tile(const uint8_t* vb, const uint8_t* pb,
                                         floatx16 (&o)[DC / 32]) {
  const uint32_t ad = (uint32_t)(uintptr_t)vb, pa = (uint32_t)(uintptr_t)pb;
  asm volatile(MLA_ASM_PVD_TILE
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15])
               : "v"(ad), "v"(pa)
               : "memory", MLA_ASM_PVD_CLOBBERS);
}

// The wave's P^T fragments of one tile (token halves 0 and 1, the B operands
// of the PV product for its 32 rows) into the P buffer: fragment (row block
// w, half k) at 1024 (2 w + k), 16 bytes per lane.
__device__ __forceinline__ void put_p(uint8_t* s_p, int wave, int lane, const uint32_t (&pk)[8]) {
  uint8_t* d = s_p + 2048 * wave + 16 * lane;
  *(u32x4*)d = u32x4{pk[0], pk[1], pk[2], pk[3]};
  *(u32x4*)(d + 1024) = u32x4{pk[4], pk[5], pk[6], pk[7]};
}

// Score-row order inside a tile: tile_row(m) (decode_tile.hpp).  The
// transposed PV reads of a half-wave cover four tile rows p, p+4, p+8, p+12
// (64 bytes each), which at the 1168-byte row pitch fall in four disjoint
// quarters of the 64 LDS banks; the score-operand reads of 16 lanes cover 16
// rows of distinct residues mod 16 (distinct bank groups).

// LDS source offset mapping of a tile (rows at a pitch of 73 granules of 16
// bytes): granule u of the slot holds granule u % 73 of token row u / 73,
// or nothing (the row's padding granule, or past the tile's 32 rows), which
// gets an offset past any valid range (the buffer load then writes zeros).
// u / 73 = (449 u) >> 15 for u < 2368.
__device__ inline uint32_t tile_src_offset(int u) {
  const int tk = (u * 449) >> 15;
  return (u - 73 * tk == NCH || tk >= TILE) ? kOOB : uint32_t(16 * (u - tk));
}

static_assert(QLOADS * 1024 == 2 * TILE_BYTES, "query halves fill ring slots 2 and 3");
static_assert(QLOADS * 64 == ROWS_WG * (QROW / 16), "whole staged rows");

// Staged query halves: 16-byte unit u holds row u / 37, unit u % 37 of the
// half (unit 36 is the row padding: an out-of-range offset, zero-filled).
// Rows are QRB bytes apart (query pairs: only the hi part is read).

// 32 E2M3 codes (6 dwords, code i at bits 6 i .. 6 i + 5) times 2^e -> 32
// bf16 values, two per dword (even element in the low half).  Exact: every
// E2M3 value times a power of two in range is a bf16 value.  The scale's
// power-of-two part is what the instruction applies.
__device__ inline void fp6x32_to_bf16x32(const uint32_t (&w)[6], float scale, u32x4 (&r)[4]) {
  typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
  const u32x6 v = {w[0], w[1], w[2], w[3], w[4], w[5]};
  u32x16 o;
  // The conversion writes its 16 result registers over several cycles and
  // a read issued right after it sees the old contents: 20 wait states
  // separate it from the first use.
  asm volatile("s_nop 1\n\tv_cvt_scalef32_pk32_bf16_fp6 %0, %1, %2\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "=&v"(o) : "v"(v), "v"(scale));
  r[0] = u32x4{o[0], o[1], o[2], o[3]};
  r[1] = u32x4{o[4], o[5], o[6], o[7]};
  r[2] = u32x4{o[8], o[9], o[10], o[11]};
  r[3] = u32x4{o[12], o[13], o[14], o[15]};
}

// KVK: cache kind, 0 = bf16, 2 = 6-bit (E2M3 codes with one power of two
// per 32 elements).  QRB: bytes between query rows (2 D, or 4 D for query
// pairs), a constant so that the staging offsets fold.
template <int KVK, int QRB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeArgs a, ItemTable tab) {
  static_assert(KVK == 0 || KVK == 2, "fp8 tiles run on decode_fp8_kernel");
  static_assert(QRB == 2 * D || QRB == 4 * D, "plain bf16 rows or query pairs");
  constexpr bool FP6 = KVK == 2, RAW = KVK != 0;
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv[NBUF][TILE_BYTES];
  __shared__ int s_restart;
  __shared__ int s_escalate;
  __shared__ __attribute__((aligned(16))) uint8_t s_p[4 * 2 * 1024];   // P^T fragments
  __shared__ float s_inv[ROWS_WG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31, g = lane >> 4, j = lane & 15;
  const int gi = xcd_logical_index(blockIdx.x, gridDim.x);
  const int item = gi / a.row_blocks, rb = gi % a.row_blocks;
  // work item -> (sequence, split, length): from the host's table when the
  // plan has few enough items, else located on the device
  int b, s_idx, L, item_id = item;      // item_id: where the partial goes
  if (tab.uniform_len > 0) {           // every sequence has the same length
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
  const int t_end = min(L, t0 + c);                       // item end
  const int rows = a.n_h * a.T;
  const int row = rb * ROWS_WG + wave * 32 + l32;         // this lane's row
  const int tau = row / a.n_h, head = row % a.n_h;
  // last visible token; the 32 rows of a wave share tau (n_h % 32 == 0)
  const int lim = __builtin_amdgcn_readfirstlane(min(t_end - 1, L - a.T + tau));
  const int tau_max = (rb * ROWS_WG + ROWS_WG - 1) / a.n_h;
  const int t_stage =                                     // tokens any row sees
      __builtin_amdgcn_readfirstlane(min(t_end, L - a.T + tau_max + 1));
  const int nq = b * a.T + tau;
  const int ntiles = (t_stage > t0) ? (t_stage - t0 + TILE - 1) / TILE : 0;

  const uint32_t lds_ring = (uint32_t)(uintptr_t)&s_kv[0][0];

  const uint8_t* cache = (const uint8_t*)a.cache;
  constexpr int ROWB = FP6 ? ROW6 : 2 * D;               // bytes per cache row
  const int seq_row0 = b * a.max_len;
  typedef __attribute__((address_space(4))) const int32_t* ConstI32;
  const ConstI32 ptab = a.page_table ? (ConstI32)(a.page_table + (size_t)b * a.max_pages) : nullptr;
  // Paged cache: the item's page ids are loaded once, one per lane (up to
  // 128 pages), and each tile takes its page from a lane with v_readlane, so
  // no tile waits for a page-table load.  Items are page-aligned (the chunk
  // is a multiple of the page size).  Longer items read the table per tile.
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

  // page id of the tile starting at token ts (ts inside the item)
#define MLA_PAGE(ts_)                                                                      \
  (pg_regs ? __builtin_amdgcn_readlane(((ts_) / kPage - pg_first) < 64 ? pg_lo : pg_hi,   \
                                       ((ts_) / kPage - pg_first) & 63)                  \
           : ptab[(ts_) / kPage])

  // ---- staging.  bf16: LDS 16-byte chunk q of a tile holds token q / 73,
  // chunk q % 73 of its row (chunk 72 is the row padding, filled with zero
  // by an out-of-range offset).  Load n of wave w fills chunks
  // 64 (w + 4n) .. +63; the last (37th) load of a tile belongs to wave 0.
  // LDS chunk q = 64 (w + 4n) + lane  <-  memory chunk q - q/73 of the tile
  // (q/73 = (449 q) >> 15 for q < 2368); the padding chunk of each row and
  // chunks past the tile take an out-of-range offset.
  const int qbase = 64 * wave + lane;
#define MLA_VOFF(n_) tile_src_offset(qbase + 256 * (n_))
  uint32_t stg6[FP6 ? 2 : 1][7];                          // fp6: 6 code dwords + exponent byte
  const uint32_t lane16 = 16 * lane;                      // fp6: lane offset of raw loads

  // Issue the loads of the tile starting at token ts into ring slot buf.  A
  // tile never crosses a page (ts is a multiple of 32, pages hold 64 tokens).
  // Everything that addresses the tile is wave-uniform: the page id comes
  // through the scalar cache and the buffer descriptor lives in SGPRs.
  // bf16 tiles are copied HBM -> LDS by buffer loads with the LDS-write
  // option, issued from inline assembly: the compiler then keeps no
  // bookkeeping of them (it would otherwise wait for every in-flight tile
  // before each LDS read, since it cannot tell the ring slots apart), and
  // the kernel's own vmcnt waits and barriers order them.
#define MLA_ISSUE_TILE(ts_, buf_)                                                          \
  do {                                                                                   \
    const int ts__ = (ts_);                                                              \
    const int nv__ = max(0, min(TILE, t_stage - ts__));                                  \
    int r0__ = 0;                                                                        \
    if (nv__ > 0)                                                                        \
      r0__ = ptab ? MLA_PAGE(ts__) * kPage + (ts__ % kPage) : seq_row0 + ts__;          \
    r0__ = __builtin_amdgcn_readfirstlane(r0__);                                         \
    const uint64_t ad__ = (uint64_t)(cache + (size_t)r0__ * ROWB);                       \
    const u32x4 rs__ = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad__),        \
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad__ >> 32)) & 0xFFFFu, \
                        (uint32_t)__builtin_amdgcn_readfirstlane(nv__ * ROWB),           \
                        0x00020000u};                                                    \
    if constexpr (!RAW) {                                                                 \
      const uint32_t lb__ = lds_ring + (buf_) * TILE_BYTES + 1024 * wave;                \
      _Pragma("unroll") for (int n = 0; n < NLD - 1; ++n)                                \
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"        \
                     :: "s"(lb__ + 4096 * n), "v"(MLA_VOFF(n)), "s"(rs__) : "memory");   \
      if (wave == 0)                                                                     \
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"        \
                     :: "s"(lds_ring + (buf_) * TILE_BYTES + 1024 * 36),                 \
                        "v"(MLA_VOFF(NLD - 1)), "s"(rs__) : "memory");                   \
    } else if constexpr (FP6) {                                                          \
      /* raw 6-bit rows (contiguous) into the slot's upper part; wave w issues */        \
      /* loads w, w+4, ...; the tail of the last load is past the range (zeros) */      \
      const uint32_t lb__ = lds_ring + (buf_) * TILE_BYTES + RAW6 + 1024 * wave;         \
      _Pragma("unroll") for (int k = 0; k < (NLD6 + 3) / 4; ++k)                         \
        if (wave + 4 * k < NLD6)                                                         \
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"     \
                       :: "s"(lb__ + 4096 * k), "v"(lane16), "s"(rs__),                  \
                          "s"(__builtin_amdgcn_readfirstlane(1024 * (wave + 4 * k))) : "memory"); \
    }                                                                                    \
  } while (0)
  // fp6: this thread's blocks q = tid, tid + 256 of the raw tile in slot buf
  // (token q / 18, elements 32 (q % 18) ..): 6 code dwords and the exponent
  // byte.  Blocks 512 .. 575 (tokens 28 .. 31) are wave 0's and are read in
  // MLA_DECODE6 itself: their raw bytes lie past every bf16 row the other
  // blocks write (rows 0 .. 28), and within wave 0 all reads precede all
  // writes.
#define MLA_READ_RAW6(buf_)                                                                \
  do {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                      \
      const int q = tid + 256 * i;                                                       \
      const int t = q / 18, k = q - 18 * (q / 18);                                       \
      const uint8_t* src = &s_kv[(buf_)][RAW6 + ROW6 * t];                               \
      _Pragma("unroll") for (int w = 0; w < 6; ++w)                                      \
        stg6[i][w] = *(const uint32_t*)(src + 24 * k + 4 * w);                           \
      stg6[i][6] = src[432 + k];                                                         \
    }                                                                                    \
  } while (0)
  // fp6: decode the blocks into the slot's bf16 rows (the raw reads of
  // blocks 0 .. 511 are done: a barrier separates the two); block (t, k) ->
  // row t, dims 32 k ..
#define MLA_DECODE6(buf_)                                                                  \
  do {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < 3; ++i) {                                      \
      const int q = tid + 256 * i;                                                       \
      if (q < NBLK6) {                                                                   \
        const int t = q / 18, k = q - 18 * (q / 18);                                     \
        uint32_t cw[6], ex;                                                              \
        if (i < 2) {                                                                     \
          _Pragma("unroll") for (int w = 0; w < 6; ++w) cw[w] = stg6[i < 2 ? i : 0][w];  \
          ex = stg6[i < 2 ? i : 0][6];                                                   \
        } else {                                                                         \
          const uint8_t* src = &s_kv[(buf_)][RAW6 + ROW6 * t];                           \
          _Pragma("unroll") for (int w = 0; w < 6; ++w)                                  \
            cw[w] = *(const uint32_t*)(src + 24 * k + 4 * w);                            \
          ex = src[432 + k];                                                             \
        }                                                                                \
        u32x4 r[4];                                                                      \
        fp6x32_to_bf16x32(cw, __builtin_bit_cast(float, ex << 23), r);                   \
        uint8_t* dst = &s_kv[(buf_)][t * LROW + 64 * k];                                 \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) *(u32x4*)(dst + 16 * u) = r[u];   \
      }                                                                                  \
    }                                                                                    \
  } while (0)
  // bf16: wait until at most one tile's loads of this wave are in flight
#define MLA_WAIT_ONE_TILE_IN_FLIGHT()                                                      \
  do {                                                                                   \
    if (wave == 0) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");                     \
    else asm volatile("s_waitcnt vmcnt(9)" ::: "memory");                                \
  } while (0)
  // bf16: buffer descriptor of the tile starting at token ts (as in
  // MLA_ISSUE_TILE), for loads issued from the step's assembly blocks
#define MLA_TILE_RSRC(ts_, rs_)                                                            \
  u32x4 rs_;                                                                             \
  {                                                                                      \
    const int ts__ = (ts_);                                                              \
    const int nv__ = max(0, min(TILE, t_stage - ts__));                                  \
    int r0__ = 0;                                                                        \
    if (nv__ > 0)                                                                        \
      r0__ = ptab ? MLA_PAGE(ts__) * kPage + (ts__ % kPage) : seq_row0 + ts__;          \
    r0__ = __builtin_amdgcn_readfirstlane(r0__);                                         \
    const uint64_t ad__ = (uint64_t)(cache + (size_t)r0__ * ROWB);                       \
    rs_ = u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad__),                \
                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad__ >> 32)) & 0xFFFFu, \
                (uint32_t)__builtin_amdgcn_readfirstlane(nv__ * ROWB), 0x00020000u};     \
  }

  // ---- per-lane LDS offsets of the MFMA operands
  const int qk_off = tile_row(l32) * LROW + 16 * h;                        // + 32 k
  // transposed reads: + 256 w selects the wave's 128 latent dims
  const int pv_off = (h + 4 * (j >> 2)) * LROW + (16 * (g & 1) + 4 * (j & 3)) * 2 + 256 * wave;
  // lane offsets of this wave's tile loads (the same for every tile)
  uint32_t voff[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) voff[n] = MLA_VOFF(n);

  // ---- absorbed query rows -> MFMA B operands (lane: head l32, 8 dims).
  // The workgroup's 128 rows are contiguous in memory (row = tau * n_h +
  // head, query token b*T + tau).  They are staged in two halves of 288
  // dims through ring slots 2 and 3, with buffer loads that write LDS
  // directly (each load 1 KB of LDS), at a row pitch of QROW bytes so that
  // the operand reads of 16 rows fall on distinct banks.  The loads of tiles
  // 0 and 1 (slots 0 and 1) go out between the first half's loads and its
  // wait, so their HBM latency overlaps the query staging.
  bf16x8 qf[D / 16];
  const uint64_t qa = (uint64_t)((const uint8_t*)a.q_abs +
                                 ((size_t)b * rows + rb * ROWS_WG) * QRB);
  const u32x4 qrs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)qa),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(qa >> 32)) & 0xFFFFu,
                     uint32_t(ROWS_WG * QRB), 0x00020000u};
  const uint32_t qlds = lds_ring + 2 * TILE_BYTES;
  const int qu0 = 64 * wave + lane;                       // staging unit of load 0
  // half p_: load n = wave + 4k (n < QLOADS) fills staging units 64n .. 64n+63
  // Loads k < QLOADS / 4 exist for every wave (wave + 4 k <= 3 + 4 (QLOADS / 4 - 1)
  // < QLOADS) and are issued with no test: a bound test per load splits them
  // into blocks, and the compiler then waits for all loads in flight before
  // each one.  The staging unit u = 64 (wave + 4 k) + lane of load k is kept
  // as row u / 37 and unit u % 37 and stepped by 256 = 6 * 37 + 34 units per
  // load (32-bit adds and selects only).
#define MLA_Q_LOAD(p_, n_, r_, c_)                                                         \
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"              \
               :: "s"(qlds + 1024 * (n_)),                                                \
                  "v"((c_) == QROW / 16 - 1 ? kOOB                                        \
                                            : uint32_t((r_) * QRB + (p_) * D + 16 * (c_))), \
                  "s"(qrs) : "memory")
#define MLA_Q_ISSUE(p_)                                                                    \
  do {                                                                                   \
    int r__ = qu0 / (QROW / 16), c__ = qu0 - (QROW / 16) * r__;                          \
    _Pragma("unroll") for (int k = 0; k < QLOADS / 4; ++k) {                             \
      MLA_Q_LOAD(p_, wave + 4 * k, r__, c__);                                            \
      c__ += 256 % (QROW / 16);                                                          \
      r__ += 256 / (QROW / 16);                                                          \
      const bool wrap__ = c__ >= QROW / 16;                                              \
      c__ = wrap__ ? c__ - QROW / 16 : c__;                                              \
      r__ = wrap__ ? r__ + 1 : r__;                                                      \
    }                                                                                    \
    if (wave < QLOADS % 4) MLA_Q_LOAD(p_, wave + 4 * (QLOADS / 4), r__, c__);            \
  } while (0)
  // half p_ -> qf[18 p_ .. 18 p_ + 17]
#define MLA_Q_READ(p_)                                                                     \
  do {                                                                                   \
    const uint8_t* qsrc__ = &s_kv[2][0] + (32 * wave + l32) * QROW + 16 * h;             \
    _Pragma("unroll") for (int k = 0; k < D / 32; ++k)                                   \
      qf[(D / 32) * (p_) + k] = *(const bf16x8*)(qsrc__ + 32 * k);                       \
  } while (0)

  floatx16 o[DC / 32];
  float m_ref = kNegInf, m_seen = kNegInf, l_run = 0.f;

  // Prologue of an attempt: issue tiles 0 and 1; 6-bit: once they have
  // landed (vmcnt(0) and a barrier), tile 0 is decoded right away, tile 1
  // in step 0.
#define MLA_ISSUE_FIRST_TILES()                                                            \
  do {                                                                                   \
    if (ntiles > 0) MLA_ISSUE_TILE(t0, 0);                                               \
    if (ntiles > 1) MLA_ISSUE_TILE(t0 + TILE, 1);                                        \
  } while (0)
#define MLA_DECODE_FIRST_TILE()                                                            \
  do {                                                                                   \
    if constexpr (FP6) {                                                                 \
      if (ntiles > 0) {                                                                  \
        MLA_READ_RAW6(0);                                                                \
        __syncthreads();                                                                 \
        MLA_DECODE6(0);                                                                  \
      }                                                                                  \
    }                                                                                    \
  } while (0)
#define MLA_PROLOGUE()                                                                     \
  do {                                                                                   \
    MLA_ISSUE_FIRST_TILES();                                                             \
    if constexpr (RAW) {                                                                 \
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                   \
      __syncthreads();                                                                   \
    }                                                                                    \
    MLA_DECODE_FIRST_TILE();                                                             \
  } while (0)

  if (tid == 0) { s_restart = 0; s_escalate = 0; }
  // first attempt: query half 0, tiles 0 and 1, query half 1
  MLA_Q_ISSUE(0);
  MLA_ISSUE_FIRST_TILES();
  {
    // wait for query half 0 only: at most the loads of the tiles issued
    // after it (the fewest any wave issues per tile) stay in flight
    const int nt = min(ntiles, 2);
    if (nt == 2) {
      if constexpr (FP6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    } else if (nt == 1) {
      if constexpr (FP6) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  }
  __syncthreads();                    // every wave's share of half 0 landed
  MLA_Q_READ(0);
  __syncthreads();                    // every wave has read half 0: the slots are free
  MLA_Q_ISSUE(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                    // half 1 and tiles 0 and 1 landed
  MLA_Q_READ(1);
#pragma unroll
  for (int k = 0; k < D / 16; ++k) asm volatile("" ::"v"(qf[k]));
  MLA_DECODE_FIRST_TILE();
#undef MLA_Q_ISSUE
#undef MLA_Q_READ
#undef MLA_Q_LOAD

  for (;;) {                          // attempts (a restart is rare)
#pragma unroll
    for (int i = 0; i < DC / 32; ++i) o[i] = floatx16{};
    l_run = 0.f;
    int restart = 0;
    if constexpr (!RAW) {
      // Step it: scores of tile it; the PV product of tile it-1 with the
      // softmax of tile it interleaved (one assembly block); the loads of
      // tile it+2 spread through both blocks; wait for tile it+1.  Ring
      // slots in use during step it: it-1 (PV), it (QK), it+1 (landing),
      // it+2 (loading).  Step 0 has no previous tile: its PV product
      // multiplies tile 0 by zero weights (adds exactly zero; the tile
      // holds finite values).  The last tile's PV product runs after the
      // loop.
      if (ntiles > 0) {
        if (ntiles > 1) MLA_WAIT_ONE_TILE_IN_FLIGHT();   // tile 0 landed
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        uint32_t pk_prev[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        for (int it = 0; it < ntiles; ++it) {
          const int ts = t0 + it * TILE;
          MLA_TILE_RSRC(ts + 2 * TILE, rs_n);
          const uint32_t lb_n = lds_ring + ((it + 2) & 3) * TILE_BYTES + 1024 * wave;
          put_p(s_p, wave, lane, pk_prev);   // weights of tile it-1 (zero at step 0)
          floatx16 s_cur;
          {
            const uint32_t ad = (uint32_t)(uintptr_t)(s_kv[it & 3] + qk_off);
            asm volatile(MLA_ASM_QK_TILE_DMA
                         : "=&v"(s_cur)
                         : "v"(ad), "v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]),
                           "v"(qf[5]), "v"(qf[6]), "v"(qf[7]), "v"(qf[8]), "v"(qf[9]),
                           "v"(qf[10]), "v"(qf[11]), "v"(qf[12]), "v"(qf[13]), "v"(qf[14]),
                           "v"(qf[15]), "v"(qf[16]), "v"(qf[17]), "v"(qf[18]), "v"(qf[19]),
                           "v"(qf[20]), "v"(qf[21]), "v"(qf[22]), "v"(qf[23]), "v"(qf[24]),
                           "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]), "v"(qf[29]),
                           "v"(qf[30]), "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]),
                           "v"(qf[35]), "s"(rs_n), "s"(lb_n), "v"(voff[0]), "v"(voff[1]),
                           "v"(voff[2]), "v"(voff[3]), "v"(voff[4])
                         : "memory", MLA_ASM_QK_CLOBBERS);
          }
          __syncthreads();                   // every wave's weights of tile it-1 are in
          // register r holds token reg_token(r, h).  The 32 rows of a
          // wave share one query token, so the visibility limit is
          // wave-uniform and only a tile that crosses it is masked.
          float sv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = s_cur[r];
          if (ts + TILE - 1 > lim) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (ts + reg_token(r, h) > lim) sv[r] = kNegInf;
          }
          float mt;
          if (m_ref == kNegInf) {
            // the first tile in which the row sees a token sets the reference
            float tmp0;
            asm volatile(MLA_ASM_SOFTMAX_MAX
                         : "=&v"(mt), "=&v"(tmp0)
                         : "v"(sv[0]), "v"(sv[1]), "v"(sv[2]), "v"(sv[3]), "v"(sv[4]),
                           "v"(sv[5]), "v"(sv[6]), "v"(sv[7]), "v"(sv[8]), "v"(sv[9]),
                           "v"(sv[10]), "v"(sv[11]), "v"(sv[12]), "v"(sv[13]), "v"(sv[14]),
                           "v"(sv[15]), "v"(a.scale_log2));
            m_ref = mt;                          // O and l are still zero here
          }
          const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
          const uint32_t vb = (uint32_t)(uintptr_t)(s_kv[(it > 0 ? it - 1 : 0) & 3] + pv_off);
          const uint32_t pb = (uint32_t)(uintptr_t)(s_p + 16 * lane);
          uint32_t pk[8];
          float tmp;
          asm volatile(MLA_ASM_PVD_SOFTMAX_TILE_DMA
                       : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]),
                         "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]),
                         "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                         "+a"(o[15]), "+v"(sv[0]), "+v"(sv[1]), "+v"(sv[2]), "+v"(sv[3]),
                         "+v"(sv[4]), "+v"(sv[5]), "+v"(sv[6]), "+v"(sv[7]), "+v"(sv[8]),
                         "+v"(sv[9]), "+v"(sv[10]), "+v"(sv[11]), "+v"(sv[12]), "+v"(sv[13]),
                         "+v"(sv[14]), "+v"(sv[15]), "=&v"(pk[0]), "=&v"(pk[1]), "=&v"(pk[2]),
                         "=&v"(pk[3]), "=&v"(pk[4]), "=&v"(pk[5]), "=&v"(pk[6]), "=&v"(pk[7]),
                         "=&v"(mt), "=&v"(tmp), "+v"(l_run)
                       : "v"(vb), "v"(pb), "v"(neg_m), "v"(a.scale_log2),
                         "s"(rs_n), "s"(lb_n), "v"(voff[5]), "v"(voff[6]), "v"(voff[7]),
                         "v"(voff[8])
                       : "memory", MLA_ASM_PVD_CLOBBERS);
          if (wave == 0)                         // the tile's 37th load
            asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(lds_ring + ((it + 2) & 3) * TILE_BYTES), "v"(voff[NLD - 1]),
                            "s"(rs_n), "i"(1024 * 36) : "memory");
#pragma unroll
          for (int i = 0; i < 8; ++i) pk_prev[i] = pk[i];
          m_seen = fmaxf(m_seen, mt);
          if (mt > m_ref + 64.0f) s_restart = 1;
          if (mt > a.esc_log2) s_escalate = 1;   // recomputed with split operands
          MLA_WAIT_ONE_TILE_IN_FLIGHT();     // tile it+1 landed (it+2 may fly)
          __syncthreads();
          restart = __builtin_amdgcn_readfirstlane(s_restart | s_escalate);   // uniform: after the barrier
          if (restart) break;
        }
        if (!restart) {
          put_p(s_p, wave, lane, pk_prev);
          __syncthreads();
          pvd_tile(s_kv[(ntiles - 1) & 3] + pv_off, s_p + 16 * lane, o);
        }
      }
    } else if constexpr (FP6) {
      // The bf16 step with 6-bit tiles: raw tile it+1 (copied during step
      // it-1) is read after the scores of step it and decoded in place after
      // its first barrier (each block of 32 codes with its power of two,
      // exact in bf16), while tile it+2 is copied.
      if (ntiles > 0) {
        __syncthreads();
        uint32_t pk_prev[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        for (int it = 0; it < ntiles; ++it) {
          const int ts = t0 + it * TILE;
          MLA_ISSUE_TILE(ts + 2 * TILE, (it + 2) & 3);
          put_p(s_p, wave, lane, pk_prev);   // weights of tile it-1 (zero at step 0)
          const floatx16 s_cur = qk_tile(s_kv[it & 3] + qk_off, qf);
          MLA_READ_RAW6((it + 1) & 3);       // after the scores: no staging registers in them
          __syncthreads();                   // weights of tile it-1 in; raw tile it+1 read
          MLA_DECODE6((it + 1) & 3);
          float sv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = s_cur[r];
          if (ts + TILE - 1 > lim) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (ts + reg_token(r, h) > lim) sv[r] = kNegInf;
          }
          float mt;
          if (m_ref == kNegInf) {
            float tmp0;
            asm volatile(MLA_ASM_SOFTMAX_MAX
                         : "=&v"(mt), "=&v"(tmp0)
                         : "v"(sv[0]), "v"(sv[1]), "v"(sv[2]), "v"(sv[3]), "v"(sv[4]),
                           "v"(sv[5]), "v"(sv[6]), "v"(sv[7]), "v"(sv[8]), "v"(sv[9]),
                           "v"(sv[10]), "v"(sv[11]), "v"(sv[12]), "v"(sv[13]), "v"(sv[14]),
                           "v"(sv[15]), "v"(a.scale_log2));
            m_ref = mt;                          // O and l are still zero here
          }
          const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
          const uint32_t vb = (uint32_t)(uintptr_t)(s_kv[(it > 0 ? it - 1 : 0) & 3] + pv_off);
          const uint32_t pb = (uint32_t)(uintptr_t)(s_p + 16 * lane);
          uint32_t pk[8];
          float tmp;
          asm volatile(MLA_ASM_PVD_SOFTMAX_TILE
                       : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]),
                         "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]),
                         "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                         "+a"(o[15]), "+v"(sv[0]), "+v"(sv[1]), "+v"(sv[2]), "+v"(sv[3]),
                         "+v"(sv[4]), "+v"(sv[5]), "+v"(sv[6]), "+v"(sv[7]), "+v"(sv[8]),
                         "+v"(sv[9]), "+v"(sv[10]), "+v"(sv[11]), "+v"(sv[12]), "+v"(sv[13]),
                         "+v"(sv[14]), "+v"(sv[15]), "=&v"(pk[0]), "=&v"(pk[1]), "=&v"(pk[2]),
                         "=&v"(pk[3]), "=&v"(pk[4]), "=&v"(pk[5]), "=&v"(pk[6]), "=&v"(pk[7]),
                         "=&v"(mt), "=&v"(tmp), "+v"(l_run)
                       : "v"(vb), "v"(pb), "v"(neg_m), "v"(a.scale_log2)
                       : "memory", MLA_ASM_PVD_CLOBBERS);
#pragma unroll
          for (int i = 0; i < 8; ++i) pk_prev[i] = pk[i];
          m_seen = fmaxf(m_seen, mt);
          if (mt > m_ref + 64.0f) s_restart = 1;
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // raw tile it+2 landed
          __syncthreads();
          restart = __builtin_amdgcn_readfirstlane(s_restart);   // uniform: read after the barrier
          if (restart) break;
        }
        if (!restart) {
          put_p(s_p, wave, lane, pk_prev);
          __syncthreads();
          pvd_tile(s_kv[(ntiles - 1) & 3] + pv_off, s_p + 16 * lane, o);
        }
      }
    }
    if (!restart) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load of this attempt in flight
    if (__builtin_amdgcn_readfirstlane(s_escalate)) {
      // A score past the escalation threshold: the split-operand kernel
      // recomputes this item's rows; nothing is written here but the flag.
      if (tid == 0) a.esc_flags[(size_t)item_id * a.fast_rb + rb] = 1;
      return;
    }
    __syncthreads();                  // everyone has read the flag
    if (tid == 0) s_restart = 0;
    m_ref = m_seen;
    MLA_PROLOGUE();
  }
#undef MLA_ISSUE_TILE
#undef MLA_PROLOGUE
#undef MLA_ISSUE_FIRST_TILES
#undef MLA_DECODE_FIRST_TILE
#undef MLA_READ_RAW6
#undef MLA_DECODE6
#undef MLA_WAIT_ONE_TILE_IN_FLIGHT
#undef MLA_TILE_RSRC
#undef MLA_VOFF
#undef MLA_PAGE

  // ---- normalise and write (the final output, or this split's partial)
  store_rows(a, o, l_run, m_ref, &s_kv[0][0], s_inv, b, rb, item_id, ns, rows, tid);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, const ItemTable& tab, hipStream_t st);

hipError_t launch_decode_mfma(const DecodeArgs& a, const ItemTable& tab, hipStream_t st) {
  // a.row_blocks counts blocks of ROWS_WG query rows
  const int grid = a.n_items * a.row_blocks;
  if (a.kv_dtype == MLA_FP8_E4M3)
    return launch_decode_fp8(a, tab, st);
  if (a.kv_dtype == MLA_FP6_E2M3 && a.q_row_bytes == 2 * D)
    hipLaunchKernelGGL((decode_mfma_kernel<2, 2 * D>), dim3(grid), dim3(256), 0, st, a, tab);
  else if (a.kv_dtype == MLA_BF16 && a.q_row_bytes == 2 * D)
    hipLaunchKernelGGL((decode_mfma_kernel<0, 2 * D>), dim3(grid), dim3(256), 0, st, a, tab);
  else if (a.kv_dtype == MLA_BF16 && a.q_row_bytes == 4 * D)
    hipLaunchKernelGGL((decode_mfma_kernel<0, 4 * D>), dim3(grid), dim3(256), 0, st, a, tab);
  else
    return hipErrorInvalidValue;     // no other query layout reaches this kernel
  return hipGetLastError();
}

}  // namespace mla
