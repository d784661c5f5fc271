// Attention output projection ("DeepSeek-V3 Technical Report" notes, MLA
// section, the equation after the attention-output equation):
//
//   u_t = W^O [o_{t,1}; o_{t,2}; ...; o_{t,n_h}],   W^O in R^{d x d_h n_h}
//
// With K = n_h d_h (16384 for DeepSeek-V2) and the few query tokens of a
// decode step, this is a skinny GEMM that streams W^O (d x K bf16, 168 MB
// for d = 5120) from HBM once per group of up to 256 tokens; the tokens'
// concatenated heads (M x K bf16) are re-read from L2 by every feature block.
//
// Matrix-core path (bf16 W^O and o, d % 4 == 0, K % 256 == 0):
//   * Workgroup (feature block of 32 NW rows of W^O, K block of up to 2048,
//     group of up to MT token tiles of 32).  Stages of 64 K pass through an
//     LDS ring, HBM/L2 -> LDS by buffer loads that write LDS directly,
//     NBUF - 1 stages ahead.  Inside a row, 16-byte unit c of the 8 sits at
//     position c ^ ((row >> 1) & 7), so the MFMA operand reads of 16
//     consecutive rows fall on 16 distinct 4-bank groups.
//   * Up to 32 tokens (out_proj_mfma_kernel): NW waves, wave w owns features
//     32w..32w+31 and copies its own W^O rows; for DeepSeek-V2 (d = 5120,
//     K = 16384) NW = 5, 6 slots, 32 x 8 = 256 workgroups, one per CU.
//   * Groups of 4 or 8 token tiles (out_proj_wide_kernel): 4 waves, each
//     computing its share of the token tiles against all of the block's
//     rows, so every SIMD carries the same number of MFMAs.
//   * Workgroups are placed so that those of one XCD share a K block: the
//     tokens' rows of that K range then come from that XCD's L2.
//   * D[feature, token] += W^O[feature, k16] x[token, k16]^T with
//     v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 16 per 32 x 32 tile).
//   * Each K block writes an fp32 partial [M, d]; out_proj_reduce_kernel sums
//     the K blocks into u (fp32 or bf16 round-to-nearest-even).
//   * W^O is read row-major, or from a panel layout (32 x 64 panels, each
//     32-row strip contiguous) written once by out_proj_pack_kernel: there a
//     stage of a strip is one 4 KB piece of memory.
// General path: any dims and dtypes, one thread per output element (slow;
// for small shapes and fp32 operands).
#include <algorithm>

#include "mla_common.hpp"

namespace mla {

namespace {
constexpr uint32_t kOpOOB = 0x40000000u;
}  // namespace

// A stage's tile holds U 16-byte units (8 K each) of every row, rows at a
// pitch of 16 U bytes.  Unit c of row r sits at position c ^ g(r), g(r) =
// (r >> 1) & 7 for U = 8 (128-byte rows: two rows share the 64 banks) and
// r & 15 for U = 16, so that the operand reads of 16 consecutive rows (same
// c) fall on 16 distinct 4-bank groups.
template <int U>
__device__ inline int op_g(int r) {
  return U == 4 ? ((r >> 2) & 3) : U == 8 ? ((r >> 1) & 7) : (r & 15);
}
template <int U>
__device__ inline int op_swz(int r, int c) {
  return r * (16 * U) + ((c ^ op_g<U>(r)) << 4);
}

// Source offset (bytes, from the tile's first row) of what lane `lane` of
// copy n brings to LDS: copy n fills LDS bytes 1024 n .. +1023, i.e. rows
// (64/U) n .. +64/U-1, unit position lane % U of row (64/U) n + lane / U.
template <int U>
__device__ inline uint32_t op_src(int n, int lane, size_t row_bytes) {
  const int r = (64 / U) * n + lane / U, pos = lane % U;
  const int c = pos ^ op_g<U>(r);
  return uint32_t(r * row_bytes + 16 * c);
}

// s_waitcnt vmcnt(n) for a wave-uniform n <= 63
__device__ inline void op_wait_vm(int n) {
  switch (n) {
#define MLA_W(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    MLA_W(0) MLA_W(1) MLA_W(2) MLA_W(3) MLA_W(4) MLA_W(5) MLA_W(6) MLA_W(7) MLA_W(8)
    MLA_W(9) MLA_W(10) MLA_W(11) MLA_W(12) MLA_W(13) MLA_W(14) MLA_W(15) MLA_W(16)
    MLA_W(17) MLA_W(18) MLA_W(19) MLA_W(20) MLA_W(21) MLA_W(22) MLA_W(23) MLA_W(24)
    MLA_W(25) MLA_W(26) MLA_W(27) MLA_W(28) MLA_W(29) MLA_W(30) MLA_W(31) MLA_W(32)
    MLA_W(33) MLA_W(34) MLA_W(35) MLA_W(36) MLA_W(37) MLA_W(38) MLA_W(39) MLA_W(40)
    MLA_W(41) MLA_W(42) MLA_W(43) MLA_W(44) MLA_W(45) MLA_W(46) MLA_W(47) MLA_W(48)
    MLA_W(49) MLA_W(50) MLA_W(51) MLA_W(52) MLA_W(53) MLA_W(54) MLA_W(55) MLA_W(56)
    MLA_W(57) MLA_W(58) MLA_W(59) MLA_W(60) MLA_W(61) MLA_W(62) MLA_W(63)
#undef MLA_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// Block coordinates of this workgroup on a 1-D grid of nfb x nkb x token
// groups.  Consecutive logical indices go to one XCD (xcd_logical_index) and
// the feature block varies fastest, so the workgroups of an XCD share their
// K block: the tokens' rows of that K range are read from HBM once per XCD
// and then hit that XCD's L2.
__device__ inline void op_block(int nfb, int nkb, int& fb, int& kb, int& tg) {
  const int L = xcd_logical_index(blockIdx.x, gridDim.x);
  fb = L % nfb;
  kb = (L / nfb) % nkb;
  tg = L / (nfb * nkb);
}

// Where the W^O operand comes from.  Row-major W^O (PK = false): the
// descriptor starts at row f0, column k0 and ends after row d_model - 1, so
// rows past d_model read as zeros; copy n of a stage (64/U rows) reads its
// rows at a pitch of K values.  Panel layout (PK = true, U = 8): element
// (f, k) at ((f/32) (K/64) + k/64) 2048 + (f%32) 64 + k%64, so a stage's 32
// rows of one strip are one contiguous 4 KB panel; copy n reads a quarter of
// the panel of strip f0/32 + n/4 (strips past d_model/32 are given an
// out-of-range offset).  op_w_stage: the byte offset of stage st.
template <bool PK>
__device__ inline u32x4 op_w_rsrc(const uint16_t* w_o, int f0, int k0, int d_model, int K) {
  const uint64_t wa = PK ? (uint64_t)w_o : (uint64_t)(w_o + (size_t)f0 * K + k0);
  const size_t bytes = PK ? (size_t)d_model * K * 2
                          : (size_t)(d_model - f0) * K * 2 - (size_t)k0 * 2;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)wa),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(wa >> 32)) & 0xFFFFu,
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bytes), 0x00020000u};
}
template <int U, bool PK>
__device__ inline uint32_t op_w_src(int n, int lane, int f0, int k0, int d_model, int K) {
  if constexpr (PK) {
    static_assert(U == 8, "panel layout: stages of 64 K");
    const int strip = f0 / 32 + n / 4;
    if (32 * strip >= d_model) return kOpOOB;
    return uint32_t(((size_t)strip * (K / 64) + k0 / 64) * 4096) + op_src<8>(n % 4, lane, 128);
  } else {
    return (f0 + (64 / U) * n + lane / U < d_model) ? op_src<U>(n, lane, (size_t)K * 2) : kOpOOB;
  }
}
template <bool PK>
__device__ inline uint32_t op_w_stage(int st, int ks) {
  return PK ? uint32_t(st) * 4096u : uint32_t(st * ks * 2);
}

// Panel layout of W^O (see op_w_rsrc) from the row-major matrix: one 16-byte
// unit per thread, written in panel order.
__global__ __launch_bounds__(256) void out_proj_pack_kernel(
    const u32x4* __restrict__ w, u32x4* __restrict__ wp, int d_model, int K) {
  const size_t units = (size_t)d_model * K / 8;
  const int kp = K / 64;
  for (size_t p = (size_t)blockIdx.x * 256 + threadIdx.x; p < units;
       p += (size_t)gridDim.x * 256) {
    const size_t panel = p >> 8;
    const int within = int(p & 255), r = within >> 3, c = within & 7;
    const size_t strip = panel / kp;
    const int kt = int(panel % kp);
    wp[p] = w[((32 * strip + r) * K + 64 * kt + 8 * c) / 8];
  }
}

// NW waves (feature block of 32 NW rows of W^O), up to MT token tiles of 32,
// NBUF ring slots (NBUF - 1 stages copied ahead of the one computed), stages
// of 8 U values of K (U 16-byte units per row).
template <int NW, int MT, int NBUF, int U, bool PK>
__global__ __launch_bounds__(64 * NW) void out_proj_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_o,
    float* __restrict__ part, int n_tok, int d_model, int K, int kb_size, int nfb, int nkb) {
  constexpr int OP_KS = 8 * U;                   // K per stage
  const int OP_NST = kb_size / OP_KS;            // stages per workgroup
  constexpr int CPR = U / 2;                     // 1 KB copies per 32 rows
  constexpr int WBYTES = 32 * NW * OP_KS * 2;    // W^O rows of a stage
  constexpr int XBYTES = 32 * OP_KS * 2;         // per token tile
  constexpr int SLOT = WBYTES + MT * XBYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF][SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int fb, kb, tg;
  op_block(nfb, nkb, fb, kb, tg);
  const int f0 = fb * 32 * NW, k0 = kb * kb_size, t0 = tg * (32 * MT);
  const int mt = min(MT, (n_tok - t0 + 31) / 32);           // token tiles in this group
  const size_t row_bytes = (size_t)K * 2;

  // buffer descriptors: W^O rows f0 .. f0+32NW-1, token rows t0 .. n_tok-1
  // (rows past n_tok are out of range: the hardware writes zeros)
  const u32x4 wrs = op_w_rsrc<PK>(w_o, f0, k0, d_model, K);
  const uint64_t xa = (uint64_t)(x + (size_t)t0 * K + k0);
  const u32x4 xrs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)xa),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(xa >> 32)) & 0xFFFFu,
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(
                         (size_t)(n_tok - t0) * row_bytes - (size_t)k0 * 2)),
                     0x00020000u};
  // wave w copies its own 32 W^O rows (copies CPR w .. CPR w + CPR-1 of the
  // stage) and, for w < 4, copies CPR/4 w .. of every token tile; the
  // stage's K offset goes in the scalar offset
  constexpr int XPW = CPR / 4;                   // token-tile copies per copying wave
  uint32_t wsrc[CPR];
#pragma unroll
  for (int j = 0; j < CPR; ++j) wsrc[j] = op_w_src<U, PK>(CPR * wave + j, lane, f0, k0, d_model, K);
  uint32_t xsrc[MT][XPW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < XPW; ++j) {
      const int n = XPW * (wave & 3) + j;
      const uint32_t o = op_src<U>(n, lane, row_bytes) + uint32_t(32 * t) * uint32_t(row_bytes);
      xsrc[t][j] = (32 * t + (64 / U) * n + lane / U < n_tok - t0) ? o : kOpOOB;
    }
  const bool x_copier = wave < 4;
  const int per_stage = CPR + (x_copier ? XPW * mt : 0);    // this wave's copies per stage
  const uint32_t lds0 = (uint32_t)(uintptr_t)&ring[0][0];

  auto issue = [&](int st) {           // copies of stage st into slot st % NBUF
    const uint32_t slot = lds0 + (st % NBUF) * SLOT;
    const uint32_t koff = __builtin_amdgcn_readfirstlane(st * OP_KS * 2);
    const uint32_t kwoff = __builtin_amdgcn_readfirstlane(op_w_stage<PK>(st, OP_KS));
#pragma unroll
    for (int j = 0; j < CPR; ++j)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :: "s"(slot + 1024 * (CPR * wave + j)), "v"(wsrc[j]), "s"(wrs), "s"(kwoff)
                   : "memory");
    if (x_copier) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if (t < mt)
#pragma unroll
          for (int j = 0; j < XPW; ++j)
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                         :: "s"(slot + WBYTES + XBYTES * t + 1024 * (XPW * wave + j)),
                            "v"(xsrc[t][j]), "s"(xrs), "s"(koff)
                         : "memory");
    }
  };

  floatx16 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx16{};
  // operand reads: row l % 32 of the wave's 32 features / of a token tile,
  // 16-byte unit 2 s + l / 32 for k16 step s of the stage
  const int r32 = lane & 31, hh = lane >> 5;

  constexpr int AHEAD = NBUF - 1;
  for (int st = 0; st < AHEAD && st < OP_NST; ++st) issue(st);
  for (int st = 0; st < OP_NST; ++st) {
    // stage st landed: the later stages' copies may still fly
    op_wait_vm(min(AHEAD - 1, OP_NST - 1 - st) * per_stage);
    __syncthreads();                   // every wave's copies landed; stage st-1 was read
    if (st + AHEAD < OP_NST) issue(st + AHEAD);
    const uint8_t* slot = &ring[st % NBUF][0];
#pragma unroll
    for (int s = 0; s < U / 2; ++s) {
      const int c = 2 * s + hh;
      const bf16x8 a = *(const bf16x8*)(slot + op_swz<U>(32 * wave + r32, c));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t < mt) {
          const bf16x8 b = *(const bf16x8*)(slot + WBYTES + XBYTES * t + op_swz<U>(r32, c));
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
        }
      }
    }
  }
  // acc[t][r]: feature f0 + 32 wave + 8 (r/4) + 4 hh + r%4, token t0 + 32 t + r32
  float* pk = part + (size_t)kb * n_tok * d_model;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tok = t0 + 32 * t + r32;
    if (t < mt && tok < n_tok) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = f0 + 32 * wave + 8 * q + 4 * hh;      // 4 features; d_model % 4 == 0
        if (f < d_model)
          *(floatx4*)(pk + (size_t)tok * d_model + f) =
              floatx4{acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
      }
    }
  }
}

// Groups of MT = 4 or 8 token tiles: 4 waves, each computing MT/4 token
// tiles against all NM M tiles (32 NM rows of W^O) of the block, so the
// four SIMDs carry the same number of MFMAs.  Stages of 64 K (U = 8) as in
// out_proj_mfma_kernel; per stage each wave copies NM KB of W^O rows and
// 1 KB of every token tile.
template <int NM, int MT, int NBUF, int U, bool PK>
__global__ __launch_bounds__(256) void out_proj_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_o,
    float* __restrict__ part, int n_tok, int d_model, int K, int kb_size, int nfb, int nkb) {
  constexpr int OP_KS = 8 * U;                   // K per stage
  const int OP_NST = kb_size / OP_KS;            // stages per workgroup
  constexpr int WBYTES = 32 * NM * OP_KS * 2;    // W^O rows of a stage
  constexpr int XBYTES = 32 * OP_KS * 2;         // per token tile
  constexpr int SLOT = WBYTES + MT * XBYTES;
  constexpr int NT = MT / 4;                     // token tiles per wave
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF][SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int fb, kb, tg;
  op_block(nfb, nkb, fb, kb, tg);
  const int f0 = fb * 32 * NM, k0 = kb * kb_size, t0 = tg * (32 * MT);
  const int mt = min(MT, (n_tok - t0 + 31) / 32);           // token tiles in this group
  const size_t row_bytes = (size_t)K * 2;

  // buffer descriptors as in out_proj_mfma_kernel: rows past d_model or
  // past n_tok are out of range (the hardware writes zeros)
  const u32x4 wrs = op_w_rsrc<PK>(w_o, f0, k0, d_model, K);
  const uint64_t xa = (uint64_t)(x + (size_t)t0 * K + k0);
  const u32x4 xrs = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)xa),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(xa >> 32)) & 0xFFFFu,
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(
                         (size_t)(n_tok - t0) * row_bytes - (size_t)k0 * 2)),
                     0x00020000u};
  // A stage holds WCP 1 KB copies of W^O rows (64/U rows each) and XCP
  // copies per token tile; wave w takes copies w, w + 4, ... of each.
  constexpr int WCP = WBYTES / 1024, XCP = XBYTES / 1024;
  constexpr int WPW = (WCP + 3) / 4, XPW = (XCP + 3) / 4;   // per wave, at most
  const int wcnt = (WCP - wave + 3) / 4, xcnt = (XCP - wave + 3) / 4;
  uint32_t wsrc[WPW];
#pragma unroll
  for (int j = 0; j < WPW; ++j) wsrc[j] = op_w_src<U, PK>(wave + 4 * j, lane, f0, k0, d_model, K);
  uint32_t xsrc[MT][XPW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < XPW; ++j) {
      const int n = wave + 4 * j;
      const uint32_t o = op_src<U>(n, lane, row_bytes) + uint32_t(32 * t) * uint32_t(row_bytes);
      xsrc[t][j] = (32 * t + (64 / U) * n + lane / U < n_tok - t0) ? o : kOpOOB;
    }
  const int per_stage = wcnt + mt * xcnt;       // this wave's copies per stage
  const uint32_t lds0 = (uint32_t)(uintptr_t)&ring[0][0];

  auto issue = [&](int st) {           // copies of stage st into slot st % NBUF
    const uint32_t slot = lds0 + (st % NBUF) * SLOT;
    const uint32_t koff = __builtin_amdgcn_readfirstlane(st * OP_KS * 2);
    const uint32_t kwoff = __builtin_amdgcn_readfirstlane(op_w_stage<PK>(st, OP_KS));
#pragma unroll
    for (int j = 0; j < WPW; ++j)
      if (j < wcnt)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(slot + 1024 * (wave + 4 * j)), "v"(wsrc[j]), "s"(wrs), "s"(kwoff)
                     : "memory");
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < XPW; ++j)
        if (t < mt && j < xcnt)
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                       :: "s"(slot + WBYTES + XBYTES * t + 1024 * (wave + 4 * j)),
                          "v"(xsrc[t][j]), "s"(xrs), "s"(koff)
                       : "memory");
  };

  floatx16 acc[NM][NT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[m][j] = floatx16{};
  const int r32 = lane & 31, hh = lane >> 5;

  constexpr int AHEAD = NBUF - 1;
  for (int st = 0; st < AHEAD && st < OP_NST; ++st) issue(st);
  for (int st = 0; st < OP_NST; ++st) {
    op_wait_vm(min(AHEAD - 1, OP_NST - 1 - st) * per_stage);
    __syncthreads();                   // every wave's copies landed; stage st-1 was read
    if (st + AHEAD < OP_NST) issue(st + AHEAD);
    const uint8_t* slot = &ring[st % NBUF][0];
#pragma unroll
    for (int s = 0; s < U / 2; ++s) {
      const int c = 2 * s + hh;
      bf16x8 b[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        b[j] = *(const bf16x8*)(slot + WBYTES + XBYTES * (NT * wave + j) + op_swz<U>(r32, c));
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x8 a = *(const bf16x8*)(slot + op_swz<U>(32 * m + r32, c));
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[m][j], 0, 0, 0);
      }
    }
  }
  // acc[m][j][r]: feature f0 + 32 m + 8 (r/4) + 4 hh + r%4, token
  // t0 + 32 (NT wave + j) + r32
  float* pk = part + (size_t)kb * n_tok * d_model;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int tok = t0 + 32 * (NT * wave + j) + r32;
    if (tok < n_tok) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = f0 + 32 * m + 8 * q + 4 * hh;       // 4 features; d_model % 4 == 0
          if (f < d_model)
            *(floatx4*)(pk + (size_t)tok * d_model + f) =
                floatx4{acc[m][j][4 * q], acc[m][j][4 * q + 1], acc[m][j][4 * q + 2],
                        acc[m][j][4 * q + 3]};
        }
    }
  }
}

// u = sum over the K blocks of the partials; four consecutive outputs per thread.
template <typename OutT>
__global__ __launch_bounds__(256) void out_proj_reduce_kernel(
    const float* __restrict__ part, OutT* __restrict__ u, size_t n4, int nkb) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  // every K block's partial is loaded before any is added (at most 16 in
  // flight), then summed in K-block order
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nkb; k0 += 16) {
    floatx4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k0 + k < nkb) v[k] = *(const floatx4*)(part + (size_t)(k0 + k) * 4 * n4 + 4 * i);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k0 + k < nkb) s += v[k];
  }
  if constexpr (sizeof(OutT) == 4) {
    *(floatx4*)(u + 4 * i) = s;
  } else {
    *(u32x2*)(u + 4 * i) = u32x2{uint32_t(f32_to_bf16_bits(s[0])) | (uint32_t(f32_to_bf16_bits(s[1])) << 16),
                                 uint32_t(f32_to_bf16_bits(s[2])) | (uint32_t(f32_to_bf16_bits(s[3])) << 16)};
  }
}

template <typename T>
__device__ inline float op_load(const T* p, size_t i) {
  if constexpr (sizeof(T) == 4) return p[i];
  else return bf16_bits_to_f32(p[i]);
}

// General path: u[n, f] = sum_k x[n, k] W^O[f, k], one thread per output.
template <typename XT, typename WT, typename OutT>
__global__ __launch_bounds__(256) void out_proj_general_kernel(
    const XT* __restrict__ x, const WT* __restrict__ w_o, OutT* __restrict__ u, int n_tok,
    int d_model, int K) {
  const size_t total = (size_t)n_tok * d_model;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * 256) {
    const size_t n = idx / d_model, f = idx % d_model;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(op_load(x, n * K + k), op_load(w_o, f * K + k), acc);
    if constexpr (sizeof(OutT) == 4) u[idx] = acc;
    else u[idx] = f32_to_bf16_bits(acc);
  }
}

// out [n_tok, d_out] = x [n_tok, K] W [d_out, K]^T.  Matrix-core path: bf16
// x and W, d_out % 4 == 0, K % 256 == 0.
bool gemm_xwt_fast(int d_out, int K, int x_dtype, int w_dtype) {
  return x_dtype == MLA_BF16 && w_dtype == MLA_BF16 && d_out > 0 && d_out % 4 == 0 &&
         K % 256 == 0;
}

namespace {
// feature blocks of 160 rows (5 waves) when they divide d_out, else 128 (the
// last block may be partial); K blocks of 2048 or less, halved (while they
// divide K and hold at least 4 stages) until there are 256 workgroups
struct GemmPlan { int nw, nfb, kb, nkb; };
GemmPlan gemm_plan(int d_out, int K) {
  GemmPlan p;
  p.nw = (d_out % 160 == 0) ? 5 : 4;
  p.nfb = (d_out + 32 * p.nw - 1) / (32 * p.nw);
  p.kb = 2048;
  while (p.kb > 256 && (K % p.kb != 0 || (int64_t)p.nfb * (K / p.kb) < kNumCU)) p.kb /= 2;
  p.nkb = K / p.kb;
  return p;
}
}  // namespace

size_t gemm_xwt_workspace(int d_out, int K, int n_tok, int x_dtype, int w_dtype) {
  if (!gemm_xwt_fast(d_out, K, x_dtype, w_dtype)) return 0;
  return (size_t)gemm_plan(d_out, K).nkb * n_tok * d_out * sizeof(float);
}

bool gemm_xwt_packable(int d_out, int K, int x_dtype, int w_dtype) {
  return gemm_xwt_fast(d_out, K, x_dtype, w_dtype) && d_out % 32 == 0 &&
         (int64_t)d_out * K * 2 <= 0x7FFFFFFF;
}

hipError_t launch_gemm_pack(const void* w, void* w_packed, int d_out, int K, hipStream_t st) {
  const size_t units = (size_t)d_out * K / 8;
  const int grid = (int)std::min<size_t>((units + 255) / 256, 8192);
  hipLaunchKernelGGL(out_proj_pack_kernel, dim3(grid), dim3(256), 0, st, (const u32x4*)w,
                     (u32x4*)w_packed, d_out, K);
  return hipGetLastError();
}

int gemm_xwt_nkb(int d_out, int K) { return gemm_plan(d_out, K).nkb; }

// The matrix-core path: partial sums [nkb, n_tok, d_out] fp32 into
// workspace, then (when out != nullptr) their sum into out.
hipError_t launch_gemm_xwt(const void* x, int x_dtype, const void* w, int w_dtype,
                           void* out, bool out_f32, int n_tok, int d_out, int K,
                           void* workspace, hipStream_t st, bool packed) {
  if (packed && !gemm_xwt_packable(d_out, K, x_dtype, w_dtype)) return hipErrorInvalidValue;
  if (!out && !gemm_xwt_fast(d_out, K, x_dtype, w_dtype)) return hipErrorInvalidValue;
  if (gemm_xwt_fast(d_out, K, x_dtype, w_dtype)) {
    // one token tile with a 6-slot ring for at most 32 tokens, groups of 4
    // token tiles with a 4-slot ring up to 128 tokens, else groups of 8
    // token tiles (W streamed once per 256 tokens) with a 3-slot ring
    const GemmPlan p = gemm_plan(d_out, K);
    const int nw = p.nw, kb = p.kb;
    int mt = (n_tok <= 32) ? 1 : (n_tok <= 128) ? 4 : 8;
    // groups of 8 token tiles that would leave more than half of the CUs
    // idle (few feature blocks, e.g. the 576 rows of the cache producer):
    // groups of 4, twice the workgroups, W streamed once per 128 tokens
    if (mt == 8 && (int64_t)p.nfb * p.nkb * ((n_tok + 255) / 256) < kNumCU / 2) mt = 4;
    const int ntg = (n_tok + 32 * mt - 1) / (32 * mt);
    const dim3 grid(p.nfb * p.nkb * ntg);
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)w;
    float* pp = (float*)workspace;
    const int nfb = p.nfb, nkb = p.nkb;
#define MLA_OPK(KER, THREADS) \
    hipLaunchKernelGGL(KER, grid, dim3(THREADS), 0, st, xp, wp, pp, n_tok, d_out, K, kb, nfb, nkb)
#define MLA_OPK_ALL(PK)                                                                     \
    if (nw == 5 && mt == 1) MLA_OPK((out_proj_mfma_kernel<5, 1, 6, 8, PK>), 320);           \
    else if (nw == 5 && mt == 4) MLA_OPK((out_proj_wide_kernel<5, 4, 4, 8, PK>), 256);      \
    else if (nw == 5) MLA_OPK((out_proj_wide_kernel<5, 8, 3, 8, PK>), 256);                 \
    else if (mt == 1) MLA_OPK((out_proj_mfma_kernel<4, 1, 6, 8, PK>), 256);                 \
    else if (mt == 4) MLA_OPK((out_proj_wide_kernel<4, 4, 4, 8, PK>), 256);                 \
    else MLA_OPK((out_proj_wide_kernel<4, 8, 3, 8, PK>), 256);
    if (packed) { MLA_OPK_ALL(true) } else { MLA_OPK_ALL(false) }
#undef MLA_OPK_ALL
#undef MLA_OPK
    if (!out) return hipGetLastError();
    const size_t n4 = (size_t)n_tok * d_out / 4;
    const dim3 rgrid((unsigned)((n4 + 255) / 256));
    if (out_f32)
      hipLaunchKernelGGL(out_proj_reduce_kernel<float>, rgrid, dim3(256), 0, st,
                         (const float*)workspace, (float*)out, n4, p.nkb);
    else
      hipLaunchKernelGGL(out_proj_reduce_kernel<uint16_t>, rgrid, dim3(256), 0, st,
                         (const float*)workspace, (uint16_t*)out, n4, p.nkb);
    return hipGetLastError();
  }
  const size_t total = (size_t)n_tok * d_out;
  const int grid = (int)std::min<size_t>((total + 255) / 256, 65535);
#define MLA_OP(XT, WT, OT)                                                               \
  hipLaunchKernelGGL((out_proj_general_kernel<XT, WT, OT>), dim3(grid), dim3(256), 0, st, \
                     (const XT*)x, (const WT*)w, (OT*)out, n_tok, d_out, K)
  if (x_dtype == MLA_F32) {
    if (w_dtype == MLA_F32) { if (out_f32) MLA_OP(float, float, float); else MLA_OP(float, float, uint16_t); }
    else { if (out_f32) MLA_OP(float, uint16_t, float); else MLA_OP(float, uint16_t, uint16_t); }
  } else {
    if (w_dtype == MLA_F32) { if (out_f32) MLA_OP(uint16_t, float, float); else MLA_OP(uint16_t, float, uint16_t); }
    else { if (out_f32) MLA_OP(uint16_t, uint16_t, float); else MLA_OP(uint16_t, uint16_t, uint16_t); }
  }
#undef MLA_OP
  return hipGetLastError();
}

}  // namespace mla
