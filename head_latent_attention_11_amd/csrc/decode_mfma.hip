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
//   * Wave w owns 32 rows.  Its absorbed queries live in VGPRs for the whole
//     item (36 MFMA operands of 8 bf16 = 144 VGPRs) and its output
//     accumulator O^T (512 x 32 fp32 = 256 registers) stays in the matrix
//     accumulators.
//   * KV tiles of 32 tokens are staged in LDS (double buffered, rows padded
//     to 1168 bytes so the 16-byte operand reads of 16 consecutive tokens hit
//     distinct banks).  fp8 tiles are decoded to bf16 while staging; the
//     per-token scale multiplies the score and is folded into P for the PV
//     product, so the fp8 values themselves enter the bf16 MFMA exactly.
//   * S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 so that each
//     lane holds one head's 16 token scores: the per-head max and sum need
//     no cross-lane reduction except with the partner lane (lane ^ 32).  The
//     probability registers are then already in the operand layout of the PV
//     product O^T += C^T P^T (token order inside the K dimension is chosen to
//     match the score layout).
//   * Softmax in the log2 domain against a per-row reference m_ref instead
//     of a running max: m_ref is the max of the first tile in which the row
//     sees a token, and p = 2^(s - m_ref) is accumulated without rescaling
//     (fp32 and bf16 share an 8-bit exponent, so p up to 2^64 is safe).  If
//     a later score exceeds m_ref by more than 64 the whole workgroup
//     restarts the work item with m_ref raised to the max seen so far; each
//     restart raises m_ref by more than 64, so restarts are rare and finite.
//     The result is exact for any reference: LSE = m_ref + log2(sum p).
#include <math.h>

#include "mla_common.hpp"
#include "plan_device.hpp"

namespace mla {

namespace {
constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int TILE = 32;                 // tokens per staged tile
constexpr int LROW = 1168;               // LDS bytes per token row (1152 + 16 pad)
constexpr int NCH = 72;                  // 16-byte bf16 chunks per row
constexpr int NSTG = TILE * NCH / 256;   // staging chunks per thread (9)
constexpr float kNegInf = -INFINITY;
}  // namespace

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 E4M3 codes -> 8 bf16 values (exact: every E4M3 value is a bf16 value).
__device__ inline u32x4 fp8x8_to_bf16x8(u32x2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true));
  return r;
}

template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][TILE * LROW];
  __shared__ float s_scale[2][TILE];
  __shared__ int s_restart;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = xcd_logical_index(blockIdx.x, gridDim.x);
  const int item = g / a.row_blocks, rb = g % a.row_blocks;
  const ItemLoc loc = locate_item(a.seq_lens, a.B, a.num_splits, a.chunk, item);
  if (loc.b < 0) return;
  const int b = loc.b;
  const int L = a.seq_lens[b];
  const int c = chunk_of(L, a.num_splits, a.chunk);
  const int t0 = loc.s * c;
  const int t_end = min(L, t0 + c);                       // item end
  const int rows = a.n_h * a.T;
  const int row = rb * 128 + wave * 32 + l32;             // this lane's row
  const int tau = row / a.n_h, head = row % a.n_h;
  const int lim = min(t_end - 1, L - a.T + tau);          // last visible token
  const int tau_max = (rb * 128 + 127) / a.n_h;
  const int t_stage = min(t_end, L - a.T + tau_max + 1);  // tokens any row sees
  const int nq = b * a.T + tau;

  // ---- absorbed query rows -> MFMA B operands (lane: head l32, 8 dims)
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = (const uint16_t*)a.q_abs + ((size_t)nq * a.n_h + head) * D;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) qf[k] = *(const bf16x8*)(qrow + 16 * k + 8 * h);
  }

  floatx16 o[DC / 32];
  float m_ref = kNegInf, m_seen = kNegInf, l_run = 0.f;

  const uint8_t* cache = (const uint8_t*)a.cache;
  constexpr int ESZ = FP8 ? 1 : 2;

  // first cache row of the tile starting at token ts (a tile never crosses
  // a page: ts is a multiple of 32 and pages hold 64 tokens)
  auto tile_row = [&](int ts) -> size_t {
    if (a.page_table)
      return (size_t)a.page_table[(size_t)b * a.max_pages + ts / kPage] * kPage + (ts % kPage);
    return (size_t)b * a.max_len + ts;
  };

  // Staging: a 32-token tile is one contiguous run of cache rows (a tile
  // never crosses a page), read with buffer loads whose range ends at the
  // last valid token: loads past it return zero, so masked tokens enter
  // the PV product as exact zeros.  Chunk ci of the tile sits at byte
  // CH*ci in memory and at 16*ci + 16*(ci/72) in LDS (rows padded).
  constexpr int CH = FP8 ? 8 : 16;     // bytes per staged chunk
  u32x4 stg16[FP8 ? 1 : NSTG];
  u32x2 stg8[FP8 ? NSTG : 1];
  float stg_scale = 0.f;

  auto stage_load = [&](int ts) {
    const size_t r0 = tile_row(ts);
    const int nvalid = min(TILE, t_stage - ts);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cache + r0 * (size_t)(D * ESZ)), (short)0, nvalid * D * ESZ, 0x00020000);
#pragma unroll
    for (int i = 0; i < NSTG; ++i) {
      if (FP8)
        stg8[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, CH * tid, CH * 256 * i, 0));
      else
        stg16[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, CH * tid, CH * 256 * i, 0));
    }
    if (FP8 && tid < TILE) stg_scale = (tid < nvalid) ? a.kv_scale[r0 + tid] : 0.f;
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NSTG; ++i) {
      const int ci = tid + 256 * i;
      u32x4 v = FP8 ? fp8x8_to_bf16x8(stg8[i]) : stg16[i];
      *(u32x4*)(&s_kv[buf][16 * ci + 16 * (ci / NCH)]) = v;
    }
    if (FP8 && tid < TILE) s_scale[buf][tid] = stg_scale;
  };

  const int ntiles = (t_stage > t0) ? (t_stage - t0 + TILE - 1) / TILE : 0;
  if (tid == 0) s_restart = 0;
  for (;;) {                          // attempts (a restart is rare)
#pragma unroll
  for (int i = 0; i < DC / 32; ++i) o[i] = floatx16{};
  l_run = 0.f;
  if (ntiles > 0) {
    stage_load(t0);
    stage_store(0);
  }
  __syncthreads();

  int restart = 0;
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int ts = t0 + it * TILE;
    if (it + 1 < ntiles) stage_load(ts + TILE);

    const uint8_t* kb = s_kv[cur];
    // ---- S^T[token, head] = sum_d K[token, d] Q[head, d]
    floatx16 sa = {};
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
      const bf16x8 a0 = *(const bf16x8*)(kb + l32 * LROW + 32 * k + 16 * h);
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[k], sa, 0, 0, 0);
    }
    // ---- scores of this lane's head: register r holds token
    //      8*(r/4) + 4*h + r%4 of the tile
    float s[16];
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tl = 8 * (r >> 2) + 4 * h + (r & 3);
      float v = sa[r] * a.scale_log2;
      if (FP8) v *= s_scale[cur][tl];
      s[r] = (ts + tl <= lim) ? v : kNegInf;
      mt = fmaxf(mt, s[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    m_seen = fmaxf(m_seen, mt);
    if (m_ref == kNegInf) m_ref = mt;          // O and l are still zero here
    if (mt > m_ref + 64.0f) s_restart = 1;
    const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r] - m_use);
      if (FP8) {
        l_run += p;
        pf[r >> 3][r & 7] = (__bf16)(p * s_scale[cur][8 * (r >> 2) + 4 * h + (r & 3)]);
      } else {
        // the normaliser sums exactly the rounded weights used in P C
        const __bf16 pb = (__bf16)p;
        l_run += (float)pb;
        pf[r >> 3][r & 7] = pb;
      }
    }
    // ---- O^T[dim, head] += sum_tok C^T[dim, tok] P^T[tok, head]
#pragma unroll
    for (int db = 0; db < DC / 32; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tl = 16 * ks + 8 * (e >> 2) + 4 * h + (e & 3);
          vf[e] = *(const __bf16*)(kb + tl * LROW + (32 * db + l32) * 2);
        }
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[db], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) stage_store(cur ^ 1);
    __syncthreads();
    restart = s_restart;              // uniform: read after the barrier
    if (restart) break;
  }
  if (!restart) break;
  __syncthreads();                    // everyone has read the flag
  if (tid == 0) s_restart = 0;
  m_ref = m_seen;
  }

  // ---- normalise and write (the final output, or this split's partial)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  const float lse = (l_tot > 0.f) ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : kNegInf;
  float* dst;
  float* dlse;
  if (loc.ns == 1) {
    dst = a.out_latent + ((size_t)nq * a.n_h + head) * DC;
    dlse = a.out_lse + (size_t)nq * a.n_h + head;
  } else {
    dst = a.part_o + ((size_t)item * rows + row) * DC;
    dlse = a.part_lse + (size_t)item * rows + row;
  }
#pragma unroll
  for (int db = 0; db < DC / 32; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 v = {o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]};
      *(floatx4*)(dst + 32 * db + 8 * j + 4 * h) = v * inv;
    }
  }
  if (h == 0) *dlse = lse;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  const int grid = a.n_items * a.row_blocks;
  if (a.kv_dtype == MLA_FP8_E4M3)
    hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(decode_mfma_kernel<false>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
