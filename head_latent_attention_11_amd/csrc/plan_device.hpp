// Device-side lookup of a split-KV work item.
//
// Work items are numbered sequence-major: the ns_b = splits_of(L_b) chunks of
// sequence 0 first, then those of sequence 1, ...  Every workgroup recomputes
// the prefix sums it needs from seq_lens (a few hundred integers, L2
// resident), so no plan has to be copied from the host.
#pragma once

#include "mla_common.hpp"

namespace mla {

struct ItemLoc {
  int b;       // sequence
  int s;       // split index within the sequence
  int ns;      // number of splits of the sequence
  int first;   // index of the sequence's first work item
};

// Block-cooperative: every thread of the workgroup must call it with the
// same arguments; blockDim.x must be a multiple of 64 and at most 1024.
// Returns b = -1 when `item` lies beyond the last work item.
__device__ inline ItemLoc locate_item(const int32_t* __restrict__ seq_lens,
                                      int B, int num_splits, int chunk,
                                      int item) {
  __shared__ int s_wave_sum[16];
  __shared__ ItemLoc s_loc;
  __shared__ int s_found;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
  if (tid == 0) { s_found = 0; s_loc.b = -1; s_loc.s = 0; s_loc.ns = 0; s_loc.first = 0; }
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < B; base += nthr) {
    const int bb = base + tid;
    const int ns = (bb < B) ? splits_of(seq_lens[bb], num_splits, chunk) : 0;
    // inclusive scan within the wave
    int incl = ns;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) s_wave_sum[wave] = incl;
    __syncthreads();
    int wave_off = 0, total = 0;
    for (int w = 0; w < nwaves; ++w) {
      if (w < wave) wave_off += s_wave_sum[w];
      total += s_wave_sum[w];
    }
    const int excl = carry + wave_off + incl - ns;
    if (ns > 0 && item >= excl && item < excl + ns) {
      s_loc.b = bb; s_loc.s = item - excl; s_loc.ns = ns; s_loc.first = excl;
      s_found = 1;
    }
    __syncthreads();
    if (s_found) break;
    carry += total;
  }
  ItemLoc r = s_loc;
  __syncthreads();
  return r;
}

}  // namespace mla
