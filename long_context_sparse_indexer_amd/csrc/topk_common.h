// Per-row radix-select state shared by the indexer epilogue and the top-k kernels.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkBins = 4096;  // bins of one 12-bit key digit

// Agent-scope acquire: invalidates this CU's view of L2 so that ordinary loads see data other blocks made
// visible (device-scope atomics, write-through stores) before the counter this block observed.
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

struct Ws {
  uint32_t* hist1;    // [R, 4096]  digit-1 histogram
  uint32_t* hist2;    // [R, 4096]  digit-2 histogram of keys inside bin b1
  uint32_t* cnt;      // [R, 4]     blocks done (digit 1), blocks done (filter), candidates reserved, unused
  uint32_t* thr;      // [R, 4]     b1, keys above b1, b2, keys above (b1, b2)
  uint32_t* seg_cnt;  // [R, nblk]  candidates of each chunk
  uint32_t* seg_off;  // [R, nblk]  where each chunk's candidates start in the row's list
  uint64_t* cand;     // [R, cap]   candidates: position << 32 | key
  int nblk;
};

// Called by all NT threads of a block after its last update of the global histogram `gh`: the block that
// finishes the row's `nparts` contributions last finds the bin b holding the need-th largest key (counting
// from the top bin) and sets b and base_above + (keys in bins above b).  Returns true in that block only.
// Histogram updates are device-scope atomics, so their completion (s_waitcnt) before the counter increment
// orders them for the last block, which acquires before reading; no cache write-back is needed.
template <int NT>
__device__ __forceinline__ bool hist_threshold_last(const uint32_t* gh, uint32_t* done, int nparts, uint32_t need,
                                                    uint32_t base_above, uint32_t* thr_b, uint32_t* thr_above,
                                                    uint32_t* scan, int* flag) {
  constexpr int kPer = kTopkBins / NT;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *flag = atomicAdd(done, 1u) == (uint32_t)(nparts - 1);
  __syncthreads();
  if (!*flag) return false;
  acquire_agent();
  const int grp = NT - 1 - threadIdx.x;  // thread 0 owns the top bins
  uint32_t c[kPer];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = gh[grp * kPer + j];
    local += c[j];
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan(local, scan, total);
  if (above < need && above + local >= need) {
    for (int j = kPer - 1; j >= 0; --j) {
      if (above + c[j] >= need) {
        *thr_b = (uint32_t)(grp * kPer + j);
        *thr_above = base_above + above;
        break;
      }
      above += c[j];
    }
  }
  __syncthreads();
  return true;
}

// Merges a block's LDS histogram `h` into the row's global histogram (one atomic per non-empty bin), then
// hist_threshold_last.  `h` must be complete (a barrier after the last LDS update).
template <int NT>
__device__ __forceinline__ void hist_merge_and_threshold(const uint32_t* h, uint32_t* gh, uint32_t* done, int nparts,
                                                         uint32_t need, uint32_t base_above, uint32_t* thr_b,
                                                         uint32_t* thr_above, uint32_t* scan, int* flag) {
  for (int i = threadIdx.x; i < kTopkBins; i += NT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  (void)hist_threshold_last<NT>(gh, done, nparts, need, base_above, thr_b, thr_above, scan, flag);
}

}  // namespace dsa
