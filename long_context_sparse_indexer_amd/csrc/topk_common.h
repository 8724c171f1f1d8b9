// Per-row radix-select state shared by the indexer epilogue and the top-k kernels.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkBins = 4096;  // bins of one 12-bit key digit

// Digit-1 histogram replicas per row: block b merges into copy b % copies.  With few rows, hundreds of blocks
// of one row hit the same popular bins, and replicas keep those atomics to a few dozen per address; with many
// rows the atomics spread over the rows' own histograms and one copy avoids clearing megabytes of replicas.
__host__ __device__ constexpr int hist_copies(int R) { return R <= 8 ? 8 : R <= 16 ? 4 : R <= 32 ? 2 : 1; }

struct Ws {
  uint32_t* hist1;    // [R, copies, 4096]  digit-1 histogram replicas
  uint32_t* hist2;    // [R, 4096]  digit-2 histogram of keys inside bin b1
  uint32_t* cnt;      // [R, 4]     unused, unused, candidates reserved, unused
  uint32_t* thr;      // [R, 4]     b1, keys above b1 (written by the filter's first block)
  uint32_t* seg_cnt;  // [R, nblk]  candidates of each chunk
  uint32_t* seg_off;  // [R, nblk]  where each chunk's candidates start in the row's list
  uint64_t* cand;     // [R, cap]   candidates: position << 32 | key
  int nblk;
  int copies;
};

// Merges a block's LDS histogram `h` (complete: a barrier after its last update) into a global histogram
// with one device-scope atomic per non-empty bin.  Consumers read the global histogram in a later kernel.
template <int NT>
__device__ __forceinline__ void hist_merge(const uint32_t* h, uint32_t* gh) {
  for (int i = threadIdx.x; i < kTopkBins; i += NT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

}  // namespace dsa
