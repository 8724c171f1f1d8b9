// Per-row radix-select state shared by the top-k kernels and the indexer that clears it in the fused step.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkBins = 4096;  // bins of a 12-bit key digit, and of the candidate histogram

struct Ws {
  uint32_t* hist;     // [R, 4096]  candidate histogram: bin of (key >> 12) - (floor << 8), the last bin open-ended
  uint32_t* cnt;      // [R, 4]     unused, unused, candidates reserved, unused
  uint32_t* thr;      // [R, 4]     floor bin of the candidates (written by the filter's first block)
  uint32_t* seg_cnt;  // [R, nblk]  candidates of each chunk
  uint32_t* seg_off;  // [R, nblk]  where each chunk's candidates start in the row's list
  uint64_t* cand;     // [R, cap]   candidates: position << 32 | key
  int nblk;
};

// Merges a block's LDS histogram `h` (complete: a barrier after its last update) into a global histogram
// with one device-scope atomic per non-empty bin.  Consumers read the global histogram in a later kernel.
template <int NT>
__device__ __forceinline__ void hist_merge(const uint32_t* h, uint32_t* gh) {
  for (int i = threadIdx.x; i < kTopkBins; i += NT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

}  // namespace dsa
