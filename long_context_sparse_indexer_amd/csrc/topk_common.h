// Per-row selection state shared by the top-k kernels and the indexer that clears it in the fused step.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkBins = 4096;  // bins of a 12-bit key digit, and of the resolve's candidate histogram

struct Ws {
  uint32_t* cnt;      // [R, 4]     unused, unused, candidates reserved, unused
  uint32_t* thr;      // [R, 4]     floor bin of the candidates (written by the filter's first block)
  uint32_t* seg_cnt;  // [R, nblk]  candidates of each chunk
  uint32_t* seg_off;  // [R, nblk]  where each chunk's candidates start in the row's list
  uint64_t* cand;     // [R, cap]   candidates: position << 32 | key
  int nblk;
};

}  // namespace dsa
