// Per-row selection state shared by the top-k kernels and the indexer that clears it in the fused step.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkBins = 4096;  // bins of a 12-bit key digit, and of the resolve's candidate histogram

// Rows whose top-k floor the fused step's indexer ranks from the row's own keys while the rest of its grid scores
// the row (indexer.hip), leaving it in the row's thr[4 r + 1] for the filter: rows of 16K..2^20 positions with
// k_eff <= 2048, and up to 2^17 positions with k_eff <= 4096, so that about n m / S <= 8192 scores reach a floor
// ranked from S samples with margin m = mu + 4 sqrt(mu) + 8 (S = 512 for a single row of up to 2^17 positions with
// k_eff <= 2048, 1024 up to 2^18 positions, else kFloorSample).  Other rows rank the filter's own sample.  One
// rule, evaluated on both sides of the kernel boundary.
constexpr int kFloorSample = 4096;     // most sampled positions: 1024 runs of four
constexpr int kFloorMinLen = 16384;
__host__ __device__ inline bool indexer_floor_row(int n, int keff) {
  return keff < n && n >= kFloorMinLen && ((n <= (1 << 17) && keff <= 4096) || (n <= (1 << 20) && keff <= 2048));
}

struct Ws {
  uint32_t* cnt;      // [R, 4]     unused, unused, candidates reserved, unused
  uint32_t* thr;      // [R, 4]     floor of the candidates (written by the filter's first block); the fused
                      //            indexer's floor (rows of indexer_floor_row)
  uint32_t* seg_cnt;  // [R, nblk]  candidates of each chunk
  uint32_t* seg_off;  // [R, nblk]  where each chunk's candidates start in the row's list
  uint64_t* cand;     // [R, cap]   candidates: position << 32 | key
  int nblk;
};

}  // namespace dsa
