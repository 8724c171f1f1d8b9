// Top-k selection on gfx950: for each row keep the k_eff = min(k, n) largest scores (DeepSeek Sparse
// Attention explained, "How Does the Selector Pick 1,024?": keep the highest budget-many positions, and a
// row shorter than the budget is read in full).  Equal scores are taken lowest position first; the result
// is written in increasing position order, padded with -1.
//
// Scores become order-preserving 32-bit keys, selected by a radix select over three digits
// (bits 31..20, 19..8, 7..0):
//   digit 1  a per-row histogram of the first digit, accumulated in LDS per block and merged with one global
//            atomic per non-empty bin -- in the indexer's epilogue (fused step) or in a histogram pass over
//            stored scores (standalone call); the last block of a row finds the bin b1 holding the k_eff-th
//            largest key and the count A1 of keys above it.
//   filter   grid (4096-score chunks, rows): keys with digit 1 >= b1 go, in position order, into a segment of
//            the row's candidate list; keys inside bin b1 also feed a histogram of digit 2, whose last block
//            finds b2 and the count A2 of keys above (b1, b2).
//   resolve  one block per row: loads the candidates (k + one bin's worth) into LDS in position order,
//            settles digit 3 among the few keys left in (b1, b2), and writes the selection in position order
//            with a two-pass wave-ballot compaction.  A row whose candidates overflow the LDS list (heavily
//            tied scores) is resolved over the whole stored score row instead.
#include "common.h"
#include "launch.h"
#include "topk_common.h"

#include <type_traits>

namespace dsa {
namespace {

constexpr int kCh = kTopkChunk;    // scores per filter / histogram block
constexpr int kTpb = 1024;         // threads of histogram / filter blocks
constexpr int kEpt = kCh / kTpb;   // scores per thread (consecutive)
constexpr int kRes = 512;          // threads of the resolve block
constexpr int kResWaves = kRes / 64;
constexpr int kCap = 12288;        // candidate entries a row keeps for the resolve step
constexpr int kTopkFusedResolveRows = 64;

Ws carve(const Geo& g, void* base) {
  Ws w;
  char* p = static_cast<char*>(base);
  w.nblk = std::max(1, (g.max_row_len + kCh - 1) / kCh);
  auto take = [&](size_t bytes) { char* q = p; p += align_up(bytes); return q; };
  w.hist1 = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * kTopkBins));
  w.hist2 = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * kTopkBins));
  w.cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 4 * (size_t)g.R));
  w.thr = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 4 * (size_t)g.R));
  w.seg_cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.seg_off = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.cand = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)g.R * kCap));
  return w;
}

// Zeroes both histograms and the counters of every row (one block per row).
__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* __restrict__ hist1, uint32_t* __restrict__ hist2,
                                                        uint32_t* __restrict__ cnt) {
  const int r = blockIdx.x;
  const v4i z = {0, 0, 0, 0};
  v4i* h1 = reinterpret_cast<v4i*>(hist1 + (int64_t)r * kTopkBins);
  v4i* h2 = reinterpret_cast<v4i*>(hist2 + (int64_t)r * kTopkBins);
  for (int i = threadIdx.x; i < kTopkBins / 4; i += blockDim.x) { h1[i] = z; h2[i] = z; }
  if (threadIdx.x == 0) reinterpret_cast<v4i*>(cnt)[r] = z;
}

// Loads the kEpt consecutive scores of this thread as keys; positions >= n give valid = false.
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int64_t first, int n, uint32_t (&key)[kEpt],
                                          bool (&valid)[kEpt]) {
  if (first + kEpt <= n) {
#pragma unroll
    for (int v = 0; v < kEpt / 4; ++v) {
      const v4f x = *reinterpret_cast<const v4f*>(row + first + 4 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) { key[4 * v + e] = order_key(x[e]); valid[4 * v + e] = true; }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
      valid[e] = first + e < n;
      key[e] = valid[e] ? order_key(row[first + e]) : 0u;
    }
  }
}

// First-digit histogram of stored scores (standalone top-k): one block per 4096-score chunk.
__global__ __launch_bounds__(kTpb) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ row_len, int max_row_len, int k,
                                                         uint32_t* __restrict__ hist1, uint32_t* __restrict__ cnt,
                                                         uint32_t* __restrict__ thr) {
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scan[kTpb / 64 + 1];
  __shared__ int flag;
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nblk = (n + kCh - 1) / kCh;
  if (keff >= n || (int)blockIdx.x >= nblk) return;  // nothing to choose, or a chunk past the row's end
  for (int i = threadIdx.x; i < kTopkBins; i += kTpb) h[i] = 0u;
  __syncthreads();
  uint32_t key[kEpt];
  bool valid[kEpt];
  load_keys(scores + (int64_t)r * ld, (int64_t)blockIdx.x * kCh + threadIdx.x * kEpt, n, key, valid);
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if (valid[e]) atomicAdd(&h[key[e] >> 20], 1u);
  __syncthreads();
  hist_merge_and_threshold<kTpb>(h, hist1 + (int64_t)r * kTopkBins, &cnt[4 * r + 0], nblk, (uint32_t)keff, 0u,
                           &thr[4 * r + 0], &thr[4 * r + 1], scan, &flag);
}

// Device-coherent accesses for data one block hands to another within a kernel (no cache flush needed).
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Candidate access for the resolve step: entries of the LDS list, or every position of the stored row.
struct LdsList {
  const uint32_t* key;
  const int32_t* pos;
  __device__ uint32_t k(int i) const { return key[i]; }
  __device__ int32_t p(int i) const { return pos[i]; }
};
struct RowList {
  const float* row;
  __device__ uint32_t k(int i) const { return order_key(row[i]); }
  __device__ int32_t p(int i) const { return i; }
};

// Among entries whose key agrees with `prefix` above bit lo+bits, find the digit (key >> lo) & (2^bits - 1)
// holding the need-th largest key; returns it and lowers `need` by the number of entries above it.
template <int NT, class List>
__device__ uint32_t refine_digit(const List& L, int len, uint32_t prefix, int lo, int bits, uint32_t& need,
                                 uint32_t* h, uint32_t* scan) {
  __shared__ uint32_t found_digit, found_above;
  const int nb = 1 << bits;
  const uint32_t mask = (uint32_t)nb - 1u;
  for (int i = threadIdx.x; i < nb; i += NT) h[i] = 0u;
  if (threadIdx.x == 0) { found_digit = 0u; found_above = 0u; }
  __syncthreads();
  for (int i = threadIdx.x; i < len; i += NT) {
    const uint32_t key = L.k(i);
    if (((uint64_t)key >> (lo + bits)) == prefix) atomicAdd(&h[(key >> lo) & mask], 1u);
  }
  __syncthreads();
  const int per = (nb + NT - 1) / NT;  // thread t owns bins [(NT-1-t)*per, +per): top bins first
  const int grp = NT - 1 - threadIdx.x;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) {
    const int b = grp * per + j;
    if (b < nb) local += h[b];
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan(local, scan, total);
  if (above < need && above + local >= need) {
    for (int j = per - 1; j >= 0; --j) {
      const int b = grp * per + j;
      if (b >= nb) continue;
      if (above + h[b] >= need) { found_digit = (uint32_t)b; found_above = above; break; }
      above += h[b];
    }
  }
  __syncthreads();
  need -= found_above;
  const uint32_t d = found_digit;
  __syncthreads();
  return d;
}

// Writes, in list (= position) order, every entry with key > T and the first eq_need entries with key == T.
// Each wave owns a contiguous stretch of the list; one pass counts, one block-level prefix, one pass writes.
template <int NT, class List>
__device__ void write_selection(const List& L, int len, uint32_t T, uint32_t eq_need, int keff, int32_t* out) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t w_gt[NW], w_eq[NW], w_eqbase[NW], w_slot[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int span = ((len + NW * 64 - 1) / (NW * 64)) * 64;
  const int lo = wave * span, hi = min(len, lo + span);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t gt = 0, eq = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const uint32_t key = i < hi ? L.k(i) : 0u;
    gt += __popcll(__ballot(i < hi && key > T));
    eq += __popcll(__ballot(i < hi && key == T));
  }
  if (lane == 0) { w_gt[wave] = gt; w_eq[wave] = eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t eq_run = 0, slot_run = 0;
    for (int w = 0; w < NW; ++w) {
      w_eqbase[w] = eq_run;
      w_slot[w] = slot_run;
      const uint32_t take_eq = eq_run >= eq_need ? 0u : min(w_eq[w], eq_need - eq_run);
      slot_run += w_gt[w] + take_eq;
      eq_run += w_eq[w];
    }
  }
  __syncthreads();
  uint32_t eq_run = w_eqbase[wave], slot_run = w_slot[wave];
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const uint32_t key = i < hi ? L.k(i) : 0u;
    const bool is_eq = i < hi && key == T;
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t rank = eq_run + (uint32_t)__popcll(eqm & below);
    const bool sel = i < hi && (key > T || (is_eq && rank < eq_need));
    const uint64_t selm = __ballot(sel);
    const uint32_t slot = slot_run + (uint32_t)__popcll(selm & below);
    if (sel && slot < (uint32_t)keff) out[slot] = L.p(i);
    eq_run += (uint32_t)__popcll(eqm);
    slot_run += (uint32_t)__popcll(selm);
  }
  __syncthreads();
}

// LDS of the resolve step.
struct ResolveLds {
  uint32_t key[kCap];
  int32_t pos[kCap];
  uint32_t h[kTopkBins];
  uint32_t seg_start[kTopkMaxBlocksPerRow + 1];
  uint32_t seg_src[kTopkMaxBlocksPerRow];
  uint32_t scan[1024 / 64 + 1];  // one word per wave of the largest block, plus the total
};

// Final selection of row r by one block of NT threads: b1 / b2 are the digit-1 / digit-2 threshold bins,
// A2 the number of keys above (b1, b2), len the row's candidate count.  The candidate data must be visible
// to ordinary loads (written by an earlier kernel, or acquired after the row's completion counter).
template <int NT>
__device__ void resolve_row(int r, int n, int keff, int k, const float* __restrict__ row, uint32_t b1, uint32_t b2,
                            uint32_t A2, uint32_t len, const uint32_t* seg_cnt, const uint32_t* seg_off,
                            const uint64_t* cand, int nblk_max, int32_t* __restrict__ out, ResolveLds& S) {
  if (len <= (uint32_t)kCap) {
    const int nblk = (n + kCh - 1) / kCh;
    {  // segment starts in chunk (= position) order; thread t owns chunks [t*CPT, (t+1)*CPT)
      constexpr int CPT = (kTopkMaxBlocksPerRow + NT - 1) / NT;
      const int c0 = threadIdx.x * CPT;
      uint32_t cc[CPT];
      uint32_t sum = 0;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int b = c0 + j;
        cc[j] = 0;
        if (b < nblk) {
          cc[j] = seg_cnt[(int64_t)r * nblk_max + b];
          S.seg_src[b] = seg_off[(int64_t)r * nblk_max + b];
        }
        sum += cc[j];
      }
      uint32_t total;
      uint32_t start = block_exclusive_scan(sum, S.scan, total);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (c0 + j < nblk) S.seg_start[c0 + j] = start;
        start += cc[j];
      }
      if (threadIdx.x == 0) S.seg_start[nblk] = total;
      __syncthreads();
    }
    // copy the segments into the LDS list: list entry i lives in the last segment starting at or before i;
    // each thread issues 8 independent loads before it stores any, so the copy costs a few round trips
    constexpr int kBatch = 8;
    for (int base = 0; base < (int)len; base += NT * kBatch) {
      uint64_t e[kBatch];
      int dst[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = base + j * NT + threadIdx.x;
        dst[j] = -1;
        if (i < (int)len) {
          int lo = 0, hi = nblk - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (S.seg_start[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
          }
          dst[j] = i;
          e[j] = cand[(int64_t)r * kCap + S.seg_src[lo] + (i - S.seg_start[lo])];
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (dst[j] >= 0) {
          S.key[dst[j]] = (uint32_t)e[j];
          S.pos[dst[j]] = (int32_t)(e[j] >> 32);
        }
      }
    }
    __syncthreads();
    uint32_t need = (uint32_t)keff - A2;  // keys of (b1, b2) still to take
    const LdsList L{S.key, S.pos};
    const uint32_t d3 = refine_digit<NT>(L, (int)len, (b1 << 12) | b2, 0, 8, need, S.h, S.scan);
    write_selection<NT>(L, (int)len, (b1 << 20) | (b2 << 8) | d3, need, keff, out);
  } else {
    const RowList L{row};
    uint32_t need = (uint32_t)keff;
    const uint32_t d1 = refine_digit<NT>(L, n, 0u, 20, 12, need, S.h, S.scan);
    const uint32_t d2 = refine_digit<NT>(L, n, d1, 8, 12, need, S.h, S.scan);
    const uint32_t d3 = refine_digit<NT>(L, n, (d1 << 12) | d2, 0, 8, need, S.h, S.scan);
    write_selection<NT>(L, n, (d1 << 20) | (d2 << 8) | d3, need, keff, out);
  }
  for (int i = keff + threadIdx.x; i < k; i += NT) out[i] = -1;
}

// kFused: the block that completes a row also resolves it (small batches); otherwise a resolve kernel follows.
template <bool kFused>
__global__ __launch_bounds__(kTpb) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ row_len, int max_row_len,
                                                           int k, uint32_t* __restrict__ thr,
                                                           uint32_t* __restrict__ hist2, uint32_t* __restrict__ cnt,
                                                           uint32_t* __restrict__ seg_cnt,
                                                           uint32_t* __restrict__ seg_off, uint64_t* __restrict__ cand,
                                                           int nblk_max, int32_t* __restrict__ topk_idx) {
  __shared__ uint32_t scan[kTpb / 64 + 1];
  __shared__ uint32_t seg_base, s_b2, s_A2;
  __shared__ int flag;
  __shared__ typename std::conditional<kFused, ResolveLds, int>::type R;
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nblk = (n + kCh - 1) / kCh;
  if (keff >= n || (int)blockIdx.x >= nblk) {
    if (kFused && blockIdx.x == 0) {  // nothing to choose: the row keeps every position
      int32_t* out = topk_idx + (int64_t)r * k;
      for (int i = threadIdx.x; i < k; i += kTpb) out[i] = i < n ? i : -1;
    }
    return;
  }
  const uint32_t b1 = thr[4 * r + 0], A1 = thr[4 * r + 1];
  const int64_t first = (int64_t)blockIdx.x * kCh + threadIdx.x * kEpt;
  uint32_t key[kEpt];
  bool valid[kEpt];
  const float* row = scores + (int64_t)r * ld;
  load_keys(row, first, n, key, valid);
  uint32_t* h2 = hist2 + (int64_t)r * kTopkBins;
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < kEpt; ++e) {
    const uint32_t d1 = key[e] >> 20;
    if (valid[e] && d1 >= b1) {
      ++c;
      if (d1 == b1) atomicAdd(&h2[(key[e] >> 8) & 0xfffu], 1u);
    }
  }
  uint32_t total;
  const uint32_t off = block_exclusive_scan(c, scan, total);
  if (threadIdx.x == 0) {
    seg_base = atomicAdd(&cnt[4 * r + 2], total);
    st_dev(&seg_cnt[(int64_t)r * nblk_max + blockIdx.x], total);
    st_dev(&seg_off[(int64_t)r * nblk_max + blockIdx.x], seg_base);
  }
  __syncthreads();
  if (seg_base + total <= (uint32_t)kCap) {  // on overflow the resolve step rescans the row
    uint64_t* dst = cand + (int64_t)r * kCap + seg_base + off;
#pragma unroll
    for (int e = 0; e < kEpt; ++e)
      if (valid[e] && (key[e] >> 20) >= b1) st_dev(dst++, ((uint64_t)(first + e) << 32) | key[e]);
  }
  // second digit: the last chunk of the row finds b2 among keys of bin b1 (need = k_eff - A1 of them)
  if (!hist_threshold_last<kTpb>(h2, &cnt[4 * r + 1], nblk, (uint32_t)keff - A1, A1, &s_b2, &s_A2, scan, &flag)) return;
  if constexpr (kFused) {
    resolve_row<kTpb>(r, n, keff, k, row, b1, s_b2, s_A2, cnt[4 * r + 2], seg_cnt, seg_off, cand, nblk_max,
                      topk_idx + (int64_t)r * k, R);
  } else {
    if (threadIdx.x == 0) { thr[4 * r + 2] = s_b2; thr[4 * r + 3] = s_A2; }
  }
}

__global__ __launch_bounds__(512) void topk_resolve_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ row_len, int max_row_len,
                                                           int k, const uint32_t* __restrict__ thr,
                                                           const uint32_t* __restrict__ cnt,
                                                           const uint32_t* __restrict__ seg_cnt,
                                                           const uint32_t* __restrict__ seg_off,
                                                           const uint64_t* __restrict__ cand, int nblk_max,
                                                           int32_t* __restrict__ topk_idx) {
  __shared__ ResolveLds S;
  const int r = blockIdx.x;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  int32_t* out = topk_idx + (int64_t)r * k;
  if (keff >= n) {
    for (int i = threadIdx.x; i < k; i += 512) out[i] = i < n ? i : -1;
    return;
  }
  resolve_row<512>(r, n, keff, k, scores + (int64_t)r * ld, thr[4 * r + 0], thr[4 * r + 2], thr[4 * r + 3],
                   cnt[4 * r + 2], seg_cnt, seg_off, cand, nblk_max, out, S);
}

}  // namespace

size_t topk_workspace_bytes(const Geo& g) {
  const size_t nblk = (size_t)std::max(1, (g.max_row_len + kCh - 1) / kCh);
  const size_t R = (size_t)g.R;
  return 2 * align_up(4 * R * kTopkBins) + 2 * align_up(16 * R) + 2 * align_up(4 * R * nblk) + align_up(8 * R * kCap);
}

TopkState topk_state(const Geo& g, void* workspace) {
  const Ws w = carve(g, workspace);
  return TopkState{w.hist1, w.cnt, w.thr};
}

hipError_t launch_topk_zero(const Geo& g, void* workspace, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  topk_zero_kernel<<<g.R, 256, 0, stream>>>(w.hist1, w.hist2, w.cnt);
  return hipGetLastError();
}

hipError_t launch_topk_select(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                              bool hist_done, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  dim3 grid(w.nblk, g.R);
  if (!hist_done)
    topk_hist_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.hist1, w.cnt, w.thr);
  // few rows: the chunk that completes a row resolves it; many rows: a resolve kernel with a block per row
  if (g.R <= kTopkFusedResolveRows) {
    topk_filter_kernel<true><<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.hist2,
                                                        w.cnt, w.seg_cnt, w.seg_off, w.cand, w.nblk, topk_idx);
  } else {
    topk_filter_kernel<false><<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.hist2,
                                                         w.cnt, w.seg_cnt, w.seg_off, w.cand, w.nblk, topk_idx);
    topk_resolve_kernel<<<g.R, 512, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.cnt, w.seg_cnt,
                                                 w.seg_off, w.cand, w.nblk, topk_idx);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                       hipStream_t stream) {
  hipError_t e = launch_topk_zero(g, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_topk_select(g, scores, ld, topk_idx, workspace, false, stream);
}

}  // namespace dsa
