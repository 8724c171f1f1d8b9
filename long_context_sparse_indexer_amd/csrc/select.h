// The resolve step of the top-k selection (the resolve kernel of topk.hip), and the whole-row radix select that the
// prefill fallback (indexer.hip) runs over a stored row.
//
// For each row keep the k_eff = min(k, n) largest scores (DeepSeek Sparse Attention explained, "How Does the
// Selector Pick 1,024?"); equal scores are taken lowest position first; the selected positions are numbered in
// increasing position order (slot 0 is the lowest selected position).
//
// Input: what the filter kernel left for the row: a floor (the 20-bit key prefix of a sampled score), a list of
// candidates (every position whose order-preserving key reaches the floor, as position << 32 | key) written in
// segments, one per 4096-score chunk, each in position order, and the segment table (count and list offset of
// each chunk's segment).  The resolve counts the candidates in an LDS histogram of their 20-bit prefixes taken
// relative to the floor (4096 bins, the last open-ended) while it places them in position order in LDS, finds the
// bin holding the k_eff-th largest key, settles the low 12 bits among the keys of that bin, and hands every
// selected (slot, position) to a sink.  A row whose sample overshot (fewer than k_eff candidates) or whose
// candidates overflowed the list is resolved over its whole stored score row instead, by a three-digit radix
// select.
#pragma once

#include "common.h"
#include "launch.h"
#include "topk_common.h"

namespace dsa {

constexpr int kCh = kTopkChunk;   // scores per filter chunk
constexpr int kCap = 12288;       // candidate entries a row keeps for the resolve step
constexpr int kResPages = 4096;   // page-table entries a resolving block stages in LDS

// The bin of an LDS histogram holding the need-th largest entry, counting from the top bin, found by wave 0
// alone in two levels: lane l sums the kBins/64 bins (63 - l) * kBins/64 .. (lane 0 the top ones) with 16-byte
// reads and a DPP scan over the lanes picks the lane L holding the bin; then lanes g < kBins/256 take L's groups
// of four bins, top group first, a second scan picks the group, and its lane walks the four bins.  The bin and the
// number of entries above it land in *b, *above (left as preset when the histogram holds fewer than `need`).
// Called by wave 0 only; the caller publishes the result with a barrier.
template <int kBins, int kInFlight = 4>
__device__ __forceinline__ void wave_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* b, uint32_t* above_out) {
  constexpr int kPer = kBins / 64, kGroups = kPer / 4;
  static_assert(kPer % 4 == 0 && kGroups <= 64, "16-byte reads of a lane's bins");
  const int lane = threadIdx.x;
  const v4i* hb = reinterpret_cast<const v4i*>(h);
  // lane l reads its kGroups 16-byte words starting at word l % kGroups (in the plain order every lane would hit the
  // same banks at once, a kGroups * 16-byte lane stride), kInFlight of them issued before any is summed: a running
  // sum over the reads had the compiler keep two in flight, eight LDS round trips in a row
  static_assert((kGroups & (kGroups - 1)) == 0, "the rotation wraps with a mask");
  constexpr int kBatch = kInFlight < kGroups ? kInFlight : kGroups;
  static_assert(kGroups % kBatch == 0, "batches tile the words");
  uint32_t local = 0;
#pragma unroll
  for (int q0 = 0; q0 < kGroups; q0 += kBatch) {
    v4i xs[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) xs[q] = hb[(63 - lane) * kGroups + ((q0 + q + lane) & (kGroups - 1))];
    __builtin_amdgcn_sched_barrier(0);  // the batch's reads issued before the first sum
#pragma unroll
    for (int q = 0; q < kBatch; ++q) local += (uint32_t)(xs[q][0] + xs[q][1] + xs[q][2] + xs[q][3]);
  }
  uint32_t tot;
  const uint32_t above = wave_exclusive_scan(local, tot);
  const uint64_t hit = __ballot(above < need && above + local >= need);
  if (!hit) return;  // uniform: fewer than `need` entries
  const int L = __builtin_ctzll(hit);
  const uint32_t above_l = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
  const v4i z = {0, 0, 0, 0};
  const v4i x = lane < kGroups ? hb[(63 - L) * kGroups + (kGroups - 1 - lane)] : z;
  const uint32_t gsum = (uint32_t)(x[0] + x[1] + x[2] + x[3]);
  uint32_t tot2;
  uint32_t a = above_l + wave_exclusive_scan(gsum, tot2);
  if (lane < kGroups && a < need && a + gsum >= need) {
    int e = 3;
    while (e > 0 && a + (uint32_t)x[e] < need) a += (uint32_t)x[e--];
    *b = (uint32_t)((63 - L) * kPer + 4 * (kGroups - 1 - lane) + e);
    *above_out = a;
  }
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

// Pool row of a position of the row's sequence, from the global row of its page table.
struct RowMap {
  const int32_t* pt;
  int max_pages, num_pages, log2ps;
  __device__ int32_t base(int32_t pos) const {  // pool row of the first position of pos's page
    const int lp = min(pos >> log2ps, max_pages - 1);
    return min(max(pt[lp], 0), num_pages - 1) << log2ps;
  }
  __device__ int32_t row(int32_t pos) const { return base(pos) | (pos & ((1 << log2ps) - 1)); }
};
// The same from the row's page ids staged in LDS.  A sink whose page-table reads may be global or LDS makes them
// flat loads, and a loop of stores and flat loads waits for every store it issued: the two are kept apart.
struct LdsRowMap {
  const __attribute__((address_space(3))) int32_t* pt;
  int max_pages, num_pages, log2ps;
  __device__ int32_t base(int32_t pos) const {
    const int lp = min(pos >> log2ps, max_pages - 1);
    return min(max(pt[lp], 0), num_pages - 1) << log2ps;
  }
  __device__ int32_t row(int32_t pos) const { return base(pos) | (pos & ((1 << log2ps) - 1)); }
};
__device__ __forceinline__ const __attribute__((address_space(3))) int32_t* lds_ptr(const int32_t* p) {
  return reinterpret_cast<const __attribute__((address_space(3))) int32_t*>(reinterpret_cast<uintptr_t>(p));
}

// Copies the page ids of a row's sequence (max_pages <= kResPages) into LDS: every load is issued before the first
// store, from an in-range address.  Called by all NT threads; the copy is visible after the caller's next barrier.
template <int NT>
__device__ __forceinline__ void stage_page_row(int32_t* __restrict__ dst, const int32_t* __restrict__ src,
                                               int max_pages) {
  constexpr int kPer = (kResPages + NT - 1) / NT;
  int32_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = src[min(j * NT + (int)threadIdx.x, max_pages - 1)];
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j * NT + (int)threadIdx.x < max_pages) dst[j * NT + threadIdx.x] = v[j];
}

// Sink of the standalone selection: the whole list of selected positions and, when rows_out is non-NULL, the pool
// row of each (Map: RowMap or LdsRowMap).
template <class Map>
struct ListSinkT {
  int32_t* out;
  int32_t* rows_out;
  Map map;
  __device__ bool wants(uint32_t, uint32_t) const { return true; }
  __device__ void put(uint32_t slot, int32_t pos) const {
    out[slot] = pos;
    if (rows_out) rows_out[slot] = map.row(pos);
  }
  __device__ void put_or_pad(uint32_t slot, int32_t pos) const {  // pos -1: a padding slot
    out[slot] = pos;
    if (rows_out) rows_out[slot] = pos >= 0 ? map.row(pos) : -1;
  }
  // A 32-aligned word of positions lies in one page (pages hold >= 32 positions): its page's first pool row, read
  // once, serves every position of the word (put_in_word), so that a loop over the word reads no page table.
  __device__ int32_t word_base(int32_t pos0) const { return rows_out ? map.base(pos0) : 0; }
  __device__ void put_in_word(uint32_t slot, int32_t pos, int32_t base) const {
    out[slot] = pos;
    if (rows_out) rows_out[slot] = base | (pos & ((1 << map.log2ps) - 1));
  }
};
using ListSink = ListSinkT<RowMap>;
using LdsListSink = ListSinkT<LdsRowMap>;

// Exclusive prefix over the block of one value per thread, and the block total, with one barrier: every wave
// scans its lanes and publishes its total in wt[0 .. NW), then every thread adds the totals of the waves before
// its own.  wt may be written again only after another barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_scan1(uint32_t v, uint32_t* wt, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t tw;
  uint32_t x = wave_exclusive_scan(v, tw);
  if (lane == 0) wt[wave] = tw;
  __syncthreads();
  static_assert(NW % 4 == 0, "wave totals are read four at a time");
  total = 0;
#pragma unroll
  for (int q = 0; q < NW / 4; ++q) {  // 16-byte reads of the wave totals (wt is 16-byte aligned)
    const v4i y = reinterpret_cast<const v4i*>(wt)[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * q + e < wave) x += (uint32_t)y[e];
      total += (uint32_t)y[e];
    }
  }
  return x;
}

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

// Hands the sink, in list (= position) order, every entry with key > T and the first eq_need entries with key == T,
// each with its slot.  Each wave owns a contiguous stretch of the list; one pass counts, one barrier publishes the
// per-wave counts, every wave adds up those of the waves before it, and a second pass hands the entries over.  A
// wave whose slots the sink does not want skips the second pass.
template <int NT, class List, class Sink>
__device__ void write_selection(const List& L, int len, uint32_t T, uint32_t eq_need, int keff, const Sink& sink) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t w_gt[NW], w_eq[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int span = ((len + NW * 64 - 1) / (NW * 64)) * 64;
  const int lo = wave * span, hi = min(len, lo + span);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int U = 4;  // 64-entry steps per iteration, their LDS reads issued together
  uint32_t gt = 0, eq = 0;
  for (int base = lo; base < hi; base += 64 * U) {
    uint32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + 64 * u + lane;
      key[u] = i < hi ? L.k(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = base + 64 * u + lane < hi;
      gt += __popcll(__ballot(in && key[u] > T));
      eq += __popcll(__ballot(in && key[u] == T));
    }
  }
  if (lane == 0) { w_gt[wave] = gt; w_eq[wave] = eq; }
  __syncthreads();
  // this wave's first slot and its rank among the keys equal to T.  The waves before it take all their keys above
  // T and, in list order, the equal ones while fewer than eq_need are taken: the share of wave w is
  // min(E_w+1, eq_need) - min(E_w, eq_need) for E_w the equal keys of the waves before w, so the shares of the
  // waves before this one add up to min(E, eq_need).  Both prefixes come from DPP scans over the wave counts.
  static_assert(NW <= 64, "one lane per wave");
  const uint32_t gl = lane < NW ? w_gt[lane] : 0u, el = lane < NW ? w_eq[lane] : 0u;
  uint32_t gsum, esum;
  const uint32_t gpre = wave_exclusive_scan(gl, gsum), epre = wave_exclusive_scan(el, esum);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t eq_run = (uint32_t)__builtin_amdgcn_readlane((int)epre, wv);
  uint32_t slot_run = (uint32_t)__builtin_amdgcn_readlane((int)gpre, wv) + min(eq_run, eq_need);
  {
    const uint32_t my_gt = (uint32_t)__builtin_amdgcn_readlane((int)gl, wv);
    const uint32_t my_eq = (uint32_t)__builtin_amdgcn_readlane((int)el, wv);
    const uint32_t take = min(eq_run + my_eq, eq_need) - min(eq_run, eq_need);
    if (!sink.wants(slot_run, slot_run + my_gt + take)) return;  // uniform over the wave
  }
  for (int base = lo; base < hi; base += 64 * U) {
    uint32_t key[U];
    int32_t pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + 64 * u + lane;
      key[u] = i < hi ? L.k(i) : 0u;
      pos[u] = i < hi ? L.p(i) : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = base + 64 * u + lane < hi;
      const bool is_eq = in && key[u] == T;
      const uint64_t eqm = __ballot(is_eq);
      const uint32_t rank = eq_run + (uint32_t)__popcll(eqm & below);
      const bool sel = in && (key[u] > T || (is_eq && rank < eq_need));
      const uint64_t selm = __ballot(sel);
      const uint32_t slot = slot_run + (uint32_t)__popcll(selm & below);
      if (sel && slot < (uint32_t)keff) sink.put(slot, pos[u]);
      eq_run += (uint32_t)__popcll(eqm);
      slot_run += (uint32_t)__popcll(selm);
    }
  }
  // no trailing barrier: every caller calls this once, as its last use of the LDS (a barrier would also wait
  // for the stores above to complete)
}

// The same hand-over for the LDS list in one pass: thread t owns the contiguous entries [t per, (t + 1) per); its
// counts of keys above T and equal to T go through two block scans, which give its first slot and the rank of its
// first equal key, and it then hands over its own entries.  The list must be at most a few entries per thread.
template <int NT, class Sink>
__device__ void write_selection_lds(const LdsList& L, int len, uint32_t T, uint32_t eq_need, int keff,
                                    const Sink& sink) {
  constexpr int NW = NT / 64;
  __shared__ __attribute__((aligned(16))) uint32_t wt[2 * NW];
  const int per = (len + NT - 1) / NT;
  const int lo = min(len, (int)threadIdx.x * per), hi = min(len, lo + per);
  uint32_t gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = L.k(i);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tg, te;
  const uint32_t pre_gt = block_scan1<NT>(gt, wt, tg);
  uint32_t eq_rank = block_scan1<NT>(eq, wt + NW, te);
  uint32_t slot = pre_gt + min(eq_rank, eq_need);
  const uint32_t take = min(eq_rank + eq, eq_need) - min(eq_rank, eq_need);
  if (!sink.wants(slot, slot + gt + take)) return;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = L.k(i);
    const bool sel = key > T || (key == T && eq_rank < eq_need);
    eq_rank += key == T;
    if (sel) {
      if (slot < (uint32_t)keff) sink.put(slot, L.p(i));
      ++slot;
    }
  }
}

// The key holding the need-th largest place among the list's entries, by a three-digit radix select; lowers
// `need` to its rank among the keys equal to it.
template <int NT, class List>
__device__ uint32_t select_key(const List& L, int len, uint32_t& need, uint32_t* h, uint32_t* scan) {
  const uint32_t d1 = refine_digit<NT>(L, len, 0u, 20, 12, need, h, scan);
  const uint32_t d2 = refine_digit<NT>(L, len, d1, 8, 12, need, h, scan);
  const uint32_t d3 = refine_digit<NT>(L, len, (d1 << 12) | d2, 0, 8, need, h, scan);
  return (d1 << 20) | (d2 << 8) | d3;
}

// The rare resolve paths (a row whose sample overshot or overflowed the list, a threshold past the candidate
// histogram's range): a three-digit radix select over the list, then the write.  Kept out of line so that the
// common path's code stays compact.
template <int NT, class List, class Sink>
__device__ __attribute__((noinline)) void select_and_write(List L, int len, uint32_t need, int keff, Sink sink,
                                                            uint32_t* h, uint32_t* scan) {
  const uint32_t T = select_key<NT>(L, len, need, h, scan);
  write_selection<NT>(L, len, T, need, keff, sink);
}

// Bin of a candidate key in the row's candidate histogram: its 20-bit prefix relative to the floor, the last bin
// taking everything 4095 or more 20-bit steps above the floor.
__device__ __forceinline__ uint32_t cand_bin(uint32_t key, uint32_t floor20) {
  return min((key >> 12) - floor20, (uint32_t)kTopkBins - 1u);
}

// LDS of the resolve step.
struct ResolveLds {
  uint32_t key[kCap];
  int32_t pos[kCap];
  alignas(16) uint32_t h[kTopkBins];  // candidate histogram, then the refine passes' digit histograms
  uint32_t seg_start[kTopkMaxBlocksPerRow];
  uint32_t seg_src[kTopkMaxBlocksPerRow];
  uint32_t scan[1024 / 64 + 1];  // one word per wave of the largest block, plus the total
  alignas(16) uint32_t scan2[2 * (1024 / 64)];
  uint32_t bin[64];               // low 12 bits of the keys of the threshold's 20-bit prefix, when at most 64
  uint32_t s_bin, s_above, s_nb, s_nbin;
  int32_t pt[kResPages];          // page ids of the row's sequence, when they fit
};

// What the filter left for one row (pointers already offset to the row).
struct RowCands {
  const uint32_t* thr;      // [4]: the floor in word 0
  const uint32_t* cnt;      // [4]: candidates reserved in word 2
  const uint32_t* seg_cnt;  // [nblk]
  const uint32_t* seg_off;  // [nblk]
  const uint64_t* cand;     // [kCap]
};

// The resolve step's first reads for one row, which depend on nothing but the row: the floor, the candidate count,
// the segment table and the first batch of candidates.  Issued by resolve_issue as early as the caller can, consumed
// by resolve_finish.
template <int NT>
struct ResolveLoads {
  static constexpr int kQ = (kTopkMaxBlocksPerRow + NT - 1) / NT;  // chunks of the segment table per thread
  static constexpr int kPer = (kCap + NT - 1) / NT;                 // candidate entries per thread
  static constexpr int kBatch = kPer < 16 ? kPer : 16;              // ... loaded per batch
  static_assert(kBatch * NT <= kCap, "the first batch lies inside the list");
  uint32_t fl, len;
  uint32_t c[kQ], src[kQ];
  uint64_t e[kBatch];
};

// Issues every read of ResolveLoads from an in-range address (entries past the row's chunks or past the candidate
// count are dropped later), so that the compiler places them all before the first wait.  nblk_max: the segment
// table's row stride.
template <int NT>
__device__ __forceinline__ void resolve_issue(const RowCands& rc, int nblk_max, ResolveLoads<NT>& L) {
  using RL = ResolveLoads<NT>;
  const int t = threadIdx.x;
  L.fl = rc.thr[0];
  L.len = rc.cnt[2];
#pragma unroll
  for (int q = 0; q < RL::kQ; ++q) {
    const int ch = min(t * RL::kQ + q, nblk_max - 1);
    L.c[q] = rc.seg_cnt[ch];
    L.src[q] = rc.seg_off[ch];
  }
#pragma unroll
  for (int j = 0; j < RL::kBatch; ++j) L.e[j] = rc.cand[j * NT + t];
}

struct NoStage {
  __device__ void operator()() const {}
};

// Resolves the selection of one row whose k_eff < n from the reads resolve_issue started and hands every selected
// (slot, position) to the sink; `row` is the row's stored scores (read only on the rare paths).  stage() runs once
// every thread has counted its candidates, before the barrier that publishes the histogram (a caller's LDS stores
// that the sink reads go there).  Called by all NT threads of the block; the block's LDS (S) is free afterwards once
// the caller has passed a barrier.
template <int NT, class Sink, class Stage, int kStamp = -1>
__device__ void resolve_finish(const float* __restrict__ row, int n, int keff, const RowCands& rc,
                               ResolveLoads<NT>& rl, ResolveLds& S, const Sink& sink, const Stage& stage) {
  constexpr int NW = NT / 64;
  using RL = ResolveLoads<NT>;
  constexpr int kQ = RL::kQ, kBatch = RL::kBatch;
  constexpr int kBatches = (RL::kPer + kBatch - 1) / kBatch;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int nblk = (n + kCh - 1) / kCh;
  const uint32_t fl = rl.fl, len = rl.len;
  uint32_t (&c)[kQ] = rl.c;
  uint32_t (&src)[kQ] = rl.src;
  uint64_t (&e)[kBatch] = rl.e;
  uint64_t f[kBatch];
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    if (t * kQ + q >= nblk) c[q] = 0u;
  for (int i = t; i < kTopkBins; i += NT) S.h[i] = 0u;  // the candidate histogram, cleared before a barrier
  if (!(len >= (uint32_t)keff && len <= (uint32_t)kCap)) {  // uniform: the rare whole-row path
    stage();
    __syncthreads();
    select_and_write<NT>(RowList{row}, n, (uint32_t)keff, keff, sink, S.h, S.scan);
    return;
  }
  // segment starts in position order: thread t holds chunks t kQ .. +kQ; the scan's barrier also publishes the
  // cleared histogram
  uint32_t mine = 0;
#pragma unroll
  for (int q = 0; q < kQ; ++q) mine += c[q];
  uint32_t ctot;
  uint32_t start = block_scan1<NT>(mine, S.scan2, ctot);
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int ch = t * kQ + q;
    if (ch < nblk) {
      S.seg_start[ch] = start;
      S.seg_src[ch] = src[q];
      start += c[q];
    }
  }
  if (t == 0) {  // the open bin, unless the scan below finds the threshold (it does: the bins hold len >= k_eff keys)
    S.s_nbin = 0;
    S.s_bin = kTopkBins - 1;
    S.s_above = 0;
    S.s_nb = 0;
  }
  __syncthreads();
  if constexpr (kStamp >= 0) DSA_STAMP(kStamp, 6);
  // every candidate counts into the histogram by its 20-bit prefix relative to the floor and goes to its chunk's
  // segment start + its offset within the segment; batch b + 1 loads while batch b is processed
  auto process = [&](const uint64_t (&x)[kBatch], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = (b * kBatch + j) * NT + t;
      if (i < (int)len) {
        const uint32_t key = (uint32_t)x[j];
        const uint32_t pos = (uint32_t)(x[j] >> 32);
        atomicAdd(&S.h[cand_bin(key, fl)], 1u);
        const int chunk = (int)(pos / kCh);
        const uint32_t dst = S.seg_start[chunk] + ((uint32_t)i - S.seg_src[chunk]);
        S.key[dst] = key;
        S.pos[dst] = (int32_t)pos;
      }
    }
  };
  auto load = [&](uint64_t (&x)[kBatch], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) x[j] = rc.cand[min((b * kBatch + j) * NT + t, kCap - 1)];  // masked in process
  };
#pragma unroll
  for (int b = 0; b < kBatches; b += 2) {
    if (b + 1 < kBatches) load(f, b + 1);
    process(e, b);
    if (b + 1 >= kBatches) break;
    if (b + 2 < kBatches) load(e, b + 2);
    process(f, b + 1);
  }
  stage();
  __syncthreads();
  if constexpr (kStamp >= 0) DSA_STAMP(kStamp, 7);
  // the bin holding the k_eff-th largest key: thread t owns bins (NT - 1 - t) * kPerBin .. (top bins first)
  constexpr int kPerBin = kTopkBins / NT;
  static_assert(kPerBin % 4 == 0, "16-byte LDS reads of histogram bins");
  uint32_t hv[kPerBin];
#pragma unroll
  for (int q = 0; q < kPerBin / 4; ++q) {
    const v4i y = reinterpret_cast<const v4i*>(S.h)[(NT - 1 - t) * (kPerBin / 4) + q];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) hv[4 * q + e2] = (uint32_t)y[e2];
  }
  uint32_t hl = 0;
#pragma unroll
  for (int j = 0; j < kPerBin; ++j) hl += hv[j];
  uint32_t htot;
  const uint32_t above = block_scan1<NT>(hl, S.scan2 + NW, htot);
  if (above < (uint32_t)keff && above + hl >= (uint32_t)keff) {
    uint32_t run = above;
#pragma unroll
    for (int j = kPerBin - 1; j >= 0; --j) {
      if (run + hv[j] >= (uint32_t)keff) {
        S.s_bin = (uint32_t)((NT - 1 - t) * kPerBin + j);
        S.s_above = run;
        S.s_nb = hv[j];
        break;
      }
      run += hv[j];
    }
  }
  __syncthreads();
  if constexpr (kStamp >= 0) DSA_STAMP(kStamp, 8);
  // nb keys share the threshold's 20-bit prefix, unless the threshold lies in the open-ended top bin
  const uint32_t bin = S.s_bin, nb = S.s_nb;
  const bool open = bin == kTopkBins - 1;
  const uint32_t prefix = fl + bin;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const LdsList L{S.key, S.pos};
  uint32_t need = (uint32_t)keff - S.s_above;  // keys of the threshold's bin still to take
  const bool few = !open && nb <= 64u;
  if (few) {
    // the low 12 bits of the keys of the threshold's prefix (their order does not matter)
    for (int base = 0; base < (int)len; base += NT) {
      const int i = base + t;
      const uint32_t key = i < (int)len ? S.key[i] : 0u;
      const bool match = i < (int)len && (key >> 12) == prefix;
      const uint64_t mm = __ballot(match);
      if (mm) {  // uniform over the wave
        const int leader = __builtin_ctzll(mm);
        uint32_t base2 = 0;
        if (lane == leader) base2 = atomicAdd(&S.s_nbin, (uint32_t)__popcll(mm));
        base2 = (uint32_t)__builtin_amdgcn_readlane((int)base2, leader);
        if (match) S.bin[base2 + (uint32_t)__popcll(mm & below)] = key & 0xfffu;
      }
    }
    __syncthreads();
  if constexpr (kStamp >= 0) DSA_STAMP(kStamp, 9);
  }
  uint32_t T = 0;
  if (few) {
    // every wave finds the low bits itself: lane x ranks the low bits of the x-th key of the prefix among all nb
    const uint32_t dx = lane < (int)nb ? S.bin[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t y = 0; y < nb; ++y) {
      const uint32_t dy = S.bin[y];
      gt += dy > dx;
      ge += dy >= dx;
    }
    const uint64_t hit = __ballot(lane < (int)nb && gt < need && need <= ge);  // lanes holding the low bits
    const int src_lane = __builtin_ctzll(hit);
    T = (prefix << 12) | (uint32_t)__builtin_amdgcn_readlane((int)dx, src_lane);
    need -= (uint32_t)__builtin_amdgcn_readlane((int)gt, src_lane);
  } else if (!open) {
    T = (prefix << 12) | refine_digit<NT>(L, (int)len, prefix, 0, 12, need, S.h, S.scan);
  }
  if constexpr (kStamp >= 0) DSA_STAMP(kStamp, 10);
  if (open) select_and_write<NT>(L, (int)len, need, keff, sink, S.h, S.scan);
  else write_selection_lds<NT>(L, (int)len, T, need, keff, sink);
}

// Selection of one row from an unordered candidate list through a bitmap over the row's positions.  The candidates
// (position << 32 | order-preserving key, every position whose key's 20-bit prefix reaches the floor `fl`; c of
// them) are counted by prefix relative to the floor in an LDS histogram, which gives the prefix of the k_eff-th
// largest key; its low 12 bits are settled among the keys of that prefix (one wave when they are at most 64, else a
// second histogram).  With T that key, the keys above T and the lowest-position keys equal to T, as many as are
// still needed, are marked in the bitmap, and a popcount scan of the bitmap hands every selected position to the
// sink at its slot, in increasing position order.  Returns false, having handed over nothing, when the list cannot
// settle the row: fewer than k_eff or more than kCap candidates, a threshold in the open-ended top bin, or more than
// kMaxTies keys equal to T.  Called by all 1024 threads (the result is uniform); `list` is the row's whole list of
// kCap entries (c of them written), `bits` holds kWpt * 1024 words, covering the row's n positions, h kTopkBins
// words.
constexpr int kMaxTies = 1024;
struct BitmapScratch {
  int32_t eq_pos[kMaxTies];
  uint32_t low[64];
  alignas(16) uint32_t wt[2 * 16];
  uint32_t bin, above, nb, nlow, neq, T, need;
};
struct NoPre {
  __device__ void operator()() const {}
};
// pre(): work of the caller's that runs while the candidates load (its LDS writes must be visible after the
// first barrier).
template <int kWpt, class Sink, class Pre = NoPre>
__device__ bool bitmap_select(int n, int keff, uint32_t fl, uint32_t c, const uint64_t* __restrict__ list,
                              const Sink& sink, uint32_t* bits, uint32_t* h, BitmapScratch& S,
                              const Pre& pre = Pre{}) {
  constexpr int NT = 1024, NW = NT / 64;
  constexpr int kPer = kCap / NT;  // candidates per thread
  static_assert(kWpt >= 1 && kWpt % 4 == 0 && kPer * NT == kCap, "bitmap and list split evenly");
  const int t = threadIdx.x, lane = t & 63;
  // a grid of at most 1024 blocks loads the whole list (kCap entries per row) whatever the count, so that the loads go
  // out together with the count's own and need not wait for its round trip (entries past c are ignored below);
  // thousands of rows (a prefill chunk) load only their c entries, since the extra bytes would then add up
  const bool speculate = gridDim.x * gridDim.y <= 1024u;
  uint64_t e[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) e[j] = list[speculate ? j * NT + t : min(j * NT + t, max((int)c, 1) - 1)];
  if (c < (uint32_t)keff || c > (uint32_t)kCap || n > kWpt * NT * 32) {
    pre();
    return false;
  }
  DSA_STAMP(1, 10);
  pre();
  for (int i = t; i < kTopkBins; i += NT) h[i] = 0u;
#pragma unroll
  for (int q = 0; q < kWpt; ++q) bits[t * kWpt + q] = 0u;
  if (t == 0) {
    S.bin = kTopkBins - 1;
    S.above = 0u;
    S.nb = 0u;
    S.nlow = 0u;
    S.neq = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j * NT + t < (int)c) atomicAdd(&h[cand_bin((uint32_t)e[j], fl)], 1u);
  __syncthreads();
  {  // the bin of the k_eff-th largest key: thread t owns bins (NT - 1 - t) * 4 .. +4, top bins first
    const v4i y = reinterpret_cast<const v4i*>(h)[NT - 1 - t];
    const uint32_t hv[4] = {(uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]};
    const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
    uint32_t tot;
    uint32_t above = block_scan1<NT>(local, S.wt, tot);
    if (above < (uint32_t)keff && above + local >= (uint32_t)keff) {
      for (int b = 3; b >= 0; --b) {
        if (above + hv[b] >= (uint32_t)keff) {
          S.bin = (uint32_t)((NT - 1 - t) * 4 + b);
          S.above = above;
          S.nb = hv[b];
          break;
        }
        above += hv[b];
      }
    }
  }
  __syncthreads();
  DSA_STAMP(1, 11);
  const uint32_t bin = S.bin, nb = S.nb;
  if (bin == kTopkBins - 1) return false;  // uniform: the threshold lies in the open-ended top bin
  const uint32_t prefix = fl + bin;
  uint32_t need = (uint32_t)keff - S.above;  // keys of the threshold's prefix still to take
  if (nb <= 64u) {
    // the low 12 bits of the keys of that prefix, ranked by one wave
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = (uint32_t)e[j];
      if (j * NT + t < (int)c && (key >> 12) == prefix) S.low[atomicAdd(&S.nlow, 1u)] = key & 0xfffu;
    }
    __syncthreads();
    if (t < 64) {
      // every low part against every other: lane y's value reaches all lanes through v_readlane, so the loop
      // runs in registers (an LDS read per step had made it a chain of LDS round trips)
      const uint32_t dx = lane < (int)nb ? S.low[lane] : 0u;
      uint32_t gt = 0, ge = 0;
      for (uint32_t y = 0; y < nb; ++y) {
        const uint32_t dy = (uint32_t)__builtin_amdgcn_readlane((int)dx, (int)y);
        gt += dy > dx;
        ge += dy >= dx;
      }
      const uint64_t hit = __ballot(lane < (int)nb && gt < need && need <= ge);
      if (lane == __builtin_ctzll(hit)) {
        S.T = (prefix << 12) | dx;
        S.need = need - gt;
      }
    }
  } else {
    for (int i = t; i < kTopkBins; i += NT) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = (uint32_t)e[j];
      if (j * NT + t < (int)c && (key >> 12) == prefix) atomicAdd(&h[key & 0xfffu], 1u);
    }
    __syncthreads();
    const v4i y = reinterpret_cast<const v4i*>(h)[NT - 1 - t];
    const uint32_t hv[4] = {(uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]};
    const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
    uint32_t tot;
    uint32_t above = block_scan1<NT>(local, S.wt + NW, tot);
    if (above < need && above + local >= need) {
      for (int b = 3; b >= 0; --b) {
        if (above + hv[b] >= need) {
          S.T = (prefix << 12) | (uint32_t)((NT - 1 - t) * 4 + b);
          S.need = need - above;
          break;
        }
        above += hv[b];
      }
    }
  }
  __syncthreads();
  DSA_STAMP(1, 12);
  const uint32_t T = S.T;
  need = S.need;  // keys equal to T to take, lowest positions first
  // mark the keys above T; list the keys equal to T
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j * NT + t >= (int)c) continue;
    const uint32_t key = (uint32_t)e[j];
    const int32_t pos = (int32_t)(e[j] >> 32);
    if (key > T) {
      atomicOr(&bits[pos >> 5], 1u << (pos & 31));
    } else if (key == T) {
      const uint32_t at = atomicAdd(&S.neq, 1u);
      if (at < (uint32_t)kMaxTies) S.eq_pos[at] = pos;
    }
  }
  __syncthreads();
  const uint32_t neq = S.neq;
  if (neq > (uint32_t)kMaxTies) return false;  // uniform: too many ties to sort out here
  if (t < (int)neq) {  // an equal key is taken when fewer than `need` equal keys lie at lower positions
    const int32_t p = S.eq_pos[t];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < neq; ++j) rank += S.eq_pos[j] < p;
    if (rank < need) atomicOr(&bits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  DSA_STAMP(1, 13);
  // slots in position order: thread t owns bitmap words t kWpt .. +kWpt
  uint32_t w[kWpt], cntw = 0;
#pragma unroll
  for (int q = 0; q < kWpt / 4; ++q) {
    const v4i y = reinterpret_cast<const v4i*>(bits)[t * (kWpt / 4) + q];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      w[4 * q + x] = (uint32_t)y[x];
      cntw += (uint32_t)__popc((uint32_t)y[x]);
    }
  }
  // each word's page base is read before the writes (one read per word, all in flight together): a read per
  // selected position had made the loop a chain of LDS round trips
  int32_t wbase[kWpt];
#pragma unroll
  for (int q = 0; q < kWpt; ++q) wbase[q] = sink.word_base((t * kWpt + q) * 32);
  uint32_t tot;
  uint32_t slot = block_scan1<NT>(cntw, S.wt, tot);
  DSA_STAMP(1, 14);
#pragma unroll
  for (int q = 0; q < kWpt; ++q) {
    uint32_t b = w[q];
    while (b) {
      const int bit = __builtin_ctz(b);
      b &= b - 1;
      if (slot < (uint32_t)keff) sink.put_in_word(slot, (t * kWpt + q) * 32 + bit, wbase[q]);
      ++slot;
    }
  }
  return true;
}

// resolve_issue then resolve_finish, for callers with nothing to overlap.
template <int NT, class Sink>
__device__ void resolve_row(const float* __restrict__ row, int n, int keff, const RowCands& rc, int nblk_max,
                            ResolveLds& S, const Sink& sink) {
  ResolveLoads<NT> rl;
  resolve_issue<NT>(rc, nblk_max, rl);
  resolve_finish<NT>(row, n, keff, rc, rl, S, sink, NoStage{});
}

}  // namespace dsa
