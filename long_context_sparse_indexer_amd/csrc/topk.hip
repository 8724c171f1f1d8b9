// Top-k selection on gfx950: for each row keep the k_eff = min(k, n) largest scores (DeepSeek Sparse
// Attention explained, "How Does the Selector Pick 1,024?": keep the highest budget-many positions, and a
// row shorter than the budget is read in full).  Equal scores are taken lowest position first; the result
// is written in increasing position order, padded with -1.
//
// Scores become order-preserving 32-bit keys, selected by a radix select over three digits
// (bits 31..20, 19..8, 7..0).  Every hand-over between blocks happens at a kernel boundary:
//   digit 1  a per-row histogram of the first digit, accumulated in LDS per block and merged with one global
//            atomic per non-empty bin -- in the indexer's epilogue (fused step) or in a histogram pass over
//            stored scores (standalone call).
//   filter   grid (4096-score chunks, rows): every block finds the threshold bin b1 (the bin holding the
//            k_eff-th largest key) from the row histogram, writes the keys with digit 1 >= b1 in position
//            order into a segment of the row's candidate list, and histograms digit 2 of the keys in bin b1.
//   resolve  one 1024-thread block per row: finds b2 from the digit-2 histogram, places the candidates
//            (k + one bin's worth) in position order in LDS, settles digit 3 among the few keys of (b1, b2),
//            and writes the selection with a two-pass wave-ballot compaction.  A row whose candidates overflow
//            the list (heavily tied scores) is resolved over its whole stored score row instead.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "topk_common.h"


namespace dsa {
namespace {

constexpr int kCh = kTopkChunk;    // scores per filter / histogram block
constexpr int kTpb = 1024;         // threads of histogram / filter blocks
constexpr int kEpt = kCh / kTpb;   // scores per thread (consecutive)
constexpr int kCap = 12288;        // candidate entries a row keeps for the resolve step

Ws carve(const Geo& g, void* base) {
  Ws w;
  char* p = static_cast<char*>(base);
  w.nblk = std::max(1, (g.max_row_len + kCh - 1) / kCh);
  w.copies = hist_copies(g.R);
  auto take = [&](size_t bytes) { char* q = p; p += align_up(bytes); return q; };
  w.hist1 = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.copies * kTopkBins));
  w.hist2 = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * kTopkBins));
  w.cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 4 * (size_t)g.R));
  w.thr = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 4 * (size_t)g.R));
  w.seg_cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.seg_off = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.cand = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)g.R * kCap));
  return w;
}

// Zeroes the histograms and the counters of every row (one block per row).
__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* __restrict__ hist1, uint32_t* __restrict__ hist2,
                                                        uint32_t* __restrict__ cnt, int copies) {
  const int r = blockIdx.x;
  const v4i z = {0, 0, 0, 0};
  v4i* h1 = reinterpret_cast<v4i*>(hist1 + (int64_t)r * copies * kTopkBins);
  v4i* h2 = reinterpret_cast<v4i*>(hist2 + (int64_t)r * kTopkBins);
  for (int i = threadIdx.x; i < copies * kTopkBins / 4; i += blockDim.x) h1[i] = z;
  for (int i = threadIdx.x; i < kTopkBins / 4; i += blockDim.x) h2[i] = z;
  if (threadIdx.x == 0) reinterpret_cast<v4i*>(cnt)[r] = z;
}

// The kEpt = 4 consecutive scores of this thread in chunk c, as one 16-byte load with no branch: the row's
// stride is a multiple of 4 and at least n, so a 4-aligned offset below n can always be read whole; past the
// row's end offset 0 is read instead and the values are marked invalid where they are used.  Keeping the raw
// load apart from the key conversion lets a chunk's load stay in flight while the previous one is processed.
static_assert(kEpt == 4, "one 16-byte load per thread and chunk");
__device__ __forceinline__ v4f load_raw(const float* __restrict__ row, int c, int n) {
  const int64_t f = (int64_t)c * kCh + threadIdx.x * kEpt;
  return *reinterpret_cast<const v4f*>(row + (f < n ? f : 0));
}

// First-digit histogram of stored scores (standalone top-k): a block covers `cpb` consecutive 4096-score
// chunks of one row, accumulates them in LDS and merges once.
__global__ __launch_bounds__(kTpb) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ row_len, int max_row_len, int k,
                                                         uint32_t* __restrict__ hist1, int copies, int cpb) {
  __shared__ uint32_t h[kTopkBins];
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if (min(k, n) >= n || c0 >= nchunk) return;  // nothing to choose, or chunks past the row's end
  for (int i = threadIdx.x; i < kTopkBins; i += kTpb) h[i] = 0u;
  __syncthreads();
  const int c1 = min(nchunk, c0 + cpb);
  const float* row = scores + (int64_t)r * ld;
  auto count = [&](int c, const v4f& x) __attribute__((always_inline)) {
    const int64_t f = (int64_t)c * kCh + threadIdx.x * kEpt;
#pragma unroll
    for (int e = 0; e < kEpt; ++e)
      if (f + e < n) atomicAdd(&h[order_key(x[e]) >> 20], 1u);
  };
  // two buffers in turn: chunk c + 1 is loading while chunk c is counted
  v4f xa = load_raw(row, c0, n), xb;
  for (int c = c0; c < c1; c += 2) {
    if (c + 1 < c1) xb = load_raw(row, c + 1, n);
    count(c, xa);
    if (c + 1 >= c1) break;
    if (c + 2 < c1) xa = load_raw(row, c + 2, n);
    count(c + 1, xb);
  }
  __syncthreads();
  hist_merge<kTpb>(h, hist1 + ((int64_t)r * copies + blockIdx.x % copies) * kTopkBins);
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

// Where the fused step wants the pool row of every selected slot ([R, k] int32, -1 for padding); `out` NULL
// when no pool rows are wanted.
struct PoolRows {
  int32_t* out;
  const int32_t* row_seq;
  const int32_t* page_table;
  int num_seqs, max_pages, num_pages, log2ps;
};

// Pool rows of selected positions, written beside the selection when `out` is non-NULL (the fused step hands
// them to the attention kernels, which then skip the page-table lookup).  The row's page table is read from
// LDS when it was staged there (`pt`), else from global memory.
struct RowMap {
  int32_t* out;
  const int32_t* pt;  // page ids of the row's sequence: LDS copy or global row of the page table
  int max_pages, num_pages, log2ps;
  __device__ int32_t row(int32_t pos) const {
    const int lp = min(pos >> log2ps, max_pages - 1);
    const int page = min(max(pt[lp], 0), num_pages - 1);
    return (page << log2ps) | (pos & ((1 << log2ps) - 1));
  }
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
// Each wave owns a contiguous stretch of the list; one pass counts, one barrier publishes the per-wave counts,
// every wave adds up those of the waves before it, and a second pass writes.
template <int NT, class List, class Rows>
__device__ void write_selection(const List& L, int len, uint32_t T, uint32_t eq_need, int keff, int32_t* out,
                                const Rows& rows) {
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
  // this wave's first slot and its rank among the keys equal to T: the waves before it take all their keys
  // above T and their share of the equal ones, in list order
  uint32_t eq_run = 0, slot_run = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t we = w_eq[w];
    slot_run += w_gt[w] + (eq_run >= eq_need ? 0u : min(we, eq_need - eq_run));
    eq_run += we;
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
      if (sel && slot < (uint32_t)keff) {
        out[slot] = pos[u];
        if (rows.out) rows.out[slot] = rows.row(pos[u]);
      }
      eq_run += (uint32_t)__popcll(eqm);
      slot_run += (uint32_t)__popcll(selm);
    }
  }
  // no trailing barrier: every caller calls this once, as its last use of the LDS (a barrier would also wait
  // for the stores above to complete)
}

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

// Exclusive prefixes over the block of two values per thread, with one barrier: every wave scans its lanes and
// publishes its totals in wt[0 .. 2 NW), then every thread adds the totals of the waves before its own.  wt may
// be written again only after another barrier.
template <int NT>
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t* wt, uint32_t& pa, uint32_t& pb) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t ta, tb;
  pa = wave_exclusive_scan(a, ta);
  pb = wave_exclusive_scan(b, tb);
  if (lane == 0) { wt[wave] = ta; wt[NW + wave] = tb; }
  __syncthreads();
  static_assert(NW % 4 == 0, "wave totals are read four at a time");
#pragma unroll
  for (int q = 0; q < NW / 4; ++q) {  // 16-byte reads of the wave totals (wt is 16-byte aligned)
    const v4i ya = reinterpret_cast<const v4i*>(wt)[q], yb = reinterpret_cast<const v4i*>(wt + NW)[q];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * q + e < wave) {
        pa += (uint32_t)ya[e];
        pb += (uint32_t)yb[e];
      }
  }
}

constexpr int kResPages = 4096;  // page-table entries a resolve block stages in LDS

// LDS of the resolve step.
struct ResolveLds {
  uint32_t key[kCap];
  int32_t pos[kCap];
  uint32_t h[kTopkBins];
  uint32_t seg_start[kTopkMaxBlocksPerRow + 1];
  uint32_t seg_src[kTopkMaxBlocksPerRow];
  uint32_t scan[1024 / 64 + 1];  // one word per wave of the largest block, plus the total
  alignas(16) uint32_t scan2[2 * (1024 / 64)];
  uint32_t bin[64];               // low digits of the keys in bin (b1, b2), when there are at most 64
  int32_t pt[kResPages];          // page ids of the row's sequence, when they fit
};

// Threshold bin of one digit: the bin b holding the need-th largest key of histogram `gh` (the sum of `copies`
// consecutive 4096-bin replicas, top bin first), and the number of keys in bins above b.  Called by all NT
// threads; the result lands in *b, *above.
template <int NT>
__device__ __forceinline__ void threshold_bin(const uint32_t* __restrict__ gh, int copies, uint32_t need,
                                              uint32_t* scan, uint32_t* b, uint32_t* above_out) {
  constexpr int kPer = kTopkBins / NT;
  const int grp = NT - 1 - threadIdx.x;  // thread 0 owns the top bins
  uint32_t c[kPer];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) c[j] = 0u;
  for (int cp = 0; cp < copies; ++cp)
#pragma unroll
    for (int j = 0; j < kPer; ++j) c[j] += gh[cp * kTopkBins + grp * kPer + j];
#pragma unroll
  for (int j = 0; j < kPer; ++j) local += c[j];
  uint32_t total;
  uint32_t above = block_scan1<NT>(local, scan, total);
  if (above < need && above + local >= need) {
    for (int j = kPer - 1; j >= 0; --j) {
      if (above + c[j] >= need) {
        *b = (uint32_t)(grp * kPer + j);
        *above_out = above;
        break;
      }
      above += c[j];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTpb) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ row_len, int max_row_len,
                                                           int k, const uint32_t* __restrict__ hist1,
                                                           uint32_t* __restrict__ hist2, uint32_t* __restrict__ cnt,
                                                           uint32_t* __restrict__ thr, uint32_t* __restrict__ seg_cnt,
                                                           uint32_t* __restrict__ seg_off, uint64_t* __restrict__ cand,
                                                           int nblk_max, int copies, int cpb) {
  __shared__ __attribute__((aligned(16))) uint32_t scan[kTpb / 64 + 1];
  __shared__ uint32_t seg_base, s_b1, s_A1;
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if (keff >= n || c0 >= nchunk) return;
  const float* row = scores + (int64_t)r * ld;
  v4f xa = load_raw(row, c0, n), xb;  // the first chunk loads while the threshold is found
  // every block finds b1 itself (a read of the row's histogram replicas) instead of waiting for one block to
  // publish it; a block covers several chunks when the row has many
  threshold_bin<kTpb>(hist1 + (int64_t)r * copies * kTopkBins, copies, (uint32_t)keff, scan, &s_b1, &s_A1);
  const uint32_t b1 = s_b1;
  if (blockIdx.x == 0 && threadIdx.x == 0) { thr[4 * r + 0] = b1; thr[4 * r + 1] = s_A1; }
  uint32_t* h2 = hist2 + (int64_t)r * kTopkBins;
  const int c1 = min(nchunk, c0 + cpb);
  auto filter = [&](int ch, const v4f& x) __attribute__((always_inline)) {
    const int64_t first = (int64_t)ch * kCh + threadIdx.x * kEpt;
    uint32_t key[kEpt];
    bool valid[kEpt];
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
      valid[e] = first + e < n;
      key[e] = order_key(x[e]);
      const uint32_t d1 = key[e] >> 20;
      if (valid[e] && d1 >= b1) {
        ++c;
        if (d1 == b1) atomicAdd(&h2[(key[e] >> 8) & 0xfffu], 1u);
      }
    }
    uint32_t total;
    const uint32_t off = block_exclusive_scan(c, scan, total);  // per chunk: cheaper than block_scan1 under load
    if (threadIdx.x == 0) {
      seg_base = atomicAdd(&cnt[4 * r + 2], total);
      seg_cnt[(int64_t)r * nblk_max + ch] = total;
      seg_off[(int64_t)r * nblk_max + ch] = seg_base;
    }
    __syncthreads();
    const uint32_t base = seg_base;
    if (base + total <= (uint32_t)kCap) {  // on overflow the resolve kernel rescans the row
      uint64_t* dst = cand + (int64_t)r * kCap + base + off;
#pragma unroll
      for (int e = 0; e < kEpt; ++e)
        if (valid[e] && (key[e] >> 20) >= b1) *dst++ = ((uint64_t)(first + e) << 32) | key[e];
    }
    // no barrier here: the next chunk writes the scan words and seg_base only after barriers that every thread
    // reaches after reading this chunk's
  };
  // two buffers in turn: chunk c + 1 is loading while chunk c is filtered
  for (int ch = c0; ch < c1; ch += 2) {
    if (ch + 1 < c1) xb = load_raw(row, ch + 1, n);
    filter(ch, xa);
    if (ch + 1 >= c1) break;
    if (ch + 2 < c1) xa = load_raw(row, ch + 2, n);
    filter(ch + 1, xb);
  }
}

// Filter for blocks that cover several chunks (long rows, large batches).  The chunk loop stages each chunk's
// candidates in LDS (position order within the chunk, chunks in order) and counts digit 2 of the keys in bin b1
// in an LDS histogram, so its only memory traffic is the next chunk's scores, loaded while the current one is
// filtered.  When the stage is full, and at the end, the block reserves one range of the row's candidate list
// with one atomic, copies the stage out and writes the segment table of the chunks it holds; the histogram is
// merged once at the end.
constexpr int kStageCap = 6144;  // staged candidates per block (48 KiB; two 1024-thread blocks fit a CU)
static_assert(kCh <= kStageCap, "one chunk always fits an empty stage");

__global__ __launch_bounds__(kTpb) void topk_filter_staged_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int max_row_len, int k,
    const uint32_t* __restrict__ hist1, uint32_t* __restrict__ hist2, uint32_t* __restrict__ cnt,
    uint32_t* __restrict__ thr, uint32_t* __restrict__ seg_cnt, uint32_t* __restrict__ seg_off,
    uint64_t* __restrict__ cand, int nblk_max, int copies, int cpb) {
  __shared__ __attribute__((aligned(16))) uint32_t scan[kTpb / 64 + 1];
  __shared__ uint64_t stage[kStageCap];
  __shared__ uint32_t h2l[kTopkBins];
  __shared__ uint32_t chunk_n[kTopkMaxBlocksPerRow];  // candidates of each staged chunk
  __shared__ uint32_t seg_base, s_b1, s_A1;
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if (keff >= n || c0 >= nchunk) return;
  const float* row = scores + (int64_t)r * ld;
  v4f x = load_raw(row, c0, n);  // the first chunk loads while the threshold is found
  for (int i = threadIdx.x; i < kTopkBins; i += kTpb) h2l[i] = 0u;
  threshold_bin<kTpb>(hist1 + (int64_t)r * copies * kTopkBins, copies, (uint32_t)keff, scan, &s_b1, &s_A1);
  const uint32_t b1 = s_b1;
  if (blockIdx.x == 0 && threadIdx.x == 0) { thr[4 * r + 0] = b1; thr[4 * r + 1] = s_A1; }
  const int c1 = min(nchunk, c0 + cpb);
  // staged chunks [cs, ch) hold `staged` candidates
  int cs = c0;
  uint32_t staged = 0;
  auto flush = [&](int ch) __attribute__((always_inline)) {
    if (threadIdx.x == 0) seg_base = atomicAdd(&cnt[4 * r + 2], staged);
    __syncthreads();
    const uint32_t base = seg_base;
    uint64_t* dst = cand + (int64_t)r * kCap;
    for (uint32_t i = threadIdx.x; i < staged; i += kTpb)
      if (base + i < (uint32_t)kCap) dst[base + i] = stage[i];  // on overflow the resolve rescans the row
    // segment table of the staged chunks: thread t holds chunk cs + t (at most kTopkMaxBlocksPerRow of them)
    const int t = threadIdx.x;
    const uint32_t cn = t < ch - cs ? chunk_n[t] : 0u;
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan(cn, scan, tot);
    if (t < ch - cs) {
      seg_cnt[(int64_t)r * nblk_max + cs + t] = cn;
      seg_off[(int64_t)r * nblk_max + cs + t] = base + pre;
    }
    cs = ch;
    staged = 0;
  };
  for (int ch = c0; ch < c1; ++ch) {
    const v4f cur = x;
    if (ch + 1 < c1) x = load_raw(row, ch + 1, n);  // next chunk in flight while this one is filtered
    const int64_t first = (int64_t)ch * kCh + threadIdx.x * kEpt;
    uint32_t key[kEpt];
    uint32_t c = 0, take = 0;
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
      key[e] = order_key(cur[e]);
      const uint32_t d1 = key[e] >> 20;
      if (first + e < n && d1 >= b1) {
        ++c;
        take |= 1u << e;
        if (d1 == b1) atomicAdd(&h2l[(key[e] >> 8) & 0xfffu], 1u);
      }
    }
    uint32_t total;
    const uint32_t off = block_exclusive_scan(c, scan, total);
    if (staged + total > (uint32_t)kStageCap) flush(ch);  // uniform: total is the block's
    uint32_t o = staged + off;
#pragma unroll
    for (int e = 0; e < kEpt; ++e)
      if (take & (1u << e)) stage[o++] = ((uint64_t)(first + e) << 32) | key[e];
    if (threadIdx.x == 0) chunk_n[ch - cs] = total;
    staged += total;
  }
  __syncthreads();  // the stage, chunk counts and histogram are complete
  flush(c1);
  hist_merge<kTpb>(h2l, hist2 + (int64_t)r * kTopkBins);
}

constexpr int kRes = 1024;  // threads of the resolve block

__global__ __launch_bounds__(kRes) void topk_resolve_kernel(const float* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ row_len, int max_row_len,
                                                            int k, const uint32_t* __restrict__ thr,
                                                            const uint32_t* __restrict__ hist2,
                                                            const uint32_t* __restrict__ cnt,
                                                            const uint32_t* __restrict__ seg_cnt,
                                                            const uint32_t* __restrict__ seg_off,
                                                            const uint64_t* __restrict__ cand, int nblk_max,
                                                            int32_t* __restrict__ topk_idx, PoolRows pr) {
  static_assert(kRes >= kTopkMaxBlocksPerRow, "one chunk per thread");
  __shared__ ResolveLds S;
  __shared__ uint32_t s_b2, s_A2, s_nb, s_nbin;
  const int r = blockIdx.x;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  int32_t* out = topk_idx + (int64_t)r * k;
  // pool rows of the selection (fused step): the sequence's page ids, staged in LDS when they fit
  const int32_t* gpt = pr.out ? pr.page_table + (int64_t)clamp_seq(pr.row_seq[r], pr.num_seqs) * pr.max_pages : nullptr;
  const bool pt_lds = pr.out && pr.max_pages <= kResPages;
  RowMap rows{pr.out ? pr.out + (int64_t)r * k : nullptr, pt_lds ? S.pt : gpt, pr.max_pages, pr.num_pages, pr.log2ps};
  if (keff >= n) {
    const RowMap grows{rows.out, gpt, pr.max_pages, pr.num_pages, pr.log2ps};
    for (int i = threadIdx.x; i < k; i += kRes) {
      out[i] = i < n ? i : -1;
      if (grows.out) grows.out[i] = i < n ? grows.row(i) : -1;
    }
    return;
  }
  if (pt_lds)  // read before the first barrier below, used after it
    for (int i = threadIdx.x; i < pr.max_pages; i += kRes) S.pt[i] = gpt[i];
  const float* row = scores + (int64_t)r * ld;
  // every read that does not depend on another is issued here, together: the thresholds, the candidate count,
  // the segment tables and the digit-2 histogram; the candidates follow as soon as their count arrives and stay
  // in flight through the two block scans
  const int nblk = (n + kCh - 1) / kCh;
  const int t = threadIdx.x;
  const uint32_t b1 = thr[4 * r + 0], A1 = thr[4 * r + 1];
  const uint32_t len = cnt[4 * r + 2];
  const uint32_t c = t < nblk ? seg_cnt[(int64_t)r * nblk_max + t] : 0u;
  const uint32_t src = t < nblk ? seg_off[(int64_t)r * nblk_max + t] : 0u;
  constexpr int kPerBin = kTopkBins / kRes;
  uint32_t h2v[kPerBin];
  {
    const uint32_t* gh = hist2 + (int64_t)r * kTopkBins + (kRes - 1 - t) * kPerBin;  // top bins first
#pragma unroll
    for (int j = 0; j < kPerBin; ++j) h2v[j] = gh[j];
  }
  // the first candidates load before their count is known (entries past it are ignored)
  constexpr int kPer = (kCap + kRes - 1) / kRes;
  constexpr int kFirst = 4;
  uint64_t e[kPer];
#pragma unroll
  for (int j = 0; j < kFirst; ++j) e[j] = cand[(int64_t)r * kCap + j * kRes + t];
  if (len <= (uint32_t)kCap) {
#pragma unroll
    for (int j = kFirst; j < kPer; ++j) {
      const int i = j * kRes + t;
      e[j] = i < (int)len ? cand[(int64_t)r * kCap + i] : 0ull;
    }
    // b2 -- the bin of digit 2 (within b1) holding the (k_eff - A1)-th largest key, thread t owning bins
    // (kRes - 1 - t) * kPerBin .. top first -- and the segment starts in position order (thread t = chunk t):
    // two scans, one barrier
    uint32_t hl = 0;
#pragma unroll
    for (int j = 0; j < kPerBin; ++j) hl += h2v[j];
    uint32_t above, start;
    if (t == 0) s_nbin = 0;
    block_scan2<kRes>(hl, c, S.scan2, above, start);
    const uint32_t need2 = (uint32_t)keff - A1;
    if (above < need2 && above + hl >= need2) {
      uint32_t run = above;
      for (int j = kPerBin - 1; j >= 0; --j) {
        if (run + h2v[j] >= need2) {
          s_b2 = (uint32_t)((kRes - 1 - t) * kPerBin + j);
          s_A2 = run;
          s_nb = h2v[j];
          break;
        }
        run += h2v[j];
      }
    }
    if (t < nblk) {
      S.seg_start[t] = start;
      S.seg_src[t] = src;
    }
    __syncthreads();
    const uint32_t b2 = s_b2, A2 = A1 + s_A2, nb = s_nb;  // nb: keys in bin (b1, b2), all in the list
    const uint32_t prefix = (b1 << 12) | b2;
    const int lane = t & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // every candidate goes to its chunk's segment start + its offset within the segment
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = j * kRes + t;
      if (i < (int)len) {
        const uint32_t pos = (uint32_t)(e[j] >> 32);
        const int chunk = (int)(pos / kCh);
        const uint32_t dst = S.seg_start[chunk] + ((uint32_t)i - S.seg_src[chunk]);
        S.key[dst] = (uint32_t)e[j];
        S.pos[dst] = (int32_t)pos;
      }
    }
    // the low digits of the keys in bin (b1, b2), when they fit one wave (their order does not matter)
    if (nb <= 64u) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = j * kRes + t;
        const uint32_t key = (uint32_t)e[j];
        const bool match = i < (int)len && (key >> 8) == prefix;
        const uint64_t mm = __ballot(match);
        if (mm) {  // uniform over the wave
          const int leader = __builtin_ctzll(mm);
          uint32_t base = 0;
          if (lane == leader) base = atomicAdd(&s_nbin, (uint32_t)__popcll(mm));
          base = __shfl(base, leader, 64);
          if (match) S.bin[base + (uint32_t)__popcll(mm & below)] = key & 0xffu;
        }
      }
    }
    __syncthreads();
    const LdsList L{S.key, S.pos};
    uint32_t need = (uint32_t)keff - A2;  // keys of (b1, b2) still to take
    uint32_t d3;
    if (nb <= 64u) {
      // every wave finds digit 3 itself: lane x ranks the low digit of the x-th key of the bin among all nb
      const uint32_t dx = lane < (int)nb ? S.bin[lane] : 0u;
      uint32_t gt = 0, ge = 0;
      for (uint32_t y = 0; y < nb; ++y) {
        const uint32_t dy = S.bin[y];
        gt += dy > dx;
        ge += dy >= dx;
      }
      const uint64_t hit = __ballot(lane < (int)nb && gt < need && need <= ge);  // lanes holding the digit
      const int src_lane = __builtin_ctzll(hit);
      d3 = __shfl(dx, src_lane, 64);
      need -= __shfl(gt, src_lane, 64);
    } else {
      d3 = refine_digit<kRes>(L, (int)len, prefix, 0, 8, need, S.h, S.scan);
    }
    write_selection<kRes>(L, (int)len, (b1 << 20) | (b2 << 8) | d3, need, keff, out, rows);
  } else {
    const RowList L{row};
    uint32_t need = (uint32_t)keff;
    const uint32_t d1 = refine_digit<kRes>(L, n, 0u, 20, 12, need, S.h, S.scan);
    const uint32_t d2 = refine_digit<kRes>(L, n, d1, 8, 12, need, S.h, S.scan);
    const uint32_t d3 = refine_digit<kRes>(L, n, (d1 << 12) | d2, 0, 8, need, S.h, S.scan);
    write_selection<kRes>(L, n, (d1 << 20) | (d2 << 8) | d3, need, keff, out, rows);
  }
  for (int i = keff + threadIdx.x; i < k; i += kRes) {
    out[i] = -1;
    if (rows.out) rows.out[i] = -1;
  }
}

}  // namespace

size_t topk_workspace_bytes(const Geo& g) {
  const size_t nblk = (size_t)std::max(1, (g.max_row_len + kCh - 1) / kCh);
  const size_t R = (size_t)g.R;
  return align_up(4 * R * hist_copies(g.R) * kTopkBins) + align_up(4 * R * kTopkBins) + 2 * align_up(16 * R) +
         2 * align_up(4 * R * nblk) + align_up(8 * R * kCap);
}

TopkState topk_state(const Geo& g, void* workspace) {
  const Ws w = carve(g, workspace);
  return TopkState{w.hist1, w.copies};
}

hipError_t launch_topk_zero(const Geo& g, void* workspace, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  topk_zero_kernel<<<g.R, 256, 0, stream>>>(w.hist1, w.hist2, w.cnt, w.copies);
  return hipGetLastError();
}

// Chunks per histogram / filter block: at most 32 blocks per row (each filter block re-reads the row's
// histogram replicas to find the threshold) and about 512 blocks overall (two 1024-thread blocks per CU) once
// there are enough chunks: a block that covers several chunks stages its candidates and keeps the next chunk's
// scores in flight (64 rows of 16 chunks: 34 -> 29 us for the top-k).
int chunks_per_block(const Geo& g, int nblk) {
  const int64_t total = (int64_t)nblk * g.R;
  return (int)std::min<int64_t>(nblk, std::max<int64_t>({1, (nblk + 31) / 32, total / 512}));
}

hipError_t launch_topk_select(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                              bool hist_done, int32_t* pool_rows, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  const int cpb = chunks_per_block(g, w.nblk);
  dim3 grid((w.nblk + cpb - 1) / cpb, g.R);
  if (!hist_done)
    topk_hist_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.hist1, w.copies, cpb);
  if (cpb > 1)
    topk_filter_staged_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.hist1, w.hist2,
                                                         w.cnt, w.thr, w.seg_cnt, w.seg_off, w.cand, w.nblk, w.copies,
                                                         cpb);
  else
  topk_filter_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.hist1, w.hist2, w.cnt,
                                                w.thr, w.seg_cnt, w.seg_off, w.cand, w.nblk, w.copies, cpb);
  topk_resolve_kernel<<<g.R, kRes, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.hist2, w.cnt,
                                                w.seg_cnt, w.seg_off, w.cand, w.nblk, topk_idx,
                                                PoolRows{pool_rows, g.row_seq, g.page_table, g.S, g.max_pages,
                                                         g.num_pages, g.log2ps});
  return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                       int32_t* pool_rows, hipStream_t stream) {
  hipError_t e = launch_topk_zero(g, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_topk_select(g, scores, ld, topk_idx, workspace, false, pool_rows, stream);
}

}  // namespace dsa
