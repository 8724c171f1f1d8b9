// Top-k selection on gfx950: for each row keep the k_eff = min(k, n) largest scores (DeepSeek Sparse
// Attention explained, "How Does the Selector Pick 1,024?": keep the highest budget-many positions, and a
// row shorter than the budget is read in full).  Equal scores are taken lowest position first; the result
// is written in increasing position order, padded with -1.
//
// Scores become order-preserving 32-bit keys.  Every hand-over between blocks happens at a kernel boundary:
//   filter   grid (4096-score chunks, rows): every block first finds the row's floor, the 20-bit key prefix of a
//            sampled score that comfortably more than k_eff scores of the row exceed.  The sample is a fixed set
//            of evenly spaced runs of the row, the same in every block, ranked through an LDS histogram.  The
//            block then writes the keys whose first 20 bits reach the floor, in position order, into a segment of
//            the row's candidate list.
//   resolve  one 1024-thread block per row: counts the candidates in an LDS histogram of their 20-bit prefixes
//            taken relative to the floor (4096 bins, the last open-ended), finds the bin holding the k_eff-th
//            largest key, places the candidates in position order in LDS, settles the low 12 bits among the few
//            keys of that bin, and writes the selection with a two-pass wave-ballot compaction.  A row whose
//            sample overshot (fewer than k_eff candidates) or whose candidates overflow the list (heavily tied
//            scores) is resolved over its whole stored score row instead, by a three-digit radix select.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "topk_common.h"


namespace dsa {
namespace {

constexpr int kCh = kTopkChunk;    // scores per filter chunk
constexpr int kTpb = 1024;         // threads of filter blocks
constexpr int kEpt = kCh / kTpb;   // scores per thread (consecutive)
constexpr int kCap = 12288;        // candidate entries a row keeps for the resolve step

Ws carve(const Geo& g, void* base) {
  Ws w;
  char* p = static_cast<char*>(base);
  w.nblk = std::max(1, (g.max_row_len + kCh - 1) / kCh);
  auto take = [&](size_t bytes) { char* q = p; p += align_up(bytes); return q; };
  w.cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 4 * (size_t)g.R));
  w.thr = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 4 * (size_t)g.R));
  w.seg_cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.seg_off = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.cand = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)g.R * kCap));
  return w;
}

// Zeroes the counters of every row (one thread per row).
__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* __restrict__ cnt, int R) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) reinterpret_cast<v4i*>(cnt)[r] = v4i{0, 0, 0, 0};
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

constexpr int kResPages = 4096;  // page-table entries a resolve block stages in LDS

// LDS of the resolve step.
struct ResolveLds {
  uint32_t key[kCap];
  int32_t pos[kCap];
  alignas(16) uint32_t h[kTopkBins];  // candidate histogram, then the refine passes' digit histograms
  uint32_t seg_start[kTopkMaxBlocksPerRow + 1];
  uint32_t seg_src[kTopkMaxBlocksPerRow];
  uint32_t scan[1024 / 64 + 1];  // one word per wave of the largest block, plus the total
  alignas(16) uint32_t scan2[2 * (1024 / 64)];
  uint32_t bin[64];               // low 12 bits of the keys of the threshold's 20-bit prefix, when at most 64
  int32_t pt[kResPages];          // page ids of the row's sequence, when they fit
};

// A sampled row of n scores is sampled about n / kSampleDiv times (n / 64 measured slower: 1.7 us more per
// 128K-position decode step, 8% more for a 4096-row prefill chunk, from the extra candidates).
constexpr int kSampleDiv = 32;

// The bin of an LDS histogram holding the need-th largest entry, counting from the top bin, found by wave 0
// alone in two levels: lane l sums the kBins/64 bins (63 - l) * kBins/64 .. (lane 0 the top ones) with 16-byte
// reads and a DPP scan over the lanes picks the lane L holding the bin; then lanes g < kBins/256 take L's groups
// of four bins, top group first, a second scan picks the group, and its lane walks the four bins.  The bin and the
// number of entries above it land in *b, *above (left as preset when the histogram holds fewer than `need`).
// Called by wave 0 only; the caller publishes the result with a barrier.
template <int kBins>
__device__ __forceinline__ void wave_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* b, uint32_t* above_out) {
  constexpr int kPer = kBins / 64, kGroups = kPer / 4;
  static_assert(kPer % 4 == 0 && kGroups <= 64, "16-byte reads of a lane's bins");
  const int lane = threadIdx.x;
  const v4i* hb = reinterpret_cast<const v4i*>(h);
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const v4i x = hb[(63 - lane) * kGroups + q];
    local += (uint32_t)(x[0] + x[1] + x[2] + x[3]);
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

// The row's floor: the first 20 bits of the m-th largest score of a sample of the row, ranked in two rounds of an
// LDS histogram: bits 31..20 of every sampled key (4096 bins in h), then bits 19..12 of those in the bin found
// (256 bins in h2), each ranked by one wave.  The sample is S scores in S/4 runs of four (one 16-byte load each)
// spread evenly over the row, with S the power of two in (n / 2d, n / d] for d = kSampleDiv, kept within
// [1024, 16384] (up to 65536 for rows past 2^21): it reads a small part of the row and is the same in every block.
// With mu = k_eff S/n the expected number of sampled scores among the row's k_eff largest, m = mu + 8 sqrt(mu) + 16
// puts the floor far enough below the k_eff-th largest score that a row rarely has fewer than k_eff scores at or
// above it, while about n m / S = k_eff + 8 sqrt(k_eff n / S) + 16 n / S scores reach it.  A row of at most one
// chunk is its own sample, with m = k_eff: its floor is exactly the 20-bit prefix of the k_eff-th largest score.
// h, h2: kTopkBins and 256 words of LDS, 16-byte aligned; s: 4 words of LDS.  Called by all NT threads; ends with
// a barrier.
template <int NT>
__device__ __forceinline__ uint32_t floor_prefix(const float* __restrict__ row, int n, int keff, uint32_t* h,
                                                 uint32_t* h2, uint32_t* s) {
  constexpr int kGroup = 4;  // runs per thread held in registers: all of them up to S = 16384
  int runs, m, step = 4;  // run j starts at position j * step (rounded down to a multiple of 4)
  if (n <= kCh) {
    runs = (n + 3) / 4;
    m = keff;
  } else {
    const int cap = n > (1 << 21) ? 65536 : 16384;
    const int S = min(cap, max(1024, 1 << (31 - __builtin_clz((unsigned)(n / kSampleDiv)))));
    runs = S / 4;
    step = n / runs;
    const float mu = (float)keff * (float)S / (float)n;
    m = min(S, (int)ceilf(mu + 8.f * sqrtf(mu) + 16.f));
  }
  const int ngroups = (runs + kGroup * NT - 1) / (kGroup * NT);
  // run j starts at a multiple of 4 below n, so its 16-byte load lies inside the row's stride (a multiple of 4
  // at least n); in a sampled row step = floor(n / runs) >= 16 and j < runs, so the run ends before n
  v4f x[kGroup];
  auto load = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int j = threadIdx.x + (g * kGroup + q) * NT;
      if (j < runs) x[q] = *reinterpret_cast<const v4f*>(row + ((j * step) & ~3));
    }
  };
  // one histogram round over the sample: bin (key >> shift) & mask of every sampled key whose bits from
  // shift + bits up equal `prefix`
  auto round = [&](uint32_t* hist, int shift, int bits, uint32_t prefix, bool reload) __attribute__((always_inline)) {
#pragma unroll 1
    for (int g = 0; g < ngroups; ++g) {
      if (g > 0 || reload) load(g);
#pragma unroll
      for (int q = 0; q < kGroup; ++q) {
        const int j = threadIdx.x + (g * kGroup + q) * NT;
        if (j < runs) {
          // the four scores of a run often share a bin: equal neighbours are counted with one atomic, which
          // keeps same-address LDS atomics of a wave few
          uint32_t bin = 0, cntb = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = order_key(x[q][e]);
            const bool in = (n > kCh || 4 * j + e < n) && (uint32_t)((uint64_t)key >> (shift + bits)) == prefix;
            const uint32_t b = (key >> shift) & ((1u << bits) - 1u);
            if (in && cntb && b != bin) {
              atomicAdd(&hist[bin], cntb);
              cntb = 0;
            }
            if (in) {
              bin = b;
              ++cntb;
            }
          }
          if (cntb) atomicAdd(&hist[bin], cntb);
        }
      }
    }
  };
  load(0);  // in flight while the histograms are cleared
  for (int i = threadIdx.x; i < kTopkBins; i += NT) h[i] = 0u;
  for (int i = threadIdx.x; i < 256; i += NT) h2[i] = 0u;
  if (threadIdx.x == 0) {  // a floor of 0 keeps every key, should the sample rank fail
    s[0] = s[1] = s[2] = s[3] = 0u;
  }
  __syncthreads();
  round(h, 20, 12, 0u, false);
  __syncthreads();
  if (threadIdx.x < 64) wave_threshold_bin<kTopkBins>(h, (uint32_t)m, &s[0], &s[1]);
  __syncthreads();
  const uint32_t b1 = s[0];
  round(h2, 12, 8, b1, ngroups > 1);
  __syncthreads();
  if (threadIdx.x < 64) wave_threshold_bin<256>(h2, (uint32_t)m - s[1], &s[2], &s[3]);
  __syncthreads();
  return (b1 << 8) | s[2];
}

// Bin of a candidate key in the row's candidate histogram: its 20-bit prefix relative to the floor, the last bin
// taking everything 4095 or more 20-bit steps above the floor.
__device__ __forceinline__ uint32_t cand_bin(uint32_t key, uint32_t floor20) {
  return min((key >> 12) - floor20, (uint32_t)kTopkBins - 1u);
}

__global__ __launch_bounds__(kTpb) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ row_len, int max_row_len,
                                                           int k, uint32_t* __restrict__ cnt,
                                                           uint32_t* __restrict__ thr,
                                                           uint32_t* __restrict__ seg_cnt,
                                                           uint32_t* __restrict__ seg_off, uint64_t* __restrict__ cand,
                                                           int nblk_max, int cpb) {
  __shared__ __attribute__((aligned(16))) uint32_t scan[kTpb / 64 + 1];
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ __attribute__((aligned(16))) uint32_t h2[256];
  __shared__ uint32_t seg_base, s_f[4];
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if (keff >= n || c0 >= nchunk) return;
  const float* row = scores + (int64_t)r * ld;
  v4f xa = load_raw(row, c0, n), xb;  // the first chunk loads together with the sample
  // every block ranks the sample itself instead of waiting for one block to publish the floor
  const uint32_t fl = floor_prefix<kTpb>(row, n, keff, h, h2, s_f);
  if (blockIdx.x == 0 && threadIdx.x == 0) thr[4 * r + 0] = fl;
  const int c1 = min(nchunk, c0 + cpb);
  auto filter = [&](int ch, const v4f& x) __attribute__((always_inline)) {
    const int64_t first = (int64_t)ch * kCh + threadIdx.x * kEpt;
    uint32_t key[kEpt];
    bool keep[kEpt];
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
      key[e] = order_key(x[e]);
      keep[e] = first + e < n && (key[e] >> 12) >= fl;
      c += keep[e];
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
        if (keep[e]) *dst++ = ((uint64_t)(first + e) << 32) | key[e];
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
// candidates in LDS (position order within the chunk, chunks in order), so its only memory traffic is the next
// chunk's scores, loaded while the current one is filtered.  When the stage is full, and at the end, the block
// reserves one range of the row's candidate list with one atomic, copies the stage out and writes the segment
// table of the chunks it holds.
constexpr int kStageCap = 6144;  // staged candidates per block (48 KiB; two 1024-thread blocks fit a CU)
static_assert(kCh <= kStageCap, "one chunk always fits an empty stage");

__global__ __launch_bounds__(kTpb) void topk_filter_staged_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int max_row_len, int k,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ thr,
    uint32_t* __restrict__ seg_cnt, uint32_t* __restrict__ seg_off, uint64_t* __restrict__ cand, int nblk_max,
    int cpb) {
  __shared__ __attribute__((aligned(16))) uint32_t scan[kTpb / 64 + 1];
  __shared__ uint64_t stage[kStageCap];
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];  // the sample's histograms
  __shared__ __attribute__((aligned(16))) uint32_t h2[256];
  __shared__ uint32_t chunk_n[kTopkMaxBlocksPerRow];  // candidates of each staged chunk
  __shared__ uint32_t seg_base, s_f[4];
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if (keff >= n || c0 >= nchunk) return;
  const float* row = scores + (int64_t)r * ld;
  v4f x = load_raw(row, c0, n);  // the first chunk loads together with the sample
  const uint32_t fl = floor_prefix<kTpb>(row, n, keff, h, h2, s_f);
  if (blockIdx.x == 0 && threadIdx.x == 0) thr[4 * r + 0] = fl;
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
      if (first + e < n && (key[e] >> 12) >= fl) {
        ++c;
        take |= 1u << e;
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
  __syncthreads();  // the stage and chunk counts are complete
  flush(c1);
}

constexpr int kRes = 1024;  // threads of the resolve block

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
template <class List>
__device__ __attribute__((noinline)) void select_and_write(List L, int len, uint32_t need, int keff, int32_t* out,
                                                            RowMap rows, uint32_t* h, uint32_t* scan) {
  const uint32_t T = select_key<kRes>(L, len, need, h, scan);
  write_selection<kRes>(L, len, T, need, keff, out, rows);
}

__global__ __launch_bounds__(kRes) void topk_resolve_kernel(const float* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ row_len, int max_row_len,
                                                            int k, const uint32_t* __restrict__ thr,
                                                            const uint32_t* __restrict__ cnt,
                                                            const uint32_t* __restrict__ seg_cnt,
                                                            const uint32_t* __restrict__ seg_off,
                                                            const uint64_t* __restrict__ cand, int nblk_max,
                                                            int32_t* __restrict__ topk_idx, PoolRows pr) {
  static_assert(kRes >= kTopkMaxBlocksPerRow, "one chunk per thread");
  __shared__ ResolveLds S;
  __shared__ uint32_t s_bin, s_above, s_nb, s_nbin;
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
  // every read that does not depend on another is issued here, together: the floor, the candidate count and the
  // segment tables; the candidates follow as soon as their count arrives
  const int nblk = (n + kCh - 1) / kCh;
  const int t = threadIdx.x;
  const uint32_t fl = thr[4 * r + 0];
  const uint32_t len = cnt[4 * r + 2];
  const uint32_t c = t < nblk ? seg_cnt[(int64_t)r * nblk_max + t] : 0u;
  const uint32_t src = t < nblk ? seg_off[(int64_t)r * nblk_max + t] : 0u;
  constexpr int kPerBin = kTopkBins / kRes;
  static_assert(kPerBin == 4, "one 16-byte LDS read of histogram bins per thread");
  for (int i = t; i < kTopkBins; i += kRes) S.h[i] = 0u;  // the candidate histogram, cleared before a barrier
  // the first candidates load before their count is known (entries past it are ignored)
  constexpr int kPer = (kCap + kRes - 1) / kRes;
  constexpr int kFirst = 4;
  uint64_t e[kPer];
#pragma unroll
  for (int j = 0; j < kFirst; ++j) e[j] = cand[(int64_t)r * kCap + j * kRes + t];
  if (len >= (uint32_t)keff && len <= (uint32_t)kCap) {
#pragma unroll
    for (int j = kFirst; j < kPer; ++j) {
      const int i = j * kRes + t;
      e[j] = i < (int)len ? cand[(int64_t)r * kCap + i] : 0ull;
    }
    // the segment starts in position order (thread t = chunk t); the scan's barrier also publishes the cleared
    // histogram, into which every candidate then counts by its 20-bit prefix relative to the floor
    uint32_t ctot;
    const uint32_t start = block_scan1<kRes>(c, S.scan2, ctot);
    if (t == 0) {  // the open bin, unless the scan finds the threshold (it does: the bins hold len >= k_eff keys)
      s_nbin = 0;
      s_bin = kTopkBins - 1;
      s_above = 0;
      s_nb = 0;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (j * kRes + t < (int)len) atomicAdd(&S.h[cand_bin((uint32_t)e[j], fl)], 1u);
    if (t < nblk) {
      S.seg_start[t] = start;
      S.seg_src[t] = src;
    }
    __syncthreads();
    // the bin holding the k_eff-th largest key, thread t owning bins (kRes - 1 - t) * kPerBin .. (top first)
    const v4i hv = reinterpret_cast<const v4i*>(S.h)[kRes - 1 - t];
    const uint32_t hl = (uint32_t)(hv[0] + hv[1] + hv[2] + hv[3]);
    uint32_t htot;
    const uint32_t above = block_scan1<kRes>(hl, S.scan2, htot);
    if (above < (uint32_t)keff && above + hl >= (uint32_t)keff) {
      uint32_t run = above;
      for (int j = kPerBin - 1; j >= 0; --j) {
        if (run + (uint32_t)hv[j] >= (uint32_t)keff) {
          s_bin = (uint32_t)((kRes - 1 - t) * kPerBin + j);
          s_above = run;
          s_nb = (uint32_t)hv[j];
          break;
        }
        run += (uint32_t)hv[j];
      }
    }
    __syncthreads();
    // nb keys share the threshold's 20-bit prefix, unless the threshold lies in the open-ended top bin
    const uint32_t bin = s_bin, nb = s_nb;
    const bool open = bin == kTopkBins - 1;
    const uint32_t prefix = fl + bin;
    const int lane = t & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // every candidate goes to its chunk's segment start + its offset within the segment; beside, the low 12 bits
    // of the keys of the threshold's prefix are collected when they fit one wave (their order does not matter)
    const bool few = !open && nb <= 64u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = j * kRes + t;
      const uint32_t key = (uint32_t)e[j];
      if (i < (int)len) {
        const uint32_t pos = (uint32_t)(e[j] >> 32);
        const int chunk = (int)(pos / kCh);
        const uint32_t dst = S.seg_start[chunk] + ((uint32_t)i - S.seg_src[chunk]);
        S.key[dst] = key;
        S.pos[dst] = (int32_t)pos;
      }
      if (few) {
        const bool match = i < (int)len && (key >> 12) == prefix;
        const uint64_t mm = __ballot(match);
        if (mm) {  // uniform over the wave
          const int leader = __builtin_ctzll(mm);
          uint32_t base = 0;
          if (lane == leader) base = atomicAdd(&s_nbin, (uint32_t)__popcll(mm));
          base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
          if (match) S.bin[base + (uint32_t)__popcll(mm & below)] = key & 0xfffu;
        }
      }
    }
    __syncthreads();
    const LdsList L{S.key, S.pos};
    uint32_t need = (uint32_t)keff - s_above;  // keys of the threshold's bin still to take
    uint32_t T;
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
      T = (prefix << 12) | refine_digit<kRes>(L, (int)len, prefix, 0, 12, need, S.h, S.scan);
    }
    if (open) select_and_write(L, (int)len, need, keff, out, rows, S.h, S.scan);
    else write_selection<kRes>(L, (int)len, T, need, keff, out, rows);
  } else {
    select_and_write(RowList{row}, n, (uint32_t)keff, keff, out, rows, S.h, S.scan);
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
  return 2 * align_up(16 * R) + 2 * align_up(4 * R * nblk) + align_up(8 * R * kCap);
}

TopkState topk_state(const Geo& g, void* workspace) {
  const Ws w = carve(g, workspace);
  return TopkState{w.cnt};
}

hipError_t launch_topk_zero(const Geo& g, void* workspace, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  topk_zero_kernel<<<(g.R + 255) / 256, 256, 0, stream>>>(w.cnt, g.R);
  return hipGetLastError();
}

// Chunks per filter block: at most 32 blocks per row (each filter block ranks the row's sample) and about 512
// blocks overall (two 1024-thread blocks per CU) once there are enough chunks: a block that covers several chunks
// stages its candidates and keeps the next chunk's scores in flight (64 rows of 16 chunks: 34 -> 29 us for the
// top-k).
int chunks_per_block(const Geo& g, int nblk) {
  const int64_t total = (int64_t)nblk * g.R;
  return (int)std::min<int64_t>(nblk, std::max<int64_t>({1, (nblk + 31) / 32, total / 512}));
}

hipError_t launch_topk_select(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                              int32_t* pool_rows, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  const int cpb = chunks_per_block(g, w.nblk);
  dim3 grid((w.nblk + cpb - 1) / cpb, g.R);
  if (cpb > 1)
    topk_filter_staged_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.cnt, w.thr,
                                                         w.seg_cnt, w.seg_off, w.cand, w.nblk, cpb);
  else
    topk_filter_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.cnt, w.thr,
                                                  w.seg_cnt, w.seg_off, w.cand, w.nblk, cpb);
  topk_resolve_kernel<<<g.R, kRes, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.cnt,
                                                w.seg_cnt, w.seg_off, w.cand, w.nblk, topk_idx,
                                                PoolRows{pool_rows, g.row_seq, g.page_table, g.S, g.max_pages,
                                                         g.num_pages, g.log2ps});
  return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                       int32_t* pool_rows, hipStream_t stream) {
  hipError_t e = launch_topk_zero(g, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_topk_select(g, scores, ld, topk_idx, workspace, pool_rows, stream);
}

}  // namespace dsa
