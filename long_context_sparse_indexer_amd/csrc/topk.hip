// Top-k selection on gfx950: for each row keep the k_eff = min(k, n) largest scores (DeepSeek Sparse
// Attention explained, "How Does the Selector Pick 1,024?": keep the highest budget-many positions, and a
// row shorter than the budget is read in full).  Equal scores are taken lowest position first; the result
// is written in increasing position order, padded with -1.
//
// Scores become order-preserving 32-bit keys.  Hand-overs between blocks happen at kernel boundaries, except that
// a single row of at most 2^17 positions is resolved by its last filter block (one acquire-release counter):
//   filter   grid (4096-score chunks, rows): every block first finds the row's floor, the 20-bit key prefix of a
//            sampled score that comfortably more than k_eff scores of the row exceed.  The sample is a fixed set
//            of evenly spaced runs of the row, the same in every block, ranked through an LDS histogram (in the
//            fused step the indexer has already ranked the floor of most decode rows from the keys).  The
//            block then writes the keys whose first 20 bits reach the floor, in position order, into a segment of
//            the row's candidate list.
//   resolve  one 1024-thread block per row runs the resolve step of select.h and writes the list (and, in the
//            fused step, the pool row of every selected slot for the attention).
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "select.h"
#include "topk_common.h"

DSA_TIMELINE_UNIT(topk)

namespace dsa {
namespace {

constexpr int kTpb = 1024;         // threads of filter blocks
constexpr int kEpt = kCh / kTpb;   // scores per thread (consecutive)

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

constexpr int kRes = 1024;  // threads of the resolve block

// Where the fused step wants the pool row of every selected slot ([R, k] int32, -1 for padding); `out` NULL
// when no pool rows are wanted.
struct PoolRows {
  int32_t* out;
  const int32_t* row_seq;
  const int32_t* page_table;
  int num_seqs, max_pages, num_pages, log2ps;
};

// LDS of a bitmap resolve over rows of at most 2^kBitsLog2 positions.
template <int kBitsLog2>
struct BitmapLds {
  static constexpr int kWords = (1 << kBitsLog2) / 32;
  static constexpr bool kStagePages = kBitsLog2 <= 17;
  alignas(16) uint32_t bits[kWords];
  alignas(16) int32_t pt[kStagePages ? kResPages : 1];
};

// The selection of row r (1024 threads): a row no longer than its budget is written whole; otherwise select.h's
// bitmap_select settles it from the candidate list (`count` candidates above the floor fl), and a row the list
// cannot settle (the sample overshot, the list overflowed, heavy ties) is selected over its stored scores.  The
// list is written in increasing position order, padded with -1, with the pool row of each slot when asked; the
// page ids of the row's sequence are staged in LDS when they fit.  h: kTopkBins words of LDS.
template <int kBitsLog2>
__device__ __forceinline__ void bitmap_resolve_row(const float* __restrict__ scores, int64_t ld, int r, int n, int k,
                                                   uint32_t fl, uint32_t count, const uint64_t* __restrict__ cand,
                                                   int32_t* __restrict__ topk_idx, const PoolRows& pr,
                                                   BitmapLds<kBitsLog2>& L, uint32_t* h, BitmapScratch& S) {
  const int t = threadIdx.x, keff = min(k, n);
  const int32_t* gpt = pr.out ? pr.page_table + (int64_t)clamp_seq(pr.row_seq[r], pr.num_seqs) * pr.max_pages : nullptr;
  const bool pt_lds = BitmapLds<kBitsLog2>::kStagePages && pr.out && pr.max_pages <= kResPages;
  int32_t* const out = topk_idx + (int64_t)r * k;
  int32_t* const rows_out = pr.out ? pr.out + (int64_t)r * k : nullptr;
  const ListSink gsink{out, rows_out, RowMap{gpt, pr.max_pages, pr.num_pages, pr.log2ps}};
  if (keff >= n) {
    for (int i = t; i < k; i += kRes) gsink.put_or_pad(i, i < n ? i : -1);
    return;
  }
  DSA_STAMP(1, 3);
  auto finish = [&](const auto& sink, auto pre) __attribute__((always_inline)) {
    if (!bitmap_select<BitmapLds<kBitsLog2>::kWords / kRes>(n, keff, fl, count, cand + (int64_t)r * kCap, sink,
                                                             L.bits, h, S, pre)) {
      __syncthreads();
      select_and_write<kRes>(RowList{scores + (int64_t)r * ld}, n, (uint32_t)keff, keff, gsink, h, S.wt);
    }
    DSA_STAMP(1, 4);
    for (int i = keff + t; i < k; i += kRes) gsink.put_or_pad(i, -1);
  };
  if (pt_lds)  // the page ids are staged while the candidates load (visible after bitmap_select's first barrier)
    finish(LdsListSink{out, rows_out, LdsRowMap{lds_ptr(L.pt), pr.max_pages, pr.num_pages, pr.log2ps}},
           [&]() { stage_page_row<kRes>(L.pt, gpt, pr.max_pages); });
  else
    finish(gsink, NoPre{});
  DSA_STAMP(1, 5);
}

// The filter blocks of a row that participate (cpb chunks each), and the hand-over to the last of them: every
// thread waits for its candidate stores, then one acquire-release atomic per block (device scope) counts the
// block in, so that one write-back of the cache per block publishes the block's stores; the block that completes
// the count has acquired the others' and resolves the row in place of a resolve launch.  (A device-scope fence
// in every thread made the hand-over cost more than the launch it saves.)
__device__ __forceinline__ bool last_filter_block(uint32_t* cnt_done, int parts, uint32_t* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(cnt_done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(parts - 1);
  __syncthreads();
  return *flag != 0u;
}
__device__ __forceinline__ uint32_t load_count(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// A sampled row of n scores is sampled about n / kSampleDiv times (n / 64 measured slower: 1.7 us more per
// 128K-position decode step, 8% more for a 4096-row prefill chunk, from the extra candidates).
constexpr int kSampleDiv = 32;

// The row's floor: the first 20 bits of the m-th largest score of a sample of the row, ranked in two rounds of an
// LDS histogram: bits 31..20 of every sampled key (4096 bins in h), then bits 19..12 of those in the bin found
// (256 bins in h2), each ranked by one wave.  The sample is S scores in S/16 runs of sixteen consecutive scores
// spread evenly over the row (four lanes read a run, so a load instruction touches 16 cache lines, not 64), with S
// the power of two in (b / 2, b] for b = (n / kSampleDiv) * max(1, k_eff / 2048), kept within [1024, 16384] (up to
// 65536 for rows past 2^21) and at most n / 8: it reads a small part of the row and is the same in every block.
// With mu = k_eff S/n the expected number of sampled scores among the row's k_eff largest, m = mu + 8 sqrt(mu) + 16
// puts the floor far enough below the k_eff-th largest score that a row rarely has fewer than k_eff scores at or
// above it, while about n m / S = k_eff + 8 sqrt(k_eff n / S) + 16 n / S scores reach it (the sample grows with the
// budget so that this stays within the candidate list up to k_eff of about 10K).  A row of at most one chunk is its
// own sample, with m = k_eff: its floor is exactly the 20-bit prefix of the k_eff-th largest score.
// h, h2: kTopkBins and 256 words of LDS, 16-byte aligned; s: 4 words of LDS.  Called by all NT threads; ends with
// a barrier.
template <int NT>
__device__ __forceinline__ uint32_t floor_prefix(const float* __restrict__ row, int n, int keff, uint32_t* h,
                                                 uint32_t* h2, uint32_t* s) {
  constexpr int kGroup = 4;  // 16-byte pieces per thread held in registers: all of them up to S = 16384
  // piece j (16 bytes) lies at `start(j)`: in a short row the row itself, piece after piece; in a sampled row the
  // j % 4-th quarter of run j / 4, which starts at a multiple of 4 below n - 16 (step >= 128), so every load lies
  // inside the row's stride (a multiple of 4 at least n)
  int runs, m, step = 0;  // runs = 16-byte pieces of the sample; step = distance between sampled runs
  if (n <= kCh) {
    runs = (n + 3) / 4;
    m = keff;
  } else {
    const int cap = min(n > (1 << 21) ? 65536 : 16384, n / 8);
    const int b = (n / kSampleDiv) * max(1, keff / 2048);
    const int S = min(cap, max(1024, 1 << (31 - __builtin_clz((unsigned)b))));
    runs = S / 4;
    step = n / (S / 16);
    const float mu = (float)keff * (float)S / (float)n;
    m = min(S, (int)ceilf(mu + 8.f * sqrtf(mu) + 16.f));
  }
  auto start = [&](int j) { return step ? (((j >> 2) * step) & ~3) + (j & 3) * 4 : 4 * j; };
  const int ngroups = (runs + kGroup * NT - 1) / (kGroup * NT);
  v4f x[kGroup];
  auto load = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int j = threadIdx.x + (g * kGroup + q) * NT;
      if (j < runs) x[q] = *reinterpret_cast<const v4f*>(row + start(j));
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
  DSA_STAMP(1, 6);
  round(h, 20, 12, 0u, false);
  __syncthreads();
  DSA_STAMP(1, 7);
  if (threadIdx.x < 64) wave_threshold_bin<kTopkBins>(h, (uint32_t)m, &s[0], &s[1]);
  __syncthreads();
  DSA_STAMP(1, 8);
  const uint32_t b1 = s[0];
  round(h2, 12, 8, b1, ngroups > 1);
  __syncthreads();
  DSA_STAMP(1, 9);
  if (threadIdx.x < 64) wave_threshold_bin<256>(h2, (uint32_t)m - s[1], &s[2], &s[3]);
  __syncthreads();
  return (b1 << 8) | s[2];
}

// kFuse: rows of at most 2^17 positions are resolved by their last filter block (bitmap_resolve_row), and a row
// no longer than its budget is written whole by block 0.
template <bool kFuse>
__global__ __launch_bounds__(kTpb) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ row_len, int max_row_len,
                                                           int k, uint32_t* __restrict__ cnt,
                                                           uint32_t* __restrict__ thr,
                                                           uint32_t* __restrict__ seg_cnt,
                                                           uint32_t* __restrict__ seg_off, uint64_t* __restrict__ cand,
                                                           int nblk_max, int cpb, int32_t* __restrict__ topk_idx,
                                                           PoolRows pr, const uint32_t* __restrict__ pre_floor) {
  __shared__ __attribute__((aligned(16))) uint32_t scan[kTpb / 64 + 1];
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ __attribute__((aligned(16))) uint32_t h2[256];
  __shared__ uint32_t seg_base, s_f[4], s_last;
  __shared__ BitmapLds<kFuse ? 17 : 5> bl;  // used when kFuse
  __shared__ BitmapScratch bs[1];  // used when kFuse
  args_to_sgprs(scores, ld, row_len, max_row_len, k, cnt, thr, seg_cnt, seg_off, cand, nblk_max, cpb);
  DSA_STAMP(1, 0);
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if constexpr (kFuse) {
    if (keff >= n) {  // the whole row, by one block
      if (blockIdx.x == 0) bitmap_resolve_row<17>(scores, ld, r, n, k, 0u, 0u, cand, topk_idx, pr, bl, h, bs[0]);
      return;
    }
  }
  if (keff >= n || c0 >= nchunk) return;
  const float* row = scores + (int64_t)r * ld;
  v4f xa = load_raw(row, c0, n), xb;  // the first chunk loads together with the sample (or the indexer's floor)
  // every block ranks the sample itself instead of waiting for one block to publish the floor, unless the fused
  // indexer ranked it
  const uint32_t fl = pre_floor && indexer_floor_row(n, keff) ? pre_floor[4 * r]
                                                              : floor_prefix<kTpb>(row, n, keff, h, h2, s_f);
  DSA_STAMP(1, 1);
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
  DSA_STAMP(1, 2);
  if constexpr (kFuse) {
    if (last_filter_block(&cnt[4 * r + 3], (nchunk + cpb - 1) / cpb, &s_last))
      bitmap_resolve_row<17>(scores, ld, r, n, k, fl, load_count(&cnt[4 * r + 2]), cand, topk_idx, pr, bl, h, bs[0]);
  }
}

// Filter for blocks that cover several chunks (long rows, large batches).  The chunk loop stages each chunk's
// candidates in LDS (position order within the chunk, chunks in order), so its only memory traffic is the next
// chunk's scores, loaded while the current one is filtered.  When the stage is full, and at the end, the block
// reserves one range of the row's candidate list with one atomic, copies the stage out and writes the segment
// table of the chunks it holds.
constexpr int kStageCap = 6144;  // staged candidates per block (48 KiB; two 1024-thread blocks fit a CU)
static_assert(kCh <= kStageCap, "one chunk always fits an empty stage");

// kFuse as for topk_filter_kernel; the resolve's bitmap and page ids take the stage's LDS once it is flushed.
template <bool kFuse>
__global__ __launch_bounds__(kTpb) void topk_filter_staged_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int max_row_len, int k,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ thr,
    uint32_t* __restrict__ seg_cnt, uint32_t* __restrict__ seg_off, uint64_t* __restrict__ cand, int nblk_max,
    int cpb, int32_t* __restrict__ topk_idx, PoolRows pr, const uint32_t* __restrict__ pre_floor) {
  static_assert(sizeof(BitmapLds<17>) <= kStageCap * sizeof(uint64_t), "the resolve's LDS fits the stage");
  __shared__ __attribute__((aligned(16))) uint32_t scan[kTpb / 64 + 1];
  __shared__ __attribute__((aligned(16))) uint64_t stage[kStageCap];
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];  // the sample's histograms
  __shared__ __attribute__((aligned(16))) uint32_t h2[256];
  __shared__ uint32_t chunk_n[kTopkMaxBlocksPerRow];  // candidates of each staged chunk
  __shared__ uint32_t seg_base, s_f[4], s_last;
  __shared__ BitmapScratch bs[1];  // used when kFuse
  args_to_sgprs(scores, ld, row_len, max_row_len, k, cnt, thr, seg_cnt, seg_off, cand, nblk_max, cpb);
  auto& bl = *reinterpret_cast<BitmapLds<17>*>(stage);
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nchunk = (n + kCh - 1) / kCh;
  const int c0 = (int)blockIdx.x * cpb;
  if constexpr (kFuse) {
    if (keff >= n) {  // the whole row, by one block
      if (blockIdx.x == 0) bitmap_resolve_row<17>(scores, ld, r, n, k, 0u, 0u, cand, topk_idx, pr, bl, h, bs[0]);
      return;
    }
  }
  if (keff >= n || c0 >= nchunk) return;
  const float* row = scores + (int64_t)r * ld;
  v4f x = load_raw(row, c0, n);  // the first chunk loads together with the sample (or the indexer's floor)
  const uint32_t fl = pre_floor && indexer_floor_row(n, keff) ? pre_floor[4 * r]
                                                              : floor_prefix<kTpb>(row, n, keff, h, h2, s_f);
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
  if constexpr (kFuse) {
    if (last_filter_block(&cnt[4 * r + 3], (nchunk + cpb - 1) / cpb, &s_last))  // its barriers end the flush
      bitmap_resolve_row<17>(scores, ld, r, n, k, fl, load_count(&cnt[4 * r + 2]), cand, topk_idx, pr, bl, h, bs[0]);
  }
}


// One block per row: the selection of the row (select.h), written as the list of selected positions in increasing
// position order, padded with -1, and, when asked, the pool row of each.
__global__ __launch_bounds__(kRes) void topk_resolve_kernel(const float* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ row_len, int max_row_len,
                                                            int k, const uint32_t* __restrict__ thr,
                                                            const uint32_t* __restrict__ cnt,
                                                            const uint32_t* __restrict__ seg_cnt,
                                                            const uint32_t* __restrict__ seg_off,
                                                            const uint64_t* __restrict__ cand, int nblk_max,
                                                            int32_t* __restrict__ topk_idx, PoolRows pr) {
  __shared__ ResolveLds S;
  args_to_sgprs(scores, ld, row_len, max_row_len, k, thr, cnt, seg_cnt, seg_off, cand, nblk_max, topk_idx, pr.out,
                pr.row_seq, pr.page_table, pr.num_seqs, pr.max_pages, pr.num_pages, pr.log2ps);
  DSA_STAMP(2, 0);
  const int r = blockIdx.x;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  int32_t* out = topk_idx + (int64_t)r * k;
  // pool rows of the selection (fused step): the sequence's page ids, staged in LDS when they fit
  const int32_t* gpt = pr.out ? pr.page_table + (int64_t)clamp_seq(pr.row_seq[r], pr.num_seqs) * pr.max_pages : nullptr;
  const bool pt_lds = pr.out && pr.max_pages <= kResPages;
  const ListSink sink{out, pr.out ? pr.out + (int64_t)r * k : nullptr,
                      RowMap{pt_lds ? S.pt : gpt, pr.max_pages, pr.num_pages, pr.log2ps}};
  if (keff >= n) {
    const RowMap gmap{gpt, pr.max_pages, pr.num_pages, pr.log2ps};
    for (int i = threadIdx.x; i < k; i += kRes) {
      out[i] = i < n ? i : -1;
      if (sink.rows_out) sink.rows_out[i] = i < n ? gmap.row(i) : -1;
    }
    return;
  }
  if (pt_lds) stage_page_row<kRes>(S.pt, gpt, pr.max_pages);  // used after the resolve's first barrier
  const RowCands rc{thr + 4 * r, cnt + 4 * r, seg_cnt + (int64_t)r * nblk_max, seg_off + (int64_t)r * nblk_max,
                    cand + (int64_t)r * kCap};
  ResolveLoads<kRes> rl;
  resolve_issue<kRes>(rc, nblk_max, rl);
  resolve_finish<kRes, ListSink, NoStage, 2>(scores + (int64_t)r * ld, n, keff, rc, rl, S, sink, NoStage{});
  for (int i = keff + threadIdx.x; i < k; i += kRes) {
    out[i] = -1;
    if (sink.rows_out) sink.rows_out[i] = -1;
  }
  DSA_STAMP(2, 5);
}

// One block per row: the selection of select.h's bitmap_select from the filter's candidate list, written in
// increasing position order, padded with -1, with the pool row of each slot when asked.  A row the list cannot
// settle (the sample overshot, the list overflowed, heavy ties) is selected over its stored scores instead.  The
// page ids of the row's sequence are staged in LDS when the bitmap leaves room (rows up to 2^17 positions).
template <int kBitsLog2>
__global__ __launch_bounds__(kRes) void topk_bitmap_resolve_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ row_len,
                                                                   int max_row_len, int k,
                                                                   const uint32_t* __restrict__ thr,
                                                                   const uint32_t* __restrict__ cnt,
                                                                   const uint64_t* __restrict__ cand,
                                                                   int32_t* __restrict__ topk_idx, PoolRows pr) {
  static_assert(kRes == 1024, "bitmap_select runs on 1024 threads");
  __shared__ BitmapLds<kBitsLog2> bl;
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ BitmapScratch S;
  args_to_sgprs(scores, ld, row_len, max_row_len, k, thr, cnt, cand, topk_idx, pr.out, pr.row_seq, pr.page_table,
                pr.num_seqs, pr.max_pages, pr.num_pages, pr.log2ps);
  const int r = blockIdx.x;
  const int n = clamp_len(row_len[r], max_row_len);
  bitmap_resolve_row<kBitsLog2>(scores, ld, r, n, k, thr[4 * r], cnt[4 * r + 2], cand, topk_idx, pr, bl, h, S);
}

}  // namespace

size_t topk_workspace_bytes(const Geo& g) {
  const size_t nblk = (size_t)std::max(1, (g.max_row_len + kCh - 1) / kCh);
  const size_t R = (size_t)g.R;
  return 2 * align_up(16 * R) + 2 * align_up(4 * R * nblk) + align_up(8 * R * kCap);
}

TopkState topk_state(const Geo& g, void* workspace) {
  const Ws w = carve(g, workspace);
  return TopkState{w.cnt, w.thr, g.k};
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
                              int32_t* pool_rows, bool indexer_floors, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const Ws w = carve(g, workspace);
  const int cpb = chunks_per_block(g, w.nblk);
  dim3 grid((w.nblk + cpb - 1) / cpb, g.R);
  const PoolRows pr{pool_rows, g.row_seq, g.page_table, g.S, g.max_pages, g.num_pages, g.log2ps};
  // a single row of at most 2^17 positions: the last filter block resolves it (one launch fewer).  With many rows
  // the resolves, a few microseconds each, would hold filter blocks' CUs while other rows' filter blocks wait
  // (64 rows of the batched decode: 20 -> 41 us), so they take a launch of their own.
  const bool fuse = g.R == 1 && g.max_row_len <= (1 << 17);
#define DSA_FILTER(KERN, F)                                                                                     \
  KERN<F><<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.cnt, w.thr, w.seg_cnt, w.seg_off, \
                                     w.cand, w.nblk, cpb, topk_idx, pr, indexer_floors ? w.thr + 1 : nullptr)
  if (cpb > 1) {
    if (fuse) DSA_FILTER(topk_filter_staged_kernel, true); else DSA_FILTER(topk_filter_staged_kernel, false);
  } else {
    if (fuse) DSA_FILTER(topk_filter_kernel, true); else DSA_FILTER(topk_filter_kernel, false);
  }
#undef DSA_FILTER
  if (fuse) return hipGetLastError();
  // the bitmap resolve up to 2^17 positions; past that the segment resolve (at 2^20 the bitmap's 32 words per thread
  // made the 8-row decode's top-k 28.6 -> 35.6 us)
  if (g.max_row_len <= (1 << 17))
    topk_bitmap_resolve_kernel<17><<<g.R, kRes, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.cnt,
                                                             w.cand, topk_idx, pr);
  else
    topk_resolve_kernel<<<g.R, kRes, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.cnt,
                                                  w.seg_cnt, w.seg_off, w.cand, w.nblk, topk_idx, pr);
  return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                       int32_t* pool_rows, hipStream_t stream) {
  hipError_t e = launch_topk_zero(g, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_topk_select(g, scores, ld, topk_idx, workspace, pool_rows, false, stream);
}

}  // namespace dsa
