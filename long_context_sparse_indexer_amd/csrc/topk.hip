// Top-k selection on gfx950: for each row keep the k_eff = min(k, n) largest scores (DeepSeek Sparse
// Attention explained, "How Does the Selector Pick 1,024?": keep the highest budget-many positions, and a
// row shorter than the budget is read in full).  Equal scores are taken lowest position first; the result
// is written in increasing position order, padded with -1.
//
// Scores become order-preserving 32-bit keys.  Selection is a radix select on those keys in three digits
// (bits 31..20, 19..8, 7..0):
//   hist    grid (chunks, rows): LDS histogram of the first digit of a 4096-score chunk, merged into a
//           per-row global histogram with one atomic per non-empty bin; the last chunk of a row to finish
//           finds the threshold bin b1 (the bin holding the k_eff-th largest key) and the count above it.
//   filter  grid (chunks, rows): every chunk writes the positions whose first digit is >= b1, in position
//           order, into a segment of a per-row candidate list (segment start from a per-row atomic).
//   resolve one 1024-thread block per row: loads the candidates (about k + one bin's worth) into LDS in
//           chunk order, refines the threshold key through the two remaining digits, and writes the
//           selection in position order with wave-ballot/block-scan compaction.  A row whose candidate
//           list overflows the LDS capacity (heavily tied scores) runs the same refinement over the whole
//           score row from global memory instead.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kCh = kTopkChunk;    // scores per chunk
constexpr int kBins = 4096;        // first-digit bins
constexpr int kTpb = 256;          // threads of hist / filter blocks
constexpr int kEpt = kCh / kTpb;   // scores per thread (consecutive)
constexpr int kRes = 1024;         // threads of the resolve block
constexpr int kCap = 12288;        // candidate entries kept per row

struct Ws {
  uint32_t* hist;     // [R, kBins]
  uint32_t* done;     // [R]   chunks finished (hist pass)
  uint32_t* fill;     // [R]   candidate entries reserved (filter pass)
  uint32_t* thr;      // [R, 2] threshold bin, count of keys above it
  uint32_t* seg_cnt;  // [R, nblk]
  uint32_t* seg_off;  // [R, nblk]
  int32_t* cand;      // [R, kCap]
  int nblk;
};

Ws carve(const Geo& g, void* base) {
  Ws w;
  char* p = static_cast<char*>(base);
  w.nblk = (g.max_row_len + kCh - 1) / kCh;
  if (w.nblk < 1) w.nblk = 1;
  auto take = [&](size_t bytes) { char* q = p; p += align_up(bytes); return q; };
  w.hist = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * kBins));
  w.done = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R));
  w.fill = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R));
  w.thr = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2 * (size_t)g.R));
  w.seg_cnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.seg_off = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)g.R * w.nblk));
  w.cand = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)g.R * kCap));
  return w;
}

__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* __restrict__ hist, uint32_t* __restrict__ done,
                                                        uint32_t* __restrict__ fill) {
  const int r = blockIdx.x;
  v4i z = {0, 0, 0, 0};
  v4i* h = reinterpret_cast<v4i*>(hist + (int64_t)r * kBins);
  for (int i = threadIdx.x; i < kBins / 4; i += blockDim.x) h[i] = z;
  if (threadIdx.x == 0) { done[r] = 0u; fill[r] = 0u; }
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

__global__ __launch_bounds__(kTpb) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ row_len, int max_row_len, int k,
                                                         uint32_t* __restrict__ hist, uint32_t* __restrict__ done,
                                                         uint32_t* __restrict__ thr) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scan[kTpb / 64 + 1];
  __shared__ int is_last;
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nblk = (n + kCh - 1) / kCh;
  if (keff >= n || (int)blockIdx.x >= nblk) return;  // nothing to choose, or a chunk past the row's end

  for (int i = threadIdx.x; i < kBins; i += kTpb) h[i] = 0u;
  __syncthreads();
  const float* row = scores + (int64_t)r * ld;
  uint32_t key[kEpt];
  bool valid[kEpt];
  load_keys(row, (int64_t)blockIdx.x * kCh + threadIdx.x * kEpt, n, key, valid);
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if (valid[e]) atomicAdd(&h[key[e] >> 20], 1u);
  __syncthreads();
  uint32_t* gh = hist + (int64_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kTpb)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(&done[r], 1u) == (uint32_t)(nblk - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // Thread t owns the 16 bins of group (255 - t), so thread 0 holds the highest keys.
  const int grp = kTpb - 1 - threadIdx.x;
  uint32_t c[kBins / kTpb];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kBins / kTpb; ++j) {
    c[j] = __hip_atomic_load(&gh[grp * (kBins / kTpb) + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    local += c[j];
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan(local, scan, total);  // keys in groups above this one
  if (above < (uint32_t)keff && above + local >= (uint32_t)keff) {
    for (int j = kBins / kTpb - 1; j >= 0; --j) {
      if (above + c[j] >= (uint32_t)keff) {
        thr[2 * r] = (uint32_t)(grp * (kBins / kTpb) + j);
        thr[2 * r + 1] = above;
        break;
      }
      above += c[j];
    }
  }
}

__global__ __launch_bounds__(kTpb) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ row_len, int max_row_len,
                                                           int k, const uint32_t* __restrict__ thr,
                                                           uint32_t* __restrict__ fill, uint32_t* __restrict__ seg_cnt,
                                                           uint32_t* __restrict__ seg_off, int32_t* __restrict__ cand,
                                                           int nblk_max) {
  __shared__ uint32_t scan[kTpb / 64 + 1];
  __shared__ uint32_t seg_base;
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  const int nblk = (n + kCh - 1) / kCh;
  if (keff >= n || (int)blockIdx.x >= nblk) return;
  const uint32_t b1 = thr[2 * r];
  const int64_t first = (int64_t)blockIdx.x * kCh + threadIdx.x * kEpt;
  uint32_t key[kEpt];
  bool valid[kEpt];
  load_keys(scores + (int64_t)r * ld, first, n, key, valid);
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < kEpt; ++e) cnt += (valid[e] && (key[e] >> 20) >= b1) ? 1u : 0u;
  uint32_t total;
  uint32_t off = block_exclusive_scan(cnt, scan, total);
  if (threadIdx.x == 0) {
    seg_base = atomicAdd(&fill[r], total);
    seg_cnt[(int64_t)r * nblk_max + blockIdx.x] = total;
    seg_off[(int64_t)r * nblk_max + blockIdx.x] = seg_base;
  }
  __syncthreads();
  if (seg_base + total > (uint32_t)kCap) return;  // overflow: the resolve pass rescans the row
  int32_t* out = cand + (int64_t)r * kCap + seg_base + off;
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if (valid[e] && (key[e] >> 20) >= b1) *out++ = (int32_t)(first + e);
}

// Candidate access for the resolve block: entries of the LDS list, or every position of the row.
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

// Among entries whose key agrees with `prefix` above bit `lo + bits`, find the digit (key >> lo) & mask
// holding the need-th largest key; returns it and lowers `need` by the count of entries above it.
template <class List>
__device__ uint32_t refine_digit(const List& L, int len, uint32_t prefix, int lo, int bits, uint32_t& need,
                                 uint32_t* h, uint32_t* scan) {
  const int nb = 1 << bits;
  const uint32_t mask = (uint32_t)nb - 1u;
  for (int i = threadIdx.x; i < nb; i += kRes) h[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < len; i += kRes) {
    const uint32_t key = L.k(i);
    if ((key >> (lo + bits)) == prefix) atomicAdd(&h[(key >> lo) & mask], 1u);
  }
  __syncthreads();
  // thread t owns bins [(kRes-1-t)*per, +per) so the scan runs from the top bin down
  const int per = (nb + kRes - 1) / kRes;
  const int grp = kRes - 1 - threadIdx.x;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) {
    const int b = grp * per + j;
    if (b < nb) local += h[b];
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan(local, scan, total);
  __shared__ uint32_t found_digit, found_above;
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

template <class List>
__device__ void select_ordered(const List& L, int len, uint32_t b1, uint32_t above1, int keff, int32_t* out,
                               uint32_t* h, uint32_t* scan) {
  uint32_t need = (uint32_t)keff - above1;  // >= 1 entries of bin b1 still to take
  const uint32_t d2 = refine_digit(L, len, b1, 8, 12, need, h, scan);
  const uint32_t d3 = refine_digit(L, len, (b1 << 12) | d2, 0, 8, need, h, scan);
  const uint32_t T = (b1 << 20) | (d2 << 8) | d3;  // the k_eff-th largest key; `need` of its ties are taken
  uint32_t taken = 0, eq_seen = 0;
  for (int base = 0; base < len; base += kRes) {
    const int i = base + threadIdx.x;
    const uint32_t key = i < len ? L.k(i) : 0u;
    const uint32_t is_eq = (i < len && key == T) ? 1u : 0u;
    uint32_t eq_total;
    const uint32_t eq_rank = eq_seen + block_exclusive_scan(is_eq, scan, eq_total);
    const uint32_t sel = (i < len && (key > T || (is_eq && eq_rank < need))) ? 1u : 0u;
    uint32_t sel_total;
    const uint32_t slot = taken + block_exclusive_scan(sel, scan, sel_total);
    if (sel && slot < (uint32_t)keff) out[slot] = L.p(i);
    taken += sel_total;
    eq_seen += eq_total;
  }
}

__global__ __launch_bounds__(kRes) void topk_resolve_kernel(const float* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ row_len, int max_row_len,
                                                            int k, const uint32_t* __restrict__ thr,
                                                            const uint32_t* __restrict__ fill,
                                                            const uint32_t* __restrict__ seg_cnt,
                                                            const uint32_t* __restrict__ seg_off,
                                                            const int32_t* __restrict__ cand, int nblk_max,
                                                            int32_t* __restrict__ topk_idx) {
  __shared__ uint32_t lkey[kCap];
  __shared__ int32_t lpos[kCap];
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t seg_start[kTopkMaxBlocksPerRow + 1];
  __shared__ uint32_t seg_src[kTopkMaxBlocksPerRow];
  __shared__ uint32_t scan[kRes / 64 + 1];
  const int r = blockIdx.x;
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  int32_t* out = topk_idx + (int64_t)r * k;
  const float* row = scores + (int64_t)r * ld;
  if (keff >= n) {
    for (int i = threadIdx.x; i < k; i += kRes) out[i] = i < n ? i : -1;
    return;
  }
  const uint32_t b1 = thr[2 * r], above1 = thr[2 * r + 1];
  const uint32_t len = fill[r];
  if (len <= (uint32_t)kCap) {
    const int nblk = (n + kCh - 1) / kCh;
    // segment starts in chunk (= position) order
    uint32_t c = 0;
    if ((int)threadIdx.x < nblk) {
      c = seg_cnt[(int64_t)r * nblk_max + threadIdx.x];
      seg_src[threadIdx.x] = seg_off[(int64_t)r * nblk_max + threadIdx.x];
    }
    uint32_t total;
    const uint32_t start = block_exclusive_scan(c, scan, total);
    if ((int)threadIdx.x < nblk) seg_start[threadIdx.x] = start;
    if (threadIdx.x == 0) seg_start[nblk] = total;
    __syncthreads();
    for (int i = threadIdx.x; i < (int)len; i += kRes) {
      int lo = 0, hi = nblk - 1;  // last segment whose start <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg_start[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
      }
      const int32_t p = cand[(int64_t)r * kCap + seg_src[lo] + (i - seg_start[lo])];
      lpos[i] = p;
      lkey[i] = order_key(row[p]);
    }
    __syncthreads();
    select_ordered(LdsList{lkey, lpos}, (int)len, b1, above1, keff, out, h, scan);
  } else {
    select_ordered(RowList{row}, n, b1, above1, keff, out, h, scan);
  }
  for (int i = keff + threadIdx.x; i < k; i += kRes) out[i] = -1;
}

}  // namespace

size_t topk_workspace_bytes(const Geo& g) {
  const size_t nblk = (size_t)std::max(1, (g.max_row_len + kCh - 1) / kCh);
  const size_t R = (size_t)g.R;
  return align_up(4 * R * kBins) + 2 * align_up(4 * R) + align_up(8 * R) + 2 * align_up(4 * R * nblk) +
         align_up(4 * R * kCap);
}

hipError_t launch_topk(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                       hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  Ws w = carve(g, workspace);
  topk_zero_kernel<<<g.R, 256, 0, stream>>>(w.hist, w.done, w.fill);
  dim3 grid(w.nblk, g.R);
  topk_hist_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.hist, w.done, w.thr);
  topk_filter_kernel<<<grid, kTpb, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.fill,
                                                w.seg_cnt, w.seg_off, w.cand, w.nblk);
  topk_resolve_kernel<<<g.R, kRes, 0, stream>>>(scores, ld, g.row_len, g.max_row_len, g.k, w.thr, w.fill,
                                                w.seg_cnt, w.seg_off, w.cand, w.nblk, topk_idx);
  return hipGetLastError();
}

}  // namespace dsa
