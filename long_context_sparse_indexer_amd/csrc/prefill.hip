// Top-k selection of a chunked prefill without the score matrix (lizeman DSA page, section 4: the indexer pass is
// tiled so that the T x T score matrix is never materialised; kgptalkie "What Does the GPU Actually Run?": the
// head-weighted scores feed a fused partial sort).  Per row r the selection is the k_eff = min(k, n_r) largest
// scores, equal scores lowest position first, written in increasing position order, padded with -1.
//
// The pipeline (rows of one sequence, the tiled fp8 indexer):
//   sample   the tiled indexer scores 4096 sampled positions of each row (128 runs of 32, spread evenly);
//   floor    one block per row ranks its sample: the floor is the 20-bit key prefix of the m-th largest sampled
//            score, m = mu + 8 sqrt(mu) + 16 for mu = k_eff * 4096 / n_r the expected number of sampled scores
//            among the row's k_eff largest, so that the row's k_eff largest scores reach it with near certainty
//            while about k_eff + 8 sqrt(k_eff n / 4096) + 16 n / 4096 scores do (rows of at most kPfCap / 2
//            positions keep every position);
//   filter   the tiled indexer again, whose epilogue keeps each score reaching its row's floor as a candidate
//            (position, order-preserving key), staged in LDS and appended to the row's list: no score is stored;
//   resolve  one block per row: an LDS histogram of the candidates' 20-bit prefixes above the floor finds the
//            prefix of the k_eff-th largest key, its low 12 bits are settled among the keys of that prefix, the
//            selected positions (keys above the threshold key T, and the lowest-position keys equal to T as many as
//            are still needed) are marked in an LDS bitmap over the row's positions, and a scan of the bitmap
//            writes them in position order;
//   fallback a row its sample misjudged (fewer candidates than k_eff, more than kPfCap, a threshold beyond the
//            histogram, more than 1024 keys tied at T) is listed and selected exactly by the fallback kernel,
//            which scores it in full into one row of workspace.
// Workspace: O(R (kPfCap + kPfSample)) plus one row, instead of the R x n score matrix.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "select.h"
#include "topk_common.h"

namespace dsa {
namespace {

constexpr int kPfSmallRow = kPfCap / 2;  // rows this short keep every position as a candidate

__device__ __forceinline__ void list_failed(const PfSel& sel, int r) {
  const uint32_t at = atomicAdd(sel.ctl, 1u);
  sel.fail[at] = r;
}

// One block of 256 threads per row.  Block 0 also clears the fallback state; every block clears its row's
// candidate counter before the filter pass runs.
__global__ __launch_bounds__(256) void pf_floor_kernel(const int32_t* __restrict__ row_len, int max_row_len, int k,
                                                       PfSel sel) {
  constexpr int NT = 256, kPer = kPfSample / NT;
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ __attribute__((aligned(16))) uint32_t h2[256];
  __shared__ uint32_t scan[NT / 64 + 1];
  __shared__ uint32_t s_b1, s_above1, s_b2;
  const int r = blockIdx.x, t = threadIdx.x;
  if (r == 0 && t < 4) sel.ctl[t] = 0u;
  if (t == 0) sel.cnt[r] = 0u;
  const int n = clamp_len(row_len[r], max_row_len), keff = min(k, n);
  const int sv = min(sel.samp_len[r], kPfSample);
  if (keff >= n || n <= kPfSmallRow || sv <= 0) {  // uniform: every position is a candidate
    if (t == 0) sel.floor[r] = 0u;
    return;
  }
  const float mu = (float)keff * (float)sv / (float)n;
  const uint32_t m = (uint32_t)min(sv, (int)ceilf(mu + 8.f * sqrtf(mu) + 16.f));
  uint32_t key[kPer];
  const float* samp = sel.samp + (int64_t)r * kPfSample;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * NT + t;
    key[j] = i < sv ? order_key(samp[i]) : 0u;
  }
  for (int i = t; i < kTopkBins; i += NT) h[i] = 0u;
  h2[t] = 0u;
  if (t == 0) {  // should the ranking fail, a floor of 0 keeps every position (the row then falls back)
    s_b1 = 0u;
    s_above1 = 0u;
    s_b2 = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j * NT + t < sv) atomicAdd(&h[key[j] >> 20], 1u);
  __syncthreads();
  {  // the 12-bit bin of the m-th largest: thread t owns bins (NT - 1 - t) * 16 .. +16, top bins first
    constexpr int kB = kTopkBins / NT;
    uint32_t hv[kB], local = 0;
#pragma unroll
    for (int q = 0; q < kB / 4; ++q) {
      const v4i y = reinterpret_cast<const v4i*>(h)[(NT - 1 - t) * (kB / 4) + q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[4 * q + e] = (uint32_t)y[e];
        local += (uint32_t)y[e];
      }
    }
    uint32_t tot;
    uint32_t above = block_exclusive_scan(local, scan, tot);
    if (above < m && above + local >= m) {
      for (int b = kB - 1; b >= 0; --b) {
        if (above + hv[b] >= m) {
          s_b1 = (uint32_t)((NT - 1 - t) * kB + b);
          s_above1 = above;
          break;
        }
        above += hv[b];
      }
    }
  }
  __syncthreads();
  const uint32_t b1 = s_b1, need = m - s_above1;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j * NT + t < sv && (key[j] >> 20) == b1) atomicAdd(&h2[(key[j] >> 12) & 255u], 1u);
  __syncthreads();
  {  // the next 8 bits: thread t owns bin 255 - t
    const uint32_t local = h2[NT - 1 - t];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(local, scan, tot);
    if (above < need && above + local >= need) s_b2 = (uint32_t)(NT - 1 - t);
  }
  __syncthreads();
  if (t == 0) sel.floor[r] = (b1 << 8) | s_b2;
}

// One block of 1024 threads per row; kBitsLog2: log2 of the longest row the LDS bitmap covers.
template <int kBitsLog2>
__global__ __launch_bounds__(1024) void pf_resolve_kernel(const int32_t* __restrict__ row_len, int max_row_len,
                                                          int k, const int32_t* __restrict__ row_seq,
                                                          const int32_t* __restrict__ page_table, int num_seqs,
                                                          int max_pages, int num_pages, int log2ps, PfSel sel,
                                                          int32_t* __restrict__ topk_idx,
                                                          int32_t* __restrict__ pool_rows) {
  constexpr int kWords = (1 << kBitsLog2) / 32;
  __shared__ __attribute__((aligned(16))) uint32_t bits[kWords];
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ BitmapScratch S;
  const int r = blockIdx.x, t = threadIdx.x;
  const int n = clamp_len(row_len[r], max_row_len), keff = min(k, n);
  int32_t* out = topk_idx + (int64_t)r * k;
  int32_t* rows_out = pool_rows ? pool_rows + (int64_t)r * k : nullptr;
  const ListSink sink{out, rows_out,
                      RowMap{page_table + (int64_t)clamp_seq(row_seq[r], num_seqs) * max_pages, max_pages, num_pages,
                             log2ps}};
  if (keff >= n) {  // the whole row
    for (int i = t; i < k; i += 1024) sink.put_or_pad(i, i < n ? i : -1);
    return;
  }
  static_assert(kPfCap == kCap, "bitmap_select reads a whole list of kCap entries");
  const bool ok = bitmap_select<kWords / 1024>(n, keff, sel.floor[r], sel.cnt[r], sel.cand + (int64_t)r * kPfCap,
                                               sink, bits, h, S);
  if (!ok) {  // uniform
    if (t == 0) list_failed(sel, r);
    return;
  }
  for (int i = keff + t; i < k; i += 1024) sink.put_or_pad(i, -1);
}

}  // namespace

// d_I = 128 keeps the stored scores: its filter pass has LDS for 64 staged candidates per row and block only (two
// blocks per CU beside the doubled query operands), and the overflow's per-candidate atomics made its step slower
// (8.8 ms against 7.0 ms for the 4096-row chunk).
bool prefill_select_supported(const Geo& g) {
  return indexer_tiled(g) && g.d_I == 64 && g.max_row_len <= (1 << 20) && g.k <= 4096;
}

size_t prefill_select_bytes(const Geo& g) {
  const size_t R = (size_t)g.R, ld = ((size_t)std::max(g.max_row_len, 1) + 63) / 64 * 64;
  return align_up(4 * R * kPfSample) + 4 * align_up(4 * R) + align_up(8 * R * kPfCap) + align_up(16) +
         align_up(4 * ld);
}

PfSel prefill_select_carve(const Geo& g, void* workspace) {
  const size_t R = (size_t)g.R;
  char* p = static_cast<char*>(workspace);
  auto take = [&](size_t bytes) { char* q = p; p += align_up(bytes); return q; };
  PfSel s;
  s.samp = reinterpret_cast<float*>(take(4 * R * kPfSample));
  s.samp_len = reinterpret_cast<int32_t*>(take(4 * R));
  s.floor = reinterpret_cast<uint32_t*>(take(4 * R));
  s.cnt = reinterpret_cast<uint32_t*>(take(4 * R));
  s.fail = reinterpret_cast<int32_t*>(take(4 * R));
  s.cand = reinterpret_cast<uint64_t*>(take(8 * R * kPfCap));
  s.ctl = reinterpret_cast<uint32_t*>(take(16));
  s.fbuf = reinterpret_cast<float*>(p);
  return s;
}

hipError_t launch_pf_floor(const Geo& g, const PfSel& sel, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  pf_floor_kernel<<<g.R, 256, 0, stream>>>(g.row_len, g.max_row_len, g.k, sel);
  return hipGetLastError();
}

hipError_t launch_pf_resolve(const Geo& g, const PfSel& sel, int32_t* topk_idx, int32_t* pool_rows,
                             hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  if (g.max_row_len <= (1 << 17))
    pf_resolve_kernel<17><<<g.R, 1024, 0, stream>>>(g.row_len, g.max_row_len, g.k, g.row_seq, g.page_table, g.S,
                                                    g.max_pages, g.num_pages, g.log2ps, sel, topk_idx, pool_rows);
  else
    pf_resolve_kernel<20><<<g.R, 1024, 0, stream>>>(g.row_len, g.max_row_len, g.k, g.row_seq, g.page_table, g.S,
                                                    g.max_pages, g.num_pages, g.log2ps, sel, topk_idx, pool_rows);
  return hipGetLastError();
}

}  // namespace dsa
