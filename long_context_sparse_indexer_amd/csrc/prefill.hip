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
constexpr int kPfMaxTies = 1024;         // keys equal to the threshold key the resolve sorts out itself

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
  constexpr int NT = 1024, NW = NT / 64;
  constexpr int kWords = (1 << kBitsLog2) / 32, kWpt = kWords / NT;  // bitmap words, per thread
  constexpr int kPer = kPfCap / NT;                                   // candidates per thread
  static_assert(kWpt >= 1 && kWpt % 4 == 0 && kPer * NT == kPfCap, "bitmap and list split evenly");
  __shared__ __attribute__((aligned(16))) uint32_t bits[kWords];
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ int32_t eq_pos[kPfMaxTies];
  __shared__ uint32_t low[64];
  __shared__ __attribute__((aligned(16))) uint32_t wt[2 * NW];
  __shared__ uint32_t scan[NW + 1];
  __shared__ uint32_t s_bin, s_above, s_nb, s_nlow, s_neq, s_T, s_need;
  const int r = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int n = clamp_len(row_len[r], max_row_len), keff = min(k, n);
  int32_t* out = topk_idx + (int64_t)r * k;
  int32_t* rows_out = pool_rows ? pool_rows + (int64_t)r * k : nullptr;
  const RowMap map{page_table + (int64_t)clamp_seq(row_seq[r], num_seqs) * max_pages, max_pages, num_pages, log2ps};
  if (keff >= n) {  // the whole row
    for (int i = t; i < k; i += NT) {
      out[i] = i < n ? i : -1;
      if (rows_out) rows_out[i] = i < n ? map.row(i) : -1;
    }
    return;
  }
  const uint32_t c = sel.cnt[r], fl = sel.floor[r];
  if (c < (uint32_t)keff || c > (uint32_t)kPfCap || n > (1 << kBitsLog2)) {  // uniform
    if (t == 0) list_failed(sel, r);
    return;
  }
  uint64_t e[kPer];
  const uint64_t* list = sel.cand + (int64_t)r * kPfCap;
#pragma unroll
  for (int j = 0; j < kPer; ++j) e[j] = list[min(j * NT + t, (int)c - 1)];  // entries past c dropped below
  for (int i = t; i < kTopkBins; i += NT) h[i] = 0u;
#pragma unroll
  for (int q = 0; q < kWpt; ++q) bits[t * kWpt + q] = 0u;
  if (t == 0) {
    s_bin = kTopkBins - 1;
    s_above = 0u;
    s_nb = 0u;
    s_nlow = 0u;
    s_neq = 0u;
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
    uint32_t above = block_scan1<NT>(local, wt, tot);
    if (above < (uint32_t)keff && above + local >= (uint32_t)keff) {
      for (int b = 3; b >= 0; --b) {
        if (above + hv[b] >= (uint32_t)keff) {
          s_bin = (uint32_t)((NT - 1 - t) * 4 + b);
          s_above = above;
          s_nb = hv[b];
          break;
        }
        above += hv[b];
      }
    }
  }
  __syncthreads();
  const uint32_t bin = s_bin, nb = s_nb;
  if (bin == kTopkBins - 1) {  // uniform: the threshold lies in the open-ended top bin
    if (t == 0) list_failed(sel, r);
    return;
  }
  const uint32_t prefix = fl + bin;
  uint32_t need = (uint32_t)keff - s_above;  // keys of the threshold's prefix still to take
  if (nb <= 64u) {
    // the low 12 bits of the keys of that prefix, ranked by one wave
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = (uint32_t)e[j];
      if (j * NT + t < (int)c && (key >> 12) == prefix) low[atomicAdd(&s_nlow, 1u)] = key & 0xfffu;
    }
    __syncthreads();
    if (t < 64) {
      const uint32_t dx = lane < (int)nb ? low[lane] : 0u;
      uint32_t gt = 0, ge = 0;
      for (uint32_t y = 0; y < nb; ++y) {
        const uint32_t dy = low[y];
        gt += dy > dx;
        ge += dy >= dx;
      }
      const uint64_t hit = __ballot(lane < (int)nb && gt < need && need <= ge);
      const int src = __builtin_ctzll(hit);
      if (lane == src) {
        s_T = (prefix << 12) | dx;
        s_need = need - gt;
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
    uint32_t above = block_scan1<NT>(local, wt + NW, tot);
    if (above < need && above + local >= need) {
      for (int b = 3; b >= 0; --b) {
        if (above + hv[b] >= need) {
          s_T = (prefix << 12) | (uint32_t)((NT - 1 - t) * 4 + b);
          s_need = need - above;
          break;
        }
        above += hv[b];
      }
    }
  }
  __syncthreads();
  const uint32_t T = s_T;
  need = s_need;  // keys equal to T to take, lowest positions first
  // mark the keys above T; list the keys equal to T
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (j * NT + t >= (int)c) continue;
    const uint32_t key = (uint32_t)e[j];
    const int32_t pos = (int32_t)(e[j] >> 32);
    if (key > T) {
      atomicOr(&bits[pos >> 5], 1u << (pos & 31));
    } else if (key == T) {
      const uint32_t at = atomicAdd(&s_neq, 1u);
      if (at < (uint32_t)kPfMaxTies) eq_pos[at] = pos;
    }
  }
  __syncthreads();
  const uint32_t neq = s_neq;
  if (neq > (uint32_t)kPfMaxTies) {  // uniform: too many ties to sort out here
    if (t == 0) list_failed(sel, r);
    return;
  }
  if (t < (int)neq) {  // an equal key is taken when fewer than `need` equal keys lie at lower positions
    const int32_t p = eq_pos[t];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < neq; ++j) rank += eq_pos[j] < p;
    if (rank < need) atomicOr(&bits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
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
  uint32_t tot;
  uint32_t slot = block_scan1<NT>(cntw, wt, tot);
#pragma unroll
  for (int q = 0; q < kWpt; ++q) {
    uint32_t b = w[q];
    while (b) {
      const int bit = __builtin_ctz(b);
      b &= b - 1;
      const int32_t pos = (t * kWpt + q) * 32 + bit;
      if (slot < (uint32_t)keff) {
        out[slot] = pos;
        if (rows_out) rows_out[slot] = map.row(pos);
      }
      ++slot;
    }
  }
  for (int i = keff + t; i < k; i += NT) {
    out[i] = -1;
    if (rows_out) rows_out[i] = -1;
  }
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
