// Lightning-indexer scores on gfx950.
//
// Per visible position s of row r:  I[r][s] = sum_j w[r][j] * max(0, <q_I[r][j], k_I[s]>)
// (DeepSeek Sparse Attention explained, "How Does the Lightning Indexer Score a Token?": H_I heads, one
// shared key per position, ReLU, head-weighted sum; head weights carry no sign constraint).
//
// fp8 path.  The per-row contraction [H_I x d_I] x [d_I x n] is a dense GEMM with K = d_I = 64, which is
// exactly the K of v_mfma_f32_32x32x64_f8f6f4.  Heads are the M dimension, positions the N dimension:
// lane l of a wave holds head (l % 32) of the A operand and position (l % 32) of the B operand, each with
// the 32 bytes of K half (l / 32); the 32x32 fp32 result leaves 16 heads of one position in each lane, so
// the ReLU and the head-weighted sum run in-lane and finish with one cross-half exchange.  The fp8 codes
// are OCP e4m3fn (the format gfx950's f8f6f4 MFMA reads with format code 0), products are exact and the 64
// terms accumulate in fp32.  Because the per-vector scales are positive they move outside the ReLU:
// max(0, sq*sk*x) = sq*sk*max(0, x), so the epilogue weight of head j is w[j]*sq[j] and sk multiplies
// the finished sum.
//
// Every key row is read once, as 32-byte pieces: one wave covers 32 consecutive positions = 2 KiB of
// contiguous pool memory (a 32-aligned run never crosses a page of >= 32 positions).
//
// In the fused step the epilogue also starts the top-k selection: each block histograms the first 12 bits
// of its scores' order-preserving keys in LDS and merges the non-empty bins into the row's histogram (see
// topk.hip).  The key loads are issued before the query operands so that both are in flight together.
#include "common.h"
#include "launch.h"
#include "topk_common.h"

namespace dsa {
namespace {

constexpr int kIdxSub = 4;                          // 32-position subtiles per wave
constexpr int kIdxTile = 4 * kIdxSub * 32;          // positions per 256-thread block

template <int HB, bool kHist>  // HB = number of 32-head blocks (H_I = 32 * HB); kHist = fused top-k histogram
__global__ __launch_bounds__(256) void indexer_f8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ head_w,
    const uint8_t* __restrict__ k_pool, const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int max_row_len, float* __restrict__ scores, int64_t ld, int k,
    uint32_t* __restrict__ hist1) {
  constexpr int H_I = 32 * HB;
  __shared__ uint32_t h[kHist ? kTopkBins : 1];
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int64_t tile0 = (int64_t)blockIdx.x * kIdxTile;
  if (tile0 >= n) return;
  const bool do_hist = kHist && k < n;  // uniform over the block; a row with k >= n keeps every position
  if (do_hist) {
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) h[i] = 0u;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int seq = clamp_seq(row_seq[r], num_seqs);

  int64_t prow[kIdxSub];
#pragma unroll
  for (int s = 0; s < kIdxSub; ++s) {
    const int64_t pos = tile0 + (s * 4 + wave) * 32 + col;
    prow[s] = pos < n ? phys_row(page_table, max_pages, num_pages, log2ps, seq, pos) : -1;
  }
  v8i b[kIdxSub];
  float sk[kIdxSub];
#pragma unroll
  for (int s = 0; s < kIdxSub; ++s) {
    if (prow[s] >= 0) {
      b[s] = *reinterpret_cast<const v8i*>(k_pool + prow[s] * 64 + half * 32);
      sk[s] = k_scale[prow[s]];
    } else {
      b[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      sk[s] = 0.f;
    }
  }

  v8i a[HB];
  float wq[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    a[hb] = *reinterpret_cast<const v8i*>(q_idx + ((int64_t)r * H_I + hb * 32 + col) * 64 + half * 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int head = hb * 32 + half * 4 + (i & 3) + 8 * (i >> 2);
      wq[hb][i] = head_w[(int64_t)r * H_I + head] * q_scale[(int64_t)r * H_I + head];
    }
  }

#pragma unroll
  for (int s = 0; s < kIdxSub; ++s) {
    float part = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[hb], b[s], acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) part = fmaf(wq[hb][i], fmaxf(acc[i], 0.f), part);
    }
    part += __shfl_xor(part, 32, 64);
    const int64_t pos = tile0 + (s * 4 + wave) * 32 + col;
    if (half == 0 && pos < n) {
      const float v = sk[s] * part;
      scores[(int64_t)r * ld + pos] = v;
      if (do_hist) atomicAdd(&h[order_key(v) >> 20], 1u);
    }
  }
  if (do_hist) {
    __syncthreads();
    hist_merge<256>(h, hist1 + ((int64_t)r * kHistCopies + blockIdx.x % kHistCopies) * kTopkBins);
  }
}

// fp32 path: one thread per position, queries and weights staged in LDS.
__global__ __launch_bounds__(256) void indexer_f32_kernel(
    const float* __restrict__ q_idx, const float* __restrict__ head_w, const float* __restrict__ k_pool,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table,
    int num_seqs, int max_pages, int num_pages, int log2ps, int max_row_len, int H_I, int d_I,
    float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sm[];  // q [H_I * d_I], w [H_I]
  const int r = blockIdx.y;
  const int n = clamp_len(row_len[r], max_row_len);
  const int64_t pos = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((int64_t)blockIdx.x * blockDim.x >= n) return;  // uniform over the block
  float* q = sm;
  float* w = sm + H_I * d_I;
  for (int i = threadIdx.x; i < H_I * d_I; i += blockDim.x) q[i] = q_idx[(int64_t)r * H_I * d_I + i];
  for (int i = threadIdx.x; i < H_I; i += blockDim.x) w[i] = head_w[(int64_t)r * H_I + i];
  __syncthreads();
  if (pos >= n) return;
  const int64_t p = phys_row(page_table, max_pages, num_pages, log2ps, clamp_seq(row_seq[r], num_seqs), pos);
  const float* kr = k_pool + p * d_I;
  float score = 0.f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.f;
    for (int d = 0; d < d_I; ++d) dot = fmaf(q[j * d_I + d], kr[d], dot);
    score = fmaf(w[j], fmaxf(dot, 0.f), score);
  }
  scores[(int64_t)r * ld + pos] = score;
}

}  // namespace

template <int HB, bool kHist>
void launch_f8(const Geo& g, dim3 grid, const uint8_t* qp, const float* q_idx_scale, const float* head_w,
               const uint8_t* kp, const float* k_idx_scale, float* scores, int64_t ld, const TopkState* fuse,
               hipStream_t stream) {
  indexer_f8_kernel<HB, kHist><<<grid, 256, 0, stream>>>(
      qp, q_idx_scale, head_w, kp, k_idx_scale, g.row_seq, g.row_len, g.page_table, g.S, g.max_pages, g.num_pages,
      g.log2ps, g.max_row_len, scores, ld, g.k, fuse ? fuse->hist1 : nullptr);
}

hipError_t launch_indexer(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                          const void* k_idx_pool, const float* k_idx_scale, float* scores, int64_t ld,
                          const TopkState* fuse, hipStream_t stream) {
  if (g.R == 0 || g.max_row_len == 0) return hipSuccess;
  if (g.idx_dtype == 2 /* F8E4M3 */) {
    dim3 grid((g.max_row_len + kIdxTile - 1) / kIdxTile, g.R);
    auto* qp = static_cast<const uint8_t*>(q_idx);
    auto* kp = static_cast<const uint8_t*>(k_idx_pool);
    if (g.H_I == 64) {
      if (fuse) launch_f8<2, true>(g, grid, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
      else launch_f8<2, false>(g, grid, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
    } else {
      if (fuse) launch_f8<1, true>(g, grid, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
      else launch_f8<1, false>(g, grid, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
    }
  } else {
    dim3 grid((g.max_row_len + 255) / 256, g.R);
    size_t lds = sizeof(float) * (size_t)(g.H_I * g.d_I + g.H_I);
    indexer_f32_kernel<<<grid, 256, lds, stream>>>(static_cast<const float*>(q_idx), head_w,
                                                    static_cast<const float*>(k_idx_pool), g.row_seq, g.row_len,
                                                    g.page_table, g.S, g.max_pages, g.num_pages, g.log2ps,
                                                    g.max_row_len, g.H_I, g.d_I, scores, ld);
  }
  return hipGetLastError();
}

}  // namespace dsa
