// Internal interface between the C-ABI entry points (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// A validated problem with its device metadata.
struct Geo {
  int R, S, H_I, d_I, H, d_c, k;
  int page_size, log2ps, max_pages, num_pages, max_row_len, rows_per_seq;
  int idx_dtype, kv_dtype;
  float softmax_scale;
  const int32_t* row_seq;
  const int32_t* row_len;
  const int32_t* page_table;
};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Per-row top-k state that must start at zero: the candidate counters.  In the fused step the indexer clears
// them (block 0 of each row, after its scores), sparing the top-k a zeroing launch.
struct TopkState {
  uint32_t* cnt;  // [R, 4]
};

// indexer.hip.  fp8 problems whose rows come in groups of at least kTiledMinRows per sequence (chunked prefill)
// run the tiled GEMM kernel, which takes no `fuse`.  Otherwise, with `fuse` non-NULL the indexer also clears the
// top-k state.
constexpr int kTiledMinRows = 8;
bool indexer_tiled(const Geo& g);
hipError_t launch_indexer(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                          const void* k_idx_pool, const float* k_idx_scale, float* scores, int64_t ld,
                          const TopkState* fuse, hipStream_t stream);

// topk.hip
constexpr int kTopkMaxBlocksPerRow = 1024;
constexpr int kTopkChunk = 4096;
size_t topk_workspace_bytes(const Geo& g);
TopkState topk_state(const Geo& g, void* workspace);
hipError_t launch_topk_zero(const Geo& g, void* workspace, hipStream_t stream);
// Selection over stored scores whose top-k state is already zero (launch_topk_zero, or the fused indexer).
// pool_rows: if non-NULL, [R, k] int32 receiving the pool row of every selected slot (-1 for padding), for the
// attention.
hipError_t launch_topk_select(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                              int32_t* pool_rows, hipStream_t stream);
hipError_t launch_topk(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                       int32_t* pool_rows, hipStream_t stream);

// attn.hip
size_t attn_workspace_bytes(const Geo& g);
// pool_rows: if non-NULL, the pool row of every selected slot (as written by the top-k), used instead of
// looking the positions up in the page table (bf16 latents).  topk_idx and pool_rows both NULL: dense
// attention, slot s of row r is position s while s < n_r (g.k = the longest row).
// append.hip.  w NULL: src holds fp32 keys [R, d_I]; otherwise latent rows [R, d_c] and W_KI [d_c, d_I] in
// g.kv_dtype.  The pool is fp8 codes + scales (g.idx_dtype F8E4M3) or fp32.
hipError_t launch_key_append(const Geo& g, const int32_t* positions, const void* src, const void* w, void* pool,
                             float* pool_scale, hipStream_t stream);
int key_append_max_latent_dim();
hipError_t launch_attn(const Geo& g, const void* q, const void* kv_pool, const int32_t* topk_idx, void* out,
                       float* lse, void* workspace, const int32_t* pool_rows, hipStream_t stream);

}  // namespace dsa
