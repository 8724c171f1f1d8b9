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
// them (block 0 of each row, after its scores), sparing the top-k a zeroing launch, and ranks the top-k floor of
// the rows of indexer_floor_row into thr (an extra block per row).
struct TopkState {
  uint32_t* cnt;  // [R, 4]
  uint32_t* thr;  // [R, 4]; entry 1 receives the floor
  int k;
};
// Whether the fused step's indexer launch carries the floor blocks (some row may have indexer_floor_row).
bool indexer_floor_blocks(const Geo& g);

// indexer.hip.  fp8 problems whose rows come in groups of at least kTiledMinRows per sequence (chunked prefill)
// run the tiled GEMM kernel, which takes no `fuse`.  Otherwise, with `fuse` non-NULL the indexer also clears the
// top-k state.
constexpr int kTiledMinRows = 8;
bool indexer_tiled(const Geo& g);
hipError_t launch_indexer(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                          const void* k_idx_pool, const float* k_idx_scale, float* scores, int64_t ld,
                          const TopkState* fuse, hipStream_t stream);

// Chunked prefill without the score matrix (prefill.hip, and the tiled indexer's sample and filter passes).
constexpr int kPfSample = 4096;  // sampled positions per row: 128 runs of 32
constexpr int kPfCap = 12288;    // candidates a row keeps
struct PfSel {
  float* samp;         // [R, kPfSample] scores of each row's sampled positions
  int32_t* samp_len;   // [R] sampled positions written for the row
  uint32_t* floor;     // [R] the row's floor: 20-bit key prefix a candidate reaches
  uint32_t* cnt;       // [R] candidates reserved (may exceed kPfCap: the row then falls back)
  uint64_t* cand;      // [R, kPfCap] candidates, position << 32 | key, in no particular order
  uint32_t* ctl;       // [4]: rows that fell back, grid-barrier counter, barrier time-outs, unused
  int32_t* fail;       // [R] rows that fell back
  float* fbuf;         // [ld] scores of the row being resolved by the fallback
};
bool prefill_select_supported(const Geo& g);
size_t prefill_select_bytes(const Geo& g);
PfSel prefill_select_carve(const Geo& g, void* workspace);
// mode 1: sampled scores into sel.samp; mode 2: candidates at or above each row's floor into sel.cand
hipError_t launch_indexer_pf(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                             const void* k_idx_pool, const float* k_idx_scale, const PfSel& sel, int mode,
                             hipStream_t stream);
// prefill.hip: floors from the samples (also clears the candidate counters and the fallback state), then, after
// the filter pass, each row's selection (pool rows too when pool_rows is non-NULL); rows the sample misjudged go
// to the fallback list
hipError_t launch_pf_floor(const Geo& g, const PfSel& sel, hipStream_t stream);
hipError_t launch_pf_resolve(const Geo& g, const PfSel& sel, int32_t* topk_idx, int32_t* pool_rows,
                             hipStream_t stream);
// indexer.hip: the fallback, which scores each listed row in full into sel.fbuf and selects over it (one
// persistent launch; it returns at once when the list is empty)
hipError_t launch_pf_fallback(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                              const void* k_idx_pool, const float* k_idx_scale, const PfSel& sel, int32_t* topk_idx,
                              int32_t* pool_rows, hipStream_t stream);

// topk.hip
constexpr int kTopkMaxBlocksPerRow = 1024;
constexpr int kTopkChunk = 4096;
size_t topk_workspace_bytes(const Geo& g);

TopkState topk_state(const Geo& g, void* workspace);
hipError_t launch_topk_zero(const Geo& g, void* workspace, hipStream_t stream);
// Selection over stored scores whose top-k state is already zero (launch_topk_zero, or the fused indexer).
// pool_rows: if non-NULL, [R, k] int32 receiving the pool row of every selected slot (-1 for padding), for the
// attention.  indexer_floors: the fused indexer ranked the floors of the rows of indexer_floor_row.
hipError_t launch_topk_select(const Geo& g, const float* scores, int64_t ld, int32_t* topk_idx, void* workspace,
                              int32_t* pool_rows, bool indexer_floors, hipStream_t stream);
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
// proj.hip: fp64-chain projections with per-group e4m3 quantisation.
const char* query_proj_unsupported(int d_model, int H_I, int d_I, bool bf16, const void* h, const void* w_q,
                                   const void* w_w);  // NULL when supported, else the reason
hipError_t launch_query_proj(int R, int d_model, int H_I, int d_I, bool bf16, bool f8, const void* h,
                             const void* w_q, const void* w_w, void* q, float* q_scale, float* head_w,
                             hipStream_t stream);
bool key_proj_supported(const Geo& g, const void* src, const void* w);
hipError_t launch_key_proj(const Geo& g, const int32_t* positions, const void* src, const void* w, void* pool,
                           float* pool_scale, hipStream_t stream);
hipError_t launch_attn(const Geo& g, const void* q, const void* kv_pool, const int32_t* topk_idx, void* out,
                       float* lse, void* workspace, const int32_t* pool_rows, hipStream_t stream);

}  // namespace dsa
