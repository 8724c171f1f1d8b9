// C-ABI entry points of libdsa (declared in include/dsa.h): argument validation on the host, workspace
// layout, and dispatch to the gfx950 kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "dsa.h"
#include "launch.h"

// Scratch of dsa_decode_step_static (see static_scratch below).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define DSA_CHECK(cond, st, ...) \
  do {                           \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ilog2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

// Checks the problem description (no device pointers) and fills the derived geometry.
dsa_status_t check_problem(const dsa_problem_t* p, const dsa_layout_t* lay, bool need_idx, bool need_attn,
                           dsa::Geo* g) {
  DSA_CHECK(p != nullptr, DSA_EINVAL, "problem is NULL");
  DSA_CHECK(p->num_rows >= 0, DSA_EINVAL, "num_rows = %d < 0", p->num_rows);
  DSA_CHECK(p->num_seqs >= 1, DSA_EINVAL, "num_seqs = %d < 1", p->num_seqs);
  DSA_CHECK(p->topk >= 1 && p->topk <= 16384, DSA_EINVAL, "topk = %d outside 1..16384", p->topk);
  const int lg = ilog2_exact(p->page_size);
  DSA_CHECK(p->page_size >= 32 && p->page_size <= 4096 && lg >= 0, DSA_EINVAL,
            "page_size = %d is not a power of two in 32..4096", p->page_size);
  DSA_CHECK(p->max_pages >= 1 && p->num_pages >= 1, DSA_EINVAL, "max_pages = %d, num_pages = %d must be >= 1",
            p->max_pages, p->num_pages);
  DSA_CHECK((int64_t)p->num_pages * p->page_size <= (int64_t)1 << 40, DSA_EINVAL, "pool too large");
  DSA_CHECK(p->max_row_len >= 0 && (int64_t)p->max_row_len <= (int64_t)p->max_pages * p->page_size, DSA_EINVAL,
            "max_row_len = %d outside 0..max_pages*page_size = %lld", p->max_row_len,
            (long long)p->max_pages * p->page_size);
  DSA_CHECK((int64_t)p->max_row_len <= (int64_t)dsa::kTopkMaxBlocksPerRow * dsa::kTopkChunk, DSA_EUNSUPPORTED,
            "max_row_len = %d above the supported %d", p->max_row_len,
            dsa::kTopkMaxBlocksPerRow * dsa::kTopkChunk);
  DSA_CHECK(p->rows_per_seq >= 1, DSA_EINVAL, "rows_per_seq = %d < 1", p->rows_per_seq);
  DSA_CHECK(p->num_rows <= 65535, DSA_EUNSUPPORTED, "num_rows = %d above 65535", p->num_rows);
  DSA_CHECK(lay != nullptr, DSA_EINVAL, "layout is NULL");
  DSA_CHECK(lay->row_seq && lay->row_len && lay->page_table, DSA_EINVAL, "layout has a NULL pointer");
  if (need_idx) {
    DSA_CHECK(p->idx_dtype == DSA_F8E4M3 || p->idx_dtype == DSA_F32, DSA_EINVAL, "idx_dtype = %d invalid",
              p->idx_dtype);
    if (p->idx_dtype == DSA_F8E4M3) {
      DSA_CHECK(p->idx_dim == 64 || p->idx_dim == 128, DSA_EUNSUPPORTED,
                "fp8 indexer needs idx_dim = 64 or 128 (got %d)", p->idx_dim);
      DSA_CHECK(p->idx_heads == 32 || p->idx_heads == 64, DSA_EUNSUPPORTED,
                "fp8 indexer needs idx_heads of 32 or 64 (got %d)", p->idx_heads);
    } else {
      DSA_CHECK(p->idx_heads >= 1 && p->idx_heads <= 64, DSA_EUNSUPPORTED, "fp32 indexer: idx_heads = %d not in 1..64",
                p->idx_heads);
      DSA_CHECK(p->idx_dim >= 1 && p->idx_dim <= 128, DSA_EUNSUPPORTED, "fp32 indexer: idx_dim = %d not in 1..128",
                p->idx_dim);
    }
  }
  if (need_attn) {
    DSA_CHECK(p->kv_dtype == DSA_BF16 || p->kv_dtype == DSA_F32 || p->kv_dtype == DSA_F8E4M3, DSA_EINVAL,
              "kv_dtype = %d invalid", p->kv_dtype);
    DSA_CHECK(p->attn_heads >= 1 && p->attn_heads <= 256, DSA_EUNSUPPORTED, "attn_heads = %d not in 1..256",
              p->attn_heads);
    DSA_CHECK(p->softmax_scale == p->softmax_scale, DSA_EINVAL, "softmax_scale is NaN");
    if (p->kv_dtype == DSA_BF16 || p->kv_dtype == DSA_F8E4M3) {
      DSA_CHECK(p->latent_dim == 512, DSA_EUNSUPPORTED, "bf16 and fp8-entry attention need latent_dim = 512 (got %d)",
                p->latent_dim);
      DSA_CHECK(p->attn_heads % 16 == 0, DSA_EUNSUPPORTED,
                "bf16 and fp8-entry attention need attn_heads %% 16 == 0 (got %d)", p->attn_heads);
      DSA_CHECK((int64_t)p->num_pages * p->page_size < ((int64_t)1 << 31), DSA_EUNSUPPORTED,
                "bf16 attention addresses latent rows with 31 bits (num_pages * page_size = %lld)",
                (long long)p->num_pages * p->page_size);
    } else {
      DSA_CHECK(p->latent_dim >= 1 && p->latent_dim <= 1024, DSA_EUNSUPPORTED, "fp32 attention: latent_dim = %d",
                p->latent_dim);
      DSA_CHECK(p->topk <= 4096, DSA_EUNSUPPORTED, "fp32 attention supports topk <= 4096 (got %d)", p->topk);
    }
  }
  g->R = p->num_rows;
  g->S = p->num_seqs;
  g->H_I = p->idx_heads;
  g->d_I = p->idx_dim;
  g->H = p->attn_heads;
  g->d_c = p->latent_dim;
  g->k = p->topk;
  g->page_size = p->page_size;
  g->log2ps = lg;
  g->max_pages = p->max_pages;
  g->num_pages = p->num_pages;
  g->max_row_len = p->max_row_len;
  g->rows_per_seq = p->rows_per_seq;
  g->idx_dtype = p->idx_dtype;
  g->kv_dtype = p->kv_dtype;
  g->softmax_scale = p->softmax_scale;
  g->row_seq = lay->row_seq;
  g->row_len = lay->row_len;
  g->page_table = lay->page_table;
  return DSA_OK;
}

dsa_status_t check_indexer_args(const dsa::Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                                const void* k_idx_pool, const float* k_idx_scale) {
  DSA_CHECK(q_idx && head_w && k_idx_pool, DSA_EINVAL, "q_idx, head_w and k_idx_pool must be non-NULL");
  DSA_CHECK(aligned16(q_idx) && aligned16(k_idx_pool), DSA_EINVAL, "q_idx and k_idx_pool must be 16-byte aligned");
  if (g.idx_dtype == DSA_F8E4M3) {
    DSA_CHECK(q_idx_scale && k_idx_scale, DSA_EINVAL, "fp8 indexer needs q_idx_scale and k_idx_scale");
    DSA_CHECK(aligned16(head_w) && aligned16(q_idx_scale), DSA_EINVAL,
              "fp8 indexer: head_w and q_idx_scale must be 16-byte aligned");
  } else
    DSA_CHECK(!q_idx_scale && !k_idx_scale, DSA_EINVAL, "fp32 indexer takes no scales (pass NULL)");
  return DSA_OK;
}

dsa_status_t check_attn_args(const dsa::Geo& g, const void* q, const void* kv_pool, const int32_t* topk_idx,
                             const void* out) {
  DSA_CHECK(q && kv_pool && topk_idx && out, DSA_EINVAL, "q, kv_pool, topk_idx and out must be non-NULL");
  DSA_CHECK(aligned16(q) && aligned16(kv_pool) && aligned16(out), DSA_EINVAL,
            "q, kv_pool and out must be 16-byte aligned");
  (void)g;
  return DSA_OK;
}

dsa_status_t check_scores(const dsa::Geo& g, const float* scores, int64_t ld) {
  DSA_CHECK(scores != nullptr, DSA_EINVAL, "scores is NULL");
  DSA_CHECK(aligned16(scores), DSA_EINVAL, "scores must be 16-byte aligned");
  DSA_CHECK(ld >= g.max_row_len && ld % 4 == 0, DSA_EINVAL, "scores_ld = %lld must be >= max_row_len = %d and a multiple of 4",
            (long long)ld, g.max_row_len);
  return DSA_OK;
}

dsa_status_t check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return DSA_OK;
  DSA_CHECK(ws != nullptr, DSA_EWORKSPACE, "workspace is NULL, %zu bytes needed", need);
  DSA_CHECK((reinterpret_cast<uintptr_t>(ws) & (dsa::kAlign - 1)) == 0, DSA_EWORKSPACE,
            "workspace must be %zu-byte aligned", dsa::kAlign);
  DSA_CHECK(have >= need, DSA_EWORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t step_ld(const dsa::Geo& g) { return ((int64_t)std::max(g.max_row_len, 1) + 63) / 64 * 64; }

// Dense attention is the sparse kernels with no selection list: slot s of row r is position s while s < n_r.
// The selection width becomes the longest row (at least 1), within what the attention kernels take (the bf16
// kernels (bf16 and fp8-entry latents) split up to 131072 slots over their blocks; the fp32 kernel stages at most
// 4096 in LDS).
dsa_status_t dense_geo(dsa::Geo* g) {
  const int cap = g->kv_dtype == DSA_F32 ? 4096 : 131072;
  DSA_CHECK(g->max_row_len <= cap, DSA_EUNSUPPORTED, "dense attention supports max_row_len <= %d (got %d)", cap,
            g->max_row_len);
  g->k = std::max(1, g->max_row_len);
  return DSA_OK;
}

size_t dense_bytes(const dsa::Geo& g) { return dsa::attn_workspace_bytes(g); }

// The fused step's workspace: scores, the selection (when the caller passes none) and the pool row of every
// selected slot, then one region that the top-k state and, once the selection is written, the attention's split
// partials share.
size_t step_bytes(const dsa::Geo& g) {
  const size_t lists = 2 * dsa::align_up(sizeof(int32_t) * (size_t)g.R * g.k);
  if (dsa::prefill_select_supported(g))  // no score matrix: candidate lists and samples, then the partials
    return lists + std::max(dsa::prefill_select_bytes(g), dsa::attn_workspace_bytes(g));
  return dsa::align_up(sizeof(float) * (size_t)g.R * step_ld(g)) + lists +
         std::max(dsa::topk_workspace_bytes(g), dsa::attn_workspace_bytes(g));
}

// A chunked prefill (rows of one sequence, fp8 indexer): sample pass, floors, filter pass, resolve and fallback,
// then the attention; the selection's workspace is reused by the attention's partials.
dsa_status_t prefill_step(const dsa::Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                          const void* k_idx_pool, const float* k_idx_scale, const void* q, const void* kv_pool,
                          int32_t* topk_idx, void* out, float* lse, void* workspace, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = reinterpret_cast<int32_t*>(ws);
  ws += dsa::align_up(sizeof(int32_t) * (size_t)g.R * g.k);
  int32_t* pool_rows = g.kv_dtype == DSA_BF16 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  ws += dsa::align_up(sizeof(int32_t) * (size_t)g.R * g.k);
  if (topk_idx) idx = topk_idx;
  const dsa::PfSel sel = dsa::prefill_select_carve(g, ws);
  dsa_status_t st;
  if ((st = hip_status(dsa::launch_indexer_pf(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, sel, 1, s),
                       "indexer sample launch")) != DSA_OK ||
      (st = hip_status(dsa::launch_pf_floor(g, sel, s), "floor launch")) != DSA_OK ||
      (st = hip_status(dsa::launch_indexer_pf(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, sel, 2, s),
                       "indexer filter launch")) != DSA_OK ||
      (st = hip_status(dsa::launch_pf_resolve(g, sel, idx, pool_rows, s), "resolve launch")) != DSA_OK ||
      (st = hip_status(dsa::launch_pf_fallback(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, sel, idx,
                                               pool_rows, s),
                       "fallback launch")) != DSA_OK)
    return st;
  return hip_status(dsa::launch_attn(g, q, kv_pool, idx, out, lse, ws, pool_rows, s), "attention launch");
}

// The step on a validated problem and workspace.
dsa_status_t decode_step(const dsa::Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                         const void* k_idx_pool, const float* k_idx_scale, const void* q, const void* kv_pool,
                         int32_t* topk_idx, void* out, float* lse, void* workspace, hipStream_t s) {
  if (dsa::prefill_select_supported(g))
    return prefill_step(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool, topk_idx, out, lse,
                        workspace, s);
  dsa_status_t st;
  char* ws = static_cast<char*>(workspace);
  const int64_t ld = step_ld(g);
  float* scores = reinterpret_cast<float*>(ws);
  ws += dsa::align_up(sizeof(float) * (size_t)g.R * ld);
  int32_t* idx = reinterpret_cast<int32_t*>(ws);
  ws += dsa::align_up(sizeof(int32_t) * (size_t)g.R * g.k);
  int32_t* pool_rows_ws = reinterpret_cast<int32_t*>(ws);
  ws += dsa::align_up(sizeof(int32_t) * (size_t)g.R * g.k);
  char* const tail = ws;  // top-k state, then the attention's split partials
  // the per-row fp8 indexer clears the top-k state once its scores are out, sparing the top-k its zeroing launch
  const bool fuse = g.idx_dtype == DSA_F8E4M3 && !dsa::indexer_tiled(g);
  const dsa::TopkState tstate = dsa::topk_state(g, tail);
  if ((st = hip_status(dsa::launch_indexer(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, scores, ld,
                                           fuse ? &tstate : nullptr, s),
                       "indexer launch")) != DSA_OK)
    return st;
  if (topk_idx) idx = topk_idx;
  // the top-k hands the bf16 attention the pool row of every selected slot, sparing it the page-table lookup
  int32_t* pool_rows = g.kv_dtype == DSA_BF16 ? pool_rows_ws : nullptr;
  if (fuse) {
    if ((st = hip_status(dsa::launch_topk_select(g, scores, ld, idx, tail, pool_rows, dsa::indexer_floor_blocks(g), s),
                         "top-k launch")) != DSA_OK)
      return st;
  } else if ((st = hip_status(dsa::launch_topk(g, scores, ld, idx, tail, pool_rows, s), "top-k launch")) != DSA_OK) {
    return st;
  }
  return hip_status(dsa::launch_attn(g, q, kv_pool, idx, out, lse, tail, pool_rows, s), "attention launch");
}

dsa_status_t check_step(const dsa_problem_t* problem, const dsa_layout_t* layout, const void* q_idx,
                        const float* q_idx_scale, const float* head_w, const void* k_idx_pool, const float* k_idx_scale,
                        const void* q, const void* kv_pool, const void* out, dsa::Geo* g) {
  dsa_status_t st = check_problem(problem, layout, true, true, g);
  if (st != DSA_OK) return st;
  if ((st = check_indexer_args(*g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale)) != DSA_OK) return st;
  DSA_CHECK(q && kv_pool && out, DSA_EINVAL, "q, kv_pool and out must be non-NULL");
  DSA_CHECK(aligned16(q) && aligned16(kv_pool) && aligned16(out), DSA_EINVAL,
            "q, kv_pool and out must be 16-byte aligned");
  return DSA_OK;
}

// The scratch of dsa_decode_step_static: a file-scope device array, one copy on every device the library runs on,
// held until the process ends.  Host code must not pass `scratch` itself to a kernel (on the host it is only a
// stand-in for the symbol); its device address is looked up once per device, with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status_t static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DSA_EHIP, "no usable current device (%d)", dev);
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return fail(DSA_EHIP, "hipStreamGetDevice failed");
    DSA_CHECK(sdev == dev, DSA_EINVAL, "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(DSA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status_t dsa_indexer_scores(const dsa_problem_t* problem, const dsa_layout_t* layout, const void* q_idx,
                                const float* q_idx_scale, const float* head_w, const void* k_idx_pool,
                                const float* k_idx_scale, float* scores, int64_t scores_ld, void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_problem(problem, layout, true, false, &g);
  if (st != DSA_OK) return st;
  if ((st = check_indexer_args(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale)) != DSA_OK) return st;
  if ((st = check_scores(g, scores, scores_ld)) != DSA_OK) return st;
  return hip_status(dsa::launch_indexer(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, scores, scores_ld,
                                        nullptr, static_cast<hipStream_t>(stream)),
                    "indexer launch");
}

dsa_status_t dsa_topk(const dsa_problem_t* problem, const dsa_layout_t* layout, const float* scores,
                      int64_t scores_ld, int32_t* topk_idx, void* workspace, size_t workspace_bytes, void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_problem(problem, layout, false, false, &g);
  if (st != DSA_OK) return st;
  if ((st = check_scores(g, scores, scores_ld)) != DSA_OK) return st;
  DSA_CHECK(topk_idx != nullptr, DSA_EINVAL, "topk_idx is NULL");
  if ((st = check_ws(workspace, workspace_bytes, dsa::topk_workspace_bytes(g))) != DSA_OK) return st;
  return hip_status(dsa::launch_topk(g, scores, scores_ld, topk_idx, workspace, nullptr, static_cast<hipStream_t>(stream)),
                    "top-k launch");
}

dsa_status_t dsa_sparse_mla_attn(const dsa_problem_t* problem, const dsa_layout_t* layout, const void* q,
                                 const void* kv_pool, const int32_t* topk_idx, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_problem(problem, layout, false, true, &g);
  if (st != DSA_OK) return st;
  if ((st = check_attn_args(g, q, kv_pool, topk_idx, out)) != DSA_OK) return st;
  if ((st = check_ws(workspace, workspace_bytes, dsa::attn_workspace_bytes(g))) != DSA_OK) return st;
  return hip_status(dsa::launch_attn(g, q, kv_pool, topk_idx, out, lse, workspace, nullptr,
                                     static_cast<hipStream_t>(stream)),
                    "attention launch");
}

dsa_status_t dsa_indexer_key_append(const dsa_problem_t* problem, const dsa_layout_t* layout,
                                    const int32_t* positions, const void* src, const void* w_k, void* k_idx_pool,
                                    float* k_idx_scale, void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_problem(problem, layout, true, false, &g);
  if (st != DSA_OK) return st;
  DSA_CHECK(positions && src && k_idx_pool, DSA_EINVAL, "positions, src and k_idx_pool must be non-NULL");
  if (g.idx_dtype == DSA_F8E4M3)
    DSA_CHECK(k_idx_scale != nullptr, DSA_EINVAL, "an fp8 indexer cache needs k_idx_scale");
  else
    DSA_CHECK(k_idx_scale == nullptr, DSA_EINVAL, "an fp32 indexer cache takes no scales (pass NULL)");
  if (w_k) {
    DSA_CHECK(g.kv_dtype == DSA_BF16 || g.kv_dtype == DSA_F32, DSA_EINVAL, "kv_dtype = %d invalid", g.kv_dtype);
    DSA_CHECK(g.d_c >= 1 && g.d_c <= dsa::key_append_max_latent_dim(), DSA_EUNSUPPORTED,
              "key projection: latent_dim = %d not in 1..%d", g.d_c, dsa::key_append_max_latent_dim());
    const uintptr_t a = g.kv_dtype == DSA_BF16 ? 1 : 3;
    DSA_CHECK(((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(w_k)) & a) == 0, DSA_EINVAL,
              "src and w_k must be aligned to their element size");
  } else {
    DSA_CHECK((reinterpret_cast<uintptr_t>(src) & 3) == 0, DSA_EINVAL, "fp32 keys must be 4-byte aligned");
  }
  if (w_k && dsa::key_proj_supported(g, src, w_k))
    return hip_status(dsa::launch_key_proj(g, positions, src, w_k, k_idx_pool, k_idx_scale,
                                           static_cast<hipStream_t>(stream)),
                      "key append launch");
  return hip_status(dsa::launch_key_append(g, positions, src, w_k, k_idx_pool, k_idx_scale,
                                           static_cast<hipStream_t>(stream)),
                    "key append launch");
}

dsa_status_t dsa_indexer_query_proj(const dsa_problem_t* problem, int32_t d_model, const void* h, const void* w_q,
                                    const void* w_w, void* q_idx, float* q_idx_scale, float* head_w,
                                    void* stream) {
  DSA_CHECK(problem != nullptr, DSA_EINVAL, "problem is NULL");
  const dsa_problem_t& p = *problem;
  DSA_CHECK(p.num_rows >= 0 && p.num_rows <= 65535 * 4, DSA_EINVAL, "num_rows = %d not in 0..262140", p.num_rows);
  DSA_CHECK(p.idx_dtype == DSA_F8E4M3 || p.idx_dtype == DSA_F32, DSA_EINVAL, "idx_dtype = %d invalid", p.idx_dtype);
  DSA_CHECK(p.kv_dtype == DSA_BF16 || p.kv_dtype == DSA_F32, DSA_EINVAL,
            "kv_dtype (the dtype of h and the weights) = %d must be BF16 or F32", p.kv_dtype);
  DSA_CHECK(d_model >= 1, DSA_EINVAL, "d_model = %d < 1", d_model);
  DSA_CHECK(p.idx_heads >= 1 && p.idx_dim >= 1, DSA_EINVAL, "idx_heads = %d, idx_dim = %d must be >= 1",
            p.idx_heads, p.idx_dim);
  DSA_CHECK(h && w_q && w_w && q_idx && head_w, DSA_EINVAL, "h, w_q, w_w, q_idx and head_w must be non-NULL");
  const bool f8 = p.idx_dtype == DSA_F8E4M3;
  if (f8)
    DSA_CHECK(q_idx_scale != nullptr, DSA_EINVAL, "an fp8 query needs q_idx_scale");
  else
    DSA_CHECK(q_idx_scale == nullptr, DSA_EINVAL, "an fp32 query takes no scales (pass NULL)");
  DSA_CHECK(((reinterpret_cast<uintptr_t>(head_w) | reinterpret_cast<uintptr_t>(q_idx_scale) |
              (f8 ? 0 : reinterpret_cast<uintptr_t>(q_idx))) & 3) == 0,
            DSA_EINVAL, "head_w, q_idx_scale and fp32 q_idx must be 4-byte aligned");
  const bool bf16 = p.kv_dtype == DSA_BF16;
  const char* why = dsa::query_proj_unsupported(d_model, p.idx_heads, p.idx_dim, bf16, h, w_q, w_w);
  DSA_CHECK(why == nullptr, why && std::strstr(why, "aligned") ? DSA_EINVAL : DSA_EUNSUPPORTED, "%s", why);
  return hip_status(dsa::launch_query_proj(p.num_rows, d_model, p.idx_heads, p.idx_dim, bf16, f8, h, w_q, w_w, q_idx,
                                           q_idx_scale, head_w, static_cast<hipStream_t>(stream)),
                    "query projection launch");
}

dsa_status_t dsa_dense_mla_attn(const dsa_problem_t* problem, const dsa_layout_t* layout, const void* q,
                                const void* kv_pool, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_problem(problem, layout, false, true, &g);
  if (st != DSA_OK) return st;
  if ((st = dense_geo(&g)) != DSA_OK) return st;
  DSA_CHECK(q && kv_pool && out, DSA_EINVAL, "q, kv_pool and out must be non-NULL");
  DSA_CHECK(aligned16(q) && aligned16(kv_pool) && aligned16(out), DSA_EINVAL,
            "q, kv_pool and out must be 16-byte aligned");
  if ((st = check_ws(workspace, workspace_bytes, dense_bytes(g))) != DSA_OK) return st;
  return hip_status(dsa::launch_attn(g, q, kv_pool, nullptr, out, lse, workspace, nullptr,
                                     static_cast<hipStream_t>(stream)),
                    "attention launch");
}

dsa_status_t dsa_decode_step(const dsa_problem_t* problem, const dsa_layout_t* layout, const void* q_idx,
                             const float* q_idx_scale, const float* head_w, const void* k_idx_pool,
                             const float* k_idx_scale, const void* q, const void* kv_pool, int32_t* topk_idx,
                             void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_step(problem, layout, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool, out,
                               &g);
  if (st != DSA_OK) return st;
  if ((st = check_ws(workspace, workspace_bytes, step_bytes(g))) != DSA_OK) return st;
  return decode_step(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool, topk_idx, out, lse,
                     workspace, static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_decode_step_static(const dsa_problem_t* problem, const dsa_layout_t* layout, const void* q_idx,
                                    const float* q_idx_scale, const float* head_w, const void* k_idx_pool,
                                    const float* k_idx_scale, const void* q, const void* kv_pool, int32_t* topk_idx,
                                    void* out, float* lse, void* stream) {
  dsa::Geo g;
  dsa_status_t st = check_step(problem, layout, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool, out,
                               &g);
  if (st != DSA_OK) return st;
  const size_t need = step_bytes(g);
  DSA_CHECK(need <= kStaticScratchBytes, DSA_EUNSUPPORTED,
            "this problem needs %zu bytes of scratch, above the static scratch of %zu bytes (use dsa_decode_step "
            "with a workspace)", need, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(static_cast<hipStream_t>(stream), &ws)) != DSA_OK) return st;
  return decode_step(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, q, kv_pool, topk_idx, out, lse, ws,
                     static_cast<hipStream_t>(stream));
}

size_t dsa_workspace_bytes(const dsa_problem_t* problem, int32_t op) {
  g_last_error.clear();  // a 0 return with an empty message means "no workspace needed"
  if (!problem) { fail(DSA_EINVAL, "problem is NULL"); return 0; }
  dsa_layout_t dummy{reinterpret_cast<const int32_t*>(16), reinterpret_cast<const int32_t*>(16),
                     reinterpret_cast<const int32_t*>(16)};
  dsa::Geo g;
  const bool idx = op == DSA_OP_STEP, attn = op == DSA_OP_ATTN || op == DSA_OP_STEP || op == DSA_OP_DENSE;
  if (check_problem(problem, &dummy, idx, attn, &g) != DSA_OK) return 0;
  switch (op) {
    case DSA_OP_TOPK: return dsa::topk_workspace_bytes(g);
    case DSA_OP_ATTN: return dsa::attn_workspace_bytes(g);
    case DSA_OP_STEP: return step_bytes(g);
    case DSA_OP_DENSE: return dense_geo(&g) == DSA_OK ? dense_bytes(g) : 0;
    default: fail(DSA_EINVAL, "unknown op %d", op); return 0;
  }
}

const char* dsa_status_str(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_EINVAL: return "DSA_EINVAL: invalid argument";
    case DSA_EUNSUPPORTED: return "DSA_EUNSUPPORTED: no kernel for this combination";
    case DSA_EWORKSPACE: return "DSA_EWORKSPACE: workspace missing or too small";
    case DSA_EHIP: return "DSA_EHIP: HIP runtime error";
  }
  return "unknown dsa_status_t";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

int32_t dsa_abi_version(void) { return 1; }

}  // extern "C"
