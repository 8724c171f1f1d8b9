/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) DeepSeek Sparse Attention decode-step library.
 *
 * For each query row the step
 *   1. scores every visible cached position with the lightning indexer: H_I narrow heads each take the
 *      dot product of their query with the position's single shared key, pass it through a ReLU, and the
 *      H_I results are summed with per-head weights that carry no sign constraint (DeepSeek Sparse Attention
 *      explained, "How Does the Lightning Indexer Score a Token?"; milos-mitrovic, "How Does the Lightning
 *      Indexer Pick Which Tokens Matter?"; lizeman DSA page, section 2 stage 1);
 *   2. keeps the min(k, n) highest-scoring positions ("How Does the Selector Pick 1,024?");
 *   3. runs softmax attention in MQA mode over only the selected 512-wide latent rows, which every query
 *      head shares and which serve as both key and value (lizeman section 2 stage 2; kiadev "How DSA works";
 *      "What Does the Whole Block Look Like?").
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library never allocates, frees or
 *     retains caller memory and keeps no state between calls; scratch space comes from the caller's
 *     workspace (size from dsa_workspace_bytes).
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null stream) and the call
 *     returns after the enqueue.  The caller synchronises.
 *   - Every argument that the host can check is checked BEFORE anything is enqueued: a non-OK return means
 *     no work was queued.  DSA_EHIP reports a failed launch.  Nothing throws or aborts across the ABI.
 *     dsa_last_error() gives a thread-local message for the last non-OK return.
 *   - Device-side metadata (row_seq, row_len, page_table) cannot be checked by the host.  Kernels clamp a
 *     row length to [0, max_row_len] and a page id to [0, num_pages) so that a bad value never reads or
 *     writes out of bounds; results for such rows are unspecified.
 *   - Positions are 0-based logical positions within a row's sequence; row r sees positions 0..n_r-1.
 *     Position s of sequence q lives at physical row page_table[q][s / page_size] * page_size +
 *     s % page_size of each pool (the selected positions are "an address list into the paged KV cache").
 *   - Calls on one stream are ordered; concurrent calls on different streams must use different
 *     workspaces.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_EINVAL = 1,        /* a NULL pointer, a bad size or an inconsistent argument */
  DSA_EUNSUPPORTED = 2,  /* a valid combination this build has no kernel for */
  DSA_EWORKSPACE = 3,    /* workspace NULL or smaller than dsa_workspace_bytes() */
  DSA_EHIP = 4           /* the HIP runtime reported an error at launch */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,     /* IEEE binary32 */
  DSA_BF16 = 1,    /* bfloat16 */
  DSA_F8E4M3 = 2   /* OCP FP8 E4M3FN codes (bias 7, max 448, no inf) with one fp32 scale per stored vector */
} dsa_dtype_t;

typedef enum { DSA_OP_TOPK = 1, DSA_OP_ATTN = 2, DSA_OP_STEP = 3, DSA_OP_DENSE = 4 } dsa_op_t;

/* Shapes, dtypes and bounds of one call.  Host memory, read during the call only. */
typedef struct {
  int32_t num_rows;      /* R: query rows in the call (one per sequence in decode, one per position in prefill) */
  int32_t num_seqs;      /* S: rows of page_table */
  int32_t idx_heads;     /* H_I: indexer heads.  F8E4M3: 32 or 64.  F32: 1..64 */
  int32_t idx_dim;       /* d_I: indexer head width.  F8E4M3: 64 or 128.  F32: 1..128 */
  int32_t attn_heads;    /* H: attention heads sharing one latent row.  BF16, F8E4M3: multiple of 16, <= 256.
                            F32: <= 256 */
  int32_t latent_dim;    /* d_c: latent width.  BF16, F8E4M3: 512.  F32: 1..1024 */
  int32_t topk;          /* k: positions kept per row, 1..16384 */
  int32_t page_size;     /* positions per page: power of two, 32..4096 */
  int32_t max_pages;     /* row stride of page_table */
  int32_t num_pages;     /* physical pages in each pool (both pools have num_pages * page_size rows) */
  int32_t max_row_len;   /* host-side bound: 0 <= row_len[r] <= max_row_len <= max_pages * page_size */
  int32_t rows_per_seq;  /* >= 1.  Consecutive groups of this many rows share one sequence (a chunked prefill);
                            the caller guarantees row_seq is constant within each group.  1 for plain decode */
  int32_t idx_dtype;     /* dsa_dtype_t of q_idx / k_idx_pool: DSA_F8E4M3 (scales required) or DSA_F32 (scales NULL) */
  int32_t kv_dtype;      /* dsa_dtype_t of the latent cache: DSA_BF16 or DSA_F32 (q, kv_pool and out in that type), or
                            DSA_F8E4M3: 656-byte cache entries (see dsa_sparse_mla_attn), bf16 q and out */
  float softmax_scale;   /* logits = softmax_scale * <q[h], c[s]> */
} dsa_problem_t;

/* Device-resident int32 metadata.  The struct itself is host memory. */
typedef struct {
  const int32_t *row_seq;     /* [R] sequence (page_table row) of each query row */
  const int32_t *row_len;     /* [R] visible positions n_r of each row */
  const int32_t *page_table;  /* [S, max_pages] physical page of each logical page, shared by both pools */
} dsa_layout_t;

/*
 * Lightning-indexer scores (step 1).
 *   q_idx       [R, H_I, d_I]   fp8 codes or fp32 indexer queries
 *   q_idx_scale [R, H_I]        fp32 dequantisation scale of each query vector (F8E4M3; NULL for F32)
 *   head_w      [R, H_I]        fp32 head weights, any sign
 *   k_idx_pool  [num_pages*page_size, d_I]  fp8 codes or fp32 keys, one per cached position
 *   k_idx_scale [num_pages*page_size]       fp32 scale of each key (F8E4M3; NULL for F32)
 *   scores      [R, scores_ld]  fp32 out: scores[r][s] = sum_j w[r][j] * max(0, <q_I[r][j], k_I[s]>) for
 *                               s < n_r, with q_I = scale * code; entries s >= n_r are not written.
 *   scores_ld   >= max_row_len
 * q_idx and k_idx_pool must be 16-byte aligned, and for F8E4M3 also head_w and q_idx_scale.
 * The fp8 path computes the per-head dot products exactly (fp8 x fp8 products, fp32 accumulation of 64
 * terms) and applies the positive scales outside the ReLU, max(0, a*b*x) = a*b*max(0, x).
 */
dsa_status_t dsa_indexer_scores(const dsa_problem_t *problem, const dsa_layout_t *layout,
                                 const void *q_idx, const float *q_idx_scale, const float *head_w,
                                 const void *k_idx_pool, const float *k_idx_scale,
                                 float *scores, int64_t scores_ld, void *stream);

/*
 * Top-k selection (step 2): for each row, the k_eff = min(k, n_r) positions with the largest scores,
 * ties broken by lower position ("keeps the highest index_topk"; "the smaller of the budget and the number
 * of tokens").
 *   scores    [R, scores_ld] fp32, read for s < n_r
 *   topk_idx  [R, k] int32 out: the selected positions in increasing position order, then -1 padding
 *   workspace >= dsa_workspace_bytes(problem, DSA_OP_TOPK) bytes of device memory, 256-byte aligned
 * Scores are ranked by an order-preserving integer key of their fp32 value (+0 and -0 are equal).
 * Cost: every row is exact, but a row settles fast only when its candidate list (the scores at or above a
 * sampled floor, about k + 8 sqrt(32 k) + 512 of them at n = 128K) fits 12288 entries, i.e. up to k of about 8K
 * at 128K; a larger budget, or heavy ties at the threshold, takes a whole-row radix select that is several times
 * slower.
 */
dsa_status_t dsa_topk(const dsa_problem_t *problem, const dsa_layout_t *layout, const float *scores,
                      int64_t scores_ld, int32_t *topk_idx, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sparse MLA attention in MQA mode (step 3) over the selected latent rows.
 *   q         [R, H, d_c]  bf16 or fp32 queries, already in latent space
 *   kv_pool   [num_pages*page_size, d_c]  bf16 or fp32 latent rows (key = value = the latent row)
 *   topk_idx  [R, k] int32 positions; entries < 0 are skipped; order does not matter
 *   out       [R, H, d_c]  bf16 or fp32 out: softmax-weighted sum of the selected rows
 *   lse       [R, H] fp32 out (may be NULL): natural-log sum of exp(logits); -inf for an empty selection,
 *             whose output is 0
 * The bf16 path runs QK^T and PV on bf16 MFMA with fp32 accumulation and an fp32 online softmax.
 * kv_dtype DSA_F8E4M3 (the FP8 cache of "What Does the GPU Actually Run?": 656 bytes per position): each kv_pool
 * row holds 512 e4m3 latent codes (bytes 0..511), 4 fp32 scales, scale t for values 128t..128t+127 (bytes
 * 512..527), and 64 bf16 RoPE values (bytes 528..655).  q is bf16 [R, H, 576] (latent dims, then RoPE dims) and
 * the logits are softmax_scale * (<q[:512], code * scale> + <q[512:], rope>); out [R, H, 512] is the softmax-
 * weighted sum of the dequantised latent rows.  The latent values are dequantised to bf16 on chip, as the bf16
 * path then computes.
 */
dsa_status_t dsa_sparse_mla_attn(const dsa_problem_t *problem, const dsa_layout_t *layout, const void *q,
                                 const void *kv_pool, const int32_t *topk_idx, void *out, float *lse,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole step on one stream: indexer scores -> top-k -> sparse attention (the four-stage decode pipeline
 * of "What Does the GPU Actually Run?", with the head weights applied in the scoring kernel).
 * Arguments as above; topk_idx may be NULL (the selection then stays in the workspace), lse may be NULL.
 * workspace >= dsa_workspace_bytes(problem, DSA_OP_STEP).
 */
dsa_status_t dsa_decode_step(const dsa_problem_t *problem, const dsa_layout_t *layout,
                             const void *q_idx, const float *q_idx_scale, const float *head_w,
                             const void *k_idx_pool, const float *k_idx_scale,
                             const void *q, const void *kv_pool, int32_t *topk_idx,
                             void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * dsa_decode_step without a workspace argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): its scratch is a 64 MiB array in the
 * library's device code, one copy per device, held until the process ends.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library call); the first call on a device looks the array's address up once.
 *   - Problems whose dsa_workspace_bytes(problem, DSA_OP_STEP) exceeds 64 MiB return DSA_EUNSUPPORTED (enough for
 *     16 rows of 128K positions or 64 rows of 64K).
 *   - `stream` must belong to the current device (DSA_EINVAL otherwise).
 *   - Every call on a device shares that device's scratch, which keeps the last call's contents (nothing in it
 *     needs to start at zero): calls that may overlap on one device (different streams, or several host threads)
 *     race and must be serialised by the caller.
 * Other arguments and results as dsa_decode_step.
 */
dsa_status_t dsa_decode_step_static(const dsa_problem_t *problem, const dsa_layout_t *layout,
                                    const void *q_idx, const float *q_idx_scale, const float *head_w,
                                    const void *k_idx_pool, const float *k_idx_scale,
                                    const void *q, const void *kv_pool, int32_t *topk_idx,
                                    void *out, float *lse, void *stream);

/*
 * Dense MLA attention in MQA mode over every visible position of each row (no indexer, no selection): the
 * short-context fallback.  Below a crossover context the indexer's fixed cost outweighs what it saves, and a
 * dense step is faster (milos-mitrovic, "When Does DSA Beat Dense Attention, and When Doesn't It?": the
 * crossover lies near 40K-64K tokens for decode; kgptalkie, "DeepSeek Sparse Attention explained", "What Does
 * It Cost?": a masked dense mode serves short prefills).  Row r attends to positions 0 .. n_r - 1 of its
 * sequence; problem->topk is not used.
 *   q, kv_pool, out, lse as for dsa_sparse_mla_attn
 *   workspace >= dsa_workspace_bytes(problem, DSA_OP_DENSE) (split partials; 0 bytes, and workspace may be
 *               NULL, when every row fits one block)
 * Supported up to max_row_len = 131072 for bf16 latents and FP8 entries, 4096 for fp32 (DSA_EUNSUPPORTED above).
 */
dsa_status_t dsa_dense_mla_attn(const dsa_problem_t *problem, const dsa_layout_t *layout, const void *q,
                                const void *kv_pool, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Indexer-query projection, the producer of step 1's query side: a token's hidden state h is projected to H_I
 * query vectors q_I = h W_QI (one d_I-wide slice per head) and to H_I head weights w = h W_w (lizeman DSA page,
 * section 2 stage 1 and the section 3 sketch; "How Does the Lightning Indexer Score a Token?": 64 small query
 * vectors plus 64 plain head weights per token).  The outputs are what dsa_indexer_scores takes.
 *   problem     num_rows (R), idx_heads (H_I, a multiple of 8 -- 4 for F32 -- and <= 128), idx_dim (d_I, a power
 *               of two, 8..128 -- 4..128 for F32), idx_dtype (F8E4M3 or F32), kv_dtype (BF16 or F32: the dtype of
 *               h, w_q and w_w) are read; no other field is
 *   d_model     width of the hidden state, a multiple of 8 (4 for F32)
 *   h           [R, d_model] hidden states, row-major
 *   w_q         [d_model, H_I * d_I] W_QI, row-major; head j owns columns j*d_I .. j*d_I + d_I - 1
 *   w_w         [d_model, H_I] the head-weight projection, row-major
 *   q_idx       [R, H_I, d_I] out.  F8E4M3: codes; F32: the fp32 projection
 *   q_idx_scale [R, H_I] out (F8E4M3; NULL for F32): per (row, head) scale = max |q| / 448 over the head's d_I
 *               values (1 for an all-zero head), code = the e4m3 value nearest to q / scale, ties to the even
 *               code, clamped to +-448, sign bit kept
 *   head_w      [R, H_I] out, fp32
 * Every output is the fp64 sum over d ascending of exact products, rounded once to fp32; scales and q / scale
 * are IEEE fp32 divisions, so codes, scales and weights are reproducible bit for bit.  h, w_q, w_w must be
 * 16-byte aligned; outputs need their element alignment.  Unsupported shapes give DSA_EUNSUPPORTED.
 */
dsa_status_t dsa_indexer_query_proj(const dsa_problem_t *problem, int32_t d_model, const void *h, const void *w_q,
                                    const void *w_w, void *q_idx, float *q_idx_scale, float *head_w, void *stream);

/*
 * Indexer-key append, the cache write before step 1: the key of each new token is its latent row times the key
 * projection, k_I = c W_KI (kiadev, "How DSA works", stage 1), written into the indexer cache at position
 * positions[r] of sequence row_seq[r] as the cache stores it ("What Does the GPU Actually Run?": FP8 numbers
 * and one scale per token).
 *   positions   [R] int32 position of row r's token; a row with a negative position, or one at or beyond
 *               max_pages * page_size, is skipped.  Rows that address the same cached position race.
 *   src         w_k non-NULL: [R, d_c] latent rows in kv_dtype (BF16 or F32), d_c = latent_dim <= 1024;
 *               w_k NULL: [R, d_I] fp32 keys, already projected
 *   w_k         [d_c, d_I] W_KI in kv_dtype, row-major, or NULL
 *   k_idx_pool, k_idx_scale  the indexer cache as dsa_indexer_scores reads it.  F8E4M3: scale = max_j |k_j| / 448
 *               (1 for a zero key) and code_j = the e4m3 value nearest to k_j / scale, ties to the even code,
 *               clamped to +-448, sign bit kept.  F32: the keys themselves (k_idx_scale NULL).
 * The projection sums exact fp64 products over d ascending and rounds each key once to fp32; the scale and
 * k_j / scale are IEEE fp32 divisions.  Codes and scales are therefore reproducible bit for bit.  Only the
 * addressed pool rows are written.  Keys must be finite.  The problem's indexer fields are checked as for
 * dsa_indexer_scores; the layout's row_len is not read.
 */
dsa_status_t dsa_indexer_key_append(const dsa_problem_t *problem, const dsa_layout_t *layout,
                                    const int32_t *positions, const void *src, const void *w_k,
                                    void *k_idx_pool, float *k_idx_scale, void *stream);

/* Workspace bytes an operation needs for this problem (0 on an invalid problem; see dsa_last_error). */
size_t dsa_workspace_bytes(const dsa_problem_t *problem, int32_t op);

const char *dsa_status_str(dsa_status_t status);
const char *dsa_last_error(void);
int32_t dsa_abi_version(void);  /* 1 */

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
