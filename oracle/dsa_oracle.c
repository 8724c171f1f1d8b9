/*
 * dsa_oracle.c -- plain fp64 CPU reference of the DeepSeek Sparse Attention (DSA) decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  It shares no source, header, table or helper with the GPU library and includes
 * nothing from it.  It is deliberately slow: every value is decoded to fp64 and every sum is a plain loop.
 *
 * What it computes, and where the pages define it:
 *   1. Element decoding.  The indexer operands are FP8 ("the whole scorer runs in FP8", DeepSeek Sparse
 *      Attention explained, "How Does the Lightning Indexer Score a Token?"; "float8_e4m3" in "What Does
 *      the GPU Actually Run?") with one fp32 scale per stored 64-vector ("128 FP8 numbers and one scale per
 *      token", same section).  The format is OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN.
 *      The latent cache and attention queries are BF16 ("attended over, in full BF16 precision",
 *      "What Does the Whole Block Look Like?").  fp32 inputs are taken as they are.
 *   2. Indexer score (same pages, "How Does the Lightning Indexer Score a Token?"; milos-mitrovic,
 *      "How Does the Lightning Indexer Pick Which Tokens Matter?"; lizeman DSA page section 2, stage 1):
 *      for every visible position s, each indexer head j takes the dot product of its query q_I[j] with
 *      the position's single shared key k_I[s]; the result goes through a ReLU; the H_I results are summed
 *      with the head weights w[j], which carry no sign constraint:
 *          I[s] = sum_j w[j] * max(0, <q_I[j], k_I[s]>),   q_I = sq * decode(q8), k_I = sk * decode(k8).
 *   3. Selection ("How Does the Selector Pick 1,024?"): sort the scores, keep the highest
 *      k_eff = min(k, n) positions (a short context is read in full).  Equal scores are ordered by
 *      position, lowest first.
 *   4. Sparse attention in MQA mode (lizeman section 2, stage 2; kiadev "How DSA works"; "What Does the
 *      Whole Block Look Like?"): every query head attends with an ordinary softmax over only the selected
 *      latent rows, which serve as both key and value:
 *          l_i = scale * <q[h], c[T_i]>,  p = softmax(l),  o[h] = sum_i p_i c[T_i],  lse[h] = log sum exp l.
 *      An empty selection gives o = 0 and lse = -inf.
 *   5. Indexer-key append, the cache write before the step (kiadev "How DSA works", stage 1: the key
 *      projection W_KI in R^{d_c x d_I} maps each cached latent row c to k_I = c W_KI; kgptalkie "What Does
 *      the GPU Actually Run?": the indexer cache holds the key's FP8 numbers and one scale per token).
 *      Reading (the pages fix one fp32 scale per key but not how it is chosen): max-abs scaling over the
 *      whole e4m3 range, scale = max_j |k_j| / 448 (1 for an all-zero key), code_j = the e4m3 value nearest
 *      to k_j / scale, ties to the even code, clamped to +-448; the code keeps the sign bit of k_j / scale.
 *      The code is an integer decided by floating point, so the decision is taken in fp32: the key is
 *      rounded once to fp32, then scale = amax / 448 and k_j / scale are IEEE fp32 divisions.  The
 *      projection is the plain fp64 sum over d = 0 .. d_c-1 of exact products (bf16 or fp32 operands).
 *   5b. Indexer-query projection, the other input of the scorer (lizeman DSA page section 2, stage 1: W_{Q_I} in
 *      R^{d_model x d_I} maps the token's hidden state h_t to q_I = h_t W_{Q_I}; kgptalkie "How Does the Lightning
 *      Indexer Score a Token?": the new token is projected into H_I query vectors plus H_I head weights).  Readings:
 *      W_QI is [d_model, H_I * d_I] (head j owns columns j d_I .. j d_I + d_I - 1) and the head weights are a
 *      second projection w = h W_w with W_w in R^{d_model x H_I}; both sums are the plain fp64 sum over d
 *      ascending of exact products, rounded once to fp32 (as for the key); each head's d_I-vector is then
 *      quantised like a key (max-abs scale, nearest e4m3 code) when the indexer runs in FP8.
 *   6. Sparse attention over the FP8 latent cache ("What Does the GPU Actually Run?": each token's entry is 656
 *      bytes, 512 values in float8_e4m3, 4 fp32 scale factors and the 64 RoPE numbers kept in bf16; "Why Is
 *      Decoding Held Back by Memory?": one 576-number entry per token).  Readings: the parts lie in that order
 *      (codes at bytes 0..511, scales at 512..527, RoPE at 528..655); scale t covers values 128t .. 128t+127;
 *      the key of a position is the 576-vector [c ; r] (dequantised latent, RoPE part) and its value is c, so
 *      with a 576-wide query q = [q_c ; q_r]:
 *          l_i = scale * (<q_c, c[T_i]> + <q_r, r[T_i]>),  o = sum_i softmax(l)_i c[T_i]  (512 wide).
 *   Cached positions are addressed through a page table: physical row = table[seq][pos / P] * P + pos % P
 *   (the selected positions are "an address list into the paged KV cache", "How Does the Selector Pick").
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F8E4M3 = 2 };

/* Threads an OpenMP parallel region of this library uses (reported beside its timings). */
int dsa_oracle_threads(void) { return omp_get_max_threads(); }

/* ---- 1. element decoding ------------------------------------------------------------------------- */

double dsa_oracle_e4m3_value(uint8_t code) {
  int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return sign ? -mag : mag;
}

double dsa_oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void *base, int dtype, int64_t i) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[i];
    case ORACLE_BF16: return dsa_oracle_bf16_value(((const uint16_t *)base)[i]);
    default: return dsa_oracle_e4m3_value(((const uint8_t *)base)[i]);
  }
}

void dsa_oracle_decode(const void *src, int32_t dtype, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = elem(src, dtype, i);
}

static int64_t phys_row(const int32_t *page_table, int32_t max_pages, int32_t page_size, int32_t seq, int64_t pos) {
  return (int64_t)page_table[(int64_t)seq * max_pages + pos / page_size] * page_size + pos % page_size;
}

/* ---- 2. indexer score ---------------------------------------------------------------------------- */

int dsa_oracle_indexer_scores(int32_t R, int32_t H_I, int32_t d_I, int32_t idx_dtype,
                              const void *q_idx, const float *q_idx_scale, const float *head_w,
                              const void *k_idx_pool, const float *k_idx_scale,
                              const int32_t *row_seq, const int32_t *row_len, const int32_t *page_table,
                              int32_t max_pages, int32_t page_size, double *scores, int64_t ld) {
  if (R < 0 || H_I <= 0 || d_I <= 0 || d_I > 1024 || page_size <= 0) return 1;
  for (int32_t r = 0; r < R; ++r) {
    const int64_t n = row_len[r];
    /* dequantised indexer queries of this row */
    double *q = (double *)malloc(sizeof(double) * (size_t)H_I * d_I);
    if (!q) return 2;
    for (int32_t j = 0; j < H_I; ++j) {
      double sq = q_idx_scale ? (double)q_idx_scale[(int64_t)r * H_I + j] : 1.0;
      for (int32_t d = 0; d < d_I; ++d) q[j * d_I + d] = sq * elem(q_idx, idx_dtype, ((int64_t)r * H_I + j) * d_I + d);
    }
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < n; ++s) {
      const int64_t p = phys_row(page_table, max_pages, page_size, row_seq[r], s);
      const double sk = k_idx_scale ? (double)k_idx_scale[p] : 1.0;
      double kv[1024];
      for (int32_t d = 0; d < d_I; ++d) kv[d] = sk * elem(k_idx_pool, idx_dtype, p * d_I + d);
      double score = 0.0;
      for (int32_t j = 0; j < H_I; ++j) {
        double dot = 0.0;
        for (int32_t d = 0; d < d_I; ++d) dot += q[j * d_I + d] * kv[d];
        score += (double)head_w[(int64_t)r * H_I + j] * (dot > 0.0 ? dot : 0.0);
      }
      scores[(int64_t)r * ld + s] = score;
    }
    free(q);
  }
  return 0;
}

/* ---- 3. selection -------------------------------------------------------------------------------- */

typedef struct { double score; int64_t pos; } scored_pos;

static int by_score_then_position(const void *a, const void *b) {
  const scored_pos *x = (const scored_pos *)a, *y = (const scored_pos *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

int dsa_oracle_topk(int32_t R, int32_t k, const int32_t *row_len, const double *scores, int64_t ld,
                    int32_t *topk_idx, double *kth_score) {
  if (R < 0 || k <= 0) return 1;
  for (int32_t r = 0; r < R; ++r) {
    const int64_t n = row_len[r];
    const int64_t keff = n < k ? n : k;
    scored_pos *all = (scored_pos *)malloc(sizeof(scored_pos) * (size_t)(n > 0 ? n : 1));
    if (!all) return 2;
    for (int64_t s = 0; s < n; ++s) { all[s].score = scores[(int64_t)r * ld + s]; all[s].pos = s; }
    qsort(all, (size_t)n, sizeof(scored_pos), by_score_then_position);
    for (int64_t i = 0; i < k; ++i) topk_idx[(int64_t)r * k + i] = i < keff ? (int32_t)all[i].pos : -1;
    if (kth_score) kth_score[r] = keff > 0 ? all[keff - 1].score : NAN;
    free(all);
  }
  return 0;
}

/* ---- 4. sparse attention over the selected latent rows ------------------------------------------ */

int dsa_oracle_sparse_attn(int32_t R, int32_t H, int32_t d_c, int32_t kv_dtype, const void *q, const void *kv_pool,
                           const int32_t *topk_idx, int32_t k, const int32_t *row_seq, const int32_t *page_table,
                           int32_t max_pages, int32_t page_size, double scale, double *out, double *lse) {
  if (R < 0 || H <= 0 || d_c <= 0 || k <= 0 || page_size <= 0) return 1;
  for (int32_t r = 0; r < R; ++r) {
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)k);
    if (!rows) return 2;
    int32_t m = 0;
    for (int32_t i = 0; i < k; ++i) {
      int32_t pos = topk_idx[(int64_t)r * k + i];
      if (pos >= 0) rows[m++] = phys_row(page_table, max_pages, page_size, row_seq[r], pos);
    }
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
      double *o = out + ((int64_t)r * H + h) * d_c;
      for (int32_t d = 0; d < d_c; ++d) o[d] = 0.0;
      if (m == 0) { lse[(int64_t)r * H + h] = -INFINITY; continue; }
      double *logit = (double *)malloc(sizeof(double) * (size_t)m);
      double mx = -INFINITY;
      for (int32_t i = 0; i < m; ++i) {
        double dot = 0.0;
        for (int32_t d = 0; d < d_c; ++d)
          dot += elem(q, kv_dtype, ((int64_t)r * H + h) * d_c + d) * elem(kv_pool, kv_dtype, rows[i] * d_c + d);
        logit[i] = scale * dot;
        if (logit[i] > mx) mx = logit[i];
      }
      double z = 0.0;
      for (int32_t i = 0; i < m; ++i) { logit[i] = exp(logit[i] - mx); z += logit[i]; }
      for (int32_t i = 0; i < m; ++i) {
        double p = logit[i] / z;
        for (int32_t d = 0; d < d_c; ++d) o[d] += p * elem(kv_pool, kv_dtype, rows[i] * d_c + d);
      }
      lse[(int64_t)r * H + h] = mx + log(z);
      free(logit);
    }
    free(rows);
  }
  return 0;
}

/* ---- 5. indexer-key append ----------------------------------------------------------------------- */

/* The e4m3 code nearest to y: every finite non-negative code is tried and the closest value to |y| kept,
 * ties going to the code with an even mantissa (the even code of the two).  For an fp32 y every distance
 * near a midpoint is exact in fp64.  |y| above 448 takes 448; the sign bit of y is kept, so a negative value
 * that rounds to zero gives 0x80. */
uint8_t dsa_oracle_e4m3_nearest(float y) {
  double a = fabs((double)y);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(a - dsa_oracle_e4m3_value((uint8_t)c));
    if (d < best_d || (d == best_d && (c & 1) == 0)) { best = c; best_d = d; }
  }
  return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* One key vector of d fp32 values -> d codes and its scale (the reading of section 5 above). */
void dsa_oracle_quantize_key(int32_t d, const float *x, uint8_t *codes, float *scale) {
  float amax = 0.0f;
  for (int32_t j = 0; j < d; ++j) if (fabsf(x[j]) > amax) amax = fabsf(x[j]);
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int32_t j = 0; j < d; ++j) {
    float y = x[j] / s;
    if (y > 448.0f) y = 448.0f;
    if (y < -448.0f) y = -448.0f;
    codes[j] = dsa_oracle_e4m3_nearest(y);
  }
  *scale = s;
}

/* k[r][j] = sum_d c[r][d] * w[d][j] in fp64, d ascending; c [R, d_c] and w [d_c, d_I] in c_dtype. */
int dsa_oracle_key_projection(int32_t R, int32_t d_c, int32_t d_I, int32_t c_dtype, const void *c, const void *w,
                              double *k) {
  if (R < 0 || d_c <= 0 || d_I <= 0 || c_dtype == ORACLE_F8E4M3) return 1;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t j = 0; j < d_I; ++j) {
      double sum = 0.0;
      for (int32_t d = 0; d < d_c; ++d)
        sum += elem(c, c_dtype, (int64_t)r * d_c + d) * elem(w, c_dtype, (int64_t)d * d_I + j);
      k[(int64_t)r * d_I + j] = sum;
    }
  return 0;
}

/* Writes the key of row r at position positions[r] of sequence row_seq[r] (rows with a negative position, or
 * one the page table cannot reach, at or beyond max_pages * page_size, are skipped): fp32 keys k32 [R, d_I] go to the pool as e4m3 codes plus a scale (pool_dtype F8E4M3) or as they are
 * (F32, no scales).  Pool rows no row addresses are left untouched. */
int dsa_oracle_key_append(int32_t R, int32_t d_I, const float *k32, const int32_t *positions, const int32_t *row_seq,
                          const int32_t *page_table, int32_t max_pages, int32_t page_size, int32_t pool_dtype,
                          void *pool, float *pool_scale) {
  if (R < 0 || d_I <= 0 || page_size <= 0 || (pool_dtype != ORACLE_F8E4M3 && pool_dtype != ORACLE_F32)) return 1;
  for (int32_t r = 0; r < R; ++r) {
    if (positions[r] < 0 || (int64_t)positions[r] >= (int64_t)max_pages * page_size) continue;
    int64_t row = phys_row(page_table, max_pages, page_size, row_seq[r], positions[r]);
    const float *x = k32 + (int64_t)r * d_I;
    if (pool_dtype == ORACLE_F8E4M3)
      dsa_oracle_quantize_key(d_I, x, (uint8_t *)pool + row * d_I, pool_scale + row);
    else
      memcpy((float *)pool + row * d_I, x, sizeof(float) * (size_t)d_I);
  }
  return 0;
}

/* ---- 5b. indexer-query projection ------------------------------------------------------------------ */

/* q_I and head weights of R tokens from their hidden states h [R, d_model] (h_dtype BF16 or F32), W_QI
 * [d_model, H_I * d_I] and W_w [d_model, H_I] in the same dtype.  idx_dtype F8E4M3: q_out receives [R, H_I, d_I]
 * e4m3 codes and q_scale [R, H_I] one scale per head vector; F32: q_out receives the fp32 values and q_scale is not
 * written.  head_w [R, H_I] fp32. */
int dsa_oracle_query_projection(int32_t R, int32_t d_model, int32_t H_I, int32_t d_I, int32_t h_dtype, const void *h,
                                const void *w_q, const void *w_w, int32_t idx_dtype, void *q_out, float *q_scale,
                                float *head_w) {
  if (R < 0 || d_model <= 0 || H_I <= 0 || d_I <= 0 || (idx_dtype != ORACLE_F8E4M3 && idx_dtype != ORACLE_F32))
    return 1;
  const int32_t nq = H_I * d_I;
  double *q = (double *)malloc(sizeof(double) * ((size_t)R * nq + (size_t)R * H_I));
  if (!q) return 2;
  double *w = q + (size_t)R * nq;
  int rc = dsa_oracle_key_projection(R, d_model, nq, h_dtype, h, w_q, q);
  if (!rc) rc = dsa_oracle_key_projection(R, d_model, H_I, h_dtype, h, w_w, w);
  if (!rc) {
    float *x = (float *)malloc(sizeof(float) * (size_t)d_I);
    if (!x) rc = 2;
    for (int32_t r = 0; !rc && r < R; ++r) {
      for (int32_t j = 0; j < H_I; ++j) {
        const double *v = q + (size_t)r * nq + (size_t)j * d_I;
        for (int32_t e = 0; e < d_I; ++e) x[e] = (float)v[e];
        const size_t o = (size_t)r * nq + (size_t)j * d_I;
        if (idx_dtype == ORACLE_F8E4M3)
          dsa_oracle_quantize_key(d_I, x, (uint8_t *)q_out + o, q_scale + (size_t)r * H_I + j);
        else
          memcpy((float *)q_out + o, x, sizeof(float) * (size_t)d_I);
        head_w[(size_t)r * H_I + j] = (float)w[(size_t)r * H_I + j];
      }
    }
    free(x);
  }
  free(q);
  return rc;
}

/* ---- 6. sparse attention over the FP8 latent cache ------------------------------------------------- */

enum { F8_ENTRY = 656, F8_LATENT = 512, F8_ROPE = 64, F8_TILE = 128 };

/* Dequantised 576-wide key of one cache entry: the 512 latent values code * scale[tile], then the 64 RoPE values. */
void dsa_oracle_fp8_entry_key(const uint8_t *entry, double *key) {
  for (int d = 0; d < F8_LATENT; ++d) {
    float sc;
    memcpy(&sc, entry + F8_LATENT + 4 * (d / F8_TILE), sizeof sc);
    key[d] = dsa_oracle_e4m3_value(entry[d]) * (double)sc;
  }
  for (int d = 0; d < F8_ROPE; ++d) {
    uint16_t b;
    memcpy(&b, entry + F8_LATENT + 16 + 2 * d, sizeof b);
    key[F8_LATENT + d] = dsa_oracle_bf16_value(b);
  }
}

/* q [R, H, 576] bf16; pool [rows, 656] bytes; out [R, H, 512] and lse [R, H] in fp64.  Entries < 0 of topk_idx are
 * ignored; an empty selection gives o = 0 and lse = -inf. */
int dsa_oracle_sparse_attn_fp8(int32_t R, int32_t H, const uint16_t *q, const uint8_t *pool, const int32_t *topk_idx,
                               int32_t k, const int32_t *row_seq, const int32_t *page_table, int32_t max_pages,
                               int32_t page_size, double scale, double *out, double *lse) {
  const int KD = F8_LATENT + F8_ROPE;
  if (R < 0 || H <= 0 || k <= 0 || page_size <= 0) return 1;
  for (int32_t r = 0; r < R; ++r) {
    double *keys = (double *)malloc(sizeof(double) * (size_t)k * KD);
    if (!keys) return 2;
    int32_t m = 0;
    for (int32_t i = 0; i < k; ++i) {
      int32_t pos = topk_idx[(int64_t)r * k + i];
      if (pos < 0) continue;
      int64_t row = phys_row(page_table, max_pages, page_size, row_seq[r], pos);
      dsa_oracle_fp8_entry_key(pool + row * F8_ENTRY, keys + (int64_t)m * KD);
      ++m;
    }
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
      double *o = out + ((int64_t)r * H + h) * F8_LATENT;
      for (int32_t d = 0; d < F8_LATENT; ++d) o[d] = 0.0;
      if (m == 0) { lse[(int64_t)r * H + h] = -INFINITY; continue; }
      const uint16_t *qh = q + ((int64_t)r * H + h) * KD;
      double *logit = (double *)malloc(sizeof(double) * (size_t)m);
      double mx = -INFINITY;
      for (int32_t i = 0; i < m; ++i) {
        double dot = 0.0;
        for (int32_t d = 0; d < KD; ++d) dot += dsa_oracle_bf16_value(qh[d]) * keys[(int64_t)i * KD + d];
        logit[i] = scale * dot;
        if (logit[i] > mx) mx = logit[i];
      }
      double z = 0.0;
      for (int32_t i = 0; i < m; ++i) { logit[i] = exp(logit[i] - mx); z += logit[i]; }
      for (int32_t i = 0; i < m; ++i) {
        double p = logit[i] / z;
        for (int32_t d = 0; d < F8_LATENT; ++d) o[d] += p * keys[(int64_t)i * KD + d];
      }
      lse[(int64_t)r * H + h] = mx + log(z);
      free(logit);
    }
    free(keys);
  }
  return 0;
}
