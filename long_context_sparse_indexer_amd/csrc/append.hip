// Indexer-key append for gfx950: the cache write that precedes the scoring step.  Each new token's indexer key
// is its latent row times the key projection, k_I = c W_KI (kiadev "How DSA works", stage 1), and the indexer
// cache keeps it as d_I e4m3 codes plus one fp32 scale (kgptalkie "DeepSeek Sparse Attention explained",
// "What Does the GPU Actually Run?"), or as fp32 in an fp32 cache.
//
// Scale and codes: scale = max_j |k_j| / 448, the largest e4m3 magnitude (1 for a zero key); code_j = the e4m3
// value nearest to k_j / scale, ties to the even code, clamped to +-448, sign bit kept.  These are integers
// decided by floating point, so every step is fixed: each product c_d w_dj of bf16 or fp32 operands is exact in
// fp64, each output sums them in fp64 over d ascending (one FMA chain), the sum is rounded once to fp32, and the
// scale and k_j / scale are IEEE fp32 divisions.  The codes are then reproducible bit for bit.
//
// The work is d_c x d_I multiply-adds per token (64 K for the shipped 512 x 128): at decode batch sizes the
// kernel is bound by the latency of its 512-step FMA chains, for long prefill chunks by the fp64 FMA rate.  A
// block of 256 threads covers all d_I columns (two 128-column or four 64-column groups) for one token per group
// and thread when the tokens fit one block per CU, and four otherwise (four independent chains per thread).
// The latent rows are staged in LDS as fp64 (exact), W_KI as bf16 when it is bf16 with d_c <= 512, so the chain
// loop reads only LDS.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kStageMaxDc = 512;     // W_KI staged in LDS up to this latent width (bf16)
constexpr int kGlobalMaxDc = 1024;   // latent width of the unstaged path

// kMode 0: the keys arrive as fp32 (no projection).  1: bf16 latent rows and W_KI, W_KI staged in LDS (d_c <= 512,
// d_I == kCols, 16-byte aligned rows).  2: latent rows and W_KI in the latent dtype, W_KI read from global memory.
// A thread runs kRpt chains (tokens) for one column; kRpt = 1 spreads few tokens over more blocks.
template <int kMode, int kCols, int kRpt>
__global__ __launch_bounds__(256) void key_append_kernel(
    const void* __restrict__ src, const void* __restrict__ w, int c_bf16, int R, int d_c, int d_I,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ page_table, int num_seqs, int max_pages, int num_pages, int log2ps, int pool_f8,
    void* __restrict__ pool, float* __restrict__ pool_scale) {
  constexpr int kGroups = 256 / kCols, kRpb = kGroups * kRpt;
  constexpr int kMaxDc = kMode == 1 ? kStageMaxDc : kGlobalMaxDc;
  // latent rows of the block's tokens as fp64, [token slot][d]; after the chains the same memory holds the
  // per-wave key maxima
  __shared__ __attribute__((aligned(16))) double c_lds[kMode == 0 ? 8 : kMaxDc * kRpb];
  __shared__ __attribute__((aligned(16))) unsigned short w_lds[kMode == 1 ? kStageMaxDc * kCols : 8];  // [d][col]
  static_assert(kMode == 0 || kMaxDc * kRpb >= 2 * 4 * kRpt, "room for the maxima");
  float* amax_lds = reinterpret_cast<float*>(c_lds);  // [wave][token of the thread]
  const int t = threadIdx.x, col = t % kCols, grp = t / kCols, lane = t & 63, wave = t >> 6;
  const int r0 = blockIdx.x * kRpb;
  float k[kRpt];

  if constexpr (kMode == 0) {
    const float* x = static_cast<const float*>(src);
#pragma unroll
    for (int i = 0; i < kRpt; ++i) {
      const int r = r0 + grp * kRpt + i;
      k[i] = r < R && col < d_I ? x[(int64_t)r * d_I + col] : 0.f;
    }
  } else {
    if constexpr (kMode == 1) {
      // W_KI [d_c, kCols] bf16 is contiguous: 16-byte pieces, up to 32 per thread in flight at a time (the
      // loads are unconditional, past the end they reread the last piece, so no branch splits them)
      constexpr int kRound = kRpt == 1 ? 32 : 16;
      const v4i* wg = static_cast<const v4i*>(w);
      const int n16 = d_c * kCols / 8;
      for (int b = 0; b < n16; b += kRound * 256) {
        v4i buf[kRound];
#pragma unroll
        for (int j = 0; j < kRound; ++j) buf[j] = wg[min(b + j * 256 + t, n16 - 1)];
#pragma unroll
        for (int j = 0; j < kRound; ++j)
          if (b + j * 256 + t < n16) *reinterpret_cast<v4i*>(&w_lds[(b + j * 256 + t) * 8]) = buf[j];
      }
      // latent rows: 8 bf16 per 16-byte piece, every piece of the thread loaded before any is stored
      constexpr int kPieces = (kRpb * kStageMaxDc / 8 + 255) / 256;
      const int per_row = d_c / 8, np = kRpb * per_row;
      v8us cp[kPieces];
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        // unconditional loads (clamped to the last token's last piece); pieces of absent tokens become zero
        const int i = min(j * 256 + t, np - 1), rs = i / per_row, r = r0 + rs;
        const int64_t off = (int64_t)min(r, R - 1) * d_c + (i - rs * per_row) * 8;
        const v8us v = *reinterpret_cast<const v8us*>(static_cast<const unsigned short*>(src) + off);
        cp[j] = r < R ? v : v8us{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int i = j * 256 + t;
        if (i < np)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            *reinterpret_cast<v2d*>(&c_lds[i * 8 + e]) =
                v2d{(double)bf16_bits_to_float(cp[j][e]), (double)bf16_bits_to_float(cp[j][e + 1])};
      }
    } else {
      for (int i = t; i < kRpb * d_c; i += 256) {
        const int rs = i / d_c, d = i - rs * d_c, r = r0 + rs;
        float v = 0.f;
        if (r < R) {
          const int64_t e = (int64_t)r * d_c + d;
          v = c_bf16 ? bf16_bits_to_float(static_cast<const unsigned short*>(src)[e])
                     : static_cast<const float*>(src)[e];
        }
        c_lds[rs * d_c + d] = (double)v;
      }
    }
    __syncthreads();
    double acc[kRpt];
#pragma unroll
    for (int i = 0; i < kRpt; ++i) acc[i] = 0.0;
    const double* cl = c_lds + grp * kRpt * d_c;  // token i of the thread at cl + i * d_c
    if constexpr (kMode == 1) {
      // steps of 8: the next step's W column entries and latent values are read from LDS while the current
      // step's FMAs run (d_c is a multiple of 8)
      float wv[2][8];
      double cv[2][kRpt][8];
      auto fetch = [&](int d, int b) {
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[b][e] = bf16_bits_to_float(w_lds[(d + e) * kCols + col]);
#pragma unroll
        for (int i = 0; i < kRpt; ++i)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const v2d p = *reinterpret_cast<const v2d*>(&cl[i * d_c + d + e]);
            cv[b][i][e] = p[0];
            cv[b][i][e + 1] = p[1];
          }
      };
      if (col < d_I) {
        fetch(0, 0);
        for (int d = 0; d < d_c; d += 16) {
          if (d + 8 < d_c) fetch(d + 8, 1);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < kRpt; ++i) acc[i] = fma(cv[0][i][e], (double)wv[0][e], acc[i]);
          if (d + 8 >= d_c) break;
          if (d + 16 < d_c) fetch(d + 16, 0);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < kRpt; ++i) acc[i] = fma(cv[1][i][e], (double)wv[1][e], acc[i]);
        }
      }
    } else if (col < d_I) {
      for (int d = 0; d < d_c; ++d) {
        const int64_t e = (int64_t)d * d_I + col;
        const float wv = c_bf16 ? bf16_bits_to_float(static_cast<const unsigned short*>(w)[e])
                                : static_cast<const float*>(w)[e];
#pragma unroll
        for (int i = 0; i < kRpt; ++i) acc[i] = fma(cl[i * d_c + d], (double)wv, acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kRpt; ++i) k[i] = (float)acc[i];
    if (pool_f8) __syncthreads();  // the maxima below reuse the latent rows' memory
  }

  // largest magnitude of each token's key: over the wave, then over the group's waves (two when kCols = 128)
  if (pool_f8) {
#pragma unroll
    for (int i = 0; i < kRpt; ++i) {
      const float m = wave_max(fabsf(k[i]));
      if (lane == 0) amax_lds[wave * kRpt + i] = m;
    }
    __syncthreads();
  }
  const int64_t cap = (int64_t)max_pages << log2ps;
#pragma unroll
  for (int i = 0; i < kRpt; ++i) {
    const int r = r0 + grp * kRpt + i;
    if (r >= R || col >= d_I) continue;
    const int pos = positions[r];
    if (pos < 0 || pos >= cap) continue;
    const int64_t row = phys_row(page_table, max_pages, num_pages, log2ps, clamp_seq(row_seq[r], num_seqs), pos);
    if (pool_f8) {
      const float amax = kCols == 128 ? fmaxf(amax_lds[2 * grp * kRpt + i], amax_lds[(2 * grp + 1) * kRpt + i])
                                      : amax_lds[grp * kRpt + i];
      const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
      const float y = fminf(fmaxf(k[i] / scale, -448.0f), 448.0f);
      static_cast<uint8_t*>(pool)[row * d_I + col] = (uint8_t)e4m3_code(y);
      if (col == 0) pool_scale[row] = scale;
    } else {
      static_cast<float*>(pool)[row * d_I + col] = k[i];
    }
  }
}

template <int kCols, int kRpt>
hipError_t launch_cols(const Geo& g, const int32_t* positions, const void* src, const void* w, int mode, void* pool,
                       float* pool_scale, hipStream_t stream) {
  constexpr int kRpb = 256 / kCols * kRpt;
  const int blocks = (g.R + kRpb - 1) / kRpb;
  const int c_bf16 = g.kv_dtype == 1 /* BF16 */;
  const int f8 = g.idx_dtype == 2 /* F8E4M3 */;
#define DSA_APPEND_ARGS                                                                                        \
  src, w, c_bf16, g.R, g.d_c, g.d_I, positions, g.row_seq, g.page_table, g.S, g.max_pages, g.num_pages, g.log2ps, \
      f8, pool, pool_scale
  switch (mode) {
    case 0: key_append_kernel<0, kCols, kRpt><<<blocks, 256, 0, stream>>>(DSA_APPEND_ARGS); break;
    case 1: key_append_kernel<1, kCols, kRpt><<<blocks, 256, 0, stream>>>(DSA_APPEND_ARGS); break;
    default: key_append_kernel<2, kCols, kRpt><<<blocks, 256, 0, stream>>>(DSA_APPEND_ARGS); break;
  }
#undef DSA_APPEND_ARGS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_key_append(const Geo& g, const int32_t* positions, const void* src, const void* w, void* pool,
                             float* pool_scale, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  const int cols = g.d_I <= 64 ? 64 : 128;
  int mode = 0;
  if (w) {
    const bool stage = g.kv_dtype == 1 && g.d_c <= kStageMaxDc && g.d_c % 8 == 0 && g.d_I == cols &&
                       ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(src)) & 15) == 0;
    mode = stage ? 1 : 2;
  }
  // one chain per thread while that still fits the tokens in one block per CU, else four
  const bool few = (g.R + 256 / cols - 1) / (256 / cols) <= 256;
  if (cols == 64)
    return few ? launch_cols<64, 1>(g, positions, src, w, mode, pool, pool_scale, stream)
               : launch_cols<64, 4>(g, positions, src, w, mode, pool, pool_scale, stream);
  return few ? launch_cols<128, 1>(g, positions, src, w, mode, pool, pool_scale, stream)
             : launch_cols<128, 4>(g, positions, src, w, mode, pool, pool_scale, stream);
}

int key_append_max_latent_dim() { return kGlobalMaxDc; }

}  // namespace dsa
