// Exact-order fp64 projections for gfx950: y = x W with every output one fp64 FMA chain over d ascending, then
// rounded once to fp32.  Two products of the indexer run on it:
//   - the indexer query of a token and its head weights, q_I = h W_QI (H_I heads of d_I columns) and w = h W_w
//     (lizeman DSA page section 2, stage 1, and the section 3 sketch; kgptalkie "DeepSeek Sparse Attention
//     explained", "How Does the Lightning Indexer Score a Token?"), each head's d_I values then quantised to e4m3
//     codes with one fp32 scale per (token, head) when the indexer runs in FP8;
//   - the indexer key k_I = c W_KI of a new cache row (kiadev "How DSA works", stage 1), quantised the same way
//     and written through the page table.
// The quantiser: scale = max |y| / 448 over the group (1 for an all-zero group), code = the e4m3 value nearest to
// y / scale, ties to even, clamped to +-448, sign kept.  Both the products (bf16 x bf16 or fp32 x fp32, exact in
// fp64) and the summation order are fixed, so codes and scales are reproducible bit for bit.
//
// Layout of the work.  A block owns one tile of kG (64 or 128) adjacent output columns, which is one or more
// whole quantisation groups, for 256 / kG x kRpt rows: thread t runs the chains of column t % kG for kRpt rows.
// W is streamed in chunks of kKC rows, loaded as 16-byte pieces kP chunks ahead into registers and widened to fp32
// in LDS, so a chain step reads one W entry (lane = column, conflict-free) and one broadcast fp64 x value (the x
// rows are widened to fp64 in LDS once per chunk), converts the W entry and issues one FMA.  For a single row
// wave 0 only computes while waves 1..3 load and widen the chunks; with one chain per thread the kernel is bound by
// the chain (one conversion at half rate plus one dependent FMA per step, d steps); with many rows each thread
// interleaves four chains, shares each conversion among them, and is bound by the fp64 FMA rate.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

struct ProjArgs {
  const void* x;   // [R, K] rows
  const void* wa;  // [K, na]: quantised groups (or plain fp32 outputs when quant == 0)
  const void* wb;  // [K, nb]: plain fp32 outputs (head weights); NULL when nb == 0
  int R, K, na, nb, tiles_a, group_log2, quant;
};

// Query side: q [R, na] codes or fp32, q_scale [R, na >> group_log2], head_w [R, nb].
struct QuerySink {
  void* q;
  float* q_scale;
  float* head_w;
  __device__ void put(const ProjArgs& a, bool in_b, int r, int col, float y, float amax) const {
    if (in_b) {
      head_w[(int64_t)r * a.nb + col] = y;
    } else if (a.quant) {
      const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
      const float v = fminf(fmaxf(y / scale, -448.0f), 448.0f);
      static_cast<uint8_t*>(q)[(int64_t)r * a.na + col] = (uint8_t)e4m3_code(v);
      if ((col & ((1 << a.group_log2) - 1)) == 0)
        q_scale[(int64_t)r * (a.na >> a.group_log2) + (col >> a.group_log2)] = scale;
    } else {
      static_cast<float*>(q)[(int64_t)r * a.na + col] = y;
    }
  }
};

// Key side: row r goes to position positions[r] of sequence row_seq[r] (skipped when negative or beyond the
// page table); one group per key (na == d_I).
struct KeySink {
  const int32_t* positions;
  const int32_t* row_seq;
  const int32_t* page_table;
  int num_seqs, max_pages, num_pages, log2ps;
  void* pool;
  float* pool_scale;
  __device__ void put(const ProjArgs& a, bool, int r, int col, float y, float amax) const {
    const int pos = positions[r];
    if (pos < 0 || (int64_t)pos >= ((int64_t)max_pages << log2ps)) return;
    const int64_t row = phys_row(page_table, max_pages, num_pages, log2ps, clamp_seq(row_seq[r], num_seqs), pos);
    if (a.quant) {
      const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
      const float v = fminf(fmaxf(y / scale, -448.0f), 448.0f);
      static_cast<uint8_t*>(pool)[row * a.na + col] = (uint8_t)e4m3_code(v);
      if (col == 0) pool_scale[row] = scale;
    } else {
      static_cast<float*>(pool)[row * a.na + col] = y;
    }
  }
};


template <bool kBf16, int kG, int kRpt, bool kSolo, int kP, class Sink>
__global__ __launch_bounds__(256) void proj_chain_kernel(ProjArgs a, Sink sink) {
  constexpr int kSlots = 256 / kG, kRB = kSlots * kRpt;
  // kSolo (a single row): wave 0 only computes and waves 1..3 stage every chunk; otherwise every thread stages.
  static_assert(!kSolo || kRpt == 1, "a single row has one chain per thread");
  constexpr int kStagers = kSolo ? 192 : 256;
  constexpr int kKC = (kSolo ? 6144 : 8192) / kG;  // W rows per chunk (24 or 32 KB as fp32)
  constexpr int kE = kBf16 ? 8 : 4;              // elements per 16-byte piece
  constexpr int kEsz = kBf16 ? 2 : 4;
  constexpr int kWRow = kG / kE;                 // pieces per W chunk row
  constexpr int kWPT = kKC * kWRow / kStagers;   // W pieces per staging thread and chunk
  constexpr int kXRow = kKC / kE;                // pieces per x chunk row
  constexpr int kXPieces = kRB * kXRow;
  constexpr int kXPT = (kXPieces + kStagers - 1) / kStagers;
  static_assert(kWPT * kStagers == kKC * kWRow, "whole W pieces per thread");
  __shared__ __attribute__((aligned(16))) float w_lds[2][kKC * kG];     // [d][column], widened to fp32
  __shared__ __attribute__((aligned(16))) double x_lds[2][kRB * kKC];   // [row slot][d], widened to fp64
  __shared__ float amax_lds[kSlots][kRpt][2];

  const int t = threadIdx.x, cl = t % kG, slot = t / kG;
  const int tile = blockIdx.x, r0 = blockIdx.y * kRB;
  const bool in_b = tile >= a.tiles_a;
  const int c0 = (in_b ? tile - a.tiles_a : tile) * kG;
  const int ncols = in_b ? a.nb : a.na;
  const char* w = static_cast<const char*>(in_b ? a.wb : a.wa);
  const char* x = static_cast<const char*>(a.x);
  const int K = a.K, R = a.R;
  const int nchunks = (K + kKC - 1) / kKC;
  const bool stager = t >= 256 - kStagers;       // the same for every lane of a wave
  const int st = (t + kStagers) % 256 % kStagers;  // staging index (wave 0 aliases the last staging wave)

  // Loads of chunk c (clamped to the last chunk, so every address is valid; such copies are never stored).
  // Columns past the matrix reread its last piece and rows past K its last row: both are masked on the way to LDS.
  v4i wr[kP][kWPT];
  v4i xr[kP][kXPT];
  auto issue = [&](int c, v4i (&wv)[kWPT], v4i (&xv)[kXPT]) {
    const int d0 = min(c, nchunks - 1) * kKC;
#pragma unroll
    for (int j = 0; j < kWPT; ++j) {
      const int i = j * kStagers + st, row = i / kWRow, pc = i % kWRow;
      const int gcol = min(c0 + pc * kE, ncols - kE), gd = min(d0 + row, K - 1);
      wv[j] = *reinterpret_cast<const v4i*>(w + ((int64_t)gd * ncols + gcol) * kEsz);
    }
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int i = min(j * kStagers + st, kXPieces - 1), rr = i / kXRow, pc = i % kXRow;
      const int gr = min(r0 + rr, R - 1), gd = min(d0 + pc * kE, K - kE);
      xv[j] = *reinterpret_cast<const v4i*>(x + ((int64_t)gr * K + gd) * kEsz);
    }
  };
  auto store = [&](int c, int b, const v4i (&wv)[kWPT], const v4i (&xv)[kXPT]) {
    const int d0 = c * kKC;
#pragma unroll
    for (int j = 0; j < kWPT; ++j) {
      const int i = j * kStagers + st, row = i / kWRow, pc = i % kWRow;
      const bool live = d0 + row < K;
      float* dst = &w_lds[b][row * kG + pc * kE];
      if constexpr (kBf16) {
        v4f lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = live ? (uint32_t)wv[j][e] : 0u;
          const float f0 = __uint_as_float(u << 16), f1 = __uint_as_float(u & 0xffff0000u);
          if (e < 2) {
            lo[2 * e] = f0;
            lo[2 * e + 1] = f1;
          } else {
            hi[2 * e - 4] = f0;
            hi[2 * e - 3] = f1;
          }
        }
        *reinterpret_cast<v4f*>(dst) = lo;
        *reinterpret_cast<v4f*>(dst + 4) = hi;
      } else {
        const v4i u = live ? wv[j] : v4i{0, 0, 0, 0};
        *reinterpret_cast<v4i*>(dst) = u;
      }
    }
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int i = j * kStagers + st;
      if (kXPieces % kStagers == 0 || i < kXPieces) {
        const int rr = i / kXRow, pc = i % kXRow;
        const bool live = d0 + pc * kE < K;
        double* dst = &x_lds[b][rr * kKC + pc * kE];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = live ? (uint32_t)xv[j][e] : 0u;
          if constexpr (kBf16) {
            *reinterpret_cast<v2d*>(dst + 2 * e) =
                v2d{(double)__uint_as_float(u << 16), (double)__uint_as_float(u & 0xffff0000u)};
          } else {
            dst[e] = (double)__uint_as_float(u);
          }
        }
      }
    }
  };

  double acc[kRpt];
#pragma unroll
  for (int i = 0; i < kRpt; ++i) acc[i] = 0.0;
  const bool active = r0 + slot * kRpt < R;  // the same for every lane of a wave (kG is a multiple of 64)
  // Zero-padded steps past K are fma(0, 0, acc) = acc: a chain that starts at +0 never holds -0.
  auto compute = [&](int b) {
    const float* wl = &w_lds[b][cl];
    const double* xl = &x_lds[b][slot * kRpt * kKC];
    if constexpr (kRpt == 1) {
      // one chain per lane: its step is latency-bound, so the LDS reads of the next 16 steps are issued before
      // the FMAs of the current 16
      constexpr int kU = 16;
      float wv[2][kU];
      v2d xv[2][kU / 2];
      auto fetch = [&](int d, int u) {
#pragma unroll
        for (int e = 0; e < kU; ++e) wv[u][e] = wl[(d + e) * kG];
#pragma unroll
        for (int e = 0; e < kU / 2; ++e) xv[u][e] = *reinterpret_cast<const v2d*>(xl + d + 2 * e);
      };
      fetch(0, 0);
#pragma unroll
      for (int d = 0; d < kKC; d += kU) {
        const int u = (d / kU) & 1;
        if (d + kU < kKC) fetch(d + kU, u ^ 1);
#pragma unroll
        for (int e = 0; e < kU; e += 2) {
          acc[0] = fma(xv[u][e / 2][0], (double)wv[u][e], acc[0]);
          acc[0] = fma(xv[u][e / 2][1], (double)wv[u][e + 1], acc[0]);
        }
      }
      return;
    }
#pragma unroll 16
    for (int d = 0; d < kKC; d += 2) {
      const double w0 = (double)wl[d * kG], w1 = (double)wl[(d + 1) * kG];
#pragma unroll
      for (int i = 0; i < kRpt; ++i) {
        const v2d xv = *reinterpret_cast<const v2d*>(xl + i * kKC + d);
        acc[i] = fma(xv[0], w0, acc[i]);
        acc[i] = fma(xv[1], w1, acc[i]);
      }
    }
  };

  // Every wave issues the loads (wave 0 repeats the last staging wave's addresses when it does not stage), so the
  // loads sit outside any branch and each chunk's data is waited for exactly, kP - 1 chunks of loads staying in
  // flight; only the staging waves convert and write.
  auto step = [&](int c, v4i (&wv)[kWPT], v4i (&xv)[kXPT]) {
    // buffer c & 1 was last read by chunk c - 2, which every wave finished before the previous barrier
    if (stager) store(c, c & 1, wv, xv);
    issue(c + kP, wv, xv);
    lds_barrier();
    if (active) compute(c & 1);
  };
#pragma unroll
  for (int s = 0; s < kP; ++s) issue(s, wr[s], xr[s]);
  int cb = 0;
  for (; cb + kP <= nchunks; cb += kP) {
#pragma unroll
    for (int s = 0; s < kP; ++s) step(cb + s, wr[s], xr[s]);
  }
#pragma unroll
  for (int s = 0; s < kP - 1; ++s)
    if (cb + s < nchunks) step(cb + s, wr[s], xr[s]);

  float y[kRpt], amax[kRpt];
  const int col = c0 + cl;
  const bool col_ok = col < ncols;
#pragma unroll
  for (int i = 0; i < kRpt; ++i) {
    y[i] = (float)acc[i];
    amax[i] = 0.f;
  }
  if (!in_b && a.quant) {  // the same for the whole block
    const int gsz = 1 << a.group_log2;
#pragma unroll
    for (int i = 0; i < kRpt; ++i) {
      float m = col_ok ? fabsf(y[i]) : 0.f;
      for (int off = 1; off < min(gsz, 64); off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
      amax[i] = m;
    }
    if (gsz > 64) {  // a 128-column group spans the two waves of a row slot
      const int half = cl >> 6;
      if ((t & 63) == 0)
#pragma unroll
        for (int i = 0; i < kRpt; ++i) amax_lds[slot][i][half] = amax[i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kRpt; ++i) amax[i] = fmaxf(amax_lds[slot][i][0], amax_lds[slot][i][1]);
    }
  }
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < kRpt; ++i) {
    const int r = r0 + slot * kRpt + i;
    if (r < R) sink.put(a, in_b, r, col, y[i], amax[i]);
  }
}

template <bool kBf16, int kG, class Sink>
hipError_t launch_g(const ProjArgs& a, const Sink& sink, hipStream_t stream) {
  constexpr int kSlots = 256 / kG, kP = kBf16 ? 4 : 2;
  const int tiles = a.tiles_a + (a.nb + kG - 1) / kG;
  // one chain per thread while the grid still has under four blocks per CU, four otherwise
  const bool few = (int64_t)tiles * ((a.R + kSlots - 1) / kSlots) <= 1024;
  if (a.R == 1) {
    proj_chain_kernel<kBf16, kG, 1, true, kP, Sink><<<dim3(tiles, 1), 256, 0, stream>>>(a, sink);
  } else if (few) {
    const dim3 grid(tiles, (a.R + kSlots - 1) / kSlots);
    proj_chain_kernel<kBf16, kG, 1, false, kP, Sink><<<grid, 256, 0, stream>>>(a, sink);
  } else {
    const dim3 grid(tiles, (a.R + 4 * kSlots - 1) / (4 * kSlots));
    proj_chain_kernel<kBf16, kG, 4, false, kP, Sink><<<grid, 256, 0, stream>>>(a, sink);
  }
  return hipGetLastError();
}

template <class Sink>
hipError_t launch_proj(ProjArgs a, const Sink& sink, bool bf16, int kG, hipStream_t stream) {
  a.tiles_a = (a.na + kG - 1) / kG;
  if (bf16)
    return kG == 64 ? launch_g<true, 64>(a, sink, stream) : launch_g<true, 128>(a, sink, stream);
  return kG == 64 ? launch_g<false, 64>(a, sink, stream) : launch_g<false, 128>(a, sink, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
int log2_exact(int v) { return (v > 0 && (v & (v - 1)) == 0) ? __builtin_ctz((unsigned)v) : -1; }

}  // namespace

const char* query_proj_unsupported(int d_model, int H_I, int d_I, bool bf16, const void* h, const void* w_q,
                                   const void* w_w) {
  const int e = bf16 ? 8 : 4;
  if (log2_exact(d_I) < 0 || d_I < e || d_I > 128) return "idx_dim must be a power of two in 8..128 (4..128 fp32)";
  if (H_I % e != 0 || H_I > 128) return "idx_heads must be a multiple of 8 (4 for fp32) and at most 128";
  if (d_model % e != 0) return "d_model must be a multiple of 8 (4 for fp32)";
  if (!aligned16(h) || !aligned16(w_q) || !aligned16(w_w)) return "h, w_q and w_w must be 16-byte aligned";
  return nullptr;
}

hipError_t launch_query_proj(int R, int d_model, int H_I, int d_I, bool bf16, bool f8, const void* h,
                             const void* w_q, const void* w_w, void* q, float* q_scale, float* head_w,
                             hipStream_t stream) {
  if (R == 0) return hipSuccess;
  ProjArgs a{h, w_q, w_w, R, d_model, H_I * d_I, H_I, 0, log2_exact(d_I), f8 ? 1 : 0};
  const int kG = d_I > 64 || H_I > 64 ? 128 : 64;
  return launch_proj(a, QuerySink{q, q_scale, head_w}, bf16, kG, stream);
}

bool key_proj_supported(const Geo& g, const void* src, const void* w) {
  const bool bf16 = g.kv_dtype == 1 /* BF16 */;
  const int e = bf16 ? 8 : 4;
  return log2_exact(g.d_I) >= 0 && g.d_I >= e && g.d_I <= 128 && g.d_c % e == 0 && aligned16(src) &&
         aligned16(w);
}

hipError_t launch_key_proj(const Geo& g, const int32_t* positions, const void* src, const void* w, void* pool,
                           float* pool_scale, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  ProjArgs a{src, w, nullptr, g.R, g.d_c, g.d_I, 0, 0, log2_exact(g.d_I), g.idx_dtype == 2 /* F8E4M3 */};
  const KeySink sink{positions, g.row_seq, g.page_table, g.S, g.max_pages, g.num_pages, g.log2ps, pool,
                     pool_scale};
  return launch_proj(a, sink, g.kv_dtype == 1, g.d_I > 64 ? 128 : 64, stream);
}

}  // namespace dsa
