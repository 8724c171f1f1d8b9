// Lightning-indexer scores on gfx950.
//
// Per visible position s of row r:  I[r][s] = sum_j w[r][j] * max(0, <q_I[r][j], k_I[s]>)
// (DeepSeek Sparse Attention explained, "How Does the Lightning Indexer Score a Token?": H_I heads, one
// shared key per position, ReLU, head-weighted sum; head weights carry no sign constraint).
//
// fp8 path.  The per-row contraction [H_I x d_I] x [d_I x n] is a dense GEMM with K = d_I = 64 or 128: one or
// two chained v_mfma_f32_32x32x64_f8f6f4 (K = 64 each).  Heads are the M dimension, positions the N dimension:
// lane l of a wave holds head (l % 32) of the A operand and position (l % 32) of the B operand, each with
// the 32 bytes of K half (l / 32); the 32x32 fp32 result leaves 16 heads of one position in each lane, so
// the ReLU and the head-weighted sum run in-lane and finish with one cross-half exchange.  The fp8 codes
// are OCP e4m3fn (the format gfx950's f8f6f4 MFMA reads with format code 0), products are exact and the d_I
// terms accumulate in fp32.  Because the per-vector scales are positive they move outside the ReLU:
// max(0, sq*sk*x) = sq*sk*max(0, x), so the epilogue weight of head j is w[j]*sq[j] and sk multiplies
// the finished sum.  The ReLU-weighted sum is formed as (sum_j wq_j x_j + sum_j wq_j |x_j|) / 2.
//
// Every key row is read once, as 32-byte pieces: one wave covers 32 consecutive positions = 32 d_I bytes of
// contiguous pool memory (a 32-aligned run never crosses a page of >= 32 positions).
//
// In the fused step block 0 of each row also clears the row's top-k state once its scores are out, so the
// selection needs no zeroing launch of its own.  The key loads are issued before the query operands so that
// both are in flight together.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "select.h"
#include "topk_common.h"

DSA_TIMELINE_UNIT(indexer)

namespace dsa {
namespace {

constexpr uint32_t kBufferWord3 = 0x00020000;  // raw buffer resource word 3 on gfx9: 32-bit, range-checked

// An empty use of a loaded value: the compiler waits for the load here, once, instead of at a later use whose
// wait it would place inside a loop.
__device__ __forceinline__ void require_loaded(const v8i& x) { asm volatile("" ::"v"(x)); }
constexpr int kIdxSub = 4;                          // 32-position subtiles per wave
constexpr int kIdxTile = 4 * kIdxSub * 32;          // positions per 256-thread block

// HB = number of 32-head blocks (H_I = 32 * HB); KB = number of 64-byte K blocks (d_I = 64 * KB), one
// v_mfma_f32_32x32x64_f8f6f4 each, chained on one accumulator.  Three waves per SIMD fit d_I = 64; the doubled key
// and query operands of d_I = 128 leave room for two.
// The work of one block: row r, tiles bx * tiles_per_block .. of 512 positions (the kernel below, and the prefill
// fallback, which scores one row with its whole grid).
template <int HB, int KB>
__device__ __forceinline__ void index_row_tiles(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ head_w,
    const uint8_t* __restrict__ k_pool, const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int max_row_len, float* __restrict__ scores, int64_t ld, TopkState clear,
    int tiles_per_block, int r, int bx) {
  constexpr int H_I = 32 * HB, D_I = 64 * KB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  // The row's query operands and epilogue weights depend on nothing but the row: they are requested first, so
  // that they arrive while the row length, the page ids and the keys make their dependent round trips.  Lane
  // half h holds heads 4 h + {0..3} + 8 m of each 32-head block (accumulator entry 4 m + e), four runs of four
  // consecutive heads: one 16-byte load each of weights and scales.
  v8i a[HB][KB];
  float wq[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      a[hb][kb] =
          *reinterpret_cast<const v8i*>(q_idx + ((int64_t)r * H_I + hb * 32 + col) * D_I + kb * 64 + half * 32);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t h0 = (int64_t)r * H_I + hb * 32 + half * 4 + 8 * m;
      const v4f w4 = *reinterpret_cast<const v4f*>(head_w + h0);
      const v4f s4 = *reinterpret_cast<const v4f*>(q_scale + h0);
#pragma unroll
      for (int e = 0; e < 4; ++e) wq[hb][4 * m + e] = w4[e] * s4[e];
    }
  }
  const int n = clamp_len(row_len[r], max_row_len);
  const int64_t first = (int64_t)bx * tiles_per_block * kIdxTile;
  // the row's top-k state, cleared by block 0 as its last work (stores issued earlier would hold up the waits
  // for its key loads, which count in the same in-order counter)
  auto clear_state = [&]() __attribute__((always_inline)) {
    if (clear.cnt && bx == 0 && threadIdx.x == 0) reinterpret_cast<v4i*>(clear.cnt)[r] = v4i{0, 0, 0, 0};
  };
  if (first >= n) {
    clear_state();
    return;
  }
  DSA_STAMP(0, 1);
  const int ntile = (int)min((int64_t)tiles_per_block, (n - first + kIdxTile - 1) / kIdxTile);
  const int seq = clamp_seq(row_seq[r], num_seqs);

  // Tile t of the block covers positions first + 512 t .. +512; wave w owns 128 of them as four 32-position
  // subtiles s.  A 32-aligned subtile lies in one page (pages hold >= 32 positions), so its page id is one
  // scalar load; lanes past the row's end use the last position instead (their scores are never stored), so
  // every key load is unconditional and stays in flight instead of waiting in a divergent branch.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto position = [&](int t, int s) { return first + (int64_t)t * kIdxTile + wave * (kIdxSub * 32) + s * 32 + col; };
  // pool row of lane `col` in subtile s of tile t: one scalar page lookup per subtile; a lane past the row's
  // end takes the row's last position (same 32-aligned block, so the same page)
  auto subtile_rows = [&](int t, int s) -> int64_t {
    const int64_t base = first + (int64_t)t * kIdxTile + wave_u * (kIdxSub * 32) + s * 32;  // uniform
    const int64_t b = base < n ? base : n - 1;
    const int lp = (int)min(b >> log2ps, (int64_t)max_pages - 1);
    int page = page_table[(int64_t)seq * max_pages + lp];
    page = min(max(page, 0), num_pages - 1);
    const int64_t row0 = ((int64_t)page << log2ps) | (b & ((1 << log2ps) - 1));
    return row0 + (base < n ? min((int64_t)col, n - 1 - base) : 0);
  };
  // per tile and lane: the key rows of the four subtiles (MFMA B operands) and the scales of the two positions
  // the lane stores (subtile 2 p + half of each pair p)
  struct TileLoad {
    v8i b[kIdxSub][KB];
    float skm[kIdxSub / 2];
  };
  auto issue = [&](int t, TileLoad& L) __attribute__((always_inline)) {
    int64_t prow[kIdxSub];
#pragma unroll
    for (int s = 0; s < kIdxSub; ++s) prow[s] = subtile_rows(t, s);
#pragma unroll
    for (int s = 0; s < kIdxSub; ++s)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        L.b[s][kb] = *reinterpret_cast<const v8i*>(k_pool + prow[s] * D_I + kb * 64 + half * 32);
#pragma unroll
    for (int p = 0; p < kIdxSub / 2; ++p) {
      // the store subtile's row, picked arithmetically (an indexed pick would put prow in scratch)
      const int64_t srow = prow[2 * p] + (prow[2 * p + 1] - prow[2 * p]) * half;
      L.skm[p] = k_scale[srow];
    }
  };

  TileLoad cur;
  issue(0, cur);
  // the row's query operands are complete before the loop (an asm use makes the compiler wait here once
  // instead of inside every iteration)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) require_loaded(a[hb][kb]);
  DSA_STAMP(0, 2);
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)r * ld, (short)0, n * 4, kBufferWord3);

  // A tile is kUnits (pair p, subtile 2 p + u of the pair, head block hb) MFMA units in that order.  The MFMA of
  // unit k + 1 is issued into a second accumulator before the epilogue of unit k (sched_barrier keeps that
  // order), so the matrix core works while the VALU reduces: with one accumulator every MFMA waited for the
  // previous epilogue and every epilogue for its MFMA.
  constexpr int kUnits = kIdxSub * HB;
  auto compute = [&](int t, const TileLoad& cur) __attribute__((always_inline)) {
    auto unit_mfma = [&](int k) __attribute__((always_inline)) {
      v16f acc = {};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k % HB][kb], cur.b[k / HB][kb], acc, 0, 0, 0, 0, 0, 0);
      return acc;
    };
    v16f acc = unit_mfma(0);
    // max(0, x) = (x + |x|) / 2: two single-instruction FMAs per element (|x| is a source modifier), where
    // fmaxf would also need a NaN-quieting max
    float lin = 0.f, ab = 0.f;
    float part[2];
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
      const int sub = k / HB, hb = k % HB, p = sub / 2, u = sub % 2;
      v16f nxt;
      if (k + 1 < kUnits) nxt = unit_mfma(k + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        lin = fmaf(wq[hb][i], acc[i], lin);
        ab = fmaf(wq[hb][i], fabsf(acc[i]), ab);
      }
      if (hb == HB - 1) {
        part[u] = lin + ab;
        lin = 0.f;
        ab = 0.f;
      }
      if (hb == HB - 1 && u == 1) {
        // half 0 finishes subtile 2 p and half 1 subtile 2 p + 1: v_permlane32_swap of the two subtiles' partial
        // sums hands each half the other half's sum of the subtile it stores
        const auto sw =
            __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
        const float v = cur.skm[p] * (0.5f * (__uint_as_float(sw[0]) + __uint_as_float(sw[1])));
        const int64_t pos = position(t, 2 * p + half);
        // the buffer ends at the row's visible length: stores past it are dropped
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, (int)pos * 4, 0, 0);
      }
      if (k + 1 < kUnits) acc = nxt;
    }
  };

  // Two tile buffers in turn: the keys of tile t + 1 are requested before tile t is computed, so a block keeps
  // a tile in flight, and a buffer is reloaded only after its tile is done (no copies between them).
  TileLoad other;
#pragma unroll 1
  for (int t = 0; t < ntile; t += 2) {
    if (t + 1 < ntile) issue(t + 1, other);
    compute(t, cur);
    if (t + 1 >= ntile) break;
    if (t + 2 < ntile) issue(t + 2, cur);
    compute(t + 1, other);
  }
  DSA_STAMP(0, 3);
  clear_state();
}


// Largest value over the 64 lanes of a wave (DPP within rows, then lane swaps between rows).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}

// The fused step's top-k floor of row r, ranked from the row's own keys by one extra block while the rest of the
// grid scores the row, so that the filter only compares (the sample used to be ranked again by every filter block
// after this kernel).  The block scores S sampled positions, S / 4 runs of four consecutive positions spread
// evenly over the row (a run lies in one page), with the tiles' contraction and epilogue, in rounds of four
// 32-position groups per wave (eight runs each, every lane loading its own position's page id); the keys go to
// LDS.  S = 512 (one round) for a single row of up to 2^17 positions with k_eff <= 2048, where this block is the
// last to finish; 1024 up to 2^18 positions (with several rows the block hides behind the other rows' tiles, and
// the larger sample admits fewer candidates); 4096 up to 2^20.  The floor is the 20-bit prefix of the m-th largest
// sampled score, m = mu + 4 sqrt(mu) + 8 with mu = k_eff S / n the expected number of sampled scores among the row's
// k_eff largest: about n m / S scores reach it (7.2 K at n = 128K, k = 2048, S = 512; 7.2 K at n = 2^20), and a
// sample holds m scores at or above the k_eff-th largest with probability below 1e-6 at these sizes.  One LDS
// histogram ranks the sample: bin 4095 - d counts the keys whose 20-bit prefix lies d below the sample's largest
// (d clamped to 4095), so the m-th largest is found without a second round unless it lies 4095 or more prefixes
// down (a spread of more than a factor of four), when the floor keeps every key.  Whatever floor comes out, the
// selection stays exact: a row whose floor admits fewer than k_eff candidates, or more than its list holds, is
// selected over its stored scores.  Rows outside indexer_floor_row return at once.
template <int HB, int KB>
__device__ __forceinline__ void sample_row_floor(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ head_w,
    const uint8_t* __restrict__ k_pool, const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int max_row_len, int k, uint32_t* __restrict__ thr, int r) {
  constexpr int H_I = 32 * HB, D_I = 64 * KB;
  constexpr int kRound = 4;  // groups per wave and round (512 positions per block)
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ uint32_t keys[kFloorSample];
  __shared__ uint32_t s[8];
  const int n = clamp_len(row_len[r], max_row_len);
  const int keff = min(k, n);
  if (!indexer_floor_row(n, keff)) return;  // uniform over the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int seq = clamp_seq(row_seq[r], num_seqs);
  const int S = gridDim.y == 1 && n <= (1 << 17) && keff <= 2048 ? 4 * 32 * kRound
                : n <= (1 << 18)                                 ? 1024
                                                                 : kFloorSample;
  const int G = S / (4 * 32);  // groups per wave
  const int runs = S / 4;
  // the row's query operands and epilogue weights, laid out as in index_row_tiles
  v8i a[HB][KB];
  float wq[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      a[hb][kb] =
          *reinterpret_cast<const v8i*>(q_idx + ((int64_t)r * H_I + hb * 32 + col) * D_I + kb * 64 + half * 32);
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      const int64_t h0 = (int64_t)r * H_I + hb * 32 + half * 4 + 8 * m4;
      const v4f w4 = *reinterpret_cast<const v4f*>(head_w + h0);
      const v4f s4 = *reinterpret_cast<const v4f*>(q_scale + h0);
#pragma unroll
      for (int e = 0; e < 4; ++e) wq[hb][4 * m4 + e] = w4[e] * s4[e];
    }
  }
  // histogram cleared while the first loads are in flight
  for (int i = threadIdx.x; i < kTopkBins; i += 256) h[i] = 0u;
  if (threadIdx.x < 8) s[threadIdx.x] = 0u;  // a floor of 0 keeps every key, should the rank fail
  // rounds of four groups: group g of wave w holds runs 8 (G w + g) + col / 4, run j starting at j n / runs rounded
  // down to a multiple of 4 (the last run ends below n since n >= kFloorMinLen); page ids, then keys and scales;
  // the MFMA of unit u + 1 is issued before the epilogue of unit u, as in the tiles, and lane half h ends with the
  // score of group 2 p + h at position col
#pragma unroll 1
  for (int g0 = 0; g0 < G; g0 += kRound) {
    int64_t prow[kRound];
#pragma unroll
    for (int g = 0; g < kRound; ++g) {
      const int j = 8 * (G * wave + g0 + g) + (col >> 2);
      const int pos = (int)(((int64_t)j * n / runs) & ~3) + (col & 3);
      const int lp = min(pos >> log2ps, max_pages - 1);
      const int page = min(max(page_table[(int64_t)seq * max_pages + lp], 0), num_pages - 1);
      prow[g] = ((int64_t)page << log2ps) | (pos & ((1 << log2ps) - 1));
    }
    DSA_STAMP(0, 4);
    v8i b[kRound][KB];
    float sk[kRound];
#pragma unroll
    for (int g = 0; g < kRound; ++g) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        b[g][kb] = *reinterpret_cast<const v8i*>(k_pool + prow[g] * D_I + kb * 64 + half * 32);
      sk[g] = k_scale[prow[g]];
    }
    auto unit_mfma = [&](int u) __attribute__((always_inline)) {
      v16f acc = {};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u % HB][kb], b[u / HB][kb], acc, 0, 0, 0, 0, 0, 0);
      return acc;
    };
    constexpr int kUnits = kRound * HB;
    v16f acc = unit_mfma(0);
    float lin = 0.f, ab = 0.f, part[2];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int g = u / HB, hb = u % HB;
      v16f nxt;
      if (u + 1 < kUnits) nxt = unit_mfma(u + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        lin = fmaf(wq[hb][i], acc[i], lin);
        ab = fmaf(wq[hb][i], fabsf(acc[i]), ab);
      }
      if (hb == HB - 1) {
        part[g % 2] = lin + ab;
        lin = 0.f;
        ab = 0.f;
      }
      if (hb == HB - 1 && g % 2 == 1) {
        const auto sw =
            __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
        const float skp = half ? sk[g] : sk[g - 1];
        keys[(G * wave + g0 + g - 1 + half) * 32 + col] =
            order_key(skp * (0.5f * (__uint_as_float(sw[0]) + __uint_as_float(sw[1]))));
      }
      if (u + 1 < kUnits) acc = nxt;
    }
  }
  DSA_STAMP(0, 5);
  const float mu = (float)keff * (float)S / (float)n;
  const uint32_t m = (uint32_t)min(S, (int)ceilf(mu + 4.f * sqrtf(mu) + 8.f));
  __syncthreads();  // the keys are in LDS
  // the sample's largest key, then one histogram of distances below it
  uint32_t mx = 0u;
  for (int i = threadIdx.x; i < S; i += 256) mx = max(mx, keys[i]);
  mx = wave_max_u32(mx);
  if (lane == 0) s[4 + wave] = mx;
  __syncthreads();
  const uint32_t top = max(max(s[4], s[5]), max(s[6], s[7])) >> 12;
  for (int i = threadIdx.x; i < S; i += 256)
    atomicAdd(&h[kTopkBins - 1 - min(top - (keys[i] >> 12), (uint32_t)kTopkBins - 1)], 1u);
  __syncthreads();
  DSA_STAMP(0, 6);
  if (threadIdx.x < 64) wave_threshold_bin<kTopkBins, 16>(h, m, &s[0], &s[1]);
  __syncthreads();
  if (threadIdx.x == 0) thr[4 * r + 1] = s[0] > 0u ? top - (kTopkBins - 1 - s[0]) : 0u;
  DSA_STAMP(0, 7);
}

template <int HB, int KB>
__global__ __launch_bounds__(256, KB == 1 ? 3 : 2) void indexer_f8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ head_w,
    const uint8_t* __restrict__ k_pool, const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int max_row_len, float* __restrict__ scores, int64_t ld, TopkState clear,
    int tiles_per_block, int floor_col) {
  args_to_sgprs(q_idx, q_scale, head_w, k_pool, k_scale, row_seq, row_len, page_table, num_seqs, max_pages, num_pages,
                log2ps, max_row_len, scores, ld, clear.cnt, clear.thr, clear.k, tiles_per_block, floor_col);
  DSA_STAMP(0, 0);
  // a grid with floor blocks has one extra column: the first R blocks in dispatch order (linear id, x fastest) rank
  // the rows' top-k floors, so that they start with the first tiles even in a batch, and the other blocks take the
  // rows' tiles in row-major order
  int r = (int)blockIdx.y, bx = (int)blockIdx.x;
  if (floor_col) {
    const int lin = (int)(blockIdx.x + blockIdx.y * gridDim.x), R = (int)gridDim.y, cols = (int)gridDim.x - 1;
    if (lin < R) {
      sample_row_floor<HB, KB>(q_idx, q_scale, head_w, k_pool, k_scale, row_seq, row_len, page_table, num_seqs,
                               max_pages, num_pages, log2ps, max_row_len, clear.k, clear.thr, lin);
      return;
    }
    r = (lin - R) / cols;
    bx = (lin - R) % cols;
  }
  index_row_tiles<HB, KB>(q_idx, q_scale, head_w, k_pool, k_scale, row_seq, row_len, page_table, num_seqs, max_pages,
                          num_pages, log2ps, max_row_len, scores, ld, clear, tiles_per_block, r, bx);
}

// Chunked prefill: consecutive rows of one sequence score the same keys, so the contraction is a real GEMM
// [rows * H_I x d_I] x [d_I x n] (DeepSeek Sparse Attention explained: over a prefill the indexer's cost stays
// quadratic in the context).  A block owns kPfRows rows of one sequence and kPfPasses * kPfTile positions.
//
// The fp8 MFMAs are cheap next to a two-instruction ReLU epilogue (64 cycles per 32x32x64 MFMA against
// 16 elements x 2 VALU ops x 4 cycles), so the epilogue is rewritten with max(0, x) = (x + |x|) / 2:
//     sum_j wq_j max(0, x_j) = ( sum_j wq_j x_j + sum_j wq_j |x_j| ) / 2,
// where x_j = <q8_j, k8> and wq_j = w_j * sq_j.  The |x| term is one v_fma_f32 with an abs source modifier
// per element.  The linear term is <u, k8> with u = sum_j wq_j q8_j, a 64-vector per row: it runs on a
// bf16 MFMA with u split into four bf16 pieces (u = p0 + p1 + p2 + p3 to 2^-32 relative, each piece the
// RNE rounding of what the previous ones leave) and the fp8 keys widened to bf16 exactly, so every product is
// exact and only fp32 accumulation rounds.  A row group of 8 rows x 4 pieces fills the 32 rows of
// v_mfma_f32_32x32x16_bf16: A row 8c + r holds piece c of row r; output register 4c + e of lane half h then
// holds piece c of row 4h + e, and the four pieces are summed in-lane.
//
// Layout per wave: 128 positions = four 32-position subtiles whose fp8 keys stay in registers as MFMA B
// operands (lane l: position l % 32, key bytes 32 (l / 32) .. +32); the same bytes, widened, feed the linear
// MFMA with K index d = 32 (l / 32) + 8 m + e for K-step m, slot e, and u is laid out to match.  Queries,
// epilogue weights and the u pieces sit in LDS, shared by the four waves.
//
// Scheduling: each row is a software pipeline over (head block, subtile pair, subtile) units, the MFMA of the
// next unit issued before the epilogue of the current one (sched_barrier keeps that order), so one wave keeps
// the matrix core and the VALU busy together; 8-row blocks need 38 KiB of LDS and 168 VGPRs, which leaves room
// for three waves per SIMD.  The finish of a subtile pair is branch-free: lane halves exchange partial sums
// with v_permlane32_swap, the half that holds a row's linear term adds it through a 0/1 factor, and scores go
// out through a raw buffer whose size is the row's visible length, so stores past it are dropped by the
// hardware.  Staging loads are all issued before the first LDS write.
constexpr int kPfRows = 8;                // query rows per block: one group of 8 for the linear MFMA
constexpr int kPfSub = 4;                 // 32-position subtiles per wave
constexpr int kPfTile = 4 * kPfSub * 32;  // positions per pass of a 256-thread block
constexpr int kPfPasses = 8;              // passes per block: the row staging is paid once per 4096 positions

// KB = d_I / 64 K blocks: each (head block, subtile) unit chains KB fp8 MFMAs, the linear MFMA takes 4 KB K-steps.
// The filter pass's hand-over of one 64-lane group of scores: the lanes in `m` (this lane's entry when `keep`)
// take consecutive places in the row's LDS stage; places past its capacity go straight to the row's list, each
// with an atomic of its own (a row far denser in candidates than its floor promised).
__device__ __forceinline__ void stage_candidates(uint64_t m, bool keep, uint64_t entry, uint64_t* stage, uint32_t* n,
                                                 int cap, uint32_t* row_cnt, uint64_t* row_list) {
  const int lane = threadIdx.x & 63;
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, (uint32_t)__popcll(m));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const uint32_t idx = base + (uint32_t)__popcll(m & below);
  if (keep) {
    if (idx < (uint32_t)cap) {
      stage[idx] = entry;
    } else {
      const uint32_t at = atomicAdd(row_cnt, 1u);
      if (at < (uint32_t)kPfCap) row_list[at] = entry;
    }
  }
}

// kMode 0: the scores of every visible position into `scores`.  kMode 1 (sample pass): the block's rows score
// kPfSample sampled positions, 128 runs of 32 consecutive positions spread evenly over the positions every row of
// the block sees (all of them when fewer), into sel.samp at the sample's own indices.  kMode 2 (filter pass): no
// score leaves the block; each position whose key reaches its row's floor is staged in LDS as a candidate, and
// the block appends each row's candidates to the row's list with one atomic.
template <int HB, int KB, int kMode>
__global__ __launch_bounds__(256, KB == 1 ? 3 : 2) void indexer_f8_tiled_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ head_w,
    const uint8_t* __restrict__ k_pool, const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int max_row_len, int R, int rows_per_seq, int tiles_per_group,
    float* __restrict__ scores, int64_t ld, PfSel sel) {
  constexpr int H_I = 32 * HB, D = 64 * KB;
  // candidates of each row staged per block (filter pass; d_I = 64 only, which keeps three blocks per CU)
  constexpr int kStage = KB == 2 ? 1 : 192;
  __shared__ uint64_t stage[kMode == 2 ? kPfRows : 1][kMode == 2 ? kStage : 1];
  __shared__ uint32_t stage_n[kPfRows], stage_base[kPfRows], floor_lds[kPfRows];
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kPfRows][HB][64][32 * KB];  // lane l's fp8 A operands
  __shared__ __attribute__((aligned(16))) float w_lds[kPfRows][HB][2][16];          // wq of each lane half's heads
  __shared__ __attribute__((aligned(16))) __bf16 u_lds[kPfRows / 8][4 * KB][64][8];  // linear-MFMA A operands
  __shared__ __attribute__((aligned(16))) int n_lds[kPfRows];
  const int group = (int)blockIdx.y / tiles_per_group;
  const int r0 = group * rows_per_seq + ((int)blockIdx.y % tiles_per_group) * kPfRows;
  const int rows = min(min(kPfRows, (group + 1) * rows_per_seq - r0), R - r0);
  if (rows <= 0) return;  // a tile past the end of a short last group (uniform)
  const int64_t span0 = (int64_t)blockIdx.x * (kPfPasses * kPfTile);
  if ((int)threadIdx.x < kPfRows)
    n_lds[threadIdx.x] = (int)threadIdx.x < rows ? clamp_len(row_len[r0 + threadIdx.x], max_row_len) : 0;
  __syncthreads();
  int nmax = 0;
  for (int q = 0; q < rows; ++q) nmax = max(nmax, n_lds[q]);
  // sample pass: virtual position v is position (v / 32) * step + v % 32; nmax becomes the sample's length
  int step = 32;
  if constexpr (kMode == 1) {
    int nmin = n_lds[0];
    for (int q = 1; q < rows; ++q) nmin = min(nmin, n_lds[q]);
    if (nmin >= kPfSample) {
      step = (nmin / (kPfSample / 32)) & ~31;
      nmax = kPfSample;
    } else {
      nmax = nmin;
    }
    if ((int)threadIdx.x < rows) sel.samp_len[r0 + threadIdx.x] = nmax;
  }
  if constexpr (kMode == 2) {
    if ((int)threadIdx.x < kPfRows) {
      stage_n[threadIdx.x] = 0u;
      floor_lds[threadIdx.x] = (int)threadIdx.x < rows ? sel.floor[r0 + threadIdx.x] : 0u;
    }
    // published by the barrier after the operand staging below
  }
  if (span0 >= nmax) return;  // uniform: no row of the tile sees these positions
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int seq = clamp_seq(row_seq[r0], num_seqs);  // shared by the group's rows

  // stage the rows' A operands (16-byte pieces: c = ((q * HB + hb) * KB + kb) * 128 + l * 2 + piece; K block kb
  // of lane l holds query bytes 64 kb + 32 (l / 32) .. +32 of head l % 32) and epilogue weights; every load is
  // issued before the first LDS write so the block pays one memory round trip, not one per piece
  {
    constexpr int kA = kPfRows * HB * KB * 128 / 256;  // A pieces per thread
    constexpr int kW = kPfRows * H_I / 256;       // weights per thread
    v4i av[kA];
    float wv[kW], sv[kW];
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int q = c / (HB * KB * 128), hb = (c / (KB * 128)) % HB, kb = (c / 128) % KB, l = (c >> 1) & 63,
                piece = c & 1;
      if (q < rows)
        av[i] = *reinterpret_cast<const v4i*>(q_idx + ((int64_t)(r0 + q) * H_I + hb * 32 + (l & 31)) * D + kb * 64 +
                                              (l >> 5) * 32 + piece * 16);
    }
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      const int c = threadIdx.x + 256 * i, q = c / H_I;
      if (q < rows) {
        wv[i] = head_w[(int64_t)r0 * H_I + c];
        sv[i] = q_scale[(int64_t)r0 * H_I + c];
      }
    }
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int q = c / (HB * KB * 128), hb = (c / (KB * 128)) % HB, kb = (c / 128) % KB, l = (c >> 1) & 63,
                piece = c & 1;
      if (q < rows) *reinterpret_cast<v4i*>(&a_lds[q][hb][l][kb * 32 + piece * 16]) = av[i];
    }
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      const int c = threadIdx.x + 256 * i, q = c / H_I, head = c % H_I, hh = head & 31;
      // lane half (hh >> 2) & 1 holds head hh as accumulator entry (hh & 3) + 4 * (hh >> 3)
      if (q < rows) w_lds[q][head >> 5][(hh >> 2) & 1][(hh & 3) + 4 * (hh >> 3)] = wv[i] * sv[i];
    }
  }
  __syncthreads();

  // u[q][d] = sum_j wq_j q8[q][j][d] in fp32, split into bf16 pieces placed as linear-MFMA A operands; dim
  // d = 64 kb + dd sits in K block kb, lane half dd / 32, byte dd % 32
  {
    constexpr int kTpr = 256 / kPfRows, kDpt = D / kTpr;  // threads per row, dims per thread
    const int q = threadIdx.x / kTpr, d0 = (threadIdx.x % kTpr) * kDpt;
    float u[kDpt];
#pragma unroll
    for (int t = 0; t < kDpt; ++t) u[t] = 0.f;
    if (q < rows) {
      for (int j = 0; j < H_I; ++j) {
        const float w = w_lds[q][j >> 5][(j >> 2) & 1][(j & 3) + 4 * ((j >> 3) & 3)];
#pragma unroll
        for (int t = 0; t < kDpt; t += 2) {
          const int d = d0 + t, dd = d & 63;
          const uint16_t codes =
              *reinterpret_cast<const uint16_t*>(&a_lds[q][j >> 5][(dd >> 5) * 32 + (j & 31)][(d >> 6) * 32 + (dd & 31)]);
          const v2f x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)codes, 1.f, false);
          u[t] = fmaf(w, x.x, u[t]);
          u[t + 1] = fmaf(w, x.y, u[t + 1]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kDpt; ++t) {
      const int d = d0 + t;
      float rest = u[t];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const __bf16 p = (__bf16)rest;  // round to nearest even; rest - p is exact
        rest -= (float)p;
        // K-step 4 kb + m, lane half h covers dims 64 kb + 32 h + 8 m .. +8
        u_lds[q >> 3][(d >> 6) * 4 + ((d >> 3) & 3)][((d >> 5) & 1) * 32 + 8 * c + (q & 7)][d & 7] = p;
      }
    }
  }
  __syncthreads();

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  v8i b[kPfSub][KB];
  for (int pass = 0; pass < kPfPasses; ++pass) {
    const int64_t tile0 = span0 + (int64_t)pass * kPfTile;
    if (tile0 >= nmax) break;  // uniform
    // Pool rows of the wave's four 32-position subtiles: a 32-aligned subtile lies in one page (pages hold >= 32
    // positions), so its page id is one scalar load; lanes past the tile's last position take that position
    // (the same page, or the last one), so every load is unconditional and in range.  Scores of positions a row
    // does not see are never stored (the row's store range ends at its length).
    int64_t prow[kPfSub];
#pragma unroll
    for (int s = 0; s < kPfSub; ++s) {
      const int64_t base = tile0 + wave_u * (kPfSub * 32) + s * 32;  // uniform
      if constexpr (kMode == 1) {
        // a sampled run: 32 consecutive positions from a multiple of 32, inside one page; a subtile past the
        // sample's end rereads the last run
        const int64_t vb = base < nmax ? base : (int64_t)((nmax - 1) & ~31);
        const int64_t pb = (vb >> 5) * step;
        const int lp = (int)min(pb >> log2ps, (int64_t)max_pages - 1);
        int page = page_table[(int64_t)seq * max_pages + lp];
        page = min(max(page, 0), num_pages - 1);
        const int64_t row0 = ((int64_t)page << log2ps) | (pb & ((1 << log2ps) - 1));
        prow[s] = row0 + min((int64_t)col, nmax - 1 - vb);
      } else {
        const int64_t bp = base < nmax ? base : nmax - 1;
        const int lp = (int)min(bp >> log2ps, (int64_t)max_pages - 1);
        int page = page_table[(int64_t)seq * max_pages + lp];
        page = min(max(page, 0), num_pages - 1);
        const int64_t row0 = ((int64_t)page << log2ps) | (bp & ((1 << log2ps) - 1));
        prow[s] = row0 + (base < nmax ? min((int64_t)col, nmax - 1 - base) : 0);
      }
    }
#pragma unroll
    for (int s = 0; s < kPfSub; ++s)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        b[s][kb] = *reinterpret_cast<const v8i*>(k_pool + prow[s] * D + kb * 64 + half * 32);

    // per pass, per lane: half 0 stores subtile 2p and half 1 subtile 2p + 1 of each pair p; 0.5 sk of that
    // position (the 1/2 of (lin + abs) folded in, exact) and its byte offset within the row
    float skm[kPfSub / 2];
    int voff[kPfSub / 2];
#pragma unroll
    for (int p = 0; p < kPfSub / 2; ++p) {
      // the store subtile's row, picked arithmetically (an indexed pick would put prow in scratch)
      const int64_t srow = prow[2 * p] + (prow[2 * p + 1] - prow[2 * p]) * half;
      skm[p] = 0.5f * k_scale[srow];
      voff[p] = (wave * (kPfSub * 32) + (2 * p + half) * 32 + col) * 4;
    }

#pragma unroll 1
    for (int g = 0; g < kPfRows / 8; ++g) {
      if (8 * g >= rows) break;  // uniform
      // linear term of rows 8 g + 4 half + e for subtile 2 p + t of each pair p
      float lin2[kPfSub / 2][2][4];
#pragma unroll
      for (int p = 0; p < kPfSub / 2; ++p) {
        float lin[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int s = 2 * p + t;
          v16f acc = {};
#pragma unroll
          for (int kq = 0; kq < KB; ++kq)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const v2bf x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)b[s][kq][2 * m], 1.f, false);
              const v2bf x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)b[s][kq][2 * m], 1.f, true);
              const v2bf x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)b[s][kq][2 * m + 1], 1.f, false);
              const v2bf x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)b[s][kq][2 * m + 1], 1.f, true);
              const v8bf kv8 = {x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  *reinterpret_cast<const v8bf*>(&u_lds[g][kq * 4 + m][lane][0]), kv8, acc, 0, 0, 0);
            }
#pragma unroll
          for (int e = 0; e < 4; ++e) lin[t][e] = ((acc[12 + e] + acc[8 + e]) + acc[4 + e]) + acc[e];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) lin2[p][t][e] = lin[t][e];
      }

#pragma unroll 1
      for (int hq = 0; hq < 2; ++hq) {
        const float ownf = hq == half ? 1.f : 0.f;  // this lane half holds the linear term of rows 8 g + 4 hq + e
        int nq[4];  // lengths of rows 8 g + 4 hq + e (0 past the tile's rows): one 16-byte LDS read
        {
          const v4i nv = *reinterpret_cast<const v4i*>(&n_lds[8 * g + 4 * hq]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            nq[e] = __builtin_amdgcn_readfirstlane(nv[e]);
            if (kMode == 1 && nq[e] > 0) nq[e] = nmax;  // a sampled row's stored length is the sample's
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = 8 * g + 4 * hq + e;
          if (tile0 >= nq[e]) continue;  // uniform; also rows past the tile's end
          v8i a[HB][KB];
          float wq[HB][16];
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) a[hb][kb] = *reinterpret_cast<const v8i*>(&a_lds[q][hb][lane][kb * 32]);
#pragma unroll
            for (int i = 0; i < 16; ++i) wq[hb][i] = w_lds[q][hb][half][i];
          }
          // the buffer starts at the pass's first position and ends at the row's visible length, so a store past
          // the row's end falls outside it (on its bounds-checked offset) and is dropped
          float* const dst_row = kMode == 1 ? sel.samp + (int64_t)(r0 + q) * kPfSample : scores + (int64_t)(r0 + q) * ld;
          const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(dst_row + tile0, (short)0, (nq[e] - (int)tile0) * 4,
                                                              kBufferWord3);
          const uint32_t fl = kMode == 2 ? floor_lds[q] : 0u;
          constexpr int U = 2 * HB;             // units per subtile pair
          constexpr int K = (kPfSub / 2) * U;   // units per row
          float ab[2] = {0.f, 0.f};
          // one unit: KB chained fp8 MFMAs over the K blocks
          auto unit = [&](int hb, int s) __attribute__((always_inline)) {
            v16f x = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[hb][0], b[s][0], v16f{}, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int kb = 1; kb < KB; ++kb)
              x = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[hb][kb], b[s][kb], x, 0, 0, 0, 0, 0, 0);
            return x;
          };
          v16f prev = unit(0, 0);
#pragma unroll
          for (int k = 1; k <= K; ++k) {
            v16f next;
            if (k < K) {
              const int p = k / U, hb = (k % U) >> 1, t = k & 1;
              next = unit(hb, 2 * p + t);
            }
            __builtin_amdgcn_sched_barrier(0);
            {
              const int kp = k - 1, p = kp / U, hb = (kp % U) >> 1, t = kp & 1;
              float acc_ab = hb == 0 ? 0.f : ab[t];
#pragma unroll
              for (int i = 0; i < 16; ++i) acc_ab = fmaf(wq[hb][i], fabsf(prev[i]), acc_ab);
              ab[t] = acc_ab;
              if (kp % U == U - 1) {  // pair p complete: half 0 finishes subtile 2p, half 1 subtile 2p + 1
                // the half that holds row q's linear term adds it to both subtiles; v_permlane32_swap of the
                // (subtile 2p, subtile 2p + 1) sums then hands each half the other half's sum of the subtile it
                // stores, so the total is the sum of the two swapped registers
                const float s0 = fmaf(ownf, lin2[p][0][e], ab[0]);
                const float s1 = fmaf(ownf, lin2[p][1][e], ab[1]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
                const float total = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                if constexpr (kMode == 2) {
                  const int pos = (int)tile0 + (voff[p] >> 2);
                  const uint32_t key = order_key(skm[p] * total);
                  const bool keep = pos < nq[e] && (key >> 12) >= fl;
                  const uint64_t m = __ballot(keep);
                  if (m) stage_candidates(m, keep, ((uint64_t)pos << 32) | key, stage[q], &stage_n[q], kStage,
                                          sel.cnt + r0 + q, sel.cand + (int64_t)(r0 + q) * kPfCap);
                } else {
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(skm[p] * total), rsrc, voff[p], 0, 0);
                }
              }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (k < K) prev = next;
          }
        }
      }
    }
  }
  if constexpr (kMode == 2) {
    // each row's staged candidates go to its list in one range, reserved with one atomic
    __syncthreads();
    if ((int)threadIdx.x < rows) {
      const uint32_t c = min(stage_n[threadIdx.x], (uint32_t)kStage);
      stage_base[threadIdx.x] = c ? atomicAdd(sel.cnt + r0 + threadIdx.x, c) : 0u;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < rows * kStage; i += 256) {
      const int q = i / kStage, j = i - q * kStage;
      const uint32_t at = stage_base[q] + (uint32_t)j;
      if (j < (int)min(stage_n[q], (uint32_t)kStage) && at < (uint32_t)kPfCap)
        sel.cand[(int64_t)(r0 + q) * kPfCap + at] = stage[q][j];
    }
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

template <int HB, int KB>
void launch_f8(const Geo& g, const uint8_t* qp, const float* q_idx_scale, const float* head_w, const uint8_t* kp,
               const float* k_idx_scale, float* scores, int64_t ld, const TopkState* fuse, hipStream_t stream) {
  // one 512-position tile per block up to kIdxTargetBlocks blocks (small, latency-bound problems spread as
  // wide as they can); beyond that a block streams several tiles so that each keeps a tile of keys in flight.
  // 4096 blocks (about 5 rounds of 3 blocks per CU) measured best on 8 x 1M and 64 x 40K rows.
  constexpr int kIdxTargetBlocks = 4096;
  const int tiles_row = (g.max_row_len + kIdxTile - 1) / kIdxTile;
  const int64_t tiles = (int64_t)tiles_row * g.R;
  const int per = (int)std::max<int64_t>(1, std::min<int64_t>(tiles_row, tiles / kIdxTargetBlocks));
  const int floor_col = fuse && indexer_floor_blocks(g) ? 1 : 0;
  dim3 grid((tiles_row + per - 1) / per + floor_col, g.R);
  indexer_f8_kernel<HB, KB><<<grid, 256, 0, stream>>>(
      qp, q_idx_scale, head_w, kp, k_idx_scale, g.row_seq, g.row_len, g.page_table, g.S, g.max_pages, g.num_pages,
      g.log2ps, g.max_row_len, scores, ld, fuse ? *fuse : TopkState{nullptr, nullptr, 0}, per, floor_col);
}

// Grid-wide barrier of a persistent launch whose blocks are all resident: each block adds one to *bar when it
// arrives (release) and waits until all nblocks blocks of this round have (acquire); the count only grows, so
// round `gen` waits for gen * nblocks.  A wait that outlasts its bound gives up and is counted in *timeouts.
__device__ __forceinline__ void grid_sync(uint32_t* bar, uint32_t nblocks, uint32_t& gen, uint32_t* timeouts) {
  __syncthreads();
  ++gen;
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = gen * nblocks;
    uint32_t spins = 0;
    while (__hip_atomic_load(bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == (1u << 22)) {
        atomicAdd(timeouts, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Rows of a chunked prefill whose sampled floor misjudged them (fewer candidates than k_eff, more than the list
// holds, a threshold beyond the candidate histogram, or more than 1024 keys tied at the threshold) are selected
// here, exactly and one at a time: the whole grid scores the row's positions into sel.fbuf with the per-row
// kernel's tiles, and block 0 runs the three-digit radix select over the stored row.  The grid is one block per
// CU, so every block is resident for the barriers; with no such row every block returns at once.
template <int HB, int KB>
__global__ __launch_bounds__(256) void pf_fallback_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ head_w,
    const uint8_t* __restrict__ k_pool, const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int max_row_len, int R, int k, PfSel sel, int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ pool_rows) {
  __shared__ __attribute__((aligned(16))) uint32_t h[kTopkBins];
  __shared__ __attribute__((aligned(16))) uint32_t scan[256 / 64 + 1];
  const uint32_t nfail = min(sel.ctl[0], (uint32_t)R);
  if (nfail == 0) return;
  uint32_t gen = 0;
  for (uint32_t i = 0; i < nfail; ++i) {
    const int r = sel.fail[i];
    const int n = clamp_len(row_len[r], max_row_len);
    const int keff = min(k, n);
    const int ntile = (n + kIdxTile - 1) / kIdxTile;
    for (int t = blockIdx.x; t < ntile; t += gridDim.x)
      index_row_tiles<HB, KB>(q_idx, q_scale, head_w, k_pool, k_scale, row_seq, row_len, page_table, num_seqs,
                              max_pages, num_pages, log2ps, max_row_len, sel.fbuf, 0, TopkState{nullptr}, 1, r, t);
    grid_sync(sel.ctl + 1, gridDim.x, gen, sel.ctl + 2);
    if (blockIdx.x == 0) {
      const int32_t* gpt = page_table + (int64_t)clamp_seq(row_seq[r], num_seqs) * max_pages;
      int32_t* out = topk_idx + (int64_t)r * k;
      int32_t* rows_out = pool_rows ? pool_rows + (int64_t)r * k : nullptr;
      const ListSink sink{out, rows_out, RowMap{gpt, max_pages, num_pages, log2ps}};
      select_and_write<256>(RowList{sel.fbuf}, n, (uint32_t)keff, keff, sink, h, scan);
      for (int j = keff + threadIdx.x; j < k; j += 256) {
        out[j] = -1;
        if (rows_out) rows_out[j] = -1;
      }
    }
    grid_sync(sel.ctl + 1, gridDim.x, gen, sel.ctl + 2);  // sel.fbuf is free for the next row
  }
}

template <int HB, int KB, int kMode>
void launch_f8_tiled(const Geo& g, const uint8_t* qp, const float* q_idx_scale, const float* head_w,
                     const uint8_t* kp, const float* k_idx_scale, float* scores, int64_t ld, const PfSel& sel,
                     hipStream_t stream) {
  const int tiles_per_group = (g.rows_per_seq + kPfRows - 1) / kPfRows;
  const int groups = (g.R + g.rows_per_seq - 1) / g.rows_per_seq;
  const int span = kMode == 1 ? kPfSample : g.max_row_len;  // the sample pass covers kPfSample virtual positions
  dim3 grid((span + kPfPasses * kPfTile - 1) / (kPfPasses * kPfTile), groups * tiles_per_group);
  indexer_f8_tiled_kernel<HB, KB, kMode><<<grid, 256, 0, stream>>>(
      qp, q_idx_scale, head_w, kp, k_idx_scale, g.row_seq, g.row_len, g.page_table, g.S, g.max_pages, g.num_pages,
      g.log2ps, g.max_row_len, g.R, g.rows_per_seq, tiles_per_group, scores, ld, sel);
}

template <int kMode>
void launch_tiled_mode(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                       const void* k_idx_pool, const float* k_idx_scale, float* scores, int64_t ld, const PfSel& sel,
                       hipStream_t stream) {
  auto* qp = static_cast<const uint8_t*>(q_idx);
  auto* kp = static_cast<const uint8_t*>(k_idx_pool);
  if constexpr (kMode != 0) {  // the sample and filter passes serve d_I = 64 (prefill_select_supported)
    if (g.H_I == 64) launch_f8_tiled<2, 1, kMode>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, sel, stream);
    else launch_f8_tiled<1, 1, kMode>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, sel, stream);
    return;
  }
  if (g.d_I == 128) {
    if (g.H_I == 64) launch_f8_tiled<2, 2, kMode>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, sel, stream);
    else launch_f8_tiled<1, 2, kMode>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, sel, stream);
  } else if (g.H_I == 64) {
    launch_f8_tiled<2, 1, kMode>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, sel, stream);
  } else {
    launch_f8_tiled<1, 1, kMode>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, sel, stream);
  }
}

// fp8 rows that come in groups sharing a sequence take the tiled kernel (d_I = 64 or 128)
bool indexer_tiled(const Geo& g) {
  return g.idx_dtype == 2 /* F8E4M3 */ && (g.d_I == 64 || g.d_I == 128) && g.rows_per_seq >= kTiledMinRows;
}

bool indexer_floor_blocks(const Geo& g) {
  return g.idx_dtype == 2 /* F8E4M3 */ && !indexer_tiled(g) && g.max_row_len >= kFloorMinLen && g.k <= 4096;
}

hipError_t launch_indexer(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                          const void* k_idx_pool, const float* k_idx_scale, float* scores, int64_t ld,
                          const TopkState* fuse, hipStream_t stream) {
  if (g.R == 0 || g.max_row_len == 0) return hipSuccess;
  if (indexer_tiled(g)) {
    if (fuse) return hipErrorInvalidValue;  // the tiled kernel does not clear the top-k state
    launch_tiled_mode<0>(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, scores, ld, PfSel{}, stream);
    return hipGetLastError();
  }
  if (g.idx_dtype == 2 /* F8E4M3 */) {
    auto* qp = static_cast<const uint8_t*>(q_idx);
    auto* kp = static_cast<const uint8_t*>(k_idx_pool);
    if (g.d_I == 128) {
      if (g.H_I == 64) launch_f8<2, 2>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
      else launch_f8<1, 2>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
    } else if (g.H_I == 64) {
      launch_f8<2, 1>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
    } else {
      launch_f8<1, 1>(g, qp, q_idx_scale, head_w, kp, k_idx_scale, scores, ld, fuse, stream);
    }
  } else {
    if (fuse) return hipErrorInvalidValue;  // only the fp8 kernel clears the top-k state
    dim3 grid((g.max_row_len + 255) / 256, g.R);
    size_t lds = sizeof(float) * (size_t)(g.H_I * g.d_I + g.H_I);
    indexer_f32_kernel<<<grid, 256, lds, stream>>>(static_cast<const float*>(q_idx), head_w,
                                                    static_cast<const float*>(k_idx_pool), g.row_seq, g.row_len,
                                                    g.page_table, g.S, g.max_pages, g.num_pages, g.log2ps,
                                                    g.max_row_len, g.H_I, g.d_I, scores, ld);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_pf(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                             const void* k_idx_pool, const float* k_idx_scale, const PfSel& sel, int mode,
                             hipStream_t stream) {
  if (g.R == 0 || g.max_row_len == 0) return hipSuccess;
  if (!indexer_tiled(g) || g.d_I != 64) return hipErrorInvalidValue;
  if (mode == 1)
    launch_tiled_mode<1>(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, nullptr, 0, sel, stream);
  else
    launch_tiled_mode<2>(g, q_idx, q_idx_scale, head_w, k_idx_pool, k_idx_scale, nullptr, 0, sel, stream);
  return hipGetLastError();
}

hipError_t launch_pf_fallback(const Geo& g, const void* q_idx, const float* q_idx_scale, const float* head_w,
                              const void* k_idx_pool, const float* k_idx_scale, const PfSel& sel, int32_t* topk_idx,
                              int32_t* pool_rows, hipStream_t stream) {
  if (g.R == 0 || g.max_row_len == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  auto* qp = static_cast<const uint8_t*>(q_idx);
  auto* kp = static_cast<const uint8_t*>(k_idx_pool);
#define DSA_PF_FALLBACK(HB, KB)                                                                                   \
  pf_fallback_kernel<HB, KB><<<std::max(1, cus), 256, 0, stream>>>(                                              \
      qp, q_idx_scale, head_w, kp, k_idx_scale, g.row_seq, g.row_len, g.page_table, g.S, g.max_pages, g.num_pages, \
      g.log2ps, g.max_row_len, g.R, g.k, sel, topk_idx, pool_rows)
  if (g.d_I == 128) {
    if (g.H_I == 64) DSA_PF_FALLBACK(2, 2);
    else DSA_PF_FALLBACK(1, 2);
  } else if (g.H_I == 64) {
    DSA_PF_FALLBACK(2, 1);
  } else {
    DSA_PF_FALLBACK(1, 1);
  }
#undef DSA_PF_FALLBACK
  return hipGetLastError();
}

}  // namespace dsa
