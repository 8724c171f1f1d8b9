// Sparse MLA attention in MQA mode on gfx950 (lizeman DSA page, section 2 stage 2; kiadev "How DSA works";
// DeepSeek Sparse Attention explained, "What Does the Whole Block Look Like?" and "What Does the GPU Actually
// Run?"): every query head attends with an ordinary softmax over only the selected latent rows; each
// 512-wide latent row is shared by all heads and serves as both key and value.
//
// bf16 path.  A block owns 16 heads of one row and a contiguous range of the k selection slots.  For each
// chunk of 64 slots it gathers the 64 selected rows (1 KiB each) through the page table into LDS, computes
// S = Q K^T with v_mfma_f32_16x16x32_bf16 (each of the 4 waves takes 16 slots over the full 512-wide
// contraction, Q held in registers), updates an fp32 online softmax, and accumulates O += P V with the same
// MFMA (each wave owns 128 output columns).  The same LDS tile is read as K (row-contiguous 16-byte reads)
// and as V (ds_read_tr16_b64 transpose reads, which hand each lane 4 consecutive-slot values of one column).
// The LDS row stride is 1040 bytes and the slots of one PV K-step are visited in the order
// 8g + {0,2,4,6,1,3,5,7}, which keeps both read patterns free of bank conflicts.  When one row's heads give
// too few blocks to fill the chip, the slot range is split and a combine kernel merges the partial
// (o, lse) pairs.
#include "common.h"
#include "launch.h"

DSA_TIMELINE_UNIT(attn)

namespace dsa {
namespace {

constexpr int kHG = 16;                  // heads per block
constexpr int kNC = 64;                  // slots per chunk
constexpr int kDC = 512;                 // latent width of the bf16 path
constexpr int kRowB = kDC * 2 + 16;      // LDS row stride (bytes)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplitLen = 4096;       // selection slots one block handles
constexpr int kChunksPerSplitSmallBatch = 1;  // gathers spread over as many CUs as possible

typedef __attribute__((address_space(3))) v4bf lds_v4bf;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of the 8-byte reads of
// lanes 4m + i/4, m = 0..3.
__device__ __forceinline__ v4bf lds_tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_v4bf*)((__attribute__((address_space(3))) char*)(const_cast<char*>(p))));
}

__device__ __forceinline__ v8bf pack8(const float (&p)[8]) {
  v8bf r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)p[e];
  return r;
}

// 16-head kernel gathers: the 16 latent rows of this wave for one chunk, one 16-byte load per lane and row into
// registers (a slot without a position reads `dummy`, a selected row of the split, and is masked later), then
// written to LDS at row stride kRowB once the current chunk is computed.  The eight head groups of a (row, split)
// read the same rows from one L2, so the LDS-DMA path's per-CU issue rate, not HBM, bounded these gathers;
// register loads measured 0.4 us faster per batch-1 step.
__device__ __forceinline__ void load_chunk_regs(const unsigned short* __restrict__ kv, const int32_t* prow, int dummy,
                                                int wave, int lane, v4i (&gv)[16]) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    int pr = prow[wave * 16 + t];
    if (pr < 0) pr = dummy;
    gv[t] = *reinterpret_cast<const v4i*>(kv + (int64_t)pr * kDC + lane * 8);
  }
}
__device__ __forceinline__ void store_chunk_regs(char* buf, int wave, int lane, const v4i (&gv)[16]) {
#pragma unroll
  for (int t = 0; t < 16; ++t) *reinterpret_cast<v4i*>(buf + (wave * 16 + t) * kRowB + lane * 16) = gv[t];
}

// FP8 latent entries of 656 bytes: 512 e4m3 codes, 4 fp32 scales (one per 128-value tile), 64 bf16 RoPE values.
// The wave's 16 rows arrive in 11 loads per lane: load t (8 of them) gives lane l codes 16 (l % 32) .. +16 of
// row 2t + l / 32, one load gives lane l scale l % 4 of row l / 4, and two give lane l RoPE bytes 16 (l % 8) ..
// +16 of row 8j + l / 8.  The store widens the codes to bf16, which is exact, at the bf16 row layout (32 bytes
// at 32 (l % 32)); the scales go to a [tile][slot] table and the RoPE values into rows of their own.  The
// scales are applied outside the MFMAs: QK accumulates each 128-dim tile apart and sums the four with the slot's
// scales, and PV multiplies each slot's probability by its scale for the tile of the wave's 128 output columns.
// No dequantised value is ever rounded.
constexpr int kF8Entry = 656;
constexpr int kRope = 64;
constexpr int kRopeRowB = kRope * 2;  // LDS row stride of the RoPE part (bytes)
struct F8Rows {
  v4i codes[8];
  float scale;
  v4i rope[2];
};
__device__ __forceinline__ void load_chunk_fp8(const uint8_t* __restrict__ kv, const int32_t* prow, int dummy,
                                               int wave, int lane, F8Rows& f) {
  auto entry = [&](int row) {
    int pr = prow[wave * 16 + row];
    if (pr < 0) pr = dummy;
    return kv + (int64_t)pr * kF8Entry;
  };
#pragma unroll
  for (int t = 0; t < 8; ++t)
    f.codes[t] = *reinterpret_cast<const v4i*>(entry(2 * t + (lane >> 5)) + (lane & 31) * 16);
  f.scale = *reinterpret_cast<const float*>(entry(lane >> 2) + 512 + 4 * (lane & 3));
#pragma unroll
  for (int j = 0; j < 2; ++j)
    f.rope[j] = *reinterpret_cast<const v4i*>(entry(8 * j + (lane >> 3)) + 528 + 16 * (lane & 7));
}
__device__ __forceinline__ void store_chunk_fp8(char* buf, char* rope_buf, float* scale_buf, int wave, int lane,
                                                const F8Rows& f) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = wave * 16 + 2 * t + (lane >> 5);
    char* dst = buf + row * kRowB + (lane & 31) * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v2bf x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.codes[t][2 * h], 1.f, false);
      const v2bf x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.codes[t][2 * h], 1.f, true);
      const v2bf x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.codes[t][2 * h + 1], 1.f, false);
      const v2bf x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.codes[t][2 * h + 1], 1.f, true);
      *reinterpret_cast<v8bf*>(dst + 16 * h) = v8bf{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
    }
  }
  scale_buf[(lane & 3) * kNC + wave * 16 + (lane >> 2)] = f.scale;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    *reinterpret_cast<v4i*>(rope_buf + (wave * 16 + 8 * j + (lane >> 3)) * kRopeRowB + 16 * (lane & 7)) = f.rope[j];
}

// Split partials.  A split's o_s is a convex combination of its rows; it is stored as fp16 scaled by 2^-e per
// (row, split, head), e being the frexp exponent of the head's largest magnitude, so every stored value lies in
// (-1, 1) and its rounding is below 2^-12 of that maximum.  e is kept beside it.
__device__ __forceinline__ int part_exponent(float maxabs) {
  int e;
  frexpf(maxabs, &e);
  return maxabs > 0.f ? e : 0;
}
__device__ __forceinline__ unsigned short part_bits(float v, int e) {
  return __builtin_bit_cast(unsigned short, (_Float16)ldexpf(v, -e));
}
// Cross-lane reductions in the register file (DPP and lane-swap moves; no LDS round trip).
// Max over each aligned group of `width` (16 or 32) lanes: within a quad (quad_perm [1,0,3,2] then [2,3,0,1]),
// then between quads by row_half_mirror and between half-rows by row_mirror, then between rows by
// v_permlane16_swap.
__device__ __forceinline__ float max_over_lanes(float v, int width) {
  v = fmaxf(v, dpp_move<0xB1>(v));
  v = fmaxf(v, dpp_move<0x4E>(v));
  v = fmaxf(v, dpp_move<0x141>(v));
  v = fmaxf(v, dpp_move<0x140>(v));
  if (width == 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  return v;
}
// Max and sum over the lanes i, i + 16, i + 32, i + 48: v_permlane16_swap pairs rows 0-1 and 2-3, then
// v_permlane32_swap the two halves; every lane ends with the same value, summed in the same order.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Work of one block: a (row, split) pair and a head group.  Workgroups are handed to the eight XCDs in turn
// (block b runs on XCD b % 8).  The head groups of one pair gather the same rows, so they get block ids 8 apart
// and share an XCD and its L2; pair p = row * nsplit + split runs on XCD p % 8, so that the splits of even a
// single row spread over the whole chip.  The grid has ceil(R nsplit / 8) * 8 * ngroups blocks; a block past
// the last pair has no work.
struct BlockWork {
  int r, split, group;
};
__device__ __forceinline__ BlockWork block_work(int nsplit, int ngroups) {
  const int b = blockIdx.x, slot = b >> 3;
  const int pair = (slot / ngroups) * 8 + (b & 7);
  return BlockWork{pair / nsplit, pair % nsplit, slot % ngroups};
}
__host__ __forceinline__ int work_blocks(int64_t pairs, int ngroups) {
  return (int)((pairs + 7) / 8 * 8 * ngroups);
}

// Where slot s of a split (row r, slots begin ..) gets its row: the pool rows the fused top-k wrote beside the
// selection (already physical), the selected positions, or, with no selection (dense attention), position
// begin + s itself while it is below n_r.
struct SlotSource {
  const int32_t* list;  // nullptr: the identity selection
  int dense_n;          // identity: slots below this are positions
  int begin;
  bool physical;        // the entries are pool rows, not positions
  __device__ __forceinline__ int at(int s) const {
    return list ? list[s] : (s < dense_n ? begin + s : -1);
  }
};
__device__ __forceinline__ SlotSource slot_source(const int32_t* topk_idx, const int32_t* pool_rows,
                                                  const int32_t* row_len, int max_row_len, int r, int k, int begin) {
  const int64_t off = (int64_t)r * k + begin;
  if (pool_rows) return SlotSource{pool_rows + off, 0, begin, true};
  if (topk_idx) return SlotSource{topk_idx + off, 0, begin, false};
  return SlotSource{nullptr, clamp_len(row_len[r], max_row_len) - begin, begin, false};
}

// kFp8: the latent rows are 656-byte FP8 entries and the queries 576 wide (latent, then RoPE dims).
template <bool kSplit, bool kFp8>
__global__ __launch_bounds__(256) void attn_bf16_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ kv, const int32_t* __restrict__ topk_idx,
    int k, const int32_t* __restrict__ pool_rows, const int32_t* __restrict__ row_len, int max_row_len,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int H, int nsplit, int units, int split_len, float scale_log2,
    unsigned short* __restrict__ out,
    float* __restrict__ lse, unsigned short* __restrict__ part_o, int32_t* __restrict__ part_exp,
    float* __restrict__ part_lse) {
  struct ChunkLds {
    char kv0[kNC * kRowB];
    char kv1[kNC * kRowB];
    float s[kHG][kNC + 4];
    // RoPE rows of the FP8 path: read only by QK, so one buffer serves (a chunk's QK ends at its mid barrier, and
    // the next chunk's rows are stored after it)
    char rope[kFp8 ? kNC * kRopeRowB : 16];
    float scale[kFp8 ? 4 * kNC : 4];  // [tile][slot], same lifetime: every read of a chunk's scales happens before
                                      // its mid barrier
  };
  __shared__ __attribute__((aligned(16))) ChunkLds U;
  __shared__ int32_t prow_lds[kMaxSplitLen];  // physical row of every slot of the split, -1 = no position
  __shared__ int wave_first[4];               // first slot with a position among each wave's slots
  char* const kv_lds0 = U.kv0;
  char* const kv_lds1 = U.kv1;
  float (*const s_lds)[kNC + 4] = U.s;
  char* const rope_lds = U.rope;
  float* const scale_lds = U.scale;
  constexpr int kQW = kFp8 ? kDC + kRope : kDC;  // query width
  args_to_sgprs(q, kv, topk_idx, k, pool_rows, row_len, max_row_len, row_seq, page_table, num_seqs, max_pages,
                num_pages, log2ps, H, nsplit, units, split_len);
  DSA_STAMP(3, 0);

  const int ngroups = H / kHG;
  const BlockWork bw = block_work(nsplit, ngroups);
  if (bw.r >= units / ngroups) return;
  const int split = bw.split, grp16 = bw.group, r = bw.r;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;

  const int begin = split * split_len;
  const int end = min(k, begin + split_len);
  const int len = max(end - begin, 0);
  const int nch = (len + kNC - 1) / kNC;

  // The group's queries (16 heads x kQW bf16, contiguous) are read once per block, each load instruction one
  // contiguous 1 KiB run, and staged in the second chunk buffer (free until chunk 0 has been computed); the MFMA
  // A operands are read from there after the prologue's barrier.  Reading them straight into the operand layout
  // would make every lane fetch 16 bytes of a different row, which the vector L1 serves about a lane per cycle.
  constexpr int kQBytes = kHG * kQW * 2;          // per block
  constexpr int kQRowB = kQW * 2 + 16;            // LDS row stride of the staged queries
  constexpr int kQPieces = (kQBytes / 16 + 255) / 256;  // 16-byte pieces per thread (the last may be partial)
  static_assert(kQBytes % 16 == 0 && kHG * kQRowB <= kNC * kRowB, "queries fit the second chunk buffer");
  v4i qpiece[kQPieces];
  {
    const char* qsrc = reinterpret_cast<const char*>(q + ((int64_t)r * H + grp16 * kHG) * kQW);
#pragma unroll
    for (int j = 0; j < kQPieces; ++j)  // a piece past the group's queries rereads its last one (not stored)
      qpiece[j] = *reinterpret_cast<const v4i*>(qsrc + (size_t)min(j * 256 + (int)threadIdx.x, kQBytes / 16 - 1) * 16);
  }
  DSA_STAMP(3, 6);

  // Every slot of the split -> physical row before any gather, so that the gathers are the only loads in
  // flight later.  With a list, every entry load is issued at once (after the queries) from an in-range address
  // (the value is dropped past the split's end); positions then take one round of page-table loads, issued
  // together, or the pool rows the top-k wrote beside the selection are used directly.
  constexpr int kSlotsPerThread = kMaxSplitLen / 256;
  int pr[kSlotsPerThread];
  {
    const SlotSource src = slot_source(topk_idx, pool_rows, row_len, max_row_len, r, k, begin);
    if (src.list) {
      if (len > 0)
#pragma unroll
        for (int j = 0; j < kSlotsPerThread; ++j) {
          // only the rounds that hold slots of the split load (uniform): a 64-slot split takes one, not sixteen
          const int s = j * 256 + threadIdx.x;
          const int v = j * 256 < len ? src.list[min(s, len - 1)] : -1;
          pr[j] = s < len ? v : -1;
        }
      else
#pragma unroll
        for (int j = 0; j < kSlotsPerThread; ++j) pr[j] = -1;
    } else {
#pragma unroll
      for (int j = 0; j < kSlotsPerThread; ++j) {
        const int s = j * 256 + threadIdx.x;
        pr[j] = s < len && s < src.dense_n ? begin + s : -1;
      }
    }
  }
  DSA_STAMP(3, 7);
  {
    const bool physical = pool_rows != nullptr;
    if (!physical) {
      const int32_t* pt = page_table + (int64_t)clamp_seq(row_seq[r], num_seqs) * max_pages;
      int pg[kSlotsPerThread];
#pragma unroll
      for (int j = 0; j < kSlotsPerThread; ++j)
        pg[j] = j * 256 < len ? pt[min(max(pr[j], 0) >> log2ps, max_pages - 1)] : 0;
#pragma unroll
      for (int j = 0; j < kSlotsPerThread; ++j)
        pr[j] = pr[j] >= 0 ? (min(max(pg[j], 0), num_pages - 1) << log2ps) | (pr[j] & ((1 << log2ps) - 1)) : -1;
    }
    // slot j * 256 + 64 wave + lane; the wave's first slot with a position comes from the ballots
    int first = 0x7fffffff;
#pragma unroll
    for (int j = kSlotsPerThread - 1; j >= 0; --j) {
      const int s = j * 256 + threadIdx.x;
      if (s < nch * kNC) prow_lds[s] = pr[j];
      const uint64_t bits = __ballot(pr[j] >= 0);
      if (bits) first = j * 256 + wave * 64 + (int)__builtin_ctzll(bits);
    }
    if (lane == 0) wave_first[wave] = first;
  }
  DSA_STAMP(3, 1);
#pragma unroll
  for (int j = 0; j < kQPieces; ++j) {
    const int piece = j * 256 + threadIdx.x, b = piece * 16;  // byte b of the group's queries
    if (b < kQBytes) *reinterpret_cast<v4i*>(kv_lds1 + (b / (kQW * 2)) * kQRowB + b % (kQW * 2)) = qpiece[j];
  }
  DSA_STAMP(3, 9);

  v4f o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running max (log2 domain) and sum for head i
  __syncthreads();
  // Q as A operands: head grp16*16 + i, d = kd*32 + g*8 .. +8 (and the RoPE dims 512 + kd*32 + g*8 .. +8)
  v8bf qa[kDC / 32];
  v8bf qr[kFp8 ? kRope / 32 : 1];
  {
    const char* qrow = kv_lds1 + i * kQRowB + g * 16;
#pragma unroll
    for (int kd = 0; kd < kDC / 32; ++kd) qa[kd] = *reinterpret_cast<const v8bf*>(qrow + kd * 64);
    if constexpr (kFp8)
#pragma unroll
      for (int kd = 0; kd < kRope / 32; ++kd) qr[kd] = *reinterpret_cast<const v8bf*>(qrow + kDC * 2 + kd * 64);
  }
  const int first_valid = min(min(wave_first[0], wave_first[1]), min(wave_first[2], wave_first[3]));
  // a split with no selected row contributes nothing; otherwise slots without a position read a selected row
  // of this split instead (their logits are -inf, so they carry zero weight)
  if (first_valid != 0x7fffffff) {
    const int dummy = prow_lds[first_valid];
    // one chunk: wait for its rows (the next chunk's gather stays in flight), then QK^T, softmax, PV.
    // `cur` and `nxt` are fixed per call site, so the compiler can tell the DMA target from the buffer read.
    const uint8_t* kv8 = reinterpret_cast<const uint8_t*>(kv);
    v4i gv[kFp8 ? 1 : 16];
    F8Rows fv;
    auto gather = [&](const int32_t* prow) __attribute__((always_inline)) {
      if constexpr (kFp8)
        load_chunk_fp8(kv8, prow, dummy, wave, lane, fv);
      else
        load_chunk_regs(kv, prow, dummy, wave, lane, gv);
    };
    auto place = [&](char* buf) __attribute__((always_inline)) {
      if constexpr (kFp8)
        store_chunk_fp8(buf, rope_lds, scale_lds, wave, lane, fv);
      else
        store_chunk_regs(buf, wave, lane, gv);
    };
    auto chunk = [&](const int c, const char* cur, char* nxt) __attribute__((always_inline)) {
      if (c + 1 < nch) gather(prow_lds + (c + 1) * kNC);
      // S for slots wave*16 + (0..15): B operand = row (wave*16 + i), d = kd*32 + g*8 .. +8
      v4f sacc = {0.f, 0.f, 0.f, 0.f};
      v4f pvs[kFp8 ? 4 : 1];  // FP8: the PV scales, read before the mid-chunk barrier (the table is rewritten after)
      if constexpr (!kFp8) {
        const char* brow = cur + (wave * 16 + i) * kRowB + g * 16;
#pragma unroll
        for (int kd = 0; kd < kDC / 32; ++kd) {
          const v8bf b = *reinterpret_cast<const v8bf*>(brow + kd * 64);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kd], b, sacc, 0, 0, 0);
        }
      } else {
        // one accumulator per 128-dim tile of codes, then the RoPE dims; the lane's slot is wave*16 + i
        v4f st[4] = {};
        const char* brow = cur + (wave * 16 + i) * kRowB + g * 16;
#pragma unroll
        for (int kd = 0; kd < kDC / 32; ++kd) {
          const v8bf b = *reinterpret_cast<const v8bf*>(brow + kd * 64);
          st[kd >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kd], b, st[kd >> 2], 0, 0, 0);
        }
        const char* rrow = rope_lds + (wave * 16 + i) * kRopeRowB + g * 16;
#pragma unroll
        for (int kd = 0; kd < kRope / 32; ++kd) {
          const v8bf b = *reinterpret_cast<const v8bf*>(rrow + kd * 64);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr[kd], b, sacc, 0, 0, 0);
        }
        const float* sl = scale_lds + wave * 16 + i;
        const float s0 = sl[0], s1 = sl[kNC], s2 = sl[2 * kNC], s3 = sl[3 * kNC];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sacc[v] = fmaf(st[3][v], s3, fmaf(st[2][v], s2, fmaf(st[1][v], s1, fmaf(st[0][v], s0, sacc[v]))));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          pvs[2 * kk] = *reinterpret_cast<const v4f*>(&scale_lds[wave * kNC + kk * 32 + 8 * g]);
          pvs[2 * kk + 1] = *reinterpret_cast<const v4f*>(&scale_lds[wave * kNC + kk * 32 + 8 * g + 4]);
        }
      }
      const bool valid = prow_lds[c * kNC + wave * 16 + i] >= 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) s_lds[g * 4 + v][wave * 16 + i] = valid ? sacc[v] * scale_log2 : -INFINITY;
      lds_barrier();

      // online softmax for head i over slots kk*32 + 8g + (0..7), kk = 0, 1
      float sv[16];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const v4f x0 = *reinterpret_cast<const v4f*>(&s_lds[i][kk * 32 + 8 * g]);
        const v4f x1 = *reinterpret_cast<const v4f*>(&s_lds[i][kk * 32 + 8 * g + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) { sv[kk * 8 + e] = x0[e]; sv[kk * 8 + 4 + e] = x1[e]; }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sv[e]);
      mx = rows_max(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) { sv[e] = exp2f(sv[e] - m_use); rs += sv[e]; }
      rs = rows_sum(rs);
      l = l * alpha + rs;
      m = m_new;

      // rescale O rows (head g*4 + v) by that head's alpha, held by lane g*4 + v (O is still zero in chunk 0)
      if (c > 0)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float av = __shfl(alpha, g * 4 + v, 64);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[dt][v] *= av;
        }

      // O += P V.  A operand element e of K-step kk is slot kk*32 + 8g + perm[e], perm = {0,2,4,6,1,3,5,7}.
      // FP8 entries: the wave's 128 output columns are tile `wave`, so each probability takes its slot's scale
      // for that tile; that product is split into its bf16 rounding and the bf16 rounding of what is left (2^-17
      // relative together), and both go through the MFMA, so no dequantised value is rounded on its way to O
      if constexpr (kFp8)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[kk * 8 + e] *= pvs[2 * kk][e];
            sv[kk * 8 + 4 + e] *= pvs[2 * kk + 1][e];
          }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const float pe[8] = {sv[kk * 8 + 0], sv[kk * 8 + 2], sv[kk * 8 + 4], sv[kk * 8 + 6],
                             sv[kk * 8 + 1], sv[kk * 8 + 3], sv[kk * 8 + 5], sv[kk * 8 + 7]};
        const v8bf pa = pack8(pe);
        v8bf pa_lo;
        if constexpr (kFp8) {
          float rest[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) rest[e] = pe[e] - (float)pa[e];  // exact: the low part of pe[e]
          pa_lo = pack8(rest);
        }
        const int row1 = kk * 32 + 8 * g + 2 * (i >> 2);
        const char* p1 = cur + row1 * kRowB + (wave * 128 + 4 * (i & 3)) * 2;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const v4bf lo4 = lds_tr_read(p1 + dt * 32);
          const v4bf hi4 = lds_tr_read(p1 + kRowB + dt * 32);
          const v8bf b = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b, o[dt], 0, 0, 0);
          if constexpr (kFp8) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b, o[dt], 0, 0, 0);
        }
      }
      if (c + 1 < nch) place(nxt);
      lds_barrier();  // every wave is done with `cur` and s_lds before they are overwritten; `nxt` is written
    };
    DSA_STAMP(3, 2);
    gather(prow_lds);
    place(kv_lds0);
    lds_barrier();
    DSA_STAMP(3, 3);
    for (int c = 0; c < nch; c += 2) {
      chunk(c, kv_lds0, kv_lds1);
      if (c + 1 < nch) chunk(c + 1, kv_lds1, kv_lds0);
    }
    DSA_STAMP(3, 4);
  }

  // finish: O rows are heads g*4 + v, columns wave*128 + dt*16 + i
  const int64_t head0 = (int64_t)r * H + grp16 * kHG;
  if (kSplit) {
    // each head's largest |o| over the block's four waves (128 columns each), for its partial exponent
    float* wmax = &s_lds[0][0];  // [4 waves][16 heads]; s_lds is free after the last chunk
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mx = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) mx = fmaxf(mx, fabsf(o[dt][v]));
      mx = max_over_lanes(mx, 16);
      if (i == 0) wmax[wave * kHG + g * 4 + v] = mx;
    }
    __syncthreads();
  }
  DSA_STAMP(3, 10);
  // split partials go out as 16-byte stores: each wave stages its 16 heads x 128 columns of fp16 bits in LDS
  // (rows padded to 136 halves so the four heads of one write land on different banks), then every lane stores
  // four 8-column pieces; the chunk buffers are free once the last chunk's barrier has passed
  constexpr int kStgRow = 136;
  unsigned short* stg = reinterpret_cast<unsigned short*>(kv_lds0) + wave * (kHG * kStgRow);
  // the four heads' sums and largest magnitudes are read before any is used (one LDS round trip, not four), and
  // each head's power-of-two partial scale folds into its 1 / l: o (2^-e / l) equals 2^-e (o / l) but for
  // subnormal values
  float lvs[4], mxs[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) lvs[v] = __shfl(l, g * 4 + v, 64);
  if (kSplit) {
    const float* wmax = &s_lds[0][0];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = g * 4 + v;
      mxs[v] = fmaxf(fmaxf(wmax[hh], wmax[kHG + hh]), fmaxf(wmax[2 * kHG + hh], wmax[3 * kHG + hh]));
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int hh = g * 4 + v;
    const float lv = lvs[v];
    const float inv = lv > 0.f ? 1.f / lv : 0.f;
    if (kSplit) {
      // l >= 1 (the largest term is 1), so 2^-e / l stays finite with e clamped at -100; values below 2^-100
      // then store as smaller fp16 codes against the same exponent
      const int e = max(part_exponent(mxs[v] * inv), -100);
      const float sc = ldexpf(inv, -e);
      const int64_t prow = ((int64_t)r * nsplit + split) * H + grp16 * kHG + hh;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        stg[hh * kStgRow + dt * 16 + i] = __builtin_bit_cast(unsigned short, (_Float16)(o[dt][v] * sc));
      if (wave == 0 && i == 0) part_exp[prow] = e;
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        out[(head0 + hh) * kDC + wave * 128 + dt * 16 + i] = float_to_bf16_bits(o[dt][v] * inv);
    }
  }
  if (kSplit) {
    // this wave's own staging rows: its LDS writes are complete before its reads (no other wave touches them);
    // the empty asm keeps the compiler from moving the 16-byte reads above the 2-byte writes
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    DSA_STAMP(3, 11);
    const int64_t prow0 = ((int64_t)r * nsplit + split) * H + grp16 * kHG;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = j * 64 + lane, hh = piece >> 4, c8 = piece & 15;  // head, 8-column piece
      const v4i x = *reinterpret_cast<const v4i*>(stg + hh * kStgRow + c8 * 8);
      // non-temporal: the combine reads the partials next, and dirty lines left in the L2 lengthen the kernel's
      // end (-0.3 us per 128K step)
      __builtin_nontemporal_store(x, reinterpret_cast<v4i*>(part_o + (prow0 + hh) * kDC + wave * 128 + c8 * 8));
    }
  }
  if (wave == 0 && g == 0) {
    const float lz = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    if (kSplit)
      part_lse[((int64_t)r * nsplit + split) * H + grp16 * kHG + i] = lz;
    else if (lse)
      lse[head0 + i] = lz;
  }
  DSA_STAMP(3, 5);
}

// ---------------------------------------------------------------------------------------------------------
// bf16 path, all heads of a row per block.  Every head of a row reads the same latent rows (MQA), so a block
// that owns up to 128 heads gathers each selected row once instead of once per 16-head group.  Wave w owns
// 32 heads and computes, per 32-slot chunk:
//   S^T = C Q^T on v_mfma_f32_32x32x16_bf16 with the gathered rows as the A operand (row-contiguous 16-byte
//       LDS reads) and Q^T held in registers (32 K-steps x 8 bf16).  Lane (half h, column n) then holds the 16
//       S^T rows 8 (i >> 2) + 4 h + (i & 3) of the chunk for head n, so the softmax of a head is an in-lane
//       reduction plus one v_permlane32_swap with the other half.
//   O += P C with P as the A operand: K position 8 h + j of K-step ks is S^T row 16 ks + 4 h + (j & 3) +
//       8 (j >> 2), which is exactly the lane's own probability i = 8 ks + j, so P needs no exchange; the B
//       operand is read with ds_read_b64_tr_b16 (four slots of one latent column per lane, two reads per
//       K-step).
// O (32 heads x 512 columns, fp32) is 256 accumulator registers per wave, so one wave runs per SIMD.  The
// gathers are LDS-DMA loads, whose throughput per CU is bounded by the loads it keeps in flight; a ring of
// four chunk buffers keeps the next three chunks' gathers in flight behind the current chunk's MFMAs.
//
// LDS bank conflicts (32 four-byte banks): the LDS row stride is 1040 bytes (260 dwords, 4 mod 32), and the
// QK A operand of lane m reads row 8 (m >> 3) + tau(m & 7), tau = {0,2,4,6,1,3,5,7}.  Eight consecutive
// lanes then read rows whose 16-byte pieces start 4 tau(x) banks apart, and the four rows behind one
// transpose read (slots 4 h + e of a K-step become rows 2 e + h) start 8 banks apart; both patterns are
// conflict-free.  The permutation is only a relabelling of which slot each S^T row holds.
constexpr int kRowW = kDC * 2 + 16;
constexpr int kWideMaxSplitLen = 2048;  // selection slots one block handles

constexpr int kCW = 32;    // slots per chunk: one S^T tile
constexpr int kBufW = 4;   // LDS ring of gathered chunks

template <int NW>  // waves per block: 32 * NW heads
__device__ __forceinline__ void gather_chunk_wide(const unsigned short* __restrict__ kv, const int32_t* prow,
                                                  int dummy, char* buf, int wave, int lane) {
  constexpr int kRows = kCW / NW;
  int prs[kRows];  // every row id first: one LDS round trip rather than one per load (the asm clobbers memory)
#pragma unroll
  for (int t = 0; t < kRows; ++t) prs[t] = prow[wave * kRows + t];
#pragma unroll
  for (int t = 0; t < kRows; ++t) {
    const int rr = wave * kRows + t;
    const int pr = prs[t] < 0 ? dummy : prs[t];
    const unsigned short* src = kv + (int64_t)pr * kDC + lane * 8;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(buf + rr * kRowW)));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
  }
}

// FP8 entries in the all-heads kernel.  A chunk's 32 entries (656 bytes each) are gathered raw by LDS-DMA into
// one of kF8Ring staging slots, packed at 656-byte strides, one load of 41 lanes per entry (wave w gathers entries
// 8 w .. 8 w + 7); loads that each cover 64 16-byte pieces, crossing entries, took twice as long to issue per byte.
// Both products read the e4m3 codes straight from the staging slot and widen them to bf16 in registers (exact: an
// e4m3 value has a 4-bit significand): QK with 16-byte reads that serve two K-steps, PV with transposed 8-bit
// reads.  The tile scales are applied outside the MFMAs: QK accumulates each 128-dim tile on its own and adds it in
// with the slot's scale; PV multiplies each probability by its slot's scale for the tile of the output columns and
// splits that product into a bf16 head and a bf16 rest, both of which go through the MFMA.  No dequantised value
// is rounded.  Register i of an S^T tile holds the same slot in every lane of a lane half, so lane l loads the four
// scales of the slot that register l % 16 holds in its half, and a DPP row_newbcast:i hands register i's scale to
// every lane of the row (rows 0-1 are half 0, rows 2-3 half 1).  The RoPE dims are read by QK from the slot too.
constexpr int kF8RopeByte = kDC + 16;          // RoPE values follow the codes and the four scales
constexpr int kF8Pieces = kF8Entry / 16;        // 41 16-byte pieces per entry: one LDS-DMA load of 41 lanes
constexpr int kF8RowsPerWave = kCW / 4;          // rows (loads) each of the four waves gathers per chunk
constexpr int kF8Slot = kCW * kF8Entry;          // staging slot bytes
constexpr int kF8Ring = 4;                       // staging slots: the chunk computed, three in flight (six spilled)
static_assert(kF8Entry % 16 == 0 && kF8Pieces <= 64, "an entry fits one load");

__device__ __forceinline__ void gather_chunk_f8(const uint8_t* __restrict__ kv, const int32_t* prow, int dummy,
                                                char* slot, int wave, int lane) {
  // The row ids first (one LDS round trip: the asm statements clobber memory), then one load per row.  The LDS
  // address is wave-uniform (scalar registers).
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)slot));
  int pr[kF8RowsPerWave];
#pragma unroll
  for (int t = 0; t < kF8RowsPerWave; ++t) pr[t] = prow[w * kF8RowsPerWave + t];
#pragma unroll
  for (int t = 0; t < kF8RowsPerWave; ++t) {
    const int r = pr[t] < 0 ? dummy : pr[t];
    const uint8_t* src = kv + (int64_t)r * kF8Entry + 16 * min(lane, kF8Pieces - 1);
    const uint32_t lds = base + (uint32_t)((w * kF8RowsPerWave + t) * kF8Entry);
    if (lane < kF8Pieces)
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
  }
}

// Slot order of the FP8 path: MFMA row m (an A row of QK, a K index of PV) holds slot f8_slot(m), which swaps
// rows 8..11 with 12..15 in each 16.  With 656-byte (164-dword, 4 banks mod 32) rows, the eight lanes of a 16-byte
// QK read (rows f8_slot(0..7), or f8_slot(8..15)) and the sixteen lanes of a PV transposed read (the rows of K
// indices 8 kh + 0..7, two 8-byte pieces each) then cover all 32 banks.
__device__ __forceinline__ int f8_slot(int m) { return m ^ (((m >> 3) & 1) << 2); }

// Register i's value of a per-row quantity held by lanes 16 r + i, applied through the DPP row_newbcast:i source
// of a VOP2 instruction, two registers (2 e, 2 e + 1) at a time: bcast_mul2 gives x = bcast_i(s) * st[i], and
// bcast_fma2 adds bcast_i(s) * a[i] to st[i].  Written out because the compiler kept a separate DPP move per use;
// two at a time so that the work can sit between MFMAs.  The s_nop covers the VALU-write-to-DPP-read hazard on s.
// All 64 lanes must be active.
template <int kE>
__device__ __forceinline__ void bcast_mul2(float& x0, float& x1, float s, float st0, float st1);
template <int kE>
__device__ __forceinline__ void bcast_fma2(float& st0, float& st1, float s, float a0, float a1);
template <>
__device__ __forceinline__ void bcast_mul2<0>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:1 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<0>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:1 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<1>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:3 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<1>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:3 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<2>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:5 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<2>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:5 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<3>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:7 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<3>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:7 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<4>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:9 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<4>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:9 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<5>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:11 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<5>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:11 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<6>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:13 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<6>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:13 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}
template <>
__device__ __forceinline__ void bcast_mul2<7>(float& x0, float& x1, float s, float st0, float st1) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %2, %3 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %2, %4 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "=&v"(x0), "=&v"(x1) : "v"(s), "v"(st0), "v"(st1));
}
template <>
__device__ __forceinline__ void bcast_fma2<7>(float& st0, float& st1, float s, float a0, float a1) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %2, %4 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "+v"(st0), "+v"(st1) : "v"(s), "v"(a0), "v"(a1));
}

// Registers 2 e, 2 e + 1 of tile scale s times the probabilities st, split into a bf16 head (the top 16 bits) and
// a bf16 rest (the exact remainder, rounded): dword e & 3 of the K-step e >> 2 operands hp and lp.
template <int kE>
__device__ __forceinline__ void split_pair(const v16f& st, float s, v4i (&hp)[2], v4i (&lp)[2]) {
  float x0, x1;
  bcast_mul2<kE>(x0, x1, s, st[2 * kE], st[2 * kE + 1]);
  const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
  const float l0 = x0 - __uint_as_float(b0 & 0xffff0000u), l1 = x1 - __uint_as_float(b1 & 0xffff0000u);
  hp[kE >> 2][kE & 3] = (int)__builtin_amdgcn_perm(b1, b0, 0x07060302u);  // top halves of b0, b1
  const v2bf lb = v2bf{(__bf16)l0, (__bf16)l1};
  lp[kE >> 2][kE & 3] = (int)__builtin_bit_cast(uint32_t, lb);
}
__device__ __forceinline__ void split_pair_n(int e, const v16f& st, float s, v4i (&hp)[2], v4i (&lp)[2]) {
  switch (e) {  // e is a constant wherever this is inlined
    case 0: split_pair<0>(st, s, hp, lp); break;
    case 1: split_pair<1>(st, s, hp, lp); break;
    case 2: split_pair<2>(st, s, hp, lp); break;
    case 3: split_pair<3>(st, s, hp, lp); break;
    case 4: split_pair<4>(st, s, hp, lp); break;
    case 5: split_pair<5>(st, s, hp, lp); break;
    case 6: split_pair<6>(st, s, hp, lp); break;
    default: split_pair<7>(st, s, hp, lp); break;
  }
}
__device__ __forceinline__ void fold_pair_n(int e, v16f& st, const v16f& a, float s) {
  float s0 = st[2 * e], s1 = st[2 * e + 1];
  switch (e) {
    case 0: bcast_fma2<0>(s0, s1, s, a[0], a[1]); break;
    case 1: bcast_fma2<1>(s0, s1, s, a[2], a[3]); break;
    case 2: bcast_fma2<2>(s0, s1, s, a[4], a[5]); break;
    case 3: bcast_fma2<3>(s0, s1, s, a[6], a[7]); break;
    case 4: bcast_fma2<4>(s0, s1, s, a[8], a[9]); break;
    case 5: bcast_fma2<5>(s0, s1, s, a[10], a[11]); break;
    case 6: bcast_fma2<6>(s0, s1, s, a[12], a[13]); break;
    default: bcast_fma2<7>(s0, s1, s, a[14], a[15]); break;
  }
  st[2 * e] = s0;
  st[2 * e + 1] = s1;
}

// kFp8: the latent rows are 656-byte FP8 entries (four waves only), dequantised into hi and lo bf16 rows; the
// queries are 576 wide (latent, then RoPE dims).
template <int NW, bool kSplit, bool kFp8>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_mqa_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ kv, const int32_t* __restrict__ topk_idx,
    int k, const int32_t* __restrict__ pool_rows, const int32_t* __restrict__ row_len, int max_row_len,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int H, int nsplit, int units, int split_len, float scale_log2,
    unsigned short* __restrict__ out,
    float* __restrict__ lse, unsigned short* __restrict__ part_o, int32_t* __restrict__ part_exp,
    float* __restrict__ part_lse) {
  static_assert(kCW % NW == 0, "every wave gathers the same number of rows");
  static_assert(!kFp8 || NW == 4, "FP8 entries: eight rows per wave and chunk");
  args_to_sgprs(q, kv, topk_idx, k, pool_rows, row_len, max_row_len, row_seq, page_table, num_seqs, max_pages,
                num_pages, log2ps, H, nsplit, units, split_len);
  DSA_STAMP(5, 0);
  constexpr int kRows = kCW / NW;  // rows each wave gathers per chunk
  // chunks gathered ahead: at the wait for chunk c, the kDepth - 1 chunks after it may still be in flight,
  // which must fit vmcnt (at most 63 outstanding loads per wave)
  constexpr int kDepth = kBufW < 63 / kRows + 1 ? kBufW : 63 / kRows + 1;
  static_assert(kDepth >= 2 && (kDepth - 1) * kRows <= 63, "gathers in flight fit vmcnt");
  // bf16 rows: a ring of kBufW chunks filled by LDS-DMA; FP8 entries: a ring of kF8Ring staging slots
  constexpr int kPool = kFp8 ? kF8Ring * kF8Slot : kBufW * kCW * kRowW;
  __shared__ __attribute__((aligned(16))) char kv_pool_lds[kPool];
  __shared__ int32_t prow_lds[kWideMaxSplitLen];           // physical row of every slot, -1 = no position
  __shared__ uint32_t valid_lds[kWideMaxSplitLen / 32];    // bit per slot: it has a position
  __shared__ int wave_first[NW], overflow;  // first slot with a position among each wave's slots

  const int ngroups = H / (32 * NW);
  const BlockWork bw = block_work(nsplit, ngroups);
  if (bw.r >= units / ngroups) return;
  const int split = bw.split, hg = bw.group, r = bw.r;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int hw = hg * 32 * NW + wave * 32;  // first head of this wave

  const int begin = split * split_len;
  const int end = min(k, begin + split_len);
  const int len = max(end - begin, 0);
  const int nch = (len + kCW - 1) / kCW;  // chunks of kCW slots
  const int n64 = (len + 63) / 64;

  // Q^T as B operands: lane (half, col) = head hw + col, latent columns 16 ks + 8 half .. +8; issued first so that
  // they load while the positions and then the page-table entries arrive
  v8bf qb[kDC / 16];
  v8bf qr[kFp8 ? kRope / 16 : 1];  // RoPE dims of the FP8 path
  {
    constexpr int kQW = kFp8 ? kDC + kRope : kDC;  // query row width
    const unsigned short* qrow = q + ((int64_t)r * H + hw + col) * kQW + 8 * half;
    // FP8 entries: K-step ks takes, in lane half h, dims 32 (ks >> 1) + 16 h + 8 (ks & 1) .. +8, so that one
    // 16-byte read of a staged row's codes serves two K-steps
#pragma unroll
    for (int ks = 0; ks < kDC / 16; ++ks)
      qb[ks] = *reinterpret_cast<const v8bf*>(kFp8 ? qrow + 8 * half + 32 * (ks >> 1) + 8 * (ks & 1) : qrow + 16 * ks);
    if constexpr (kFp8)
#pragma unroll
      for (int ks = 0; ks < kRope / 16; ++ks) qr[ks] = *reinterpret_cast<const v8bf*>(qrow + kDC + 16 * ks);
  }
  v16f o[kDC / 32];  // O tile dt: column 32 dt + col, head 8 (i >> 2) + 4 half + (i & 3)

  // Slots -> physical rows: all position loads are issued together (from in-range addresses, the values dropped
  // past the split's end), then all page-table loads.  Slot j * 64 NW + 64 wave + lane belongs to 64-slot group
  // j NW + wave, so a ballot gives the validity bits of two chunks.
  constexpr int kSlotsPerThread = kWideMaxSplitLen / (64 * NW);
  const SlotSource src = slot_source(topk_idx, pool_rows, row_len, max_row_len, r, k, begin);
  int pr[kSlotsPerThread];
  if (src.list && len > 0) {
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      // only the rounds that hold slots of the split load (uniform over the block)
      const int sl = (j * NW + wave) * 64 + lane;
      const int v = j * NW * 64 < len ? src.list[min(sl, len - 1)] : -1;
      pr[j] = sl < len ? v : -1;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int sl = (j * NW + wave) * 64 + lane;
      pr[j] = !src.list && sl < len && sl < src.dense_n ? begin + sl : -1;
    }
  }
  if (!src.physical) {
    const int32_t* pt = page_table + (int64_t)clamp_seq(row_seq[r], num_seqs) * max_pages;
    int pg[kSlotsPerThread];
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j)
      pg[j] = j * NW * 64 < len ? pt[min(max(pr[j], 0) >> log2ps, max_pages - 1)] : 0;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j)
      pr[j] = pr[j] >= 0 ? (min(max(pg[j], 0), num_pages - 1) << log2ps) | (pr[j] & ((1 << log2ps) - 1)) : -1;
  }
  {
    int first = 0x7fffffff;
#pragma unroll
    for (int j = kSlotsPerThread - 1; j >= 0; --j) {
      const int c = j * NW + wave;
      if (c < n64) {
        prow_lds[c * 64 + lane] = pr[j];
        const uint64_t bits = __ballot(pr[j] >= 0);
        if (lane == 0) {
          valid_lds[2 * c] = (uint32_t)bits;
          valid_lds[2 * c + 1] = (uint32_t)(bits >> 32);
        }
        if (bits) first = c * 64 + (int)__builtin_ctzll(bits);
      }
    }
    if (lane == 0) wave_first[wave] = first;
    if (threadIdx.x == 0) overflow = 0;
  }
  __syncthreads();
  DSA_STAMP(5, 1);
  int first_valid = wave_first[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) first_valid = min(first_valid, wave_first[w]);

  // Softmax without rescaling O.  Every head accumulates p = 2^(s - m_ref) against a fixed reference: the
  // largest logit of the first chunk in which it has one.  O and l are then plain sums, and o = O / l,
  // lse = m_ref + log2 l are exact; probabilities of later, larger logits exceed 1, which fp32 sums and bf16
  // MFMA operands hold without loss of relative precision.  Only a logit more than kHeadroom above the
  // reference could overflow; then the block recomputes against the exact maximum of a QK-only pass.
  constexpr float kHeadroom = 64.f;
  float m_ref = -INFINITY, l = 0.f;  // of head hw + col (the same in both lane halves)
  if (first_valid != 0x7fffffff) {
    const int dummy = prow_lds[first_valid];
    const int S16 = lane & 15, qh = (lane >> 4) & 1;  // transpose-read lane roles
    // One chunk: S^T tile, softmax, O += P C.  qk_only: only track the per-head maximum (into m_ref);
    // otherwise accumulate O and l.
    // FP8 entries: `cur` is the chunk's code buffer and `raw` its staging slot (RoPE dims).
    auto chunk = [&](const int c, const char* cur, const char* raw, const bool qk_only) __attribute__((always_inline)) {
      // S^T: slots 0..31 of the chunk (A rows) x this wave's 32 heads (B columns).  The A operands are read
      // kQkDepth K-steps ahead of their MFMAs; sched_barrier keeps the compiler from hoisting further.
      v16f st = {};
      // the slot this lane's A row holds (FP8: see f8_slot)
      const int arow_i = kFp8 ? f8_slot(col) : 8 * (col >> 3) + 2 * (col & 3) + ((col >> 2) & 1);
      // FP8: the four tile scales of the slot register (lane % 16) holds in this lane's half
      v4f sc = {};
      if constexpr (kFp8) {
        const int sl = f8_slot(8 * ((lane & 15) >> 2) + 4 * half + (lane & 3));
        sc = *reinterpret_cast<const v4f*>(raw + sl * kF8Entry + kDC);
      }
      if constexpr (kFp8) {
        // Each 128-dim tile of codes on an accumulator of its own, added in with the scales of this lane's rows
        // (row_newbcast:i gives register i's), then the RoPE K-steps straight onto st.  The A operands are read
        // from the staged entries as e4m3 codes, 16 bytes (two K-steps) per read, and widened to bf16 in
        // registers: half the LDS bytes of reading the widened rows, which the four waves' QK reads saturate.
        constexpr int kQkDepth = 2;  // reads (K-step pairs) ahead
        const char* araw = raw + arow_i * kF8Entry + 16 * half;
        v4i abuf[kQkDepth];
#pragma unroll
        for (int j = 0; j < kQkDepth; ++j) abuf[j] = *reinterpret_cast<const v4i*>(araw + 32 * j);
        auto widen = [](v4i c, int odd) __attribute__((always_inline)) {  // codes of K-step 2 j + odd
          const uint32_t d0 = (uint32_t)c[2 * odd], d1 = (uint32_t)c[2 * odd + 1];
          const v2bf x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.f, false);
          const v2bf x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.f, true);
          const v2bf x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.f, false);
          const v2bf x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.f, true);
          return v8bf{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
        };
        v16f acc[2];
#pragma unroll
        for (int t = 0; t < 5; ++t) {
          // tile t's K-steps, each followed by a quarter of the previous tile's fold (two registers), so that
          // the fold's VALU work runs while the MFMAs do
          if (t < 4) acc[t & 1] = v16f{};
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const int ks = 8 * t + kk, j = ks >> 1;
            if (t < 4) {
              acc[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen(abuf[j % kQkDepth], ks & 1), qb[ks],
                                                                   acc[t & 1], 0, 0, 0);
              if ((ks & 1) && j + kQkDepth < kDC / 32)
                abuf[j % kQkDepth] = *reinterpret_cast<const v4i*>(araw + 32 * (j + kQkDepth));
            }
            if (t > 0) fold_pair_n(kk, st, acc[(t - 1) & 1], sc[t - 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        const char* rrow = raw + arow_i * kF8Entry + kF8RopeByte + 16 * half;
#pragma unroll
        for (int ks = 0; ks < kRope / 16; ++ks)
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const v8bf*>(rrow + 32 * ks), qr[ks], st, 0,
                                                       0, 0);
      } else {
        constexpr int kQkDepth = 8;
        const char* arow = cur + arow_i * kRowW + 16 * half;
        v8bf abuf[kQkDepth];
#pragma unroll
        for (int ks = 0; ks < kQkDepth; ++ks) abuf[ks] = *reinterpret_cast<const v8bf*>(arow + 32 * ks);
#pragma unroll
        for (int ks = 0; ks < kDC / 16; ++ks) {
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abuf[ks % kQkDepth], qb[ks], st, 0, 0, 0);
          if (ks + kQkDepth < kDC / 16)
            abuf[ks % kQkDepth] = *reinterpret_cast<const v8bf*>(arow + 32 * (ks + kQkDepth));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // logits in the log2 domain; slots without a position get -inf
      const uint32_t vw = valid_lds[c];
#pragma unroll
      for (int i = 0; i < 16; ++i) st[i] *= scale_log2;
      if (vw != ~0u) {  // uniform: a chunk with slots that hold no position
        // register i holds slot 8 (i >> 2) + 2 (i & 3) + half (bf16 rows), f8_slot(8 (i >> 2) + 4 half + (i & 3))
        // (FP8 entries)
        if constexpr (kFp8) {
          // register 4 a + b holds slot 8 a + 4 (half ^ (a & 1)) + b: gather those nibbles of vw into bits 4 a ..
          uint32_t wp = 0;
#pragma unroll
          for (int a = 0; a < 4; ++a) wp |= ((vw >> (8 * a + 4 * (half ^ (a & 1)))) & 0xfu) << (4 * a);
#pragma unroll
          for (int i = 0; i < 16; ++i) st[i] = (wp >> i) & 1u ? st[i] : -INFINITY;
        } else {
          const uint32_t w = vw >> half;
#pragma unroll
          for (int i = 0; i < 16; ++i) st[i] = (w >> (8 * (i >> 2) + 2 * (i & 3))) & 1u ? st[i] : -INFINITY;
        }
      }
      float mx = st[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[i]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(mx, __uint_as_float(half ? sw[0] : sw[1]));
      }
      if (qk_only) {
        m_ref = fmaxf(m_ref, mx);
      } else {
        if (m_ref == -INFINITY) m_ref = mx;
        if (mx > m_ref + kHeadroom) overflow = 1;  // any wave; read after the loop
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // v_exp_f32: 2^x for x <= kHeadroom, 0 for -inf
          st[i] = __builtin_amdgcn_exp2f(st[i] - m_use);
          rs += st[i];
        }
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
          rs += __uint_as_float(half ? sw[0] : sw[1]);
        }
        l += rs;
        // O += P C over the chunk's two K-steps of 16 slots; the transposed B reads run kPvDepth MFMAs ahead
        constexpr int kPvDepth = 4;
        constexpr int kSteps = (kCW / 16) * (kDC / 32);  // (K-step, column tile) pairs
        const char* pbase = cur + (2 * (S16 >> 2) + half) * kRowW + (16 * qh + 4 * (S16 & 3)) * 2;
        auto bread = [&](int u) __attribute__((always_inline)) {
          const int ks = u / (kDC / 32), dt = u % (kDC / 32);
          const char* p = pbase + 16 * ks * kRowW + dt * 64;
          const v4bf lo4 = lds_tr_read(p);
          const v4bf hi4 = lds_tr_read(p + 8 * kRowW);
          return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        if constexpr (kFp8) {
          // tile t of the output columns (dt = 4 t .. 4 t + 3): each probability times its slot's scale for the
          // tile, x, as the bf16 head h = x cut to its top 16 bits and the rest x - h (exact) rounded to bf16
          // (together x to 2^-16 relative), on two MFMAs per (K-step, column tile).  The B operands come straight
          // from the staged codes: ds_read_b64_tr_b8 gives lane (n, kh) the codes of column n in the eight slots
          // of K indices 8 kh .., widened to bf16 in registers.  In each 16-lane group lane 2 e + hh addresses
          // slot f8_slot(16 ks + 8 (e >> 2) + 4 kh + (e & 3)), columns 16 nh + 8 hh .. +8 of the tile; lane l of
          // the group receives byte l & 7 of the addresses of lanes 2 e + (l >> 3), e = 0..7.
          constexpr int kTileSteps = (kCW / 16) * 4;  // (K-step, column tile) pairs of one tile, K-step major
          const char* pb8;
          {
            const int g = lane >> 4, L = lane & 15, e = L >> 1, hh = L & 1, kh = g >> 1, nh = g & 1;
            pb8 = raw + f8_slot(8 * (e >> 2) + 4 * kh + (e & 3)) * kF8Entry + 16 * nh + 8 * hh;
          }
          auto bread8 = [&](int ks, int dt) __attribute__((always_inline)) {
            const v2i c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)((__attribute__((address_space(3))) char*)(
                    const_cast<char*>(pb8 + 16 * kF8Entry * ks + 32 * dt))));
            const v2bf x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c.x, 1.f, false);
            const v2bf x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c.x, 1.f, true);
            const v2bf x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c.y, 1.f, false);
            const v2bf x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c.y, 1.f, true);
            return v8bf{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
          };
          v8bf bbuf[kPvDepth];
          auto pvb = [&](int v) __attribute__((always_inline)) {  // v: tile-major index of the pairs
            const int t = v / kTileSteps, w = v % kTileSteps;
            return bread8(w >> 2, 4 * t + (w & 3));
          };
#pragma unroll
          for (int v = 0; v < kPvDepth; ++v) bbuf[v] = pvb(v);
          // hp / lp [K-step]: bf16 pairs (2 e, 2 e + 1) of registers 8 ks ..  Skewed so that one set suffices:
          // while a tile's K-step 0 MFMAs run, its K-step 1 operands are made (the previous tile's are spent);
          // while its K-step 1 MFMAs run, the next tile's K-step 0 operands.
          v4i hp[2], lp[2];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_pair_n(e, st, sc[0], hp, lp);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int w = 0; w < kTileSteps; ++w) {
              const int v = t * kTileSteps + w, ks = w >> 2, dt = 4 * t + (w & 3);
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, hp[ks]), bbuf[v % kPvDepth],
                                                              o[dt], 0, 0, 0);
              if (w < 4) split_pair_n(4 + w, st, sc[t], hp, lp);
              else if (t < 3) split_pair_n(w - 4, st, sc[t + 1], hp, lp);
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lp[ks]), bbuf[v % kPvDepth],
                                                              o[dt], 0, 0, 0);
              if (v + kPvDepth < 4 * kTileSteps) bbuf[v % kPvDepth] = pvb(v + kPvDepth);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else {
          v8bf pa[kCW / 16];
#pragma unroll
          for (int ks = 0; ks < kCW / 16; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) pa[ks][j] = (__bf16)st[8 * ks + j];
          v8bf bbuf[kPvDepth];
#pragma unroll
          for (int u = 0; u < kPvDepth; ++u) bbuf[u] = bread(u);
#pragma unroll
          for (int u = 0; u < kSteps; ++u) {
            const int ks = u / (kDC / 32), dt = u % (kDC / 32);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], bbuf[u % kPvDepth], o[dt], 0, 0, 0);
            if (u + kPvDepth < kSteps) bbuf[u % kPvDepth] = bread(u + kPvDepth);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    // Wait until chunk c has landed while the `ahead` chunks gathered after it stay in flight.  The gathers
    // are opaque to the compiler's wait insertion, so these waits are the only ones on them.
    auto buf = [&](int c) { return kv_pool_lds + (c % kBufW) * (kCW * kRowW); };
    auto wait_chunk = [&](const int ahead) __attribute__((always_inline)) {
      switch (ahead) {
        case 0: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(kRows)); break;
        case 2: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(2 * kRows < 63 ? 2 * kRows : 63)); break;
        default: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(3 * kRows < 63 ? 3 * kRows : 63)); break;
      }
    };
    // One pass over the chunks.  bf16 rows: kDepth chunks are gathered ahead into a ring of kBufW LDS buffers;
    // after the barrier that ends chunk c, chunk c + kDepth is gathered into a buffer no wave still reads.
    // FP8 entries: kF8Ring - 1 chunks are gathered ahead into a ring of kF8Ring staging slots; at the barrier that
    // opens chunk c, chunk c has landed and every wave is done with chunk c - 1, whose slot takes chunk
    // c + kF8Ring - 1.
    auto run = [&](const bool qk_only) __attribute__((always_inline)) {
      if constexpr (kFp8) {
        const uint8_t* kv8 = reinterpret_cast<const uint8_t*>(kv);
        auto slot = [&](int c) { return kv_pool_lds + (c % kF8Ring) * kF8Slot; };
        // waits until this wave's gathers of chunk c have landed, `ahead` later chunks staying in flight
        // (kF8RowsPerWave loads per chunk)
        auto wait_f8 = [&](const int ahead) __attribute__((always_inline)) {
          static_assert((kF8Ring - 2) * kF8RowsPerWave <= 63, "gathers in flight fit vmcnt");
          switch (ahead) {
            case 0: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(kF8RowsPerWave)); break;
            case 2: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(2 * kF8RowsPerWave)); break;
            case 3: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(3 * kF8RowsPerWave)); break;
            default: __builtin_amdgcn_s_waitcnt(kWaitVmOnly(4 * kF8RowsPerWave)); break;
          }
        };
        static_assert(kF8Ring - 2 <= 4, "wait_f8 covers the ring");
        __builtin_amdgcn_s_waitcnt(0);  // from here the gathers are the only loads in flight
        for (int c = 0; c < kF8Ring - 1 && c < nch; ++c)
          gather_chunk_f8(kv8, prow_lds + c * kCW, dummy, slot(c), wave, lane);
        DSA_STAMP(5, 2);
        for (int c = 0; c < nch; ++c) {
          wait_f8(min(nch - 1 - c, kF8Ring - 2));
          lds_barrier();
          if (c + kF8Ring - 1 < nch)
            gather_chunk_f8(kv8, prow_lds + (c + kF8Ring - 1) * kCW, dummy, slot(c + kF8Ring - 1), wave, lane);
          chunk(c, nullptr, slot(c), qk_only);
          if ((c & 3) == 3 && c < 16) DSA_STAMP(5, 3 + (c >> 2));
        }
        __syncthreads();
      } else {
        __builtin_amdgcn_s_waitcnt(0);  // from here the gathers are the only loads in flight
        for (int c = 0; c < kDepth && c < nch; ++c)
          gather_chunk_wide<NW>(kv, prow_lds + c * kCW, dummy, buf(c), wave, lane);
        for (int c = 0; c < nch; ++c) {
          wait_chunk(min(nch - 1 - c, kDepth - 1));
          lds_barrier();
          chunk(c, buf(c), nullptr, qk_only);
          if ((c & 3) == 3 && c < 16) DSA_STAMP(5, 3 + (c >> 2));
          lds_barrier();  // every wave is done with this buffer before a gather overwrites it
          if (c + kDepth < nch) gather_chunk_wide<NW>(kv, prow_lds + (c + kDepth) * kCW, dummy, buf(c + kDepth), wave, lane);
        }
        __syncthreads();
      }
    };
#pragma unroll
    for (int dt = 0; dt < kDC / 32; ++dt) o[dt] = v16f{};
    run(false);       // reference = each head's first-chunk maximum
    if (overflow) {  // uniform and rare: exact maxima first, then accumulate against them
#pragma unroll
      for (int dt = 0; dt < kDC / 32; ++dt) o[dt] = v16f{};
      l = 0.f;
      m_ref = -INFINITY;
      run(true);
      run(false);
    }
  }

  DSA_STAMP(5, 7);
  // finish: normalise O rows by their head's sum (held in lane (0, head))
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  const bool any = first_valid != 0x7fffffff;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int hh = 8 * (i >> 2) + 4 * half + (i & 3);
    const float inv = __shfl(inv_l, hh, 64);
    if (kSplit) {  // head hh's 512 columns: tiles dt = 0..15 across the 32 lanes of this half
      // O is only initialised when the split has a selected row (`any`, uniform); otherwise store zeros
      float mx = 0.f;
      if (any)
#pragma unroll
        for (int dt = 0; dt < kDC / 32; ++dt) mx = fmaxf(mx, fabsf(o[dt][i]));
      const int ex = part_exponent(max_over_lanes(mx, 32) * inv);
      const int64_t prow = ((int64_t)r * nsplit + split) * H + hw + hh;
#pragma unroll
      for (int dt = 0; dt < kDC / 32; ++dt)
        __builtin_nontemporal_store(part_bits(any ? o[dt][i] * inv : 0.f, ex), part_o + prow * kDC + 32 * dt + col);
      if (col == 0) part_exp[prow] = ex;
    } else {
      const int64_t orow = (int64_t)r * H + hw + hh;
#pragma unroll
      for (int dt = 0; dt < kDC / 32; ++dt)
        out[orow * kDC + 32 * dt + col] = float_to_bf16_bits(any ? o[dt][i] * inv : 0.f);
    }
  }
  if (half == 0) {
    const float lz = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    if (kSplit)
      part_lse[((int64_t)r * nsplit + split) * H + hw + col] = lz;
    else if (lse)
      lse[(int64_t)r * H + hw + col] = lz;
  }
  DSA_STAMP(5, 8);
}

// Merge the per-split (o, lse) pairs of one (row, head): o = sum_s exp(lse_s - L) o_s, L = log sum exp lse_s,
// in fp32.  One block of 4 L waves per (row, head) and up to 64 L splits: lane l holds the lse and exponent of
// splits l, l + 64, ... and latent columns 8l .. 8l+7 (d_c = 512); wave 4 i + u takes the 16 splits 64 i + u,
// 64 i + u + 4, ... as one 16-byte load each.  Every load is issued before any is used, so the weights and the
// rows arrive in one round trip; the other waves hand their sums to wave 0 through LDS.
constexpr int kMaxSplit = 64;       // splits of the 16-head kernel
constexpr int kMaxSplitWide = 256;  // splits of the all-heads kernel (the combine's limit)
constexpr int64_t kCombineWavePairs = 1024;  // (row, head) pairs from which the merge runs a wave per pair
// kP blocks share one (row, head): block part p merges columns 512 p / kP .. +512 / kP (8 / kP per lane), so that
// a small batch still spreads the merge over the chip.
template <int L, int kP>
__global__ __launch_bounds__(256 * L) void attn_combine_kernel(const unsigned short* __restrict__ part_o,
                                                               const int32_t* __restrict__ part_exp,
                                                               const float* __restrict__ part_lse, int H, int nsplit,
                                                               unsigned short* __restrict__ out,
                                                               float* __restrict__ lse) {
  static_assert(kDC == 8 * 64, "eight latent columns per lane and part");
  constexpr int kE = 8 / kP;  // columns per lane
  typedef unsigned short vcol __attribute__((ext_vector_type(kE)));
  constexpr int kNW = 4 * L, kPerWave = 16;
  __shared__ float red[kNW - 1][kE][64];  // waves 1..: their partial sums, column-major per lane
  args_to_sgprs(part_o, part_exp, part_lse, H, nsplit, out, lse);
  DSA_STAMP(4, 0);
  const int rh = blockIdx.x / kP, col0 = (blockIdx.x % kP) * (kDC / kP) + (int)(threadIdx.x & 63) * kE;
  const int r = rh / H, h = rh % H;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int grp = wave >> 2, u = wave & 3;         // this wave's 64 splits, and its offset among them
  const int64_t row0 = (int64_t)r * nsplit * H + h;  // partial row of split 0; split j is j * H further
  float ls[L];
  int ex[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int j = 64 * i + lane;
    ls[i] = j < nsplit ? part_lse[row0 + (int64_t)j * H] : -INFINITY;
    ex[i] = j < nsplit ? part_exp[row0 + (int64_t)j * H] : 0;
  }
  vcol v[kPerWave];
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    const int j = 64 * grp + u + 4 * q;
    if (j < nsplit) v[q] = *reinterpret_cast<const vcol*>(part_o + (row0 + (int64_t)j * H) * kDC + col0);
  }
  // split weights w_j = exp(lse_j - max) / sum, each wave for itself; the lane that holds split j also folds in
  // its exponent
  float m = ls[0];
#pragma unroll
  for (int i = 1; i < L; ++i) m = fmaxf(m, ls[i]);
  const float mx = wave_max(m);
  float w[L], part = 0.f;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    w[i] = ls[i] == -INFINITY ? 0.f : expf(ls[i] - mx);
    part += w[i];
  }
  const float wsum = wave_sum(part);
  DSA_STAMP(4, 1);
  float wl = 0.f;  // weight of split 64 grp + lane
#pragma unroll
  for (int i = 0; i < L; ++i)
    if (i == grp) wl = ldexpf(wsum > 0.f ? w[i] / wsum : 0.f, ex[i]);
  auto half_f = [](unsigned short b) { return (float)__builtin_bit_cast(_Float16, b); };
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    if (64 * grp + u + 4 * q < nsplit) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u + 4 * q));
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] = fmaf(wj, half_f(v[q][e]), acc[e]);
    }
  }
  DSA_STAMP(4, 2);
  if (wave > 0)
#pragma unroll
    for (int e = 0; e < kE; ++e) red[wave - 1][e][lane] = acc[e];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < kNW - 1; ++t)
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] += red[t][e][lane];
    vcol b;
#pragma unroll
    for (int e = 0; e < kE; ++e) b[e] = float_to_bf16_bits(acc[e]);
    *reinterpret_cast<vcol*>(out + ((int64_t)r * H + h) * kDC + col0) = b;  // 16- or 8-byte aligned
    if (lane == 0 && col0 == 0 && lse) lse[(int64_t)r * H + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
  }
  DSA_STAMP(4, 3);
}

// The same merge for batches with many (row, head) pairs: one wave per pair, lane l merging columns 8 l .. +8 of
// all nsplit <= kJ partials.  Lane j also reads split j's log-sum-exp and exponent, every load of the wave is
// issued before the first is used, and no LDS or barrier is needed: a pair costs one round trip, and the
// 256-thread blocks (four pairs each) all fit on the chip at once at the batched shapes.
template <int kJ>
__global__ __launch_bounds__(256) void attn_combine_wave_kernel(const unsigned short* __restrict__ part_o,
                                                                const int32_t* __restrict__ part_exp,
                                                                const float* __restrict__ part_lse, int H, int nsplit,
                                                                int pairs, unsigned short* __restrict__ out,
                                                                float* __restrict__ lse) {
  static_assert(kDC == 8 * 64 && kJ <= 64, "eight latent columns per lane, one split per lane");
  typedef unsigned short v8us __attribute__((ext_vector_type(8)));
  args_to_sgprs(part_o, part_exp, part_lse, H, nsplit, pairs, out, lse);
  const int lane = threadIdx.x & 63;
  const int rh = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (rh >= pairs) return;  // uniform per wave
  const int r = rh / H, h = rh % H;
  const int64_t row0 = (int64_t)r * nsplit * H + h;  // partial row of split 0; split j is j * H further
  const float ls = lane < nsplit ? part_lse[row0 + (int64_t)lane * H] : -INFINITY;
  const int ex = lane < nsplit ? part_exp[row0 + (int64_t)lane * H] : 0;
  v8us v[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j)
    if (j < nsplit) v[j] = *reinterpret_cast<const v8us*>(part_o + (row0 + (int64_t)j * H) * kDC + lane * 8);
  const float mx = wave_max(ls);
  const float w = ls == -INFINITY ? 0.f : expf(ls - mx);
  const float wsum = wave_sum(w);
  const float wl = ldexpf(wsum > 0.f ? w / wsum : 0.f, ex);  // weight of split `lane`
  auto half_f = [](unsigned short b) { return (float)__builtin_bit_cast(_Float16, b); };
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int j = 0; j < kJ; ++j)
    if (j < nsplit) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wj, half_f(v[j][e]), acc[e]);
    }
  v8us b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = float_to_bf16_bits(acc[e]);
  *reinterpret_cast<v8us*>(out + (int64_t)rh * kDC + lane * 8) = b;
  if (lane == 0 && lse) lse[rh] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// fp32 path: one block per (row, head); logits and physical rows staged in LDS.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kv,
                                                       const int32_t* __restrict__ topk_idx, int k,
                                                       const int32_t* __restrict__ row_len, int max_row_len,
                                                       const int32_t* __restrict__ row_seq,
                                                       const int32_t* __restrict__ page_table, int num_seqs,
                                                       int max_pages, int num_pages, int log2ps, int H, int d_c,
                                                       float scale,
                                                       float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int64_t* prow = reinterpret_cast<int64_t*>(smem);          // [k]
  float* logit = reinterpret_cast<float*>(prow + k);        // [k]
  float* qs = logit + k;                                    // [d_c]
  __shared__ float red[256 / 64];
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int seq = clamp_seq(row_seq[r], num_seqs);
  const float* qrow = q + ((int64_t)r * H + h) * d_c;
  for (int d = threadIdx.x; d < d_c; d += blockDim.x) qs[d] = qrow[d];
  const SlotSource src = slot_source(topk_idx, nullptr, row_len, max_row_len, r, k, 0);
  for (int s = threadIdx.x; s < k; s += blockDim.x) {
    const int pos = src.at(s);
    prow[s] = pos >= 0 ? phys_row(page_table, max_pages, num_pages, log2ps, seq, pos) : -1;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < k; s += blockDim.x) {
    float v = -INFINITY;
    if (prow[s] >= 0) {
      const float* c = kv + prow[s] * d_c;
      float dot = 0.f;
      for (int d = 0; d < d_c; ++d) dot = fmaf(qs[d], c[d], dot);
      v = scale * dot;
    }
    logit[s] = v;
    mx = fmaxf(mx, v);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x / 64;
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < nw; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  const float mu = mx == -INFINITY ? 0.f : mx;
  float z = 0.f;
  for (int s = threadIdx.x; s < k; s += blockDim.x) {
    const float p = logit[s] == -INFINITY ? 0.f : expf(logit[s] - mu);
    logit[s] = p;
    z += p;
  }
  z = wave_sum(z);
  if (lane == 0) red[wave] = z;
  __syncthreads();
  z = 0.f;
  for (int w = 0; w < nw; ++w) z += red[w];
  const float inv = z > 0.f ? 1.f / z : 0.f;
  for (int d = threadIdx.x; d < d_c; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < k; ++s)
      if (prow[s] >= 0) acc = fmaf(logit[s], kv[prow[s] * d_c + d], acc);
    out[((int64_t)r * H + h) * d_c + d] = acc * inv;
  }
  if (threadIdx.x == 0 && lse) lse[(int64_t)r * H + h] = z > 0.f ? mu + logf(z) : -INFINITY;
}

struct AttnPlan {
  int nsplit;
  int split_len;
  int nw;  // > 0: all-heads kernel with nw waves (32 nw heads per block); 0: 16-head kernel
};

AttnPlan plan(const Geo& g) {
  const int chunks = std::max(1, (g.k + kNC - 1) / kNC);
  AttnPlan p{1, chunks * kNC, 0};
  if (g.kv_dtype == 0 /* F32 */) return p;
  const int nw = g.H % 128 == 0 ? 4 : g.H % 64 == 0 ? 2 : 1;  // waves per block divide the 64 gathers of a chunk
  // FP8 entries take the all-heads kernel with four waves only (128 heads per block)
  const bool wide_ok = g.kv_dtype == 1 ? g.H % 32 == 0 : g.H % 128 == 0;
  if (wide_ok && (int64_t)g.R * (g.H / (32 * nw)) * chunks >= 128) {
    // all-heads kernel: one block per (row, head group of <= 128, split), one block per CU at a time; split
    // the selection only as far as needed to give every CU a block.  With fewer than 128 (row, group, chunk)
    // units it could not spread over the chip, and the 16-head kernel below runs instead.
    p.nw = nw;
    const int64_t groups = (int64_t)g.R * (g.H / (32 * p.nw));
    const int min_split = (chunks * kNC + kWideMaxSplitLen - 1) / kWideMaxSplitLen;
    int64_t want = (256 + groups - 1) / groups;
    int nsplit = (int)std::max<int64_t>(min_split, std::min<int64_t>(want, std::min(chunks, kMaxSplitWide)));
    const int per = (chunks + nsplit - 1) / nsplit;
    p.nsplit = (chunks + per - 1) / per;
    p.split_len = per * kNC;
    return p;
  }
  // a block handles at most kMaxSplitLen slots; below ~2 blocks per CU the selection is split further into
  // pieces of about kChunksPerSplitSmallBatch chunks (double buffering needs a few), at most kMaxSplit of them
  const int64_t groups = (int64_t)g.R * (g.H / kHG);
  int per = std::min(chunks, kMaxSplitLen / kNC);
  if (groups * ((chunks + per - 1) / per) < 256) per = std::min(per, kChunksPerSplitSmallBatch);
  int nsplit = (chunks + per - 1) / per;
  if (nsplit > kMaxSplit) {
    per = (chunks + kMaxSplit - 1) / kMaxSplit;
    nsplit = (chunks + per - 1) / per;
  }
  p.nsplit = nsplit;
  p.split_len = per * kNC;
  return p;
}

// Split partials in the workspace: o [R, nsplit, H, d_c] fp16, lse [R, nsplit, H] fp32, exponents
// [R, nsplit, H] int32.
struct Partials {
  unsigned short* o;
  float* lse;
  int32_t* ex;
};
Partials carve_partials(const Geo& g, int nsplit, void* workspace) {
  if (nsplit <= 1) return Partials{nullptr, nullptr, nullptr};
  const size_t rows = (size_t)g.R * nsplit * g.H;
  char* p = static_cast<char*>(workspace);
  Partials w;
  w.o = reinterpret_cast<unsigned short*>(p);
  p += align_up(sizeof(uint16_t) * rows * g.d_c);
  w.lse = reinterpret_cast<float*>(p);
  p += align_up(sizeof(float) * rows);
  w.ex = reinterpret_cast<int32_t*>(p);
  return w;
}

template <int NW, bool kFp8>
void launch_mqa(const Geo& g, const AttnPlan& p, const unsigned short* qp, const unsigned short* kp,
                const int32_t* topk_idx, const int32_t* pool_rows, void* out, float* lse, const Partials& pt,
                float scale_log2, hipStream_t stream) {
  const int64_t units = (int64_t)g.R * (g.H / (32 * NW));
  const int nblocks = work_blocks((int64_t)g.R * p.nsplit, g.H / (32 * NW));
  if (p.nsplit == 1)
    attn_bf16_mqa_kernel<NW, false, kFp8><<<nblocks, NW * 64, 0, stream>>>(
        qp, kp, topk_idx, g.k, pool_rows, g.row_len, g.max_row_len, g.row_seq, g.page_table, g.S, g.max_pages,
        g.num_pages, g.log2ps, g.H, 1, (int)units, p.split_len, scale_log2, static_cast<unsigned short*>(out), lse,
        nullptr, nullptr, nullptr);
  else
    attn_bf16_mqa_kernel<NW, true, kFp8><<<nblocks, NW * 64, 0, stream>>>(
        qp, kp, topk_idx, g.k, pool_rows, g.row_len, g.max_row_len, g.row_seq, g.page_table, g.S, g.max_pages,
        g.num_pages, g.log2ps, g.H, p.nsplit, (int)units, p.split_len, scale_log2, nullptr, nullptr, pt.o, pt.ex,
        pt.lse);
}

}  // namespace

size_t attn_workspace_bytes(const Geo& g) {
  const AttnPlan p = plan(g);
  if (p.nsplit <= 1) return 0;
  const size_t rows = (size_t)g.R * p.nsplit * g.H;
  return align_up(sizeof(uint16_t) * rows * g.d_c) + align_up(sizeof(float) * rows) +
         align_up(sizeof(int32_t) * rows);
}

hipError_t launch_attn(const Geo& g, const void* q, const void* kv_pool, const int32_t* topk_idx, void* out,
                       float* lse, void* workspace, const int32_t* pool_rows, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  if (g.kv_dtype == 1 /* BF16 */ || g.kv_dtype == 2 /* FP8 entries */) {
    const bool fp8 = g.kv_dtype == 2;
    const AttnPlan p = plan(g);
    const float scale_log2 = g.softmax_scale * kLog2e;
    auto* qp = static_cast<const unsigned short*>(q);
    auto* kp = static_cast<const unsigned short*>(kv_pool);
    const Partials pt = carve_partials(g, p.nsplit, workspace);
    if (p.nw > 0) {
      switch (p.nw) {
        case 1: launch_mqa<1, false>(g, p, qp, kp, topk_idx, pool_rows, out, lse, pt, scale_log2, stream); break;
        case 2: launch_mqa<2, false>(g, p, qp, kp, topk_idx, pool_rows, out, lse, pt, scale_log2, stream); break;
        default:
          if (fp8) launch_mqa<4, true>(g, p, qp, kp, topk_idx, pool_rows, out, lse, pt, scale_log2, stream);
          else launch_mqa<4, false>(g, p, qp, kp, topk_idx, pool_rows, out, lse, pt, scale_log2, stream);
          break;
      }
    } else {
      const int64_t units = (int64_t)g.R * (g.H / kHG);
      const int nblocks = work_blocks((int64_t)g.R * p.nsplit, g.H / kHG);
      auto go = [&](auto kern, bool split) {
        kern<<<nblocks, 256, 0, stream>>>(qp, kp, topk_idx, g.k, pool_rows, g.row_len, g.max_row_len, g.row_seq,
                                          g.page_table, g.S, g.max_pages, g.num_pages, g.log2ps, g.H,
                                          split ? p.nsplit : 1, (int)units, p.split_len, scale_log2,
                                          split ? nullptr : static_cast<unsigned short*>(out), split ? nullptr : lse,
                                          pt.o, pt.ex, pt.lse);
      };
      if (p.nsplit > 1) go(fp8 ? attn_bf16_kernel<true, true> : attn_bf16_kernel<true, false>, true);
      else go(fp8 ? attn_bf16_kernel<false, true> : attn_bf16_kernel<false, false>, false);
    }
    if (p.nsplit > 1) {
      // fewer (row, head) pairs than CUs: two blocks per pair, half the columns each
      auto* o = static_cast<unsigned short*>(out);
      const int64_t rh = (int64_t)g.R * g.H;
      const bool two = rh < 256;
      const int nb = (int)(two ? 2 * rh : rh);
#define DSA_COMBINE(L_, P_) \
  attn_combine_kernel<L_, P_><<<nb, 256 * L_, 0, stream>>>(pt.o, pt.ex, pt.lse, g.H, p.nsplit, o, lse)
#define DSA_COMBINE_WAVE(J_)                                                                                     \
  attn_combine_wave_kernel<J_><<<(int)((rh + 3) / 4), 256, 0, stream>>>(pt.o, pt.ex, pt.lse, g.H, p.nsplit, \
                                                                         (int)rh, o, lse)
      if (rh >= kCombineWavePairs && p.nsplit <= 16) {
        // at least a wave per SIMD of the chip, each with few splits to load: one wave per (row, head).  With
        // more splits a pair's loads spread over the four waves of a block (at 8 rows x 128 heads of 32 splits
        // the attention phase measured 27.6 us that way against 29.0 us with a wave per pair)
        if (p.nsplit <= 4) DSA_COMBINE_WAVE(4);
        else if (p.nsplit <= 8) DSA_COMBINE_WAVE(8);
        else DSA_COMBINE_WAVE(16);
      } else if (p.nsplit <= 64) {
        if (two) DSA_COMBINE(1, 2); else DSA_COMBINE(1, 1);
      } else if (p.nsplit <= 128) {
        if (two) DSA_COMBINE(2, 2); else DSA_COMBINE(2, 1);
      } else {
        if (two) DSA_COMBINE(4, 2); else DSA_COMBINE(4, 1);
      }
#undef DSA_COMBINE
#undef DSA_COMBINE_WAVE
    }
  } else {
    const size_t lds = (size_t)g.k * (sizeof(int64_t) + sizeof(float)) + sizeof(float) * (size_t)g.d_c;
    attn_f32_kernel<<<g.R * g.H, 256, lds, stream>>>(static_cast<const float*>(q), static_cast<const float*>(kv_pool),
                                                      topk_idx, g.k, g.row_len, g.max_row_len, g.row_seq,
                                                      g.page_table, g.S,
                                                      g.max_pages, g.num_pages, g.log2ps, g.H, g.d_c, g.softmax_scale,
                                                      static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
