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

// Gathers the 16 latent rows of this wave for chunk c straight into LDS: global_load_lds_dwordx4 lands the 64
// lanes' 16-byte pieces contiguously at the LDS address in M0, one 1 KiB row per instruction.  Every wave
// issues exactly 16 such loads per chunk (a slot without a position reads `dummy`, a selected row of the split,
// and is masked later), so "this chunk has arrived" is a fixed vmcnt once the next chunk has been issued.
// The loads are written as asm so that the compiler's wait insertion, which cannot tell which LDS buffer a
// pending DMA targets across the chunk loop, does not add a full vmcnt(0) before every LDS read; the waits
// on them are explicit (kWaitVm16 / s_waitcnt 0).  No output register is involved: the data goes to LDS and
// the address operands are read when the instruction issues.
__device__ __forceinline__ void gather_chunk(const unsigned short* __restrict__ kv, const int32_t* prow, int dummy,
                                             char* buf, int wave, int lane) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int rr = wave * 16 + t;
    int pr = prow[rr];
    if (pr < 0) pr = dummy;
    const unsigned short* src = kv + (int64_t)pr * kDC + lane * 8;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(buf + rr * kRowB)));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int kWaitVm16 = (16 & 15) | ((16 >> 4) << 14) | (7 << 4) | (15 << 8);  // vmcnt <= 16 only
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);                               // lgkmcnt == 0 only

// Workgroup barrier for data this wave wrote with ds_* instructions.  Unlike __syncthreads() it does not wait
// for vector-memory operations, so the next chunk's LDS-DMA gather stays in flight across it; the empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool kSplit>
__global__ __launch_bounds__(256) void attn_bf16_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ kv, const int32_t* __restrict__ topk_idx,
    int k, const int32_t* __restrict__ row_seq, const int32_t* __restrict__ page_table, int num_seqs, int max_pages,
    int num_pages, int log2ps, int H, int nsplit, int split_len, float scale_log2, unsigned short* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) char kv_lds0[kNC * kRowB];
  __shared__ __attribute__((aligned(16))) char kv_lds1[kNC * kRowB];
  __shared__ __attribute__((aligned(16))) float s_lds[kHG][kNC + 4];
  __shared__ int32_t prow_lds[kMaxSplitLen];  // physical row of every slot of the split, -1 = no position
  __shared__ int first_valid;

  const int ngroups = H / kHG;
  const int split = blockIdx.x % nsplit;
  const int rg = blockIdx.x / nsplit;
  const int grp16 = rg % ngroups;
  const int r = rg / ngroups;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;

  // Q as A operands: head grp16*16 + i, d = kd*32 + g*8 .. +8
  v8bf qa[kDC / 32];
  {
    const unsigned short* qrow = q + ((int64_t)r * H + grp16 * kHG + i) * kDC + g * 8;
#pragma unroll
    for (int kd = 0; kd < kDC / 32; ++kd) qa[kd] = *reinterpret_cast<const v8bf*>(qrow + kd * 32);
  }

  v4f o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running max (log2 domain) and sum for head i

  const int seq = clamp_seq(row_seq[r], num_seqs);
  const int begin = split * split_len;
  const int end = min(k, begin + split_len);
  const int len = max(end - begin, 0);
  const int nch = (len + kNC - 1) / kNC;
  const int32_t* idx = topk_idx + (int64_t)r * k + begin;

  // every slot of the split -> physical row before any gather (so gathers are the only loads in flight)
  if (threadIdx.x == 0) first_valid = 0x7fffffff;
  __syncthreads();
  for (int s = threadIdx.x; s < nch * kNC; s += blockDim.x) {
    const int pos = s < len ? idx[s] : -1;
    const int pr = pos >= 0 ? (int)phys_row(page_table, max_pages, num_pages, log2ps, seq, pos) : -1;
    prow_lds[s] = pr;
    if (pr >= 0) atomicMin(&first_valid, s);
  }
  __syncthreads();
  // a split with no selected row contributes nothing; otherwise slots without a position read a selected row
  // of this split instead (their logits are -inf, so they carry zero weight)
  if (first_valid != 0x7fffffff) {
    const int dummy = prow_lds[first_valid];
    // one chunk: wait for its rows (the next chunk's gather stays in flight), then QK^T, softmax, PV.
    // `cur` and `nxt` are fixed per call site, so the compiler can tell the DMA target from the buffer read.
    auto chunk = [&](const int c, const char* cur, char* nxt) __attribute__((always_inline)) {
      if (c + 1 < nch) {
        gather_chunk(kv, prow_lds + (c + 1) * kNC, dummy, nxt, wave, lane);
        __builtin_amdgcn_s_waitcnt(kWaitVm16);  // chunk c has landed; chunk c+1 stays in flight
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      lds_barrier();
      // S for slots wave*16 + (0..15): B operand = row (wave*16 + i), d = kd*32 + g*8 .. +8
      v4f sacc = {0.f, 0.f, 0.f, 0.f};
      {
        const char* brow = cur + (wave * 16 + i) * kRowB + g * 16;
#pragma unroll
        for (int kd = 0; kd < kDC / 32; ++kd) {
          const v8bf b = *reinterpret_cast<const v8bf*>(brow + kd * 64);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kd], b, sacc, 0, 0, 0);
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
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) { sv[e] = exp2f(sv[e] - m_use); rs += sv[e]; }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l = l * alpha + rs;
      m = m_new;

      // rescale O rows (head g*4 + v) by that head's alpha, held by lane g*4 + v
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, g * 4 + v, 64);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][v] *= av;
      }

      // O += P V.  A operand element e of K-step kk is slot kk*32 + 8g + perm[e], perm = {0,2,4,6,1,3,5,7}.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const float pe[8] = {sv[kk * 8 + 0], sv[kk * 8 + 2], sv[kk * 8 + 4], sv[kk * 8 + 6],
                             sv[kk * 8 + 1], sv[kk * 8 + 3], sv[kk * 8 + 5], sv[kk * 8 + 7]};
        const v8bf pa = pack8(pe);
        const int row1 = kk * 32 + 8 * g + 2 * (i >> 2);
        const char* p1 = cur + row1 * kRowB + (wave * 128 + 4 * (i & 3)) * 2;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const v4bf lo4 = lds_tr_read(p1 + dt * 32);
          const v4bf hi4 = lds_tr_read(p1 + kRowB + dt * 32);
          const v8bf b = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, b, o[dt], 0, 0, 0);
        }
      }
      lds_barrier();  // every wave is done with `cur` and s_lds before they are overwritten
    };
    __builtin_amdgcn_s_waitcnt(0);  // Q operands and slot rows are in; from here the gathers are the only loads
    gather_chunk(kv, prow_lds, dummy, kv_lds0, wave, lane);
    for (int c = 0; c < nch; c += 2) {
      chunk(c, kv_lds0, kv_lds1);
      if (c + 1 < nch) chunk(c + 1, kv_lds1, kv_lds0);
    }
  }

  // finish: O rows are heads g*4 + v, columns wave*128 + dt*16 + i
  const int64_t head0 = (int64_t)r * H + grp16 * kHG;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int hh = g * 4 + v;
    const float lv = __shfl(l, hh, 64);
    const float inv = lv > 0.f ? 1.f / lv : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = wave * 128 + dt * 16 + i;
      const float val = o[dt][v] * inv;
      if (kSplit)
        part_o[(((int64_t)r * nsplit + split) * H + grp16 * kHG + hh) * kDC + d] = val;
      else
        out[(head0 + hh) * kDC + d] = float_to_bf16_bits(val);
    }
  }
  if (wave == 0 && g == 0) {
    const float lz = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    if (kSplit)
      part_lse[((int64_t)r * nsplit + split) * H + grp16 * kHG + i] = lz;
    else if (lse)
      lse[head0 + i] = lz;
  }
}

// Merge the per-split (o, lse) pairs of one (row, head): o = sum_s exp(lse_s - L) o_s, L = log sum exp lse_s.
// Block (row*H + head, column slice): the split weights are computed once by the first wave.
constexpr int kMaxSplit = 64;
template <bool kBf16Out>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse, int H, int d_c,
                                                           int nsplit, void* __restrict__ out, float* __restrict__ lse) {
  __shared__ float wts[kMaxSplit];
  const int rh = blockIdx.x;
  const int r = rh / H, h = rh % H;
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float ls = s < nsplit ? part_lse[((int64_t)r * nsplit + s) * H + h] : -INFINITY;
    const float mx = wave_max(ls);
    const float w = ls == -INFINITY ? 0.f : expf(ls - mx);
    const float wsum = wave_sum(w);
    wts[s] = wsum > 0.f ? w / wsum : 0.f;
    if (s == 0 && lse && blockIdx.y == 0) lse[(int64_t)r * H + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
  }
  __syncthreads();
  const int d = blockIdx.y * blockDim.x + threadIdx.x;
  if (d >= d_c) return;
  const float* src = part_o + ((int64_t)r * nsplit * H + h) * d_c + d;
  const int64_t stride = (int64_t)H * d_c;
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[(s + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(wts[s + j], v[j], acc);
  }
  for (; s < nsplit; ++s) acc = fmaf(wts[s], src[s * stride], acc);
  if (kBf16Out)
    static_cast<unsigned short*>(out)[((int64_t)r * H + h) * d_c + d] = float_to_bf16_bits(acc);
  else
    static_cast<float*>(out)[((int64_t)r * H + h) * d_c + d] = acc;
}

// fp32 path: one block per (row, head); logits and physical rows staged in LDS.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kv,
                                                       const int32_t* __restrict__ topk_idx, int k,
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
  for (int s = threadIdx.x; s < k; s += blockDim.x) {
    const int pos = topk_idx[(int64_t)r * k + s];
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
};

AttnPlan plan(const Geo& g) {
  const int chunks = std::max(1, (g.k + kNC - 1) / kNC);
  AttnPlan p{1, chunks * kNC};
  if (g.kv_dtype != 1 /* BF16 */) return p;
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

}  // namespace

size_t attn_workspace_bytes(const Geo& g) {
  const AttnPlan p = plan(g);
  if (p.nsplit <= 1) return 0;
  return align_up(sizeof(float) * (size_t)g.R * p.nsplit * g.H * g.d_c) + align_up(sizeof(float) * (size_t)g.R * p.nsplit * g.H);
}

hipError_t launch_attn(const Geo& g, const void* q, const void* kv_pool, const int32_t* topk_idx, void* out,
                       float* lse, void* workspace, hipStream_t stream) {
  if (g.R == 0) return hipSuccess;
  if (g.kv_dtype == 1 /* BF16 */) {
    const AttnPlan p = plan(g);
    const float scale_log2 = g.softmax_scale * kLog2e;
    const int nblocks = g.R * (g.H / kHG) * p.nsplit;
    auto* qp = static_cast<const unsigned short*>(q);
    auto* kp = static_cast<const unsigned short*>(kv_pool);
    if (p.nsplit == 1) {
      attn_bf16_kernel<false><<<nblocks, 256, 0, stream>>>(qp, kp, topk_idx, g.k, g.row_seq, g.page_table,
                                                           g.S, g.max_pages, g.num_pages, g.log2ps, g.H, 1, p.split_len,
                                                           scale_log2, static_cast<unsigned short*>(out), lse,
                                                           nullptr, nullptr);
    } else {
      float* part_o = static_cast<float*>(workspace);
      float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                 align_up(sizeof(float) * (size_t)g.R * p.nsplit * g.H * g.d_c));
      attn_bf16_kernel<true><<<nblocks, 256, 0, stream>>>(qp, kp, topk_idx, g.k, g.row_seq, g.page_table,
                                                          g.S, g.max_pages, g.num_pages, g.log2ps, g.H, p.nsplit,
                                                          p.split_len, scale_log2, nullptr, nullptr, part_o, part_lse);
      attn_combine_kernel<true><<<dim3(g.R * g.H, (g.d_c + 255) / 256), 256, 0, stream>>>(part_o, part_lse, g.H, g.d_c,
                                                                                       p.nsplit, out, lse);
    }
  } else {
    const size_t lds = (size_t)g.k * (sizeof(int64_t) + sizeof(float)) + sizeof(float) * (size_t)g.d_c;
    attn_f32_kernel<<<g.R * g.H, 256, lds, stream>>>(static_cast<const float*>(q), static_cast<const float*>(kv_pool),
                                                      topk_idx, g.k, g.row_seq, g.page_table, g.S,
                                                      g.max_pages, g.num_pages, g.log2ps, g.H, g.d_c, g.softmax_scale,
                                                      static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
