// Device helpers shared by the gfx950 kernels of libdsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Timeline probes for profiling builds.  Compiled out unless DSA_TIMELINE is defined; a profiling build then
// records s_memrealtime (a 100 MHz clock common to the whole device) at marked points of each block into a
// device buffer that the host installs with dsa_timeline_set_<unit>(), one per translation unit.
#ifdef DSA_TIMELINE
static __constant__ unsigned long long* g_timeline;  // constant: stamps never reload it
#define DSA_TIMELINE_UNIT(name)                                                               \
  extern "C" int dsa_timeline_set_##name(void* p) {                                           \
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &p, sizeof p);                      \
  }
#define DSA_STAMP(kernel, point)                                                              \
  do {                                                                                        \
    if (threadIdx.x == 0 && g_timeline) {                                                     \
      const unsigned blk = blockIdx.x + blockIdx.y * gridDim.x;                               \
      if (blk < 4096) g_timeline[((kernel) * 4096u + blk) * 16u + (point)] = __builtin_amdgcn_s_memrealtime(); \
    }                                                                                         \
  } while (0)
#else
#define DSA_TIMELINE_UNIT(name)
#define DSA_STAMP(kernel, point) ((void)0)
#endif

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef double v2d __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned short v8us __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int kWaitVmOnly(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }  // vmcnt <= n only
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);                               // lgkmcnt == 0 only

// Workgroup barrier for data this wave wrote with ds_* instructions.  Unlike __syncthreads() it does not wait
// for vector-memory operations, so loads issued for later chunks stay in flight across it; the empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// fp32 -> OCP e4m3fn code for |y| <= 448, round to nearest even; the sign bit of y is kept.  Below 2^-6 the codes
// are the subnormals m * 2^-9 (m = 8 is the smallest normal, code 0x08); above, the fp32 mantissa is cut to three
// bits with a carry into the exponent field.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  const uint32_t b = __float_as_uint(a);
  const uint32_t e = (b >> 23) - 127 + 7;  // biased e4m3 exponent, 1 .. 15
  uint32_t m3 = (b >> 20) & 7u;
  const uint32_t rest = b & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
  return sign | ((e << 3) + m3);  // m3 = 8 carries into the exponent
}

// Physical pool row of logical position `pos` (>= 0) of sequence `seq`.  The logical page is clamped to
// [0, max_pages) and the page id to [0, num_pages), so corrupt metadata never addresses memory outside the
// table or the pools.
__device__ __forceinline__ int64_t phys_row(const int32_t* __restrict__ page_table, int max_pages, int num_pages,
                                            int log2ps, int seq, int64_t pos) {
  const int lp = (int)min(pos >> log2ps, (int64_t)max_pages - 1);
  int page = page_table[(int64_t)seq * max_pages + lp];
  page = min(max(page, 0), num_pages - 1);
  return ((int64_t)page << log2ps) | (pos & ((1 << log2ps) - 1));
}

// Makes the compiler read kernel arguments into scalar registers at this point.  Left to itself it sinks each
// argument's load into the first block that uses it, and a prologue then pays a separate load-and-wait round for
// each group of arguments; called at a kernel's entry with the arguments of its prologue, it turns those rounds
// into one.
template <class T>
__device__ __forceinline__ void arg_to_sgpr(const T& a) {
  asm volatile("" ::"s"(a));
}
template <class... T>
__device__ __forceinline__ void args_to_sgprs(const T&... a) {
  (arg_to_sgpr(a), ...);
}

__device__ __forceinline__ int clamp_len(int n, int max_len) { return min(max(n, 0), max_len); }
__device__ __forceinline__ int clamp_seq(int seq, int num_seqs) { return min(max(seq, 0), num_seqs - 1); }

// Order-preserving unsigned key of an fp32 score: a > b  <=>  key(a) > key(b); +0 and -0 share one key.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (the gfx950 conversion instruction).
__device__ __forceinline__ unsigned short float_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(unsigned short, h);
}

// A DPP lane move of a float (every lane's source lies in its own row for the controls used here).
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Reduction over the 64 lanes of a wave in the register file, every lane receiving the same value: within each
// 16-lane row by DPP (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror), then between rows by
// v_permlane16_swap and v_permlane32_swap.  Each step combines a lane with its partner in the same order on both
// sides, so a sum is bit-identical in every lane.  All 64 lanes must be active.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_move<0xB1>(v));
  v = op(v, dpp_move<0x4E>(v));
  v = op(v, dpp_move<0x141>(v));
  v = op(v, dpp_move<0x140>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

// Exclusive prefix of `v` over the lanes of a wave (and the wave total), with DPP lane moves instead of LDS-routed
// shuffles: shifts by 1, 2, 4 and 8 lanes scan each row of 16 (a lane whose source falls outside its row adds 0),
// then row_bcast:15 adds row 0's total into row 1 and row 2's into row 3, and row_bcast:31 adds the total of rows
// 0-1 into rows 2-3.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t v, uint32_t& total) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  total = (uint32_t)__builtin_amdgcn_readlane(x, 63);
  return (uint32_t)x - v;
}

// Block-wide exclusive scan of one value per thread.  `scratch` holds blockDim.x / 64 + 1 words of LDS.  Every
// wave scans its lanes and publishes its total; after one barrier every wave scans the wave totals itself (one
// per lane, DPP) and takes the prefix of its own with v_readlane.  A trailing barrier lets the next call reuse
// `scratch`.  Must be called by every thread of the block.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
  uint32_t wt;
  uint32_t x = wave_exclusive_scan(v, wt);
  if (lane == 0) scratch[wave] = wt;
  __syncthreads();
  const uint32_t t = lane < nwaves ? scratch[lane] : 0u;  // at most 64 waves per block
  uint32_t tot;
  const uint32_t pre = wave_exclusive_scan(t, tot);
  x += (uint32_t)__builtin_amdgcn_readlane((int)pre, __builtin_amdgcn_readfirstlane(wave));
  total = tot;
  __syncthreads();
  return x;
}

}  // namespace dsa
