// Internal helpers shared by the HIP translation units of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- errors (host)
moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status check_launch(const char* what);
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

#define MOE_REQUIRE(cond, code, ...)            \
  do {                                          \
    if (!(cond)) return ::moe::fail(code, __VA_ARGS__); \
  } while (0)

// ---------------------------------------------------------------- limits
constexpr int64_t kMaxExperts = 1024;
constexpr int64_t kMaxTopK = 64;
constexpr int kCountBlock = 16;  // tokens per counting block (route hist, drop, permute)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------- per-block expert counts and their scan
// hist[b*E + e]   = number of tokens of block b (kCountBlock tokens) routed to e
// blkoff[b*E + e] = number of tokens routed to e in blocks before b
size_t count_ws_bytes(int64_t T, int64_t E);  // hist + blkoff + kept[E]
// Fill n int32 with v by a kernel (graph-capture friendly, no memset node).
void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
void launch_block_hist(const uint8_t* map, int64_t T, int64_t E, int32_t* hist, hipStream_t s);
// One workgroup per expert: blkoff = exclusive prefix over blocks,
// kept[e] = min(total, cap) (cap < 0: total).
void launch_count_scan(const int32_t* hist, int64_t nblk, int64_t E, int64_t cap, int32_t* blkoff,
                       int32_t* kept, hipStream_t s);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Exclusive scan over a workgroup of NW waves.  Returns this thread's
// exclusive prefix; *total receives the sum.  `scratch` is >= NW LDS
// entries.  Every thread of the workgroup must call it.
template <int NW>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* scratch, int64_t* total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t s = scratch[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ int64_t block_exclusive_scan256(int64_t v, int64_t* scratch,
                                                           int64_t* total) {
  return block_exclusive_scan<4>(v, scratch, total);
}

// LDS layout for tiles of 64-byte rows (32 bf16 of k) read as 16-byte MFMA
// fragments: rows 2L and 2L+1 share 128-byte line L, and logical chunk
// lc = (row & 1) * 4 + c (c = 0..3) sits at physical chunk lc ^ ((L >> 1) & 3),
// so 16 lanes reading one chunk of 16 consecutive rows hit 16 different
// 16-byte bank groups (gfx950: 64 banks of 4 bytes, 16 lanes per cycle).
__device__ __forceinline__ uint32_t lds_swz64b(int row, int c) {
  const int line = row >> 1;
  const int lc = ((row & 1) << 2) | c;
  return static_cast<uint32_t>(line * 128 + ((lc ^ ((line >> 1) & 3)) << 4));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace moe
