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
// hist[e*nblk + b] = number of tokens of block b (kCountBlock tokens) routed
//                    to e (expert-major, so that the per-expert scan reads a
//                    contiguous run)
// blkoff[b*E + e]  = number of tokens routed to e in blocks before b (with a
//                    capacity: of those kept, min(that number, cap))
size_t count_ws_bytes(int64_t T, int64_t E);  // hist + blkoff + kept[E]
// Fill n int32 with v by a kernel (graph-capture friendly, no memset node).
void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
void launch_block_hist(const uint8_t* map, int64_t T, int64_t E, int32_t* hist, hipStream_t s);
// Workgroups per expert and chunk of blocks: blkoff = exclusive prefix over
// blocks (min(prefix, cap) when cap >= 0), kept[e] = min(total, cap) (cap <
// 0: total).  With cap >= 0 and rmap/probs ([T,E]), also drops the entries
// ranked >= cap (earliest tokens kept), so that blkoff and kept then count
// the final map.
void launch_count_scan(const int32_t* hist, int64_t nblk, int64_t E, int64_t cap, int32_t* blkoff,
                       int32_t* kept, hipStream_t s, int64_t T = 0, float* probs = nullptr,
                       uint8_t* rmap = nullptr);

// moe_permute's argument checks (no GPU call).
moe_status permute_check(int64_t T, int64_t h, int64_t E, int64_t K, int32_t dtype, const void* x,
                         const uint8_t* routing_map, const float* probs, int64_t max_rows,
                         const void* permuted_x, const float* permuted_probs,
                         const int32_t* sorted_token, const int32_t* row_id_map,
                         const int32_t* expert_offsets);

// moe_permute's body.  With given_blkoff (per-block exclusive offsets of each
// expert's entries, block-major [nblk, E]) and given_totals (entries per
// expert), the counting passes are skipped and the workspace is not used.
moe_status permute_impl(int64_t T, int64_t h, int64_t E, int64_t K, int32_t dtype, const void* x,
                        const uint8_t* routing_map, const float* probs, int64_t max_rows,
                        void* permuted_x, float* permuted_probs, int32_t* sorted_token,
                        int32_t* row_id_map, int32_t* expert_offsets, void* workspace,
                        size_t workspace_bytes, hipStream_t s, const int32_t* given_blkoff,
                        const int32_t* given_totals);

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

// ------------------------------------------ LDS staging of MFMA operand tiles
// A stage holds rows of one SBK-wide k slab of bf16 values (SBK*2 bytes per
// row) in 16-byte chunks.  gfx950's LDS serves a 16-byte-per-lane read 16 lanes
// at a time across 64 four-byte banks (256 bytes), so chunks are
// XOR-swizzled such that sixteen lanes reading the same logical chunk of
// sixteen consecutive rows touch sixteen different 16-byte bank groups,
// while a direct-to-LDS load still fills a contiguous 1 KB piece (lane i ->
// bytes 16i):
//   SBK = 32 (64-byte rows): rows 2L and 2L+1 share 128-byte line L;
//     logical chunk lc = (row & 1) * 4 + c sits at lc ^ ((L >> 1) & 3);
//   SBK = 64 (128-byte rows): chunk c of row r sits at c ^ ((r >> 1) & 7);
//   SBK >= 128: chunk c of row r sits at (c & ~15) | ((c & 15) ^ (r & 15)).
template <int SBK>
__device__ __forceinline__ uint32_t lds_chunk_byte(int row, int c) {
  if constexpr (SBK == 32) {
    const int line = row >> 1;
    const int lc = ((row & 1) << 2) | c;
    return static_cast<uint32_t>(line * 128 + ((lc ^ ((line >> 1) & 3)) << 4));
  } else if constexpr (SBK == 64) {
    return static_cast<uint32_t>(row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
  } else {
    const int pc = (c & ~15) | ((c & 15) ^ (row & 15));
    return static_cast<uint32_t>(row * (SBK * 2) + (pc << 4));
  }
}

// Inverse of lds_chunk_byte for a 16-byte piece at stage byte offset o.
template <int SBK>
__device__ __forceinline__ void lds_piece(int o, int& row, int& c) {
  if constexpr (SBK == 32) {
    const int line = o >> 7;
    const int lc = ((o >> 4) & 7) ^ ((line >> 1) & 3);
    row = 2 * line + (lc >> 2);
    c = lc & 3;
  } else if constexpr (SBK == 64) {
    row = o >> 7;
    c = ((o >> 4) & 7) ^ ((row >> 1) & 7);
  } else {
    row = o / (SBK * 2);
    const int pc = (o % (SBK * 2)) >> 4;
    c = (pc & ~15) | ((pc & 15) ^ (row & 15));
  }
}

// Direct global -> LDS 16-byte load: lane i writes LDS bytes
// [lds_base + 16 i, lds_base + 16 i + 16).  Issued as inline assembly so the
// compiler does not serialise the pipeline with conservative waits; the
// kernel waits for these loads itself (vmcnt) before a barrier.  The LDS
// destination goes in m0 as an input operand of the statement, so the
// compiler writes m0 itself and knows the statement reads it; the s_nop
// covers the wait state between that write and the load.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// dma16 with the source as a 32-bit byte offset (per lane) from a 64-bit base
// held in SGPRs (the saddr form), so that a lane's source takes one VGPR.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// dma4 with the source as a 32-bit byte offset from a base held in SGPRs.
__device__ __forceinline__ void dma4s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// A pointer the compiler can keep in SGPRs (its value taken from the first
// active lane; callers pass wave-uniform pointers).
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Direct 4-byte global -> LDS load: lane i writes LDS bytes [base + 4 i, +4).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// Wait until at most n of this wave's vector-memory loads are outstanding.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] bits 3:0, vmcnt[5:4] bits 15:14; expcnt and
  // lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkm0() {
  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int LPW, int STAGES>
__device__ __forceinline__ void wait_stage(int n_after) {
  // wait until at most n_after later stages (of this wave's loads) are in
  // flight; n_after <= STAGES - 1
  if constexpr (STAGES >= 6) { if (n_after >= 5) { wait_vmcnt<LPW * 5>(); return; } }
  if constexpr (STAGES >= 5) { if (n_after >= 4) { wait_vmcnt<LPW * 4>(); return; } }
  if constexpr (STAGES >= 4) { if (n_after >= 3) { wait_vmcnt<LPW * 3>(); return; } }
  if constexpr (STAGES >= 3) { if (n_after >= 2) { wait_vmcnt<LPW * 2>(); return; } }
  if (n_after >= 1) { wait_vmcnt<LPW * 1>(); return; }
  wait_vmcnt<0>();
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
