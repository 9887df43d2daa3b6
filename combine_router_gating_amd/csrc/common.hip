// Error reporting, interface version, and the per-block expert counting
// kernels shared by the router (capacity drop) and the permute.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "moe_internal.h"

namespace moe {

static thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

size_t count_ws_bytes(int64_t T, int64_t E) {
  const int64_t nblk = ceil_div(T, kCountBlock);
  return 2 * align_up(static_cast<size_t>(nblk * E) * sizeof(int32_t), 256) +
         align_up(static_cast<size_t>(E) * sizeof(int32_t), 256);
}

// One workgroup per block of kCountBlock tokens: count the routed entries of
// each expert in LDS (integer atomics: the sum does not depend on order).
__global__ void __launch_bounds__(256) block_hist_kernel(const uint8_t* __restrict__ map,
                                                         int64_t T, int E,
                                                         int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(b) * kCountBlock;
  const int64_t nt = min(static_cast<int64_t>(kCountBlock), T - t0);
  const uint8_t* base = map + t0 * E;
  const int n = static_cast<int>(nt) * E;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    if (base[i]) atomicAdd(&cnt[i % E], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<int64_t>(e) * gridDim.x + b] = cnt[e];
}

// Workgroup (e, s) scans chunk s of expert e's blocks: the counts before
// and after the chunk are summed, the chunk's own blocks are split into
// contiguous runs, one per thread, and scanned across the workgroup; each
// thread writes the exclusive prefixes of its run.  With a capacity and the
// map, the same pass drops expert e's entries ranked >= cap (rank = entries
// of e in earlier tokens, so the earliest tokens are kept): the one block
// whose ranks cross cap is walked in token order, and every entry of the
// blocks after it (all ranked >= cap) is cleared by the whole workgroup.
__global__ void __launch_bounds__(256) count_scan_kernel(const int32_t* __restrict__ hist,
                                                         int nblk, int E, int64_t cap,
                                                         int32_t* __restrict__ blkoff,
                                                         int32_t* __restrict__ kept, int64_t T,
                                                         float* __restrict__ probs,
                                                         uint8_t* __restrict__ rmap) {
  constexpr int kPre = 1024;  // map column bytes of a chunk held in LDS (up to 64 blocks)
  __shared__ int64_t scratch[4];
  __shared__ int s_past;  // first block of the chunk whose entries all rank >= cap
  __shared__ uint8_t s_m[kPre];
  const int e = blockIdx.x;
  const int cb = (nblk + static_cast<int>(gridDim.y) - 1) / static_cast<int>(gridDim.y);
  const int c0 = min(nblk, static_cast<int>(blockIdx.y) * cb);
  const int c1 = min(nblk, c0 + cb);
  const int32_t* h = hist + static_cast<int64_t>(e) * nblk;
  // With a capacity, the chunk's map column is read together with the counts
  // (one round trip), so the drop below reads it from LDS.
  const int64_t ct0 = static_cast<int64_t>(c0) * kCountBlock;
  const int64_t ct1 = min(T, static_cast<int64_t>(c1) * kCountBlock);
  const bool pref = rmap && cap >= 0 && ct1 - ct0 <= kPre;
  uint8_t pm[kPre / 256];
  if (pref) {
#pragma unroll
    for (int u = 0; u < kPre / 256; ++u) {
      const int64_t t = ct0 + threadIdx.x + 256 * u;
      pm[u] = t < ct1 ? rmap[t * E + e] : 0;
    }
  }
  const int per = (c1 - c0 + 255) / 256;
  const int b0 = c0 + static_cast<int>(threadIdx.x) * per;
  const int b1 = min(c1, b0 + per);
  int64_t sum = 0, pre = 0, post = 0;
  for (int b = b0; b < b1; ++b) sum += h[b];
  for (int b = threadIdx.x; b < c0; b += 256) pre += h[b];
  for (int b = c1 + static_cast<int>(threadIdx.x); b < nblk; b += 256) post += h[b];
  int64_t chunk, outside;
  int64_t run = block_exclusive_scan256(sum, scratch, &chunk);
  // counts are below 2^31, so both sums fit one 64-bit word without a carry
  block_exclusive_scan256((pre << 32) | post, scratch, &outside);
  const int64_t before = outside >> 32;
  const int64_t total = before + chunk + (outside & 0xffffffffll);
  run += before;
  const bool drop = rmap && cap >= 0 && total > cap;
  if (threadIdx.x == 0) {
    s_past = c1;
    if (blockIdx.y == 0) kept[e] = static_cast<int32_t>((cap >= 0 && total > cap) ? cap : total);
  }
  if (pref) {
#pragma unroll
    for (int u = 0; u < kPre / 256; ++u) s_m[threadIdx.x + 256 * u] = pm[u];
  }
  __syncthreads();
  auto map_at = [&](int64_t t) -> uint8_t { return pref ? s_m[t - ct0] : rmap[t * E + e]; };
  for (int b = b0; b < b1; ++b) {
    const int c = h[b];
    blkoff[static_cast<int64_t>(b) * E + e] = static_cast<int32_t>(cap >= 0 && run > cap ? cap : run);
    if (drop && run >= cap) atomicMin(&s_past, b);
    if (drop && run < cap && run + c > cap) {
      const int64_t t0 = static_cast<int64_t>(b) * kCountBlock;
      const int nt = static_cast<int>(min(static_cast<int64_t>(kCountBlock), T - t0));
      uint8_t m[kCountBlock];
#pragma unroll
      for (int i = 0; i < kCountBlock; ++i) m[i] = i < nt ? map_at(t0 + i) : 0;
      int64_t r = run;
#pragma unroll
      for (int i = 0; i < kCountBlock; ++i) {
        if (m[i]) {
          if (r >= cap) {
            rmap[(t0 + i) * E + e] = 0;
            probs[(t0 + i) * E + e] = 0.f;
          }
          ++r;
        }
      }
    }
    run += c;
  }
  if (drop) {
    __syncthreads();
    const int64_t end = min(T, static_cast<int64_t>(c1) * kCountBlock);
    constexpr int kU = 4;
    for (int64_t t = static_cast<int64_t>(s_past) * kCountBlock + threadIdx.x; t < end;
         t += 256 * kU) {
      uint8_t m[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) m[u] = t + 256 * u < end ? map_at(t + 256 * u) : 0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (m[u]) {
          rmap[(t + 256 * u) * E + e] = 0;
          probs[(t + 256 * u) * E + e] = 0.f;
        }
      }
    }
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s,
                     p, n, v);
}

void launch_block_hist(const uint8_t* map, int64_t T, int64_t E, int32_t* hist, hipStream_t s) {
  const int64_t nblk = ceil_div(T, kCountBlock);
  hipLaunchKernelGGL(block_hist_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, map, T,
                     static_cast<int>(E), hist);
}

void launch_count_scan(const int32_t* hist, int64_t nblk, int64_t E, int64_t cap, int32_t* blkoff,
                       int32_t* kept, hipStream_t s, int64_t T, float* probs, uint8_t* rmap) {
  // chunks of about 32 blocks, at most 32 per expert (each reads the whole
  // row); on the Switch-shaped router 9.0 us against 9.8 with 64-block
  // chunks and 13.1 with 128
  const int64_t chunks = std::min<int64_t>(32, std::max<int64_t>(1, ceil_div(nblk, 32)));
  hipLaunchKernelGGL(count_scan_kernel, dim3(static_cast<unsigned>(E), static_cast<unsigned>(chunks)),
                     dim3(256), 0, s, hist,
                     static_cast<int>(nblk), static_cast<int>(E), cap, blkoff, kept, T, probs, rmap);
}

}  // namespace moe

namespace moe {

// One wave; lane 0 sleeps in short steps until `ticks` of the constant
// 100 MHz counter have passed, then stores the shader-clock cycles
// (s_memtime) and real-time ticks (s_memrealtime) that elapsed meanwhile.
__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long* __restrict__ out,
                                                         unsigned long long ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_readcyclecounter();
  unsigned long long r = r0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  out[0] = c1 - c0;
  out[1] = r - r0;
}

}  // namespace moe

extern "C" moe_status moe_clock_probe(uint64_t* out, int64_t spin_us, void* stream) {
  if (!out) return moe::fail(MOE_ERR_ARG, "moe_clock_probe: out is null");
  if (spin_us <= 0 || spin_us > 1000000)
    return moe::fail(MOE_ERR_ARG, "moe_clock_probe: spin_us %lld outside (0, 1e6]",
                     static_cast<long long>(spin_us));
  hipLaunchKernelGGL(moe::clock_probe_kernel, dim3(1), dim3(64), 0, moe::as_stream(stream),
                     reinterpret_cast<unsigned long long*>(out),
                     static_cast<unsigned long long>(spin_us) * 100ull);
  return moe::check_launch("moe_clock_probe");
}

extern "C" int moe_abi_version(void) { return 8; }

extern "C" const char* moe_last_error(void) { return moe::g_last_error.c_str(); }
