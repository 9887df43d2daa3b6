// Error reporting, interface version, and the per-block expert counting
// kernels shared by the router (capacity drop) and the permute.
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
  return 2 * align_up(static_cast<size_t>(nblk * E) * sizeof(int32_t), 256);
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
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<int64_t>(b) * E + e] = cnt[e];
}

// One workgroup; thread e walks the blocks of expert e (loads are coalesced
// across threads), then the kept totals are scanned over experts in LDS.
__global__ void __launch_bounds__(1024) count_scan_kernel(const int32_t* __restrict__ hist,
                                                          int nblk, int E, int64_t cap,
                                                          int32_t* __restrict__ blkoff,
                                                          int32_t* __restrict__ tokens_per_expert,
                                                          int32_t* __restrict__ expert_offsets) {
  __shared__ int part[1024];
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E) {
    int run = 0;
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) {
      const int64_t i = static_cast<int64_t>(b) * E + e;
      const int c = hist[i];
      blkoff[i] = run;
      run += c;
    }
    kept = (cap >= 0 && run > cap) ? static_cast<int>(cap) : run;
    if (tokens_per_expert) tokens_per_expert[e] = kept;
  }
  part[e] = kept;
  __syncthreads();
  // Hillis-Steele inclusive scan over blockDim entries
  for (int off = 1; off < static_cast<int>(blockDim.x); off <<= 1) {
    int v = (e >= off) ? part[e - off] : 0;
    __syncthreads();
    part[e] += v;
    __syncthreads();
  }
  if (expert_offsets && e < E) {
    expert_offsets[e] = part[e] - kept;
    if (e == E - 1) expert_offsets[E] = part[e];
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
                       int32_t* tokens_per_expert, int32_t* expert_offsets, hipStream_t s) {
  const int threads = static_cast<int>(ceil_div(E, 64) * 64);
  hipLaunchKernelGGL(count_scan_kernel, dim3(1), dim3(threads), 0, s, hist,
                     static_cast<int>(nblk), static_cast<int>(E), cap, blkoff, tokens_per_expert,
                     expert_offsets);
}

}  // namespace moe

extern "C" int moe_abi_version(void) { return 1; }

extern "C" const char* moe_last_error(void) { return moe::g_last_error.c_str(); }
