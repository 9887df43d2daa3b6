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
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<int64_t>(b) * E + e] = cnt[e];
}

// One workgroup per expert: each thread sums a contiguous run of blocks,
// the runs are scanned across the workgroup, then each thread writes the
// exclusive prefixes of its run.
__global__ void __launch_bounds__(256) count_scan_kernel(const int32_t* __restrict__ hist,
                                                         int nblk, int E, int64_t cap,
                                                         int32_t* __restrict__ blkoff,
                                                         int32_t* __restrict__ kept) {
  __shared__ int64_t scratch[4];
  const int e = blockIdx.x;
  const int per = (nblk + 255) / 256;
  const int b0 = threadIdx.x * per;
  const int b1 = min(nblk, b0 + per);
  int64_t sum = 0;
  for (int b = b0; b < b1; ++b) sum += hist[static_cast<int64_t>(b) * E + e];
  int64_t total;
  int64_t run = block_exclusive_scan256(sum, scratch, &total);
  for (int b = b0; b < b1; ++b) {
    const int64_t i = static_cast<int64_t>(b) * E + e;
    const int c = hist[i];
    blkoff[i] = static_cast<int32_t>(run);
    run += c;
  }
  if (threadIdx.x == 0) kept[e] = static_cast<int32_t>((cap >= 0 && total > cap) ? cap : total);
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
                       int32_t* kept, hipStream_t s) {
  hipLaunchKernelGGL(count_scan_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, s, hist,
                     static_cast<int>(nblk), static_cast<int>(E), cap, blkoff, kept);
}

}  // namespace moe

extern "C" int moe_abi_version(void) { return 2; }

extern "C" const char* moe_last_error(void) { return moe::g_last_error.c_str(); }
