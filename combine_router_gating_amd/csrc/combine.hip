// Combine: unpermute the expert outputs and weight them by the router probs.
//
// Megatron Core MoE 源码路径解析 §2: the combine step takes the expert outputs
// and the probs and returns rows in token order; the shared expert's output
// is added to that result (§11).  MoE Internals: DeepSpeed-Megatron Expert
// Parallel Implementation §8, last step: unpermute and combine with the gate
// weights.
//
// One wave per token gathers its K rows (row_id_map), accumulates
// p_k * y_k in fp32 in ascending k order, adds the shared output, and rounds
// once.  No atomics: the result is bitwise reproducible.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16>
struct Chunk;  // 16 bytes of one row, as fp32 values

template <>
struct Chunk<true> {
  static constexpr int N = 8;
  __device__ static void load(const uint4* p, float* v) {
    const uint4 u = *p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(uint4* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
    *p = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <>
struct Chunk<false> {
  static constexpr int N = 4;
  __device__ static void load(const uint4* p, float* v) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
  __device__ static void store(uint4* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

constexpr int kUnroll = 4;  // 16-byte chunks per lane in flight

template <bool BF16>
__global__ void __launch_bounds__(256) combine_kernel(const uint4* __restrict__ y,
                                                      const float* __restrict__ pprobs,
                                                      const int32_t* __restrict__ row_id_map,
                                                      int64_t T, int chunks, int K,
                                                      int64_t max_rows,
                                                      const uint4* __restrict__ shared,
                                                      uint4* __restrict__ out) {
  using C = Chunk<BF16>;
  const int lane = threadIdx.x % 64;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (t >= T) return;  // whole wave
  int my_row = -1;
  float my_p = 0.f;
  if (lane < K) {
    const int r = row_id_map[t * K + lane];
    if (r >= 0 && r < max_rows) {
      my_row = r;
      my_p = pprobs[r];
    }
  }
  for (int c0 = 0; c0 < chunks; c0 += 64 * kUnroll) {
    float acc[kUnroll][C::N];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < C::N; ++i) acc[u][i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int r = __shfl(my_row, k, 64);
      if (r < 0) continue;  // wave-uniform
      const float p = __shfl(my_p, k, 64);
      const uint4* src = y + static_cast<int64_t>(r) * chunks;
      float v[kUnroll][C::N];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < chunks) C::load(src + c, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int i = 0; i < C::N; ++i) acc[u][i] = fmaf(p, v[u][i], acc[u][i]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c >= chunks) continue;
      if (shared) {
        float sv[C::N];
        C::load(shared + t * chunks + c, sv);
#pragma unroll
        for (int i = 0; i < C::N; ++i) acc[u][i] += sv[i];
      }
      C::store(out + t * chunks + c, acc[u]);
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(int64_t T, int64_t h, int64_t K, int32_t dtype,
                                  const void* expert_out, const float* permuted_probs,
                                  const int32_t* row_id_map, int64_t max_rows,
                                  const void* shared_out, void* out, void* stream) {
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "moe_combine: T out of range");
  MOE_REQUIRE(K >= 1 && K <= kMaxTopK, MOE_ERR_ARG, "moe_combine: bad K=%lld", (long long)K);
  MOE_REQUIRE(h >= 1 && h % 8 == 0, MOE_ERR_UNSUPPORTED, "moe_combine: h=%lld must be a multiple of 8",
              (long long)h);
  MOE_REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_ARG, "moe_combine: bad dtype %d", dtype);
  MOE_REQUIRE(max_rows >= 0, MOE_ERR_ARG, "moe_combine: max_rows < 0");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(row_id_map && out && (max_rows == 0 || (expert_out && permuted_probs)), MOE_ERR_ARG,
              "moe_combine: NULL tensor argument");
  const hipStream_t s = as_stream(stream);
  const int esize = dtype == MOE_BF16 ? 2 : 4;
  const int chunks = static_cast<int>(h * esize / 16);
  const dim3 grid(static_cast<unsigned>(ceil_div(T, 4)));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s,
                       static_cast<const uint4*>(expert_out), permuted_probs, row_id_map, T, chunks,
                       static_cast<int>(K), max_rows, static_cast<const uint4*>(shared_out),
                       static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s,
                       static_cast<const uint4*>(expert_out), permuted_probs, row_id_map, T, chunks,
                       static_cast<int>(K), max_rows, static_cast<const uint4*>(shared_out),
                       static_cast<uint4*>(out));
  return check_launch("moe_combine");
}
