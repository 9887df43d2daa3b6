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
  __device__ static void load(const uint4* p, float* v) { from(*p, v); }
  __device__ static void from(const uint4 u, float* v) {
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
  __device__ static void load(const uint4* p, float* v) { from(*p, v); }
  __device__ static void from(const uint4 u, float* v) {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
  }
  __device__ static void store(uint4* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// A wave's loads for KG of its token's K rows (KU 16-byte chunks per lane of
// each) are all issued before any is accumulated, so a token keeps KG*KU*1 KB
// in flight instead of one row's chunks at a time; the accumulation order
// (ascending k, one fma per element) is unchanged.  Expert rows and shared
// rows are read exactly once, so their loads are non-temporal (measured on
// the DeepSeek-V3-shaped layer: 247 -> 219 us, 4.8 -> 5.35 TB/s; the
// output stores keep the default policy, non-temporal stores were slower).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool BF16, int KG, int KU>
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
  for (int c0 = 0; c0 < chunks; c0 += 64 * KU) {
    uint4 sh[KU];
    if (shared) {
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < chunks) sh[u] = load_once(shared + t * chunks + c);
      }
    }
    float acc[KU][C::N];
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int i = 0; i < C::N; ++i) acc[u][i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KG) {
      int r[KG];
      float p[KG];
      uint4 raw[KG][KU];
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        r[g] = __shfl(my_row, min(k0 + g, 63), 64);
        p[g] = __shfl(my_p, min(k0 + g, 63), 64);
        if (k0 + g >= K) r[g] = -1;
      }
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        if (r[g] < 0) continue;  // wave-uniform
        const uint4* src = y + static_cast<int64_t>(r[g]) * chunks;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < chunks) raw[g][u] = load_once(src + c);
        }
      }
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        if (r[g] < 0) continue;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          float v[C::N];
          C::from(raw[g][u], v);
#pragma unroll
          for (int i = 0; i < C::N; ++i) acc[u][i] = fmaf(p[g], v[i], acc[u][i]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c >= chunks) continue;
      if (shared) {
        float sv[C::N];
        C::from(sh[u], sv);
#pragma unroll
        for (int i = 0; i < C::N; ++i) acc[u][i] += sv[i];
      }
      C::store(out + t * chunks + c, acc[u]);
    }
  }
}

template <bool BF16, int KG, int KU>
void launch_combine(dim3 grid, hipStream_t s, const void* y, const float* pp, const int32_t* rim,
                    int64_t T, int chunks, int K, int64_t max_rows, const void* shared, void* out) {
  hipLaunchKernelGGL((combine_kernel<BF16, KG, KU>), grid, dim3(256), 0, s,
                     static_cast<const uint4*>(y), pp, rim, T, chunks, K, max_rows,
                     static_cast<const uint4*>(shared), static_cast<uint4*>(out));
}

template <bool BF16>
void dispatch_combine(dim3 grid, hipStream_t s, const void* y, const float* pp, const int32_t* rim,
                      int64_t T, int chunks, int K, int64_t max_rows, const void* shared, void* out) {
  if (K <= 1) launch_combine<BF16, 1, 8>(grid, s, y, pp, rim, T, chunks, K, max_rows, shared, out);
  else if (K <= 2) launch_combine<BF16, 2, 4>(grid, s, y, pp, rim, T, chunks, K, max_rows, shared, out);
  else if (K <= 4) launch_combine<BF16, 4, 4>(grid, s, y, pp, rim, T, chunks, K, max_rows, shared, out);
  else launch_combine<BF16, 8, 2>(grid, s, y, pp, rim, T, chunks, K, max_rows, shared, out);
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
  const int Ki = static_cast<int>(K);
  if (dtype == MOE_BF16)
    dispatch_combine<true>(grid, s, expert_out, permuted_probs, row_id_map, T, chunks, Ki, max_rows,
                           shared_out, out);
  else
    dispatch_combine<false>(grid, s, expert_out, permuted_probs, row_id_map, T, chunks, Ki, max_rows,
                            shared_out, out);
  return check_launch("moe_combine");
}
