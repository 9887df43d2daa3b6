// MXFP8 (OCP Microscaling, E4M3 elements) block quantisation.
//
// Scalable Training of Mixture-of-Experts Models with Megatron Core (FP8/FP4
// 低精度训练) names FP8 GEMMs among the MoE optimisations without a scaling
// recipe; this library uses the OCP MX v1.0 MXFP8-E4M3 format, which
// gfx950's scaled MFMA consumes directly: 32 consecutive values share a
// power-of-two scale X = 2^(floor(log2 amax) - 8) (8 = exponent of E4M3's
// largest normal, 448), stored as an E8M0 byte (exponent + 127, clamped to
// [0, 254]; an all-zero block gets 0, i.e. 2^-127); each element is V / X
// rounded to the nearest E4M3 value, ties to even, saturated to +-448.
// E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals
// m * 2^-9, no infinities.
//
// Scale layouts: row-major [rows, cols/32], or k-tiled for GEMM operands
// whose rows a tile reads contiguously: [rows/R, cols/128, R, 4], so that
// the 4 scales of one 128-wide k stage of R consecutive rows are one
// contiguous run of 4R bytes (R = rows per expert for a weight).
#include "mx_codec.h"

namespace moe {

namespace {

// One lane per 32-value block; a wave covers 64 consecutive blocks of a row.
template <typename T>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const T* __restrict__ src, int64_t rows,
                                                          int64_t cols, int64_t tile_rows,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t nb = cols / 32;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (blk >= rows * nb) return;
  const int64_t row = blk / nb, b = blk % nb;
  const T* p = src + row * cols + b * 32;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (sizeof(T) == 2) v[i] = bf16_bits_to_f32(p[i]);
    else v[i] = p[i];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_scale_exp(amax);
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e, exact
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_code(v[4 * q + i] * inv) << (8 * i);
    w[q] = word;
  }
  uint4* out = reinterpret_cast<uint4*>(codes + row * cols + b * 32);
  out[0] = make_uint4(w[0], w[1], w[2], w[3]);
  out[1] = make_uint4(w[4], w[5], w[6], w[7]);
  int64_t si;
  if (tile_rows > 0) {  // [rows/tile_rows, cols/128, tile_rows, 4]
    const int64_t g = row / tile_rows, r = row % tile_rows;
    si = ((g * (cols / 128) + b / 4) * tile_rows + r) * 4 + (b & 3);
  } else {
    si = row * nb + b;
  }
  scales[si] = static_cast<uint8_t>(e + 127);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_mxfp8_quantize(int64_t rows, int64_t cols, int64_t tile_rows,
                                         int32_t dtype, const void* src, uint8_t* codes,
                                         uint8_t* scales, void* stream) {
  MOE_REQUIRE(rows >= 0 && cols >= 0, MOE_ERR_ARG, "moe_mxfp8_quantize: negative size");
  MOE_REQUIRE(cols % 32 == 0, MOE_ERR_UNSUPPORTED, "moe_mxfp8_quantize: cols=%lld is not a multiple of 32",
              (long long)cols);
  MOE_REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_ARG, "moe_mxfp8_quantize: bad dtype %d", dtype);
  MOE_REQUIRE(tile_rows >= 0, MOE_ERR_ARG, "moe_mxfp8_quantize: tile_rows < 0");
  MOE_REQUIRE(tile_rows == 0 || (cols % 128 == 0 && rows % tile_rows == 0), MOE_ERR_UNSUPPORTED,
              "moe_mxfp8_quantize: the k-tiled scale layout needs cols %% 128 == 0 and rows %% "
              "tile_rows == 0");
  MOE_REQUIRE(rows * (cols / 32) < (int64_t(1) << 40), MOE_ERR_UNSUPPORTED, "moe_mxfp8_quantize: too large");
  if (rows == 0 || cols == 0) return MOE_OK;
  MOE_REQUIRE(src && codes && scales, MOE_ERR_ARG, "moe_mxfp8_quantize: NULL tensor argument");
  const int64_t blocks = rows * (cols / 32);
  const dim3 grid(static_cast<unsigned>(ceil_div(blocks, 256)));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(mx_quantize_kernel<uint16_t>, grid, dim3(256), 0, as_stream(stream),
                       static_cast<const uint16_t*>(src), rows, cols, tile_rows, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize_kernel<float>, grid, dim3(256), 0, as_stream(stream),
                       static_cast<const float*>(src), rows, cols, tile_rows, codes, scales);
  return check_launch("moe_mxfp8_quantize");
}
