// MXFP8-E4M3 element and scale encoding shared by the quantisation kernel
// and the grouped GEMM's fused activation quantisation (see mx.hip for the
// format).
#pragma once

#include "moe_internal.h"

namespace moe {

// E4M3 code of fp32 v (any finite value): nearest, ties to even, saturating.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0x1p-6f) {                       // subnormal range: multiples of 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.0f));  // 0..8 (8 = smallest normal)
  } else {
    const uint32_t b = __float_as_uint(a);
    // round the 23-bit mantissa to 3 bits, ties to even (a carry bumps the exponent)
    const uint32_t r = b + 0x7ffffu + ((b >> 20) & 1u);
    const int e = static_cast<int>((r >> 23) & 255u) - 127;  // -6 .. (saturated below)
    code = (e > 8) ? 0x7eu : ((static_cast<uint32_t>(e + 7) << 3) | ((r >> 20) & 7u));
    if (code > 0x7eu) code = 0x7eu;        // 1.875 * 2^8 = 480 > 448: saturate
  }
  return sign | code;
}

// E8M0 exponent (unbiased) of a block whose largest magnitude is amax.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  // floor(log2 amax) - 8, clamped to [-127, 127]; a zero or subnormal amax
  // (floor(log2) <= -127) clamps to -127
  const int be = static_cast<int>((__float_as_uint(amax) >> 23) & 255u);
  if (be == 0) return -127;
  const int e = be - 127 - 8;
  return e < -127 ? -127 : e;
}

}  // namespace moe
