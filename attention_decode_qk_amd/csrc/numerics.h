// numerics.h -- exact number-format helpers of the gated-attention kernel
// (device code only).  Formats: IEEE bfloat16 and OCP float8 e4m3 ("fn": bias
// 7, largest finite 448, S.1111.111 NaN, no infinities), the formats of the
// projection row and of the KV cache on the page "012-attention-local-splits.py".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355x_ga {

__device__ inline float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> nearest-even bf16 bit pattern (NaN -> quiet NaN).
__device__ inline uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> nearest-even bf16, returned as the fp32 value it represents.
__device__ inline float round_bf16(float f) { return __uint_as_float(bf16_bits(f) << 16); }

// Two fp32 values -> two OCP e4m3 codes (low half-word: a, then b) with the
// gfx950 converter, which rounds to nearest even and keeps the sign of zero.
// Magnitudes are first clamped to 448 so overflow and infinities saturate to
// the largest finite code; a NaN input gives the NaN code with its sign.
__device__ inline uint32_t e4m3x2(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xffffu;
  if (a != a) w = (w & 0xff00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7fu;
  if (b != b) w = (w & 0x00ffu) | ((((__float_as_uint(b) >> 24) & 0x80u) | 0x7fu) << 8);
  return w;
}

// Correctly rounded fp32 1/sqrt(a) for finite a > 0: the hardware estimate is
// within two fp32 steps; each neighbour midpoint m (25 significant bits, m*m
// exact in fp64) is tested exactly through the sign of fma(m*m, a, -1).
__device__ inline float rsqrt_exact(float a) {
  float y = __builtin_amdgcn_rsqf(a);
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const uint32_t yb = __float_as_uint(y);
    const float up = __uint_as_float(yb + 1u);
    const double mu = ((double)y + (double)up) * 0.5;
    if (fma(mu * mu, (double)a, -1.0) < 0.0) {
      y = up;
      continue;
    }
    const float dn = __uint_as_float(yb - 1u);
    const double md = ((double)y + (double)dn) * 0.5;
    if (fma(md * md, (double)a, -1.0) > 0.0) {
      y = dn;
      continue;
    }
    break;
  }
  return y;
}

}  // namespace mi355x_ga
