// numerics.h -- exact number-format helpers of the gated-attention kernel
// (device code only).  Formats: IEEE bfloat16 and OCP float8 e4m3 ("fn": bias
// 7, largest finite 448, S.1111.111 NaN, no infinities), the formats of the
// projection row and of the KV cache on the page "012-attention-local-splits.py".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355x_ga {

__device__ inline float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> nearest-even bf16 bit pattern (NaN -> the positive quiet NaN 0x7fc0),
// on the gfx950 converter (v_cvt_pk_bf16_f32).  Checked against the integer
// rounding (add 0x7fff plus the kept lowest bit, truncate) over all 2^32 fp32
// patterns: equal on every non-NaN input, subnormals and infinities included;
// a NaN keeps its own sign and payload there, hence the select.
__device__ inline uint32_t bf16_bits(float f) {
  const uint32_t h = __builtin_bit_cast(unsigned short, (__bf16)f);
  return __builtin_isnan(f) ? 0x7fc0u : h;
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

// Correctly rounded fp32 1/sqrt(a) for finite a > 0.  The hardware estimate y
// is within two fp32 steps of the true value t; the result is y moved by one
// step for each of the four midpoints between y-2..y+2 that t lies beyond.
// Each midpoint m has 25 significant bits, so m*m is exact in fp64 and the
// sign of fma(m*m, a, -1) tells exactly whether t > m (negative) or t < m.
__device__ inline float rsqrt_exact(float a) {
  const float y = __builtin_amdgcn_rsqf(a);
  const uint32_t yb = __float_as_uint(y);
  const double ad = (double)a;
  auto side = [&](uint32_t lo) {  // fma(m*m, a, -1) for m between lo and lo + 1
    const double m = ((double)__uint_as_float(lo) + (double)__uint_as_float(lo + 1u)) * 0.5;
    return fma(m * m, ad, -1.0);
  };
  int step = 0;
  step += side(yb) < 0.0;           // t above the midpoint y | y+1
  step += side(yb + 1u) < 0.0;      // t above y+1 | y+2
  step -= side(yb - 1u) > 0.0;      // t below y-1 | y
  step -= side(yb - 2u) > 0.0;      // t below y-2 | y-1
  return __uint_as_float(yb + (uint32_t)step);
}

}  // namespace mi355x_ga
