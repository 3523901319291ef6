// prologue.hip -- kernel 1 of the gated-attention step: per-head unweighted
// RMSNorm of q and k, interleaved RoPE, the q cast to e4m3 and the e4m3 K/V
// store at each new token's cache row.
//
// Definition: page "012-attention-local-splits.py", the `_prepare_qkv` Triton
// kernel and the `_cos_sin` table recipe.  Every fp32 step the page writes is
// rounded exactly once here (contraction is off for this file), so the stored
// bytes are a deterministic function of the inputs:
//   * sum of squares: each square of a bf16 value is exact in fp32 and the sum
//     of 64 of them is formed in fp64, where it is exact, then rounded once;
//   * 1/sqrt(ms + 1e-5) is the correctly rounded fp32 value;
//   * cos/sin of the fp32 angle are evaluated in fp64 and rounded once, the
//     page's 2^21 x 64 table is never built;
//   * bf16 and e4m3 roundings are to nearest even; e4m3 saturates at 448.
//
// Mapping: 16 lanes per head row (4 columns each, one 8-byte load), 4 head rows
// per wave, 16 head rows per 256-thread workgroup; the 20 head rows of a token
// are its 16 q heads, 2 k heads and 2 v heads.  RoPE pairs (2i, 2i+1) stay
// inside a lane.
#include "kernels.h"

#pragma clang fp contract(off)

namespace mi355x_ga {
namespace {

__device__ inline float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> nearest-even bf16, returned as the fp32 value it represents.
__device__ inline float round_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return __uint_as_float(0x7fc00000u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

// fp32 -> OCP float8 e4m3 code, nearest even, signed zero kept, |x| >= 448
// saturating to the largest finite code, NaN to the NaN code.
__device__ inline uint32_t to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (!(ax == ax)) return sign | 0x7fu;
  if (ax >= 448.0f) return sign | 0x7eu;
  if (ax < 0.015625f) {  // below 2^-6: subnormal step 2^-9
    return sign | (uint32_t)__builtin_rintf(ax * 512.0f);
  }
  int e = (int)((__float_as_uint(ax) >> 23) & 0xffu) - 127;  // 2^e <= ax < 2^(e+1)
  float m = __builtin_rintf(__builtin_ldexpf(ax, 3 - e));    // 8..16, nearest even
  if (m == 16.0f) {
    m = 8.0f;
    e += 1;
  }
  return sign | (uint32_t)(((e + 7) << 3) | ((int)m - 8));
}

// Correctly rounded fp32 1/sqrt(a) for finite a > 0: an fp64 estimate is within
// one fp32 step; each neighbour midpoint m (25 significant bits, m*m exact in
// fp64) is tested exactly through the sign of fma(m*m, a, -1).
__device__ inline float rsqrt_exact(float a) {
  float y = (float)(1.0 / sqrt((double)a));
#pragma unroll
  for (int it = 0; it < 2; ++it) {
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

__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
  constexpr int kHeads = kQHeads + 2 * kKvHeads;  // 20 head rows per token
  const int lane16 = threadIdx.x & 15;
  const int64_t hr = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool active = hr < (int64_t)p.tokens * kHeads;
  const int64_t t = active ? hr / kHeads : 0;
  const int head = active ? (int)(hr % kHeads) : 0;
  const int col = lane16 * 4;

  const uint2 raw = *reinterpret_cast<const uint2*>(p.qkv + t * kWidth + head * kHeadDim + col);
  float x[4] = {bf16_value(raw.x & 0xffffu), bf16_value(raw.x >> 16), bf16_value(raw.y & 0xffffu),
                bf16_value(raw.y >> 16)};

  // Sum of squares over the head row (16 lanes): exact in fp64.
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) ss += (double)(x[k] * x[k]);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 16);

  const bool is_v = head >= kQHeads + kKvHeads;
  float y[4];
  if (!is_v) {
    const float ms = (float)ss / 64.0f;
    const float inv = rsqrt_exact(ms + 1.0e-5f);
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = round_bf16(x[k] * inv);
    if (p.rope) {
      const float pos = (float)p.positions[t];
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const float ang = pos * p.inv_freq[lane16 * 2 + pr];
        const float c = (float)cos((double)ang);
        const float s = (float)sin((double)ang);
        const float e = y[2 * pr], o = y[2 * pr + 1];
        const float ec = e * c, os = o * s, oc = o * c, es = e * s;
        y[2 * pr] = round_bf16(ec - os);
        y[2 * pr + 1] = round_bf16(oc + es);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = x[k];  // values are stored un-normed
  }
  if (!active) return;

  if (head < kQHeads) {
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) packed |= to_e4m3(y[k]) << (8 * k);
    *reinterpret_cast<uint32_t*>(p.q_out + (t * kQHeads + head) * kHeadDim + col) = packed;
    return;
  }
  const int64_t slot = p.cache_loc[t];
  if (slot < 0 || slot >= p.num_rows) return;
  const bool is_k = !is_v;
  const int g = is_k ? head - kQHeads : head - kQHeads - kKvHeads;
  if (p.scaled) {
    const float sc = is_k ? *p.k_scale : *p.v_scale;
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = round_bf16(y[k] / sc);
  }
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) packed |= to_e4m3(y[k]) << (8 * k);
  uint8_t* dst = (is_k ? p.k_cache : p.v_cache) + (slot * kKvHeads + g) * kHeadDim + col;
  *reinterpret_cast<uint32_t*>(dst) = packed;
}

}  // namespace

hipError_t launch_prologue(const PrologueParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.tokens * (kQHeads + 2 * kKvHeads);
  const unsigned grid = (unsigned)((rows + 15) / 16);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prologue_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mi355x_ga
