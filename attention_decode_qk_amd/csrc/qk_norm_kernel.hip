// qk_norm_kernel.hip -- per-head unweighted RMSNorm with an output scale, the
// operation of the page "qk_norm" (vLLM's CuTeDSL fused QK-norm for
// MuseSpark1x attention: the `qk_norm` function and QKNormDirectKernel's
// kernel).  Each head_dim-wide group of a row of x [M, heads * D] (rows
// `row_stride` elements apart, the last dimension contiguous) becomes
// round(x * rstd [* scale]) with rstd = 1/sqrt(sum(x^2)/D + eps); the product
// stays fp32 and the store is the only rounding.
//
// gfx950 layout: a head group is D/8 consecutive lanes holding 16 bytes (8
// values) each, so one wave reads 1 KB of whole groups per load; the sum of
// squares (each square exact in fp32) is formed exactly in fp64, reduced over
// the group's lanes, rounded once to fp32; rsqrt is correctly rounded (the
// estimate corrected by exact midpoint tests).  The operation streams: HBM
// bandwidth bounds it, so there is no LDS and no matrix-core work.
#include <algorithm>

#include "kernels.h"
#include "numerics.h"

namespace mi355x_ga {
namespace {

// Sum over the n consecutive lanes of a group (n a power of two <= 32).
template <int N>
__device__ inline double group_sum(double v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v += __shfl_xor(v, m, N);
  return v;
}

// binary16 <-> fp32 in integer arithmetic, subnormals included (the hardware
// conversions flush binary16 subnormals under the default float mode).
__device__ inline float half_value(uint32_t h) {
  const uint32_t sign = (h & 0x8000u) << 16, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  if (e == 0) {  // zero or subnormal: m * 2^-24, exact in fp32
    const float v = (float)m * 0x1p-24f;
    return __uint_as_float(__float_as_uint(v) | sign);
  }
  if (e == 0x1f) return __uint_as_float(sign | 0x7f800000u | (m << 13));  // inf, NaN
  return __uint_as_float(sign | ((e + 112u) << 23) | (m << 13));
}

// fp32 -> binary16, round to nearest even; overflow to infinity, NaN quiet.
__device__ inline uint32_t half_bits(float f) {
  const uint32_t u = __float_as_uint(f), sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00u;
  if (a >= 0x477ff000u) return sign | 0x7c00u;  // >= 65520: infinity
  if (a >= 0x38800000u) {                        // >= 2^-14: normal binary16
    const uint32_t r = a + 0xfffu + ((a >> 13) & 1u);
    return sign | ((r >> 13) - (112u << 10));
  }
  // Subnormal (quantum 2^-24) or zero: the scaled value is exact in fp32 and
  // rint rounds it to the nearest even integer (1024 is the smallest normal).
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 0x1p24f);
}

template <bool FP16>
__device__ inline float value16(uint32_t bits16) {
  return FP16 ? half_value(bits16) : bf16_value(bits16);
}

template <bool FP16>
__device__ inline uint32_t round16(float y) {
  if constexpr (FP16) return half_bits(y);
  else return bf16_bits(y);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Thread t of a workgroup handles lane t % (D/8) of head groups; groups are
// (row, head) in row-major order.  Each pass a thread takes U groups, the
// workgroup's groups in U slices of G = 256 / (D/8), and issues their U loads
// before any arithmetic, so a wave keeps U KB of rows in flight.  Both streams
// are touched once: nontemporal loads and stores.  The grid strides.
template <int D, bool FP16, bool SCALE, int U>
__global__ __launch_bounds__(256) void qk_norm_kernel(const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ out, int64_t groups,
                                                      int32_t heads, int64_t row_stride, float eps,
                                                      float scale) {
  constexpr int kLanes = D / 8;  // lanes per head group
  constexpr int kG = 256 / kLanes;  // groups per slice of a workgroup
  const int lane_in_group = threadIdx.x % kLanes;
  const int64_t stride = (int64_t)gridDim.x * kG * U;
  for (int64_t g0 = (int64_t)blockIdx.x * kG * U + threadIdx.x / kLanes; g0 < groups;
       g0 += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // past the last group: reload it (in bounds)
      const int64_t g = min(g0 + (int64_t)u * kG, groups - 1);
      const int64_t row = g / heads;
      const int h = (int)(g - row * heads);
      const v4u t = __builtin_nontemporal_load(
          reinterpret_cast<const v4u*>(x + row * row_stride + (int64_t)h * D + lane_in_group * 8));
      v[u] = make_uint4(t[0], t[1], t[2], t[3]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + (int64_t)u * kG;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float xs[8];
      double ss = 0.0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xs[2 * k] = value16<FP16>(w[k] & 0xffffu);
        xs[2 * k + 1] = value16<FP16>(w[k] >> 16);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) ss += (double)(xs[k] * xs[k]);  // squares rounded in fp32 (exact unless below its normal range)
      ss = group_sum<kLanes>(ss);
      const float ms = (float)ss * (1.0f / D);  // D is a power of two: exact
      const float a = ms + eps;
      // rsqrt_exact takes a finite positive normal argument: a subnormal one is
      // scaled by 2^64 first (exactly: 1/sqrt scales by 2^-32); 0, inf and NaN
      // take the hardware value (inf, 0, NaN: the exact results).
      float rstd;
      if (a >= 0x1p-126f && a < INFINITY) rstd = rsqrt_exact(a);
      else if (a > 0.0f) rstd = rsqrt_exact(a * 0x1p64f) * 0x1p32f;
      else rstd = __builtin_amdgcn_rsqf(a);
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float y0 = xs[2 * k] * rstd, y1 = xs[2 * k + 1] * rstd;
        if constexpr (SCALE) {
          y0 = y0 * scale;
          y1 = y1 * scale;
        }
        o[k] = round16<FP16>(y0) | (round16<FP16>(y1) << 16);
      }
      if (g < groups) {
        const int64_t row = g / heads;
        const int h = (int)(g - row * heads);
        __builtin_nontemporal_store(
            v4u{o[0], o[1], o[2], o[3]},
            reinterpret_cast<v4u*>(out + row * ((int64_t)heads * D) + (int64_t)h * D + lane_in_group * 8));
      }
    }
  }
}

template <int D, bool FP16, bool SCALE>
hipError_t launch_d(const QkNormParams& p, hipStream_t stream) {
  constexpr int kThreads = 256;
  constexpr int kGroupsPerSlice = kThreads / (D / 8);
  constexpr unsigned kMaxGrid = 256 * 8;  // eight workgroups per compute unit
  const int64_t groups = p.rows * p.heads;
  // Four groups per thread once they fill the capped grid (measured on 64 MB
  // calls: 13.6 against 16.5 us with one); a smaller call spreads one group
  // per thread over as many workgroups as it has slices.
  const bool unroll = groups >= (int64_t)kMaxGrid * kGroupsPerSlice * 4;
  const int64_t per_block = kGroupsPerSlice * (unroll ? 4 : 1);
  const unsigned grid = (unsigned)std::min<int64_t>((groups + per_block - 1) / per_block, kMaxGrid);
  if (unroll)
    hipLaunchKernelGGL((qk_norm_kernel<D, FP16, SCALE, 4>), dim3(grid), dim3(kThreads), 0, stream, p.x,
                       p.out, groups, p.heads, p.row_stride, p.eps, p.scale);
  else
    hipLaunchKernelGGL((qk_norm_kernel<D, FP16, SCALE, 1>), dim3(grid), dim3(kThreads), 0, stream, p.x,
                       p.out, groups, p.heads, p.row_stride, p.eps, p.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dtype(const QkNormParams& p, hipStream_t stream) {
  const bool scale = p.scale != 1.0f;
  if (p.fp16) return scale ? launch_d<D, true, true>(p, stream) : launch_d<D, true, false>(p, stream);
  return scale ? launch_d<D, false, true>(p, stream) : launch_d<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_qk_norm(const QkNormParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  switch (p.head_dim) {
    case 64: return launch_dtype<64>(p, stream);
    case 128: return launch_dtype<128>(p, stream);
    case 256: return launch_dtype<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mi355x_ga
