// combine.hip -- kernel 3 of the gated-attention step: merge the split
// partials of each (token, query head) row, round the attention output to bf16,
// then per-head unweighted RMSNorm times sigmoid(gate), rounded once to bf16.
//
// Definition: page "012-attention-local-splits.py", kernel_fn: the FA3 split
// combine (its bf16 output) and rms_norm_gate(out, gate, None, eps=1e-5,
// has_norm=True) with gate = qkv[:, (Hq + 2Hkv) * D:].
//
// Mapping: one wave per row, lane = output column; the S partials of a row are
// contiguous 256-byte reads.
#include "kernels.h"

namespace mi355x_ga {
namespace {

__device__ inline uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)p.tokens * kQHeads) return;  // whole waves exit together
  const int64_t t = row / kQHeads;
  const int h = (int)(row - t * kQHeads);
  const int64_t b = t / p.q_len;
  const int i = (int)(t - b * p.q_len);

  const int64_t stride = (int64_t)p.q_len * kQHeads;  // rows per split
  const int64_t base = (b * p.splits) * stride + (int64_t)i * kQHeads + h;
  float mmax = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mmax = fmaxf(mmax, p.part_ml[(base + s * stride) * 2]);
  float o = 0.0f;
  if (mmax != -INFINITY) {
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < p.splits; ++s) {
      const int64_t pr = base + s * stride;
      const float w = exp2f(p.part_ml[pr * 2] - mmax);
      den += w * p.part_ml[pr * 2 + 1];
      num += w * p.part_o[pr * kHeadDim + lane];
    }
    o = num / den;
    if (p.scaled) o *= *p.v_scale;
  }
  // The attention result is bf16 before the epilogue.
  o = __uint_as_float(bf16_bits(o) << 16);

  float ss = o * o;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = (float)(1.0 / sqrt((double)ss / 64.0 + 1.0e-5));
  const float gate = __uint_as_float((uint32_t)p.qkv[t * kWidth + kGateOffset + h * kHeadDim + lane] << 16);
  const float sig = 1.0f / (1.0f + expf(-gate));
  p.out[t * (kQHeads * kHeadDim) + h * kHeadDim + lane] = (uint16_t)bf16_bits(o * r * sig);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.tokens * kQHeads;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mi355x_ga
