// attention.hip -- kernel 2 of the gated-attention step: paged, causal,
// sliding-window grouped-query attention over the e4m3 KV cache, split along
// the keys (flash-decoding), writing one (o, max, sum) partial per split.
//
// Definition: page "012-attention-local-splits.py", the flash_attn_with_kvcache
// call in kernel_fn (causal, window (W-1, 0), fp8 q/k/v, descales only when the
// cache scales are set, softmax scale sm_scale * qk_scale_factor, split-KV).
// Query i of request b sits at p = cache_seqlens[b] - L + i and sees keys
// max(0, p-W+1)..p (W = 0: 0..p); query head h reads KV head h / 8.
//
// gfx950 design (not the page's H200 kernel):
//  * Work unit = (request, split) workgroup of 4 waves; it covers ALL 16 query
//    heads of the request, i.e. both KV heads, so every 128-byte cache row it
//    fetches (one key, both heads) is used whole.  Waves take 32-key blocks
//    round-robin and merge through LDS at the end.
//  * Rows = (token, query head) pairs, grouped per KV head (8L rows per head),
//    in blocks of 16 rows.
//  * QK^T on the fp8 MFMA v_mfma_f32_16x16x32_fp8_fp8, A = 16 keys (straight
//    from global memory: lane (q4, j) holds 16 bytes of key j's row), B = q.
//    fp8 x fp8 products are exact in fp32.
//  * Softmax in base 2 in fp32; P is rounded to f16 (11 significant bits) for
//    the PV product; never to e4m3.
//  * PV as O^T = V^T P^T on v_mfma_f32_16x16x32_f16: V's e4m3 bytes are
//    transposed in registers (v_perm_b32) and widened exactly to f16 with
//    v_cvt_scalef32_pk_f16_fp8; the P operand is the QK accumulator layout
//    itself, so no cross-lane shuffles are needed for P, and each lane ends
//    with 16 contiguous output columns of one row.
#include "kernels.h"

namespace mi355x_ga {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ inline int64_t key_row(const AttnParams& p, const int32_t* pt_row, int key) {
  int page, off;
  if (p.page_shift >= 0) {
    page = key >> p.page_shift;
    off = key & (p.page_size - 1);
  } else {
    page = key / p.page_size;
    off = key - page * p.page_size;
  }
  page = min(page, p.max_pages - 1);
  int64_t phys = pt_row[page];
  if (phys < 0 || phys >= p.num_pages) phys = 0;  // only for invalid inputs: stay in bounds
  return phys * p.page_size + off;
}

__device__ inline long as_long(uint32_t lo, uint32_t hi) {
  return (long)(((unsigned long)hi << 32) | (unsigned long)lo);
}

template <int L>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnParams p) {
  constexpr int kRowsPerGroup = L * kGroup;
  constexpr int NRB = (kRowsPerGroup + 15) / 16;  // 16-row blocks per KV head
  constexpr int kLdsRows = kKvHeads * NRB * 16;
  __shared__ float lds_o[2][kLdsRows][kHeadDim];
  __shared__ float lds_ml[2][kLdsRows][2];

  const int b = blockIdx.x / p.splits;
  const int s = blockIdx.x - b * p.splits;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int q4 = lane >> 4;

  // Key range of the request (union over its L queries) and this split's chunk.
  const int cs = p.cache_seqlens[b];
  const int p0 = cs - L;
  const int last = cs - 1;
  const int first = p.window > 0 ? max(0, p0 - p.window + 1) : 0;
  const int n = max(0, last - first + 1);
  int chunk = (n + p.splits - 1) / p.splits;
  chunk = (chunk + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
  const int start = first + s * chunk;
  const int end = min(start + chunk, last + 1);
  const int nblk = end > start ? (end - start + kKeyBlock - 1) / kKeyBlock : 0;

  const int32_t* pt_row = p.page_table + (int64_t)b * p.max_pages;
  const float ks = p.scaled ? *p.k_scale : 1.0f;
  const float scale = p.sm_scale_log2 * ks;

  // q operands and per-row visible key ranges.  Row r = 16*rb + j of KV head g
  // is query token r / 8, query head 8g + r % 8.
  long qop[kKvHeads][NRB][2];
  int rlo[NRB], rhi[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = 16 * rb + j;
    const int i = r >> 3;
    const bool valid = i < L;
    const int pi = p0 + i;
    rlo[rb] = valid ? (p.window > 0 ? max(0, pi - p.window + 1) : 0) : 1;
    rhi[rb] = valid ? pi : 0;
#pragma unroll
    for (int g = 0; g < kKvHeads; ++g) {
      uint4 qv = make_uint4(0, 0, 0, 0);
      if (valid) {
        const int h = g * kGroup + (r & 7);
        qv = *reinterpret_cast<const uint4*>(
            p.q + ((int64_t)(b * L + i) * kQHeads + h) * kHeadDim + 16 * q4);
      }
      qop[g][rb][0] = as_long(qv.x, qv.y);
      qop[g][rb][1] = as_long(qv.z, qv.w);
    }
  }

  float mrow[kKvHeads][NRB], lrow[kKvHeads][NRB];
  v4f acc[kKvHeads][NRB][4];
#pragma unroll
  for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      mrow[g][rb] = -INFINITY;
      lrow[g][rb] = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[g][rb][c] = v4f{0.f, 0.f, 0.f, 0.f};
    }

  for (int kb = wave; kb < nblk; kb += kAttnWaves) {
    const int kbase = start + kb * kKeyBlock;
    // K: lane (q4, j) reads 16 bytes of key kbase+16t+j for each KV head.
    uint4 kd[2][kKvHeads];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = min(kbase + 16 * t + j, end - 1);
      const uint8_t* row = p.k_cache + key_row(p, pt_row, key) * kRowBytes + 16 * q4;
      kd[t][0] = *reinterpret_cast<const uint4*>(row);
      kd[t][1] = *reinterpret_cast<const uint4*>(row + kHeadDim);
    }
    // V: lane (q4, j) reads columns 4j..4j+3 of each KV head for the 8 keys
    // kbase + 16t + 4q4 + ii (t < 2, ii < 4) -- the keys whose scores it holds.
    uint32_t vd[kKvHeads][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = min(kbase + 16 * (r >> 2) + 4 * q4 + (r & 3), end - 1);
      const uint8_t* row = p.v_cache + key_row(p, pt_row, key) * kRowBytes + 4 * j;
      vd[0][r] = *reinterpret_cast<const uint32_t*>(row);
      vd[1][r] = *reinterpret_cast<const uint32_t*>(row + kHeadDim);
    }

    // V^T operand: for each KV head and column c (of the lane's 4), the 8 keys
    // as f16 pairs.  perm gathers byte c (and c+1) of two key rows.
    v8h va[kKvHeads][4];
#pragma unroll
    for (int g = 0; g < kKvHeads; ++g) {
#pragma unroll
      for (int rp = 0; rp < 4; ++rp) {
        const uint32_t lo = __builtin_amdgcn_perm(vd[g][2 * rp + 1], vd[g][2 * rp], 0x05010400u);
        const uint32_t hi = __builtin_amdgcn_perm(vd[g][2 * rp + 1], vd[g][2 * rp], 0x07030602u);
        const v2h c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
        const v2h c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
        const v2h c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
        const v2h c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
        va[g][0][2 * rp] = c0[0];
        va[g][0][2 * rp + 1] = c0[1];
        va[g][1][2 * rp] = c1[0];
        va[g][1][2 * rp + 1] = c1[1];
        va[g][2][2 * rp] = c2[0];
        va[g][2][2 * rp + 1] = c2[1];
        va[g][3][2 * rp] = c3[0];
        va[g][3][2 * rp + 1] = c3[1];
      }
    }

#pragma unroll
    for (int g = 0; g < kKvHeads; ++g) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float sv[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v4f z = {0.f, 0.f, 0.f, 0.f};
          z = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(kd[t][g].x, kd[t][g].y),
                                                          qop[g][rb][0], z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(kd[t][g].z, kd[t][g].w),
                                                          qop[g][rb][1], z, 0, 0, 0);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int key = kbase + 16 * t + 4 * q4 + ii;
            const bool vis = key < end && key >= rlo[rb] && key <= rhi[rb];
            sv[t * 4 + ii] = vis ? z[ii] * scale : -INFINITY;
          }
        }
        float mx = sv[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sv[k]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrow[g][rb], mx);
        const float muse = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = exp2f(mrow[g][rb] - muse);
        mrow[g][rb] = mnew;
        v8h pb;
        float psum = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float pk = exp2f(sv[k] - muse);
          psum += pk;
          pb[k] = (_Float16)pk;
        }
        lrow[g][rb] = lrow[g][rb] * alpha + psum;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[g][rb][c] *= alpha;
          acc[g][rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[g][c], pb, acc[g][rb][c], 0, 0, 0);
        }
      }
    }
  }

  // Row sums: each lane summed its own keys; add the four lane groups of a row.
#pragma unroll
  for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      lrow[g][rb] += __shfl_xor(lrow[g][rb], 16);
      lrow[g][rb] += __shfl_xor(lrow[g][rb], 32);
    }

  // Merge the four waves: 2,3 -> 0,1, then 1 -> 0.  Lane (q4, j) holds columns
  // 16*q4 + 4*ii + c of its row in acc[g][rb][c][ii].
  auto put = [&](int slot) {
#pragma unroll
    for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int row = (g * NRB + rb) * 16 + j;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          *reinterpret_cast<float4*>(&lds_o[slot][row][16 * q4 + 4 * ii]) =
              make_float4(acc[g][rb][0][ii], acc[g][rb][1][ii], acc[g][rb][2][ii], acc[g][rb][3][ii]);
        if (q4 == 0) {
          lds_ml[slot][row][0] = mrow[g][rb];
          lds_ml[slot][row][1] = lrow[g][rb];
        }
      }
  };
  auto take = [&](int slot) {
#pragma unroll
    for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int row = (g * NRB + rb) * 16 + j;
        const float mo = lds_ml[slot][row][0];
        const float lo = lds_ml[slot][row][1];
        const float mnew = fmaxf(mrow[g][rb], mo);
        const float muse = mnew == -INFINITY ? 0.0f : mnew;
        const float a = exp2f(mrow[g][rb] - muse);
        const float bo = exp2f(mo - muse);
        mrow[g][rb] = mnew;
        lrow[g][rb] = lrow[g][rb] * a + lo * bo;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float4 v = *reinterpret_cast<const float4*>(&lds_o[slot][row][16 * q4 + 4 * ii]);
          acc[g][rb][0][ii] = acc[g][rb][0][ii] * a + v.x * bo;
          acc[g][rb][1][ii] = acc[g][rb][1][ii] * a + v.y * bo;
          acc[g][rb][2][ii] = acc[g][rb][2][ii] * a + v.z * bo;
          acc[g][rb][3][ii] = acc[g][rb][3][ii] * a + v.w * bo;
        }
      }
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) take(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave != 0) return;
  take(0);

#pragma unroll
  for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = 16 * rb + j;
      const int i = r >> 3;
      if (i >= L) continue;
      const int h = g * kGroup + (r & 7);
      const int64_t prow = ((int64_t)(b * p.splits + s) * L + i) * kQHeads + h;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        *reinterpret_cast<float4*>(p.part_o + prow * kHeadDim + 16 * q4 + 4 * ii) =
            make_float4(acc[g][rb][0][ii], acc[g][rb][1][ii], acc[g][rb][2][ii], acc[g][rb][3][ii]);
      if (q4 == 0) {
        p.part_ml[prow * 2] = mrow[g][rb];
        p.part_ml[prow * 2 + 1] = lrow[g][rb];
      }
    }
}

template <int L>
hipError_t launch_l(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.batch * (unsigned)p.splits;
  hipLaunchKernelGGL(attn_split_kernel<L>, dim3(grid), dim3(64 * kAttnWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int q_len, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  switch (q_len) {
    case 1: return launch_l<1>(p, stream);
    case 2: return launch_l<2>(p, stream);
    case 3: return launch_l<3>(p, stream);
    case 4: return launch_l<4>(p, stream);
    case 5: return launch_l<5>(p, stream);
    case 6: return launch_l<6>(p, stream);
    case 7: return launch_l<7>(p, stream);
    case 8: return launch_l<8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mi355x_ga
