// step_kernel.hip -- the whole gated-attention layer-step as ONE gfx950 kernel.
//
// Definition: page "012-attention-local-splits.py" -- module docstring (step
// order), `_prepare_qkv` (norm, RoPE, q cast, K/V store), `_cos_sin` (RoPE
// frequencies), kernel_fn's flash_attn_with_kvcache call (paged causal window
// attention over the e4m3 cache, split-KV) and its rms_norm_gate epilogue.
//
// One workgroup (4 waves) per work unit (request b, split s).  A unit covers all
// 16 query heads of its request, i.e. both KV heads, so every 128-byte cache row
// it fetches (one key, both heads) is used whole.
//
//  A. Geometry and early loads: cache_seqlens[b] gives the request's key range
//     and this unit's chunk; the projection rows, positions and the page-table
//     entries of the first key blocks are requested, then the first two blocks'
//     K/V rows.  While those are in flight the unit computes its request's q
//     (norm, RoPE, e4m3) into LDS; the unit whose chunk holds a new token's key
//     also computes that token's K/V codes, stores them at cache_loc and uses
//     them in place of the cache row, so no unit reads a row being written.
//  B. Key loop (waves take 32-key blocks round-robin, two blocks in flight):
//     QK^T on v_mfma_f32_16x16x32_fp8_fp8 straight from the cache bytes; base-2
//     softmax with a lazily moved running max (rescale only when the max grows
//     by more than 2^8); P in f16; PV as O^T = V^T P^T on
//     v_mfma_f32_16x16x32_f16 with V transposed in registers and widened
//     exactly to f16.
//  C. The four waves merge through LDS and publish the unit's partial (o, m, l)
//     with device-coherent stores; an atomic counter per request elects the last
//     unit, which reads the request's partials with device-coherent loads,
//     merges them, rounds the attention output to bf16, applies RMSNorm x
//     sigmoid(gate), writes bf16 out and re-arms the counter.
//
// Cross-workgroup visibility (C): partials are written and read only with
// agent-scope atomic accesses (sc1: coherent across the XCDs' L2 caches), and
// each wave waits for its own stores to complete (s_waitcnt vmcnt(0)) before
// the workgroup barrier that precedes the counter increment.  No L2 write-back
// or invalidate is needed, unlike a generic device-scope fence.
#include "kernels.h"
#include "numerics.h"

namespace mi355x_ga {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kHeadRows = kQHeads + 2 * kKvHeads;  // 20 head rows per token
constexpr float kLazyRescale = 8.0f;               // log2 units: P stays <= 2^8

__device__ inline long as_long(uint32_t lo, uint32_t hi) {
  return (long)(((unsigned long)hi << 32) | (unsigned long)lo);
}

__device__ inline void store_coherent(float* dst, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float2 load_coherent(const float* src) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Page-table entry of logical key `key` (the load only; nothing waits on it).
__device__ inline int page_entry(const StepParams& p, const int32_t* pt, int key) {
  const int page = p.page_shift >= 0 ? key >> p.page_shift : key / p.page_size;
  return pt[min(page, p.max_pages - 1)];
}

// Flat cache row of logical key `key` from its page-table entry.
__device__ inline int key_row(const StepParams& p, int entry, int key) {
  const int off = p.page_shift >= 0 ? key & (p.page_size - 1) : key % p.page_size;
  const int64_t phys = (entry < 0 || entry >= p.num_pages) ? 0 : entry;  // invalid input: stay in bounds
  return (int)(phys * p.page_size + off);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load of the wave, which would stall on the K/V blocks
// kept in flight across the prologue.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct KvBlock {
  uint4 k[2][kKvHeads];      // lane (q4, j): 16 bytes of key 16t+j, both KV heads
  uint32_t v[kKvHeads][8];   // lane (q4, j): columns 4j..4j+3 of keys 16(r/4)+4q4+r%4
};

// `entry`: this lane's page-table entry for key `key` (= block base + lane % 32,
// clamped); the rows are shared by lane shuffles, so each lane issues one
// page-table load per block.
__device__ inline KvBlock load_kv(const StepParams& p, int entry, int key, int j, int q4) {
  const int myrow = key_row(p, entry, key);
  KvBlock d;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = __shfl(myrow, 16 * t + j);
    const uint8_t* kr = p.k_cache + (int64_t)row * kRowBytes + 16 * q4;
    d.k[t][0] = *reinterpret_cast<const uint4*>(kr);
    d.k[t][1] = *reinterpret_cast<const uint4*>(kr + kHeadDim);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = __shfl(myrow, 16 * (r >> 2) + 4 * q4 + (r & 3));
    const uint8_t* vr = p.v_cache + (int64_t)row * kRowBytes + 4 * j;
    d.v[0][r] = *reinterpret_cast<const uint32_t*>(vr);
    d.v[1][r] = *reinterpret_cast<const uint32_t*>(vr + kHeadDim);
  }
  return d;
}

// Norm (+ RoPE) of one 8-column slice of a head row, page order, every fp32 step
// rounded once (no contraction): fp64-exact sum of squares over the 8 lanes of
// the row, exact rsqrt, fp32 product, bf16; RoPE pairs (2i, 2i+1) with fp32
// products and sum, bf16.
__device__ inline void norm_rope8(const float (&x)[8], bool rope, const float (*cs)[2], int c8,
                                  float (&y)[8]) {
#pragma clang fp contract(off)
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += (double)(x[k] * x[k]);
  ss += __shfl_xor(ss, 1, 8);
  ss += __shfl_xor(ss, 2, 8);
  ss += __shfl_xor(ss, 4, 8);
  const float ms = (float)ss / 64.0f;
  const float inv = rsqrt_exact(ms + 1.0e-5f);
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = round_bf16(x[k] * inv);
  if (rope) {
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const float c = cs[c8 * 4 + pr][0], s = cs[c8 * 4 + pr][1];
      const float e = y[2 * pr], o = y[2 * pr + 1];
      const float ec = e * c, os = o * s, oc = o * c, es = e * s;
      y[2 * pr] = round_bf16(ec - os);
      y[2 * pr + 1] = round_bf16(oc + es);
    }
  }
}

__device__ inline uint2 pack_e4m3x8(const float (&y)[8]) {
  const uint32_t lo = e4m3x2(y[0], y[1]) | (e4m3x2(y[2], y[3]) << 16);
  const uint32_t hi = e4m3x2(y[4], y[5]) | (e4m3x2(y[6], y[7]) << 16);
  return make_uint2(lo, hi);
}

template <int L>
__global__ __launch_bounds__(256) void fused_step_kernel(StepParams p) {
  constexpr int NRB = (L * kGroup + 15) / 16;  // 16-row blocks per KV head
  constexpr int kItems = L * kHeadRows * 8;    // (token, head row, 8-column slice)
  constexpr int kItemIters = (kItems + 255) / 256;
  __shared__ __align__(16) uint8_t s_q[L][kQHeads][kHeadDim];
  __shared__ __align__(16) uint8_t s_newk[L][kRowBytes];
  __shared__ __align__(16) uint8_t s_newv[L][kRowBytes];
  __shared__ float s_cs[L][kHeadDim / 2][2];
  __shared__ __align__(16) float s_mo[kAttnWaves][L * kQHeads][kHeadDim];
  __shared__ __align__(16) float s_ml[kAttnWaves][L * kQHeads][2];
  __shared__ int s_last;

  const int b = blockIdx.x / p.splits;
  const int s = blockIdx.x - b * p.splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;
  const int q4 = lane >> 4;
  const int64_t tok0 = (int64_t)b * L;

  // ---------------- A. geometry and early loads ----------------
  const int cs = p.cache_seqlens[b];
  const uint16_t* qkv_b = p.qkv + tok0 * kWidth;
  uint4 xv[kItemIters];
#pragma unroll
  for (int it = 0; it < kItemIters; ++it) {
    const int item = tid + 256 * it;
    xv[it] = make_uint4(0, 0, 0, 0);
    if (item < kItems) {
      const int i = item / (kHeadRows * 8), rem = item - i * (kHeadRows * 8);
      xv[it] = *reinterpret_cast<const uint4*>(qkv_b + i * kWidth + (rem >> 3) * kHeadDim +
                                                (rem & 7) * 8);
    }
  }
  const bool cs_thread = p.rope && tid < 32 * L;
  int64_t my_slot = p.cache_loc[tok0 + min(tid, L - 1)];
  float my_ang = p.rope ? (float)p.positions[tok0 + min(tid >> 5, L - 1)] * p.inv_freq[tid & 31] : 0.0f;
  float ks = p.scaled ? *p.k_scale : 1.0f;
  float vs = p.scaled ? *p.v_scale : 1.0f;
  // Take these small values now, while waiting for cache_seqlens anyway: a load
  // left for later would be consumed after the K/V loads, and since vector
  // memory counters complete in order, waiting for it would wait for them too.
  asm volatile("" : "+v"(my_ang), "+v"(ks), "+v"(vs), "+v"(my_slot));

  const int p0 = cs - L;  // key index (position) of the block's first new token
  const int last = cs - 1;
  const int first = p.window > 0 ? max(0, p0 - p.window + 1) : 0;
  const int n = max(0, last - first + 1);
  int chunk = (n + p.splits - 1) / p.splits;
  chunk = (chunk + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
  const int start = first + s * chunk;
  const int end = min(start + chunk, last + 1);
  const int nblk = end > start ? (end - start + kKeyBlock - 1) / kKeyBlock : 0;
  const int nb = nblk > wave ? (nblk - wave + kAttnWaves - 1) / kAttnWaves : 0;  // this wave's
  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  // Key of this lane in the wave's block i.  Blocks past the wave's last are
  // clamped to it, so the pipeline's loads are unconditional (which keeps the
  // compiler's memory-counter waits exact) and the extra ones hit cache lines
  // already fetched.
  auto lane_key = [&](int i) {
    const int blk = min(i, max(nb - 1, 0));
    return max(0, min(start + (wave + kAttnWaves * blk) * kKeyBlock + (lane & 31), end - 1));
  };
  auto load_pte = [&](int i) { return page_entry(p, pt, lane_key(i)); };

  // Issue order matters (vector memory counters complete in order): each block's
  // page-table load follows the K/V loads two blocks earlier, so waiting for it
  // never waits for the next block's K/V.
  const int pte0 = load_pte(0);
  const int pte1 = load_pte(1);
  KvBlock bufA = load_kv(p, pte0, lane_key(0), j, q4);
  int pa = load_pte(2);
  KvBlock bufB = load_kv(p, pte1, lane_key(1), j, q4);
  int pb = load_pte(3);

  // New token i's key is stored and substituted by the unit whose chunk holds
  // it (by unit 0 when it has no place in any chunk, e.g. a padded slot).
  auto owns = [&](int i) {
    const int key = p0 + i;
    return (key >= start && key < end) || (key < first && s == 0);
  };

  // RoPE table for the request's tokens: (token, frequency) per thread.
  if (cs_thread) {
    double sd, cd;
    sincos((double)my_ang, &sd, &cd);
    s_cs[tid >> 5][tid & 31][0] = (float)cd;
    s_cs[tid >> 5][tid & 31][1] = (float)sd;
  }
  lds_barrier();

#pragma unroll
  for (int it = 0; it < kItemIters; ++it) {
    const int item = tid + 256 * it;
    const int i = min(item / (kHeadRows * 8), L - 1);
    const int rem = item - (item / (kHeadRows * 8)) * (kHeadRows * 8);
    const int hr = rem >> 3, c8 = rem & 7;
    // Whole 8-lane groups are skipped together (the norm shuffles stay in-group).
    if (item >= kItems || (hr >= kQHeads && !owns(i))) continue;
    float x[8], y[8];
    const uint32_t w[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_value(w[k] & 0xffffu);
      x[2 * k + 1] = bf16_value(w[k] >> 16);
    }
    if (hr < kQHeads + kKvHeads) {
      norm_rope8(x, p.rope != 0, s_cs[i], c8, y);
      if (hr >= kQHeads && p.scaled) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = round_bf16(y[k] / ks);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = p.scaled ? round_bf16(x[k] / vs) : x[k];  // raw value
    }
    const uint2 codes = pack_e4m3x8(y);
    if (hr < kQHeads) {
      *reinterpret_cast<uint2*>(&s_q[i][hr][c8 * 8]) = codes;
      if (s == 0)
        *reinterpret_cast<uint2*>(p.q_out + ((tok0 + i) * kQHeads + hr) * kHeadDim + c8 * 8) = codes;
    } else if (hr < kQHeads + kKvHeads) {
      *reinterpret_cast<uint2*>(&s_newk[i][(hr - kQHeads) * kHeadDim + c8 * 8]) = codes;
    } else {
      *reinterpret_cast<uint2*>(&s_newv[i][(hr - kQHeads - kKvHeads) * kHeadDim + c8 * 8]) = codes;
    }
  }
  lds_barrier();

  if (tid < L && owns(tid) && my_slot >= 0 && my_slot < p.num_rows) {
    const uint4* kk = reinterpret_cast<const uint4*>(s_newk[tid]);
    const uint4* vv = reinterpret_cast<const uint4*>(s_newv[tid]);
    uint4* kd = reinterpret_cast<uint4*>(p.k_cache + my_slot * kRowBytes);
    uint4* vd = reinterpret_cast<uint4*>(p.v_cache + my_slot * kRowBytes);
#pragma unroll
    for (int c = 0; c < kRowBytes / 16; ++c) {
      kd[c] = kk[c];
      vd[c] = vv[c];
    }
  }

  // q operands and per-row visible ranges.  Row r = 16*rb + j of KV head g is
  // query token r / 8, query head 8g + r % 8.
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
      const uint4 qv = *reinterpret_cast<const uint4*>(&s_q[min(i, L - 1)][g * kGroup + (r & 7)][16 * q4]);
      qop[g][rb][0] = valid ? as_long(qv.x, qv.y) : 0;
      qop[g][rb][1] = valid ? as_long(qv.z, qv.w) : 0;
    }
  }
  // A block is visible to every row when it lies in [lo_all, hi_all].
  const int lo_all = p.window > 0 ? max(0, p0 + L - 1 - p.window + 1) : 0;
  const int hi_all = min(p0, end - 1);
  const float scale = p.sm_scale_log2 * ks;

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

  // ---------------- B. key loop ----------------
  auto process = [&](KvBlock& d, const int kbase) {
    if (kbase + kKeyBlock - 1 >= p0) {  // the block holds new keys: use their codes
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = kbase + 16 * t + j;
        const int i = min(max(key - p0, 0), L - 1);
        const bool nk = key >= p0;
#pragma unroll
        for (int g = 0; g < kKvHeads; ++g) {
          const uint4 nv = *reinterpret_cast<const uint4*>(&s_newk[i][g * kHeadDim + 16 * q4]);
          d.k[t][g].x = nk ? nv.x : d.k[t][g].x;
          d.k[t][g].y = nk ? nv.y : d.k[t][g].y;
          d.k[t][g].z = nk ? nv.z : d.k[t][g].z;
          d.k[t][g].w = nk ? nv.w : d.k[t][g].w;
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int key = kbase + 16 * (r >> 2) + 4 * q4 + (r & 3);
        const int i = min(max(key - p0, 0), L - 1);
        const bool nk = key >= p0;
#pragma unroll
        for (int g = 0; g < kKvHeads; ++g) {
          const uint32_t nv = *reinterpret_cast<const uint32_t*>(&s_newv[i][g * kHeadDim + 4 * j]);
          d.v[g][r] = nk ? nv : d.v[g][r];
        }
      }
    }

    // V^T operand: per KV head and column c (of the lane's 4), the 8 keys as f16
    // pairs; perm gathers byte c (and c+1) of two key rows.
    v8h va[kKvHeads][4];
#pragma unroll
    for (int g = 0; g < kKvHeads; ++g) {
#pragma unroll
      for (int rp = 0; rp < 4; ++rp) {
        const uint32_t lo = __builtin_amdgcn_perm(d.v[g][2 * rp + 1], d.v[g][2 * rp], 0x05010400u);
        const uint32_t hi = __builtin_amdgcn_perm(d.v[g][2 * rp + 1], d.v[g][2 * rp], 0x07030602u);
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

    // Per KV head: the scores of all its row blocks first (their MFMAs overlap),
    // then one wave-uniform running-max decision, then P and PV.
    const bool full = kbase >= lo_all && kbase + kKeyBlock - 1 <= hi_all;
#pragma unroll
    for (int g = 0; g < kKvHeads; ++g) {
      float sv[NRB][8];
      float lmx[NRB];     // this lane's maximum over its 8 keys
      bool grow = false;  // some lane's maximum passes its row's lazy bound
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v4f z = {0.f, 0.f, 0.f, 0.f};
          z = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(d.k[t][g].x, d.k[t][g].y),
                                                          qop[g][rb][0], z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(d.k[t][g].z, d.k[t][g].w),
                                                          qop[g][rb][1], z, 0, 0, 0);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) sv[rb][t * 4 + ii] = z[ii] * scale;
        }
        if (!full) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int key = kbase + 16 * (k >> 2) + 4 * q4 + (k & 3);
            const bool vis = key < end && key >= rlo[rb] && key <= rhi[rb];
            sv[rb][k] = vis ? sv[rb][k] : -INFINITY;
          }
        }
        const float* v = sv[rb];
        lmx[rb] = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                        fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
        grow |= lmx[rb] > mrow[g][rb] + kLazyRescale;
      }
      // A row's maximum moves only when its full maximum (over the four lane
      // groups) passes the bound, which no lane's own maximum does in the common
      // case: then nothing moves and the cross-lane reduction is skipped.
      if (__any(grow)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          float mx = lmx[rb];
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mold = mrow[g][rb];
          const float mnew = mx > mold + kLazyRescale ? mx : mold;
          const float alpha = __builtin_amdgcn_exp2f(mold - (mnew == -INFINITY ? 0.0f : mnew));
          lrow[g][rb] *= alpha;  // alpha is exactly 1 for a row that kept its maximum
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[g][rb][c] *= alpha;
          mrow[g][rb] = mnew;
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float muse = mrow[g][rb] == -INFINITY ? 0.0f : mrow[g][rb];
        v8h pb;
        float psum = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float pk = __builtin_amdgcn_exp2f(sv[rb][k] - muse);
          psum += pk;
          pb[k] = (_Float16)pk;
        }
        lrow[g][rb] += psum;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[g][rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[g][c], pb, acc[g][rb][c], 0, 0, 0);
      }
    }
  };

  for (int bi = 0; bi < nb; bi += 2) {
    process(bufA, start + (wave + kAttnWaves * bi) * kKeyBlock);
    bufA = load_kv(p, pa, lane_key(bi + 2), j, q4);
    pa = load_pte(bi + 4);
    if (bi + 1 < nb) process(bufB, start + (wave + kAttnWaves * (bi + 1)) * kKeyBlock);
    bufB = load_kv(p, pb, lane_key(bi + 3), j, q4);
    pb = load_pte(bi + 5);
  }

  // Row sums: each lane summed its own keys; add the four lane groups of a row.
#pragma unroll
  for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      lrow[g][rb] += __shfl_xor(lrow[g][rb], 16);
      lrow[g][rb] += __shfl_xor(lrow[g][rb], 32);
    }

  // ---------------- C. merge the waves, publish the partial ----------------
  // Every wave parks (m, l, o) of its valid rows in its LDS slot (compact row
  // i*16 + h); after one barrier all 256 threads merge 4 columns of a row each
  // and publish the unit's partial.
#pragma unroll
  for (int g = 0; g < kKvHeads; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = 16 * rb + j;
      const int i = r >> 3;
      if (i >= L) continue;
      const int cr = i * kQHeads + g * kGroup + (r & 7);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        *reinterpret_cast<float4*>(&s_mo[wave][cr][16 * q4 + 4 * ii]) =
            make_float4(acc[g][rb][0][ii], acc[g][rb][1][ii], acc[g][rb][2][ii], acc[g][rb][3][ii]);
      if (q4 == 0) *reinterpret_cast<float2*>(&s_ml[wave][cr][0]) = make_float2(mrow[g][rb], lrow[g][rb]);
    }
  lds_barrier();
  const int64_t prow0 = (int64_t)(b * p.splits + s) * (L * kQHeads);
  for (int idx = tid; idx < L * kQHeads * 16; idx += 256) {
    const int cr = idx >> 4, c4 = (idx & 15) * 4;
    float mw[kAttnWaves], lw[kAttnWaves];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float2 ml = *reinterpret_cast<const float2*>(&s_ml[w][cr][0]);
      mw[w] = ml.x;
      lw[w] = ml.y;
      mx = fmaxf(mx, ml.x);
    }
    const float muse = mx == -INFINITY ? 0.0f : mx;
    float lsum = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float a = __builtin_amdgcn_exp2f(mw[w] - muse);
      const float4 v = *reinterpret_cast<const float4*>(&s_mo[w][cr][c4]);
      lsum += a * lw[w];
      o.x += a * v.x;
      o.y += a * v.y;
      o.z += a * v.z;
      o.w += a * v.w;
    }
    float* dst = p.part_o + (prow0 + cr) * kHeadDim + c4;
    store_coherent(dst, o.x, o.y);
    store_coherent(dst + 2, o.z, o.w);
    if (c4 == 0) store_coherent(p.part_ml + (prow0 + cr) * 2, mx, lsum);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&p.counters[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             p.splits - 1;
  __syncthreads();
  if (!s_last) return;

  // ---------------- D. combine + gated epilogue (last unit) ----------------
  // Thread (h, c4) takes columns c4..c4+3 of head h for every token of the
  // request.  The partials are read KS splits at a time for all tokens at once,
  // so the chain of device-coherent round trips is ceil(splits / KS) long
  // whatever the number of tokens.
  constexpr int KS = L >= 8 ? 4 : (32 / L > 16 ? 16 : 32 / L);
  const int c4 = (tid & 15) * 4;
  const int h = tid >> 4;
  const int64_t stride = (int64_t)L * kQHeads;  // partial rows per split
  const int64_t base = (int64_t)b * p.splits * stride + h;
  uint2 graw[L];
#pragma unroll
  for (int i = 0; i < L; ++i)
    graw[i] = *reinterpret_cast<const uint2*>(p.qkv + (tok0 + i) * kWidth + kGateOffset + h * kHeadDim + c4);
  float mrun[L], lrun[L], o[L][4];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[i][c] = 0.0f;
  }
  for (int s0 = 0; s0 < p.splits; s0 += KS) {
    float2 ml[L][KS], o01[L][KS], o23[L][KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        ml[i][k] = make_float2(-INFINITY, 0.0f);
        o01[i][k] = o23[i][k] = make_float2(0.0f, 0.0f);
        if (s0 + k < p.splits) {
          const int64_t pr = base + (int64_t)(s0 + k) * stride + i * kQHeads;
          ml[i][k] = load_coherent(p.part_ml + pr * 2);
          o01[i][k] = load_coherent(p.part_o + pr * kHeadDim + c4);
          o23[i][k] = load_coherent(p.part_o + pr * kHeadDim + c4 + 2);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      float mc = mrun[i];
#pragma unroll
      for (int k = 0; k < KS; ++k) mc = fmaxf(mc, ml[i][k].x);
      const float muse = mc == -INFINITY ? 0.0f : mc;
      const float a = __builtin_amdgcn_exp2f(mrun[i] - muse);
      lrun[i] *= a;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[i][c] *= a;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float wk = __builtin_amdgcn_exp2f(ml[i][k].x - muse);
        lrun[i] += wk * ml[i][k].y;
        o[i][0] += wk * o01[i][k].x;
        o[i][1] += wk * o01[i][k].y;
        o[i][2] += wk * o23[i][k].x;
        o[i][3] += wk * o23[i][k].y;
      }
      mrun[i] = mc;
    }
  }
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const float inv = lrun[i] > 0.0f ? vs / lrun[i] : 0.0f;
    float y[4];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      y[c] = round_bf16(o[i][c] * inv);  // the attention result is bf16 before the epilogue
      ss += y[c] * y[c];
    }
    ss += __shfl_xor(ss, 1, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 8, 16);
    const float r = (float)(1.0 / sqrt((double)ss / 64.0 + 1.0e-5));
    const float gate[4] = {bf16_value(graw[i].x & 0xffffu), bf16_value(graw[i].x >> 16),
                           bf16_value(graw[i].y & 0xffffu), bf16_value(graw[i].y >> 16)};
    uint32_t ob[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ob[c] = bf16_bits(y[c] * r * (1.0f / (1.0f + __expf(-gate[c]))));
    *reinterpret_cast<uint2*>(p.out + (tok0 + i) * (kQHeads * kHeadDim) + h * kHeadDim + c4) =
        make_uint2(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16));
  }
  if (tid == 0) __hip_atomic_store(&p.counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int L>
hipError_t launch_l(const StepParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.batch * (unsigned)p.splits;
  hipLaunchKernelGGL(fused_step_kernel<L>, dim3(grid), dim3(64 * kAttnWaves), 0, stream, p);
  return hipGetLastError();
}

__global__ void zero_counters_kernel(int32_t* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0;
}

}  // namespace

hipError_t launch_step(const StepParams& p, int q_len, hipStream_t stream) {
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

hipError_t launch_zero_counters(int32_t* counters, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, counters, n);
  return hipGetLastError();
}

}  // namespace mi355x_ga
