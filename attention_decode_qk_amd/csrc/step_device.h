// step_device.h -- device helpers shared by the step's kernels (decode /
// verify in step_kernel.hip, extend / prefill in extend_kernel.hip): MFMA
// operand types, cross-lane reductions, paged-cache addressing, the LDS-only
// barrier and the prologue's per-slice norm, RoPE and e4m3 packing.  Internal
// linkage: each kernel file gets its own copy.
#pragma once

#include "kernels.h"
#include "numerics.h"

namespace mi355x_ga {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr float kLazyRescale = 8.0f;               // log2 units: P stays <= 2^8

__device__ inline long as_long(uint32_t lo, uint32_t hi) {
  return (long)(((unsigned long)hi << 32) | (unsigned long)lo);
}

// Device-coherent (agent-scope) accesses for partial results exchanged
// between workgroups of one launch.
__device__ inline void store_coherent(float* dst, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float2 load_coherent(const float* src) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Four f16 values (round to nearest even) in one 8-byte agent-scope store.
__device__ inline void store_coherent_h4(_Float16* dst, float a, float b, float c, float d) {
  const v2h lo = {(_Float16)a, (_Float16)b}, hi = {(_Float16)c, (_Float16)d};
  const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint2 load_coherent_h4(const _Float16* src) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}

// The decode step's split exchange.  Every 8-byte word of a partial slot
// holds the sentinel (all bits set) between steps: a producer stores its words
// (never the sentinel: a value with that pattern, which only a NaN payload
// could give, is stored as a canonical NaN instead) and the group's combiner
// polls them until no sentinel is left, then stores the sentinel back.
constexpr uint64_t kPartialSentinel = ~0ull;
constexpr uint64_t kEmptyPartialMl = 0x00000000FF800000ull;  // (m, l) = (-inf, 0)
constexpr uint64_t kPartialWaitTicks = 10000000;             // 100 ms of the 100 MHz wall clock

__device__ inline void publish_word(void* dst, uint64_t v, uint64_t nan_form) {
  if (v == kPartialSentinel) v = nan_form;
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void publish_ml(float* dst, float m, float l) {
  publish_word(dst, (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(l) << 32),
               0x7FC000007FC00000ull);
}

__device__ inline void publish_h4(_Float16* dst, float a, float b, float c, float d) {
  const v2h lo = {(_Float16)a, (_Float16)b}, hi = {(_Float16)c, (_Float16)d};
  publish_word(dst, (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32),
               0x7E007E007E007E00ull);
}

__device__ inline uint64_t poll_word(const void* src) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void reset_word(void* dst) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), kPartialSentinel, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float h_lo(uint32_t w) { return (float)__builtin_bit_cast(v2h, w)[0]; }
__device__ inline float h_hi(uint32_t w) { return (float)__builtin_bit_cast(v2h, w)[1]; }

// Cross-lane moves on the VALU (DPP and the gfx950 lane swaps) rather than LDS
// permutes.  DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1]
// (lane ^ 2), row_half_mirror (lane i <-> 7 - i in each 8), row_mirror (lane
// i <-> 15 - i in each 16-lane row), row_newbcast n (lane n of each row to the
// whole row).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowBcast = 0x150;

template <int C>
__device__ inline int dpp(int x) { return __builtin_amdgcn_mov_dpp(x, C, 0xF, 0xF, false); }
template <int C>
__device__ inline float dpp(float x) { return __int_as_float(dpp<C>(__float_as_int(x))); }
template <int C>
__device__ inline double dpp(double x) {
  const long v = __double_as_longlong(x);
  const int lo = dpp<C>((int)v), hi = dpp<C>((int)(v >> 32));
  return __longlong_as_double((long)(((unsigned long)(unsigned)hi << 32) | (unsigned)lo));
}

// Sum over each aligned group of 8 (16) lanes.  Every step adds the same two
// values in every lane of a pair, so all lanes of a group end with one value.
__device__ inline double sum8(double s) {
  s += dpp<kDppXor1>(s);
  s += dpp<kDppXor2>(s);
  return s + dpp<kDppHalfMirror>(s);
}
__device__ inline float sum16(float s) {
  s += dpp<kDppXor1>(s);
  s += dpp<kDppXor2>(s);
  s += dpp<kDppHalfMirror>(s);
  return s + dpp<kDppMirror>(s);
}

// Maximum of three values in one v_maximum3_f32: without the quieting moves the
// compiler puts before fmaxf on values it cannot prove canonical (MFMA
// results), and visible to the compiler, which then keeps the wait states a
// matrix-core result needs before a vector read (it adds none ahead of inline
// assembly).  NaN-propagating; the scores it serves hold none.
__device__ inline float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// `acc` plus the sum of the f16 weights of n blocks (the values the PV products
// take), two per v_dot2_f32_f16 against ones: half the instructions of fp32
// adds, and the row's sum then matches the weights its output is formed from.
template <int N>
__device__ inline float row_weights(const v8h (&pv)[N], float acc) {
  const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int q = 0; q < N; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(v2h{pv[q][2 * i], pv[q][2 * i + 1]}, ones, acc, false);
  return acc;
}

// Maximum / sum of lane j over the four 16-lane rows: the 16-row swap pairs
// rows (0,1) and (2,3), the 32-row swap then pairs the halves.
__device__ inline float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ inline float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
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

// The norm alone (norm_rope8 without its RoPE) and the RoPE alone, for a
// prologue that computes the sincos table while the norms run.
__device__ inline void norm8(const float (&x)[8], float scale, float (&y)[8]) {
#pragma clang fp contract(off)
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += (double)(x[k] * x[k]);
  ss = sum8(ss);
  const float ms = (float)ss / 64.0f;
  const float inv = rsqrt_exact(ms + 1.0e-5f);
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = x[k] * inv;
  if (scale != 1.0f) {
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = y[k] * scale;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = round_bf16(y[k]);
}

__device__ inline void rope8(const float (*cs)[2], int c8, float (&y)[8]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const float c = cs[c8 * 4 + pr][0], s = cs[c8 * 4 + pr][1];
    const float e = y[2 * pr], o = y[2 * pr + 1];
    const float ec = e * c, os = o * s, oc = o * c, es = e * s;
    y[2 * pr] = round_bf16(ec - os);
    y[2 * pr + 1] = round_bf16(oc + es);
  }
}

__device__ inline uint2 pack_e4m3x8(const float (&y)[8]) {
  const uint32_t lo = e4m3x2(y[0], y[1]) | (e4m3x2(y[2], y[3]) << 16);
  const uint32_t hi = e4m3x2(y[4], y[5]) | (e4m3x2(y[6], y[7]) << 16);
  return make_uint2(lo, hi);
}

}  // namespace
}  // namespace mi355x_ga
