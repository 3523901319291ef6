// step_kernel.hip -- the whole gated-attention layer-step as ONE gfx950 kernel.
//
// Definition: page "012-attention-local-splits.py" -- module docstring (step
// order), `_prepare_qkv` (norm, RoPE, q cast, K/V store), `_cos_sin` (RoPE
// frequencies), kernel_fn's flash_attn_with_kvcache call (paged causal window
// attention over the e4m3 cache, split-KV) and its rms_norm_gate epilogue.
//
// One workgroup per work unit (request b, token group tg, split s).  A
// request's L new tokens form one group or groups of at most two or four
// consecutive tokens (the plan's choice).  Four waves each cover both KV heads
// of the group's rows, so every 128-byte cache row a wave fetches (one key,
// both heads) is used whole; or, for multi-token groups over a short key range
// and for one group of five to eight tokens, eight waves each cover one KV
// head.  Groups of fewer tokens shorten a unit's prologue at the price of
// reading each key chunk once per group (workgroups are dealt to the 8 XCDs
// round-robin, so the units of a chunk share an XCD and its L2 when batch x
// splits is a multiple of 8).
//
//  A. Geometry and early loads: cache_seqlens[b] gives the request's key range
//     and this unit's chunk; the projection rows, positions and the page-table
//     entries of the first key blocks are requested, then the first two blocks'
//     K/V rows.  While those are in flight the unit computes its group's q
//     (norm, RoPE, e4m3) into LDS; the units whose chunk holds a new token's key
//     also compute that token's K/V codes and use them in place of the cache
//     row (the group-0 one stores them at cache_loc), so no unit reads a row
//     being written.
//  B. Key loop (waves take 32-key blocks round-robin, two blocks in flight):
//     QK^T on v_mfma_f32_16x16x32_fp8_fp8 straight from the cache bytes; base-2
//     softmax with a lazily moved running max (rescale only when the max grows
//     by more than 2^8); P in f16; PV as O^T = V^T P^T on
//     v_mfma_f32_16x16x32_f16 with V transposed in registers and widened
//     exactly to f16.
//  C. The waves merge through LDS.  Token t of a group is combined by split
//     t mod S of its request; the other splits publish their partial rows of t
//     (o / l in f16, m and l in fp32), each 8-byte word one device-coherent
//     store, and do not wait for them.
//  D. A combiner keeps its own partial in registers, polls the others' words
//     until none holds the empty-slot sentinel, merges them (log-sum-exp),
//     rounds the attention output to bf16, applies RMSNorm x sigmoid(gate),
//     writes bf16 out and sets the consumed words back to the sentinel.
//
// Cross-workgroup visibility (C, D): the partials are written and read only
// with agent-scope atomic accesses (sc1: coherent across the XCDs' L2 caches;
// workgroup-scope loads can return a stale line even within one XCD), and an
// 8-byte aligned atomic access is single-copy atomic, so a word is either the
// sentinel or the producer's value.  No unit waits for its own stores, no
// counter is taken, and no L2 write-back or invalidate is needed.  The
// combiner's wait is bounded (100 ms): a split that never arrives (the launch's
// workgroups could not all run) gives NaN output instead of a hang.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "numerics.h"
#include "step_device.h"

namespace mi355x_ga {
namespace {

constexpr int kHeadRows = kQHeads + 2 * kKvHeads;  // 20 head rows per token

// K/V operands of one 32-key block for NG KV heads starting at head g0.
template <int NG>
struct KvBlock {
  uint4 k[2][NG];      // lane (q4, j): 16 bytes of key 16t+j per head
  uint32_t v[NG][8];   // lane (q4, j): columns 4j..4j+3 of keys 16(r/4)+4q4+r%4 per head
};

// Offset in a 32-key block of the key whose page-table entry lane l fetches for
// the V operand: lane (q4, n) of row q4, n < 8, takes key 16(n/4) + 4q4 + n%4,
// the keys every lane of row q4 reads V from.
__device__ inline int v_key_offset(int lane) {
  return 16 * ((lane & 7) >> 2) + 4 * (lane >> 4) + (lane & 3);
}

// `kk`, `kv`: this lane's keys and page-table entries for the K operand (block
// base + lane % 32) and the V operand (block base + v_key_offset), clamped.
// Rows reach the lanes that read them by lane swaps and row broadcasts.
template <int NG>
__device__ inline KvBlock<NG> load_kv(const StepParams& p, int2 entry, int kk, int kv, int g0, int j,
                                      int q4) {
  const int krow = key_row(p, entry.x, kk);
  const int vrow = key_row(p, entry.y, kv);
  // Lanes 32..63 repeat lanes 0..31, so the 16-row swap leaves row 0's rows
  // (keys 0..15) in a[0] and row 1's (keys 16..31) in a[1], in every row.
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)krow, (unsigned)krow, false, false);
  KvBlock<NG> d;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint8_t* kr = p.k_cache + (int64_t)(int)a[t] * kRowBytes + g0 * kHeadDim + 16 * q4;
#pragma unroll
    for (int g = 0; g < NG; ++g) d.k[t][g] = *reinterpret_cast<const uint4*>(kr + g * kHeadDim);
  }
  int vr[8];
  vr[0] = dpp<kDppRowBcast + 0>(vrow);
  vr[1] = dpp<kDppRowBcast + 1>(vrow);
  vr[2] = dpp<kDppRowBcast + 2>(vrow);
  vr[3] = dpp<kDppRowBcast + 3>(vrow);
  vr[4] = dpp<kDppRowBcast + 4>(vrow);
  vr[5] = dpp<kDppRowBcast + 5>(vrow);
  vr[6] = dpp<kDppRowBcast + 6>(vrow);
  vr[7] = dpp<kDppRowBcast + 7>(vrow);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint8_t* vp = p.v_cache + (int64_t)vr[r] * kRowBytes + g0 * kHeadDim + 4 * j;
#pragma unroll
    for (int g = 0; g < NG; ++g) d.v[g][r] = *reinterpret_cast<const uint32_t*>(vp + g * kHeadDim);
  }
  return d;
}

// load_kv for a block that lies in one page (32-aligned blocks, power-of-two
// pages of 32 keys or more): the page's base row in scalar registers (`entry`
// and `kb`, the block's first key, are wave-uniform), each lane's rows at fixed
// offsets from it (the loads' immediates), so no per-lane page lookups or row
// addresses.  All 32 rows lie in the block's page, so they are in bounds; in a
// block that runs past the chunk's end the rows of the keys beyond it may hold
// anything: their scores are masked, and the kernel zeroes their V bytes where
// the block is consumed (zero_v_past), so that no NaN code reaches the PV
// products (load_kv clamps such keys to end - 1 instead).
template <int NG>
__device__ inline KvBlock<NG> load_kv_page(const StepParams& p, int entry, int kb, int g0, int j, int q4) {
  const int e = __builtin_amdgcn_readfirstlane(entry);  // uniform: keep the base scalar
  const int phys = (uint32_t)e < (uint32_t)p.num_pages ? e : 0;  // invalid input: stay in bounds
  const int64_t row0 = ((int64_t)phys << p.page_shift) + (kb & ((1 << p.page_shift) - 1));
  const uint8_t* kbase = p.k_cache + row0 * kRowBytes + g0 * kHeadDim;
  const uint8_t* vbase = p.v_cache + row0 * kRowBytes + g0 * kHeadDim;
  const uint32_t ok = (uint32_t)(j * kRowBytes + 16 * q4);
  const uint32_t ov = (uint32_t)(4 * q4 * kRowBytes + 4 * j);
  KvBlock<NG> d;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int g = 0; g < NG; ++g)
      d.k[t][g] = *reinterpret_cast<const uint4*>(kbase + ok + (16 * t * kRowBytes + g * kHeadDim));
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int g = 0; g < NG; ++g)
      d.v[g][r] =
          *reinterpret_cast<const uint32_t*>(vbase + ov + ((16 * (r >> 2) + (r & 3)) * kRowBytes + g * kHeadDim));
  return d;
}

// V bytes of the keys past offset `lim` of a block loaded by load_kv_page set
// to zero (lim < 0: every key).
template <int NG>
__device__ inline void zero_v_past(KvBlock<NG>& d, int lim, int q4) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int g = 0; g < NG; ++g) d.v[g][r] = 16 * (r >> 2) + 4 * q4 + (r & 3) <= lim ? d.v[g][r] : 0u;
}

// Norm (+ RoPE) of one 8-column slice of a head row, page order, every fp32 step
// rounded once (no contraction): fp64-exact sum of squares over the 8 lanes of
// the row, exact rsqrt, fp32 product (times `scale`, exact when 1), bf16; RoPE
// pairs (2i, 2i+1) with fp32 products and sum, bf16.
__device__ inline void norm_rope8(const float (&x)[8], bool rope, const float (*cs)[2], int c8,
                                  float scale, float (&y)[8]) {
#pragma clang fp contract(off)
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += (double)(x[k] * x[k]);
  ss = sum8(ss);
  const float ms = (float)ss / 64.0f;
  const float inv = rsqrt_exact(ms + 1.0e-5f);
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = x[k] * inv;
  if (scale != 1.0f) {  // page 1's norm (scale 1) skips the product
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = y[k] * scale;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = round_bf16(y[k]);
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

// The balanced deal (batch <= 64; lane l stands for request l): the first of
// the token group's B * S units that request l gets, R_l = l + floor(X * K_<l
// / K) with X = B * (S - 1), K_<l the keys of the requests before l and K all
// of them (R_B = B * S), so that every unit carries about K / (B * S) keys;
// csl receives request l's cached length.  Every wave of a workgroup computes
// the same values.
__device__ inline int balanced_first_unit(const StepParams& p, int L, int lane, int& csl) {
  const int bs = p.batch * p.splits;
  csl = lane < p.batch ? p.cache_seqlens[lane] : 0;
  const int firstl = p.window > 0 ? max(0, csl - L - p.window + 1) : 0;
  const long long kl = max(0, csl - firstl);
  long long incl = kl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const long long ktot = __shfl(incl, 63);
  const int x = bs - p.batch;
  // Exact in double (x * keys < 2^53); correctly rounded division is monotonic,
  // so the boundaries strictly increase and the last one is bs.
  return ktot > 0 ? lane + (int)floor((double)x * (double)(incl - kl) / (double)ktot) : lane * p.splits;
}

// The gated epilogue of one thread's 4 columns (c4..c4+3 of a head: 16
// consecutive lanes hold the head's 64 columns): the attention output o / l
// (times the value descale vs) rounded to bf16, RMSNorm over the head,
// times sigmoid(gate); bf16 bits of the 4 results packed in a uint2.  Output-
// side arithmetic runs in fp32 on the hardware reciprocal, rsqrt and exp (each
// within a couple of fp32 ulps); the result is rounded to bf16 (2^-9
// relative) once at the end.  A lost split (lost) gives NaN.
__device__ inline uint2 gated_epilogue(const float (&o)[4], float l, float vs, uint2 graw, bool lost) {
  const float inv = lost ? __builtin_nanf("") : (l > 0.0f ? vs * __builtin_amdgcn_rcpf(l) : 0.0f);
  float y[4];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    y[c] = round_bf16(o[c] * inv);  // the attention result is bf16 before the epilogue
    ss += y[c] * y[c];
  }
  ss = sum16(ss);
  const float r = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + 1.0e-5f);
  const float gate[4] = {bf16_value(graw.x & 0xffffu), bf16_value(graw.x >> 16), bf16_value(graw.y & 0xffffu),
                         bf16_value(graw.y >> 16)};
  uint32_t ob[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) ob[c] = bf16_bits(y[c] * r * __builtin_amdgcn_rcpf(1.0f + __expf(-gate[c])));
  return make_uint2(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16));
}

template <int LU, bool HS, int KW, bool SP, bool BAL, bool PG>
__global__ __launch_bounds__(64 * KW * (HS ? 2 : 1)) void fused_step_kernel(StepParams p) {
  // LU: tokens per unit.  A request's L tokens form p.tgroups groups of at most
  // LU consecutive tokens; the unit (request b, token group tg, key chunk kc)
  // attends its group's query rows over chunk kc of the request's keys.
  // KW waves per KV head take the chunk's 32-key blocks round-robin.  HS (head
  // split): 2*KW waves, each working on one KV head's rows; otherwise KW waves
  // working on both heads.  PG (balanced units of a whole verify block, pages
  // of a power of two >= 32 keys): every block starts at a multiple of 32 keys
  // (no window, chunks of whole blocks), so it lies in one page, and its rows
  // come from one scalar page-table load (load_kv_page).
  constexpr int NG = HS ? 1 : kKvHeads;           // KV heads a wave works on
  constexpr int kWaves = HS ? 2 * KW : KW;
  constexpr int kThreads = 64 * kWaves;
  constexpr int NRB = (LU * kGroup + 15) / 16;  // 16-row blocks per KV head
  constexpr int kQItems = LU * kQHeads * 8;     // (token, q head, 8-column slice)
  constexpr int kMaxL = max_q_len_for(LU);
  static_assert(kMaxL >= LU, "no q_len is served by this unit size");
  static_assert(!SP || (HS && LU == 1), "page-list-driven decode: q_len 1, one KV head per wave");
  static_assert(!PG || (BAL && HS && NRB >= 4), "page-blocks: balanced whole-block units only");
  constexpr int kMaxItems = kQItems + kMaxL * 2 * kKvHeads * 8;  // + K/V rows of every token
  constexpr int kItemIters = (kMaxItems + kThreads - 1) / kThreads;
  constexpr int kRows = LU * kQHeads;           // partial rows of a unit
  __shared__ __align__(16) uint8_t s_q[LU][kQHeads][kHeadDim];
  __shared__ __align__(16) uint8_t s_newk[kMaxQLen][kRowBytes];
  __shared__ __align__(16) uint8_t s_newv[kMaxQLen][kRowBytes];
  __shared__ float s_cs[kMaxQLen][kHeadDim / 2][2];
  // Wave partials for the merge: rows KV-head-major (row g * LU * 8 + r of
  // head g's row r), padded by 4 floats so that a wave's 16 consecutive rows
  // start on distinct banks.
  __shared__ __align__(16) float s_mo[KW][kRows][kHeadDim + 4];
  __shared__ __align__(16) float s_ml[KW][kRows][2];
  // SP (page-list-driven decode): the request's block lists, one per KV head.
  __shared__ int s_blk[SP ? kKvHeads : 1][SP ? kMaxSparseTopk : 1];

  // Units of one token serve q_len 1 only, as one group.
  constexpr bool kOneGroup = LU == 1;
  const int L = kOneGroup ? LU : p.q_len;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // A token group's B * S units, in order, are the requests' splits: unit ru
  // is split kc of request b, whose nsp splits are units sbase .. sbase + nsp - 1
  // (ru is also the unit's partial slot).  Uniform: S splits per request.
  // BAL (balanced): request l gets 1 + floor(X * K_<=l / K) - floor(X * K_<l / K)
  // of them, X = B * (S - 1), K_<l the keys of the requests before l and K all
  // of them, so that every unit carries about K / (B * S) keys: the step then
  // lasts as long as the average request rather than the longest.
  int b, kc, nsp, sbase, cs, tg, ru;
  if constexpr (BAL) {  // batch <= 64: request `lane` per lane, every wave alike
    const int bs = p.batch * p.splits;
    ru = kOneGroup ? blockIdx.x : blockIdx.x % bs;
    tg = kOneGroup ? 0 : blockIdx.x / bs;
    int csl;
    const int rl = balanced_first_unit(p, L, lane, csl);
    b = __popcll(__ballot(lane >= 1 && lane < p.batch && rl <= ru));
    sbase = __builtin_amdgcn_readlane(rl, b);
    nsp = (b + 1 < p.batch ? __builtin_amdgcn_readlane(rl, b + 1) : bs) - sbase;
    kc = ru - sbase;
    cs = __builtin_amdgcn_readlane(csl, b);
  } else {
    kc = blockIdx.x % p.splits;
    const int bt = blockIdx.x / p.splits;
    b = kOneGroup ? bt : bt % p.batch;
    tg = kOneGroup ? 0 : bt / p.batch;
    nsp = p.splits;
    sbase = b * p.splits;
    ru = sbase + kc;
    cs = p.cache_seqlens[b];
  }
  const int t_lo = tg * LU;              // the group's first token (request-local)
  const int t_n = min(LU, L - t_lo);     // its tokens, >= 1
  // The wave index as a scalar keeps the block indices and branches of the
  // windowed kernels scalar (B = 32, L = 1, W = 2048: 10.39 against 10.53 us);
  // the balanced kernels' long key loops run faster with it in a vector
  // register (B = 64, L = 1, 32k keys: 101.1 against 119.6 us; B = 8, L = 8,
  // 64k-128k keys: 82.3 against 89.6 us).
  const int wave = BAL ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % KW;            // this wave's place among its head's waves
  const int g0 = HS ? wave / KW : 0;   // first KV head this wave works on
  const int j = lane & 15;
  const int q4 = lane >> 4;
  const int64_t tok0 = (int64_t)b * L;
  const int kItems = kQItems + L * 2 * kKvHeads * 8;

  // ---------------- A. geometry and early loads ----------------
  // The chain cache_seqlens -> page table -> K/V rows bounds the step's
  // latency, so the first two blocks' page-table entries are requested before
  // any load off that chain: vector memory counters complete in order, and a
  // slower load issued earlier (a cold projection row) would hold up the wait
  // for the page table.  The other small loads follow, then the K/V loads.
  // The cache scales: tiny, shared by every unit, issued with cache_seqlens so
  // that every path reaches the page-table wait with the same loads in flight.
  const float ks = p.scaled ? *p.k_scale : 1.0f;
  const float vs = p.scaled ? *p.v_scale : 1.0f;
  if constexpr (SP) {  // both KV heads' lists of request b into LDS (2 * topk <= threads)
    if (tid < kKvHeads * p.sparse_topk) {
      const int g = tid / p.sparse_topk, s = tid - g * p.sparse_topk;
      s_blk[g][s] = p.block_idx[((int64_t)g * p.batch + b) * p.sparse_topk + s];
    }
    lds_barrier();
  }
  asm volatile("" ::: "memory");
  const int p0 = cs - L;  // key index (position) of the request's first new token
  const int last = cs - 1;
  // SP: the unit's chunk is a range of virtual key indices v in [0, topk * BS):
  // list slot v / BS, offset v % BS within that block.
  const int first = SP ? 0 : (p.window > 0 ? max(0, p0 - p.window + 1) : 0);
  // Units of three or more tokens over a window split only the cached keys
  // (first .. p0 - 1); the request's new keys, whose codes the prologue leaves
  // in LDS, are one more block for the last split (kNewApart).  A window of W
  // then splits as W - 1 keys instead of W + L - 1: B 32, L 8, W 2048 gives 64
  // blocks, four per wave, where 65 left one wave of most units a fifth.
  constexpr bool kNewApart = LU > 2 && !BAL && !SP;
  const int n = SP ? p.sparse_topk * p.sparse_block : max(0, (kNewApart ? p0 - 1 : last) - first + 1);
  int chunk = (n + nsp - 1) / nsp;
  chunk = (chunk + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
  const int start = first + kc * chunk;
  const int end = min(start + chunk, SP ? n : (kNewApart ? p0 : last + 1));
  const int nblk = end > start ? (end - start + kKeyBlock - 1) / kKeyBlock : 0;
  const int nb = nblk > kw ? (nblk - kw + KW - 1) / KW : 0;  // this wave's
  const int pt_row = SP && p.token_req ? min(max(p.token_req[b], 0), p.pt_rows - 1) : b;
  const int32_t* pt = p.page_table + (int64_t)pt_row * p.max_pages;
  // Key of this lane in the wave's block i.  Blocks past the wave's last are
  // clamped to it, so the pipeline's loads are unconditional (which keeps the
  // compiler's memory-counter waits exact) and the extra ones hit cache lines
  // already fetched.
  const int voff = v_key_offset(lane);
  auto block_key = [&](int i, int off) {
    const int blk = min(i, max(nb - 1, 0));
    return max(0, min(start + (kw + KW * blk) * kKeyBlock + off, end - 1));
  };
  // SP: virtual index -> key of the request; false (and key 0, a row in bounds)
  // when the slot is empty or the key lies at or past the cached length.
  // SP: list slot of virtual index v (>= 0) and its offset in the slot's block
  // (a shift when the block size is a power of two).
  auto sp_slot = [&](int v) { return p.sparse_shift >= 0 ? v >> p.sparse_shift : v / p.sparse_block; };
  auto sp_key = [&](int v, int& key) {
    if constexpr (SP) {
      const int slot = sp_slot(v);
      const int bid = s_blk[g0][slot];
      key = bid * p.sparse_block + (v - slot * p.sparse_block);
      const bool ok = bid >= 0 && key < cs;
      key = ok ? key : 0;
      return ok;
    } else {
      key = v;
      return true;
    }
  };
  auto mapped = [&](int v) {
    int key;
    sp_key(v, key);
    return key;
  };
  auto k_key = [&](int i) { return SP ? mapped(block_key(i, lane & 31)) : block_key(i, lane & 31); };
  auto v_key = [&](int i) { return SP ? mapped(block_key(i, voff)) : block_key(i, voff); };
  // PG: the wave's block i (clamped like block_key) from scalars: its first key
  // and its page's entry (a uniform load), in .x of the int2 the other kernels
  // fill with the lane's K and V entries.
  const int kw_s = __builtin_amdgcn_readfirstlane(kw);
  const int nb_s = __builtin_amdgcn_readfirstlane(nb);
  auto pg_key = [&](int i) { return start + (kw_s + KW * min(i, max(nb_s - 1, 0))) * kKeyBlock; };
  auto load_pte = [&](int i) {
    if constexpr (PG) return make_int2(pt[min(pg_key(i) >> p.page_shift, p.max_pages - 1)], 0);
    else return make_int2(page_entry(p, pt, k_key(i)), page_entry(p, pt, v_key(i)));
  };
  auto load_block = [&](int2 e, int i) {
    if constexpr (PG) return load_kv_page<NG>(p, e.x, pg_key(i), g0, j, q4);
    else return load_kv<NG>(p, e, k_key(i), v_key(i), g0, j, q4);
  };

  const int2 pte0 = load_pte(0);
  const int2 pte1 = load_pte(1);
  asm volatile("" ::: "memory");  // the loads below stay behind the page-table loads

  const uint16_t* qkv_b = p.qkv + tok0 * kWidth;
  // Item -> (request-local token, head row, 8-column slice): q rows of the
  // group's tokens first, then the K and V rows of every token.
  auto item_token = [&](int item) {
    return item < kQItems ? t_lo + (item >> 7) : (item - kQItems) >> 5;
  };
  auto item_row = [&](int item) {
    return item < kQItems ? (item >> 3) & (kQHeads - 1) : kQHeads + (((item - kQItems) >> 3) & 3);
  };
  // Unconditional loads (slots past the items read a valid row and are never
  // used): a load skipped on some path would leave the compiler's memory-counter
  // waits counting for the longest path, and the page-table wait would then
  // also wait for a projection row.
  uint4 xv[kItemIters];
#pragma unroll
  for (int it = 0; it < kItemIters; ++it) {
    const int item = min(tid + kThreads * it, kItems - 1);
    xv[it] = *reinterpret_cast<const uint4*>(qkv_b + min(item_token(item), L - 1) * kWidth +
                                              item_row(item) * kHeadDim + (item & 7) * 8);
  }
  // The sincos table's (token, frequency) threads: the first 32 L, or, when a
  // one-token unit leaves threads without an item, the last 32, which then
  // compute it while the item threads compute their norms.
  constexpr bool kIdleCs = kOneGroup && kMaxItems + 32 * LU <= kThreads;
  constexpr int kCsBase = kIdleCs ? kThreads - 32 * LU : 0;
  const bool cs_thread = kIdleCs ? p.rope && tid >= kCsBase && tid < kCsBase + 32 * L
                                 : p.rope && tid < 32 * L;
  int64_t my_slot = p.cache_loc[tok0 + min(tid, L - 1)];
  // Raw position and frequency now; the angle (which waits for them) after the
  // K/V loads.  Without RoPE, positions may be absent: read a cache row index
  // instead (same type, always present) and ignore it.
  const int64_t* pos_src = p.rope ? p.positions : p.cache_loc;
  int64_t my_pos = kIdleCs ? pos_src[tok0 + min(max((tid - kCsBase) >> 5, 0), L - 1)]
                           : pos_src[tok0 + min(tid >> 5, L - 1)];
  float my_freq = p.inv_freq[tid & 31];
  asm volatile("" ::: "memory");  // ... and ahead of the K/V loads, so waiting for them never waits for K/V

  // Each block's page-table load follows the K/V loads two blocks earlier, so
  // waiting for it never waits for the next block's K/V.
  // Units of one or two tokens issue block A's loads only: a wave's loads
  // issue slowly once the compute unit's misses in flight reach their limit,
  // and in-order issue would hold the q prologue behind block B's loads, which
  // follow the prologue instead (their chunks are often one pair per wave).
  // Larger units keep both blocks ahead of their longer prologue.
  constexpr bool kLateB = LU <= 2;
  KvBlock<NG> bufA = load_block(pte0, 0);
  int2 pa = load_pte(2);
  // PG: the single-block walk issues A's successor, its entry, then B's; the
  // same order here (not left to the scheduler) keeps the memory-counter waits
  // on the loop's entry path no tighter than on its back edge.
  if constexpr (PG) asm volatile("" ::: "memory");
  KvBlock<NG> bufB;
  int2 pb;
  if constexpr (!kLateB) {
    bufB = load_block(pte1, 1);
    pb = load_pte(3);
  }
  // The small values are taken only now (the compiler would otherwise move
  // them, uniform ones into scalar registers, right after their loads, and
  // that wait would also wait for the page table's slower neighbours).
  asm volatile("" : "+v"(my_pos), "+v"(my_freq), "+v"(my_slot));

  // New token i's K/V codes are needed by the units whose chunk holds its key
  // (one per token group); the group-0 one stores them.  A key with no place in
  // any chunk (a padded slot) goes to chunk 0.
  auto chunk_has = [&](int i) {
    if constexpr (SP) return true;  // the new key may sit in any chunk's blocks
    if constexpr (kNewApart) return kc == nsp - 1;
    const int key = p0 + i;
    return (key >= start && key < end) || (key < first && kc == 0);
  };

  // RoPE table for the request's tokens: (token, frequency) per thread.
  auto sincos_table = [&]() {  // (one-token units with idle threads)
    if (cs_thread) {
      const float my_ang = (float)my_pos * my_freq;
      double sd, cd;
      sincos((double)my_ang, &sd, &cd);
      s_cs[(tid - kCsBase) >> 5][tid & 31][0] = (float)cd;
      s_cs[(tid - kCsBase) >> 5][tid & 31][1] = (float)sd;
    }
  };
  if constexpr (kIdleCs) {
    // One item per thread: its norm, then (after the table) RoPE and the codes.
    static_assert(kItemIters == 1, "one item per thread");
    const int item = tid;
    const int i = min(item_token(item), L - 1);
    const int hr = item_row(item), c8 = item & 7;
    const bool is_q = item < kQItems;
    const bool active = !(item >= kItems || item_token(item) >= L || (!is_q && !chunk_has(i)));
    float y[8];
    if (active) {
      float x[8];
      const uint32_t w[4] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_value(w[k] & 0xffffu);
        x[2 * k + 1] = bf16_value(w[k] >> 16);
      }
      if (hr < kQHeads + kKvHeads) {
        norm8(x, is_q ? p.q_scale : 1.0f, y);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = p.scaled ? round_bf16(x[k] / vs) : x[k];  // raw value
      }
    }
    sincos_table();
    lds_barrier();
    if (active) {
      if (hr < kQHeads + kKvHeads) {
        if (p.rope) rope8(s_cs[i], c8, y);
        if (hr >= kQHeads && p.scaled) {
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = round_bf16(y[k] / ks);
        }
      }
      const uint2 codes = pack_e4m3x8(y);
      if (is_q) {
        *reinterpret_cast<uint2*>(&s_q[i - t_lo][hr][c8 * 8]) = codes;
        if (kc == 0)
          *reinterpret_cast<uint2*>(p.q_out + ((tok0 + i) * kQHeads + hr) * kHeadDim + c8 * 8) = codes;
      } else if (hr < kQHeads + kKvHeads) {
        *reinterpret_cast<uint2*>(&s_newk[i][(hr - kQHeads) * kHeadDim + c8 * 8]) = codes;
      } else {
        *reinterpret_cast<uint2*>(&s_newv[i][(hr - kQHeads - kKvHeads) * kHeadDim + c8 * 8]) = codes;
      }
    }
  } else {
  if (cs_thread) {
    const float my_ang = (float)my_pos * my_freq;
    double sd, cd;
    sincos((double)my_ang, &sd, &cd);
    s_cs[tid >> 5][tid & 31][0] = (float)cd;
    s_cs[tid >> 5][tid & 31][1] = (float)sd;
  }
  lds_barrier();

#pragma unroll
  for (int it = 0; it < kItemIters; ++it) {
    const int item = tid + kThreads * it;
    const int i = min(item_token(item), L - 1);
    const int hr = item_row(item), c8 = item & 7;
    const bool is_q = item < kQItems;
    // Whole 8-lane groups are skipped together (the norm shuffles stay in-group).
    if (item >= kItems || item_token(item) >= L || (!is_q && !chunk_has(i))) continue;
    float x[8], y[8];
    const uint32_t w[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_value(w[k] & 0xffffu);
      x[2 * k + 1] = bf16_value(w[k] >> 16);
    }
    if (hr < kQHeads + kKvHeads) {
      norm_rope8(x, p.rope != 0, s_cs[i], c8, is_q ? p.q_scale : 1.0f, y);
      if (hr >= kQHeads && p.scaled) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = round_bf16(y[k] / ks);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = p.scaled ? round_bf16(x[k] / vs) : x[k];  // raw value
    }
    const uint2 codes = pack_e4m3x8(y);
    if (is_q) {
      *reinterpret_cast<uint2*>(&s_q[i - t_lo][hr][c8 * 8]) = codes;
      if (kc == 0)
        *reinterpret_cast<uint2*>(p.q_out + ((tok0 + i) * kQHeads + hr) * kHeadDim + c8 * 8) = codes;
    } else if (hr < kQHeads + kKvHeads) {
      *reinterpret_cast<uint2*>(&s_newk[i][(hr - kQHeads) * kHeadDim + c8 * 8]) = codes;
    } else {
      *reinterpret_cast<uint2*>(&s_newv[i][(hr - kQHeads - kKvHeads) * kHeadDim + c8 * 8]) = codes;
    }
  }
  }  // kIdleCs
  lds_barrier();

  if (tid < L && tg == 0 && (SP ? kc == 0 : chunk_has(tid)) && my_slot >= 0 && my_slot < p.num_rows) {
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
  // the group's token r / 8, query head 8g + r % 8.
  long qop[NG][NRB][2];
  int rlo[NRB], rhi[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = 16 * rb + j;
    const int ti = r >> 3;
    const bool valid = ti < t_n;
    const int pi = p0 + t_lo + ti;
    rlo[rb] = valid ? (p.window > 0 ? max(0, pi - p.window + 1) : 0) : 1;
    rhi[rb] = valid ? pi : 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint4 qv =
          *reinterpret_cast<const uint4*>(&s_q[min(ti, LU - 1)][(g0 + g) * kGroup + (r & 7)][16 * q4]);
      qop[g][rb][0] = valid ? as_long(qv.x, qv.y) : 0;
      qop[g][rb][1] = valid ? as_long(qv.z, qv.w) : 0;
    }
  }
  // A block is visible to every row of the group when it lies in [lo_all, hi_all].
  const int lo_all = p.window > 0 ? max(0, p0 + t_lo + t_n - 1 - p.window + 1) : 0;
  const int hi_all = min(p0 + t_lo, end - 1);
  const float scale = p.sm_scale_log2 * ks;

  float mrow[NG][NRB], lrow[NG][NRB];
  // Single-block walks (four row blocks): the exponent's offset, -mrow once a
  // row has a reference; before that 2^30 for a valid row, so that any visible
  // key's weight overflows and asks for the maximum, and 0 for a padding row.
  float nmr[NG][NRB];
  v4f acc[NG][NRB][4];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      mrow[g][rb] = -INFINITY;
      nmr[g][rb] = ((16 * rb + j) >> 3) < t_n ? 0x1p30f : 0.0f;
      lrow[g][rb] = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[g][rb][c] = v4f{0.f, 0.f, 0.f, 0.f};
    }

  // ---------------- B. key loop ----------------
  // New keys' codes replace the cache bytes of a block that holds them.
  auto substitute = [&](KvBlock<NG>& d, const int kbase) {
    if constexpr (SP) {
      // q_len 1: the new key p0, wherever this block's list slot holds it (a
      // 32-key block lies in one slot: BS and the chunks are multiples of 32).
      if (kbase >= end) return;
      const int slot = sp_slot(kbase);
      const int bid = s_blk[g0][slot];
      const int k0 = bid * p.sparse_block + (kbase - slot * p.sparse_block);
      if (bid < 0 || p0 < k0 || p0 >= k0 + kKeyBlock) return;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool nk = k0 + 16 * t + j == p0;
        const uint4 nv = *reinterpret_cast<const uint4*>(&s_newk[0][g0 * kHeadDim + 16 * q4]);
        d.k[t][0].x = nk ? nv.x : d.k[t][0].x;
        d.k[t][0].y = nk ? nv.y : d.k[t][0].y;
        d.k[t][0].z = nk ? nv.z : d.k[t][0].z;
        d.k[t][0].w = nk ? nv.w : d.k[t][0].w;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool nk = k0 + 16 * (r >> 2) + 4 * q4 + (r & 3) == p0;
        const uint32_t nv = *reinterpret_cast<const uint32_t*>(&s_newv[0][g0 * kHeadDim + 4 * j]);
        d.v[0][r] = nk ? nv : d.v[0][r];
      }
      return;
    }
    if (kbase + kKeyBlock - 1 < p0) return;
    // kNewApart: cached blocks stop before p0 (their keys past it are masked and
    // loaded from clamped cached rows); only the new-key block, at p0, takes the
    // codes, which only the last split computes.
    if constexpr (kNewApart)
      if (kbase < p0) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = kbase + 16 * t + j;
      const int i = min(max(key - p0, 0), L - 1);
      const bool nk = key >= p0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint4 nv = *reinterpret_cast<const uint4*>(&s_newk[i][(g0 + g) * kHeadDim + 16 * q4]);
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
      for (int g = 0; g < NG; ++g) {
        const uint32_t nv = *reinterpret_cast<const uint32_t*>(&s_newv[i][(g0 + g) * kHeadDim + 4 * j]);
        d.v[g][r] = nk ? nv : d.v[g][r];
      }
    }
  };

  // V^T operand: per KV head and column c (of the lane's 4), the 8 keys as f16
  // pairs; perm gathers byte c (and c+1) of two key rows.
  auto v_operand = [&](const KvBlock<NG>& d, v8h (&va)[NG][4]) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
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
  };

  // Raw q.k of one block for every row block: lane (q4, j) gets keys
  // 16t + 4q4 + i (slot 4t + i) of row j.
  auto qk = [&](const KvBlock<NG>& d, float (&z)[NG][NRB][8]) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v4f c = {0.f, 0.f, 0.f, 0.f};
          c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(d.k[t][g].x, d.k[t][g].y),
                                                          qop[g][rb][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(d.k[t][g].z, d.k[t][g].w),
                                                          qop[g][rb][1], c, 0, 0, 0);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) z[g][rb][t * 4 + ii] = c[ii];
        }
  };

  // Invisible keys (at or past kend, outside a row's window) get a -inf score.
  auto mask = [&](const int kbase, float (&z)[NG][NRB][8], const int kend) {
    if constexpr (SP) {
      // A block past the chunk is invisible; otherwise its keys are visible when
      // their slot is used and they lie below the cached length (q_len 1).
      const int slot = sp_slot(min(kbase, kend - 1));
      const int bid = kbase < kend ? s_blk[g0][slot] : -1;
      const int k0 = bid * p.sparse_block + (kbase - slot * p.sparse_block);
      if (bid >= 0 && k0 + kKeyBlock - 1 < cs) return;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool vis = bid >= 0 && k0 + 16 * (k >> 2) + 4 * q4 + (k & 3) < cs;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int g = 0; g < NG; ++g) z[g][rb][k] = vis ? z[g][rb][k] : -INFINITY;
      }
      return;
    }
    if (kbase >= lo_all && kbase + kKeyBlock - 1 <= hi_all) return;  // visible to every row
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int key = kbase + 16 * (k >> 2) + 4 * q4 + (k & 3);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const bool vis = (key < kend) & (key >= rlo[rb]) & (key <= rhi[rb]);
#pragma unroll
        for (int g = 0; g < NG; ++g) z[g][rb][k] = vis ? z[g][rb][k] : -INFINITY;
      }
    }
  };

  if constexpr (kLateB) {
    bufB = load_block(pte1, 1);
    pb = load_pte(3);
  }

  // Scores of one block -> running max -> P and PV, for KV head g.  z holds
  // raw q.k for NB blocks (the lazy max decision covers them all).
  auto softmax_pv = [&](int g, auto& zs, auto& vas, auto nblocks) {
    constexpr int NB = decltype(nblocks)::value;
    // This lane's scaled maximum over its keys of the blocks in row block rb.
    auto lane_max = [&](int rb) {
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const float* u = zs[q][g][rb];
        m = fmax3(m, fmax3(u[0], u[1], u[2]), fmax3(u[3], u[4], u[5]));
        m = fmax3(m, u[6], u[7]);
      }
      return m * scale;
    };
    // Rows whose full maximum (over the four lane groups) passes their
    // reference by more than kLazyRescale move it there; acc and l rescale.
    auto move_refs = [&](const float (&lmx)[NRB]) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mx = rows_max(lmx[rb]);
        const float mold = mrow[g][rb];
        const float mnew = mx > mold + kLazyRescale ? mx : mold;
        const float alpha = __builtin_amdgcn_exp2f(mold - (mnew == -INFINITY ? 0.0f : mnew));
        lrow[g][rb] *= alpha;  // alpha is exactly 1 for a row that kept its maximum
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[g][rb][c] *= alpha;
        mrow[g][rb] = mnew;
        if (mnew != -INFINITY) nmr[g][rb] = -mnew;
      }
    };
    // f16 weights of row block rb against the row's reference (exponent offset nmuse).
    auto weights = [&](int rb, float nmuse, v8h (&pv)[NB]) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int q = 0; q < NB; ++q)
          pv[q][k] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(zs[q][g][rb][k], scale, nmuse));
    };
    auto products = [&](int rb, const v8h (&pv)[NB]) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < NB; ++q)
          acc[g][rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vas[q][g][c], pv[q], acc[g][rb][c], 0, 0, 0);
    };
    if constexpr (NRB >= 4) {
      // Long walks of single blocks: the weights are formed against the rows'
      // references first and the maximum is taken only when some lane's sum
      // passes NB * 8 * 2^8 (a weight may have passed 2^8; a valid row without
      // a reference overflows, see nmr); a row's weights therefore stay below
      // 2^11 (f16 holds them to its 11-bit precision), and the maximum's
      // instructions leave the common block.
      v8h pv[NRB][NB];
      float bs[NRB];
      bool redo = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        weights(rb, nmr[g][rb], pv[rb]);
        bs[rb] = row_weights(pv[rb], 0.0f);
        redo |= !(bs[rb] <= NB * 8 * 256.0f);
      }
      if (__any(redo)) {
        float lmx[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) lmx[rb] = lane_max(rb);
        move_refs(lmx);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          weights(rb, nmr[g][rb], pv[rb]);
          bs[rb] = row_weights(pv[rb], 0.0f);
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        lrow[g][rb] += bs[rb];
        products(rb, pv[rb]);
      }
    } else {
      float lmx[NRB];     // this lane's scaled maximum over its keys of the blocks
      bool grow = false;  // some lane's maximum passes its row's lazy bound
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        lmx[rb] = lane_max(rb);
        grow |= lmx[rb] > mrow[g][rb] + kLazyRescale;
      }
      // A row's maximum moves only when its full maximum passes the bound,
      // which no lane's own maximum does in the common case: then nothing
      // moves and the cross-lane reduction is skipped.
      if (__any(grow)) move_refs(lmx);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        v8h pv[NB];
        weights(rb, mrow[g][rb] == -INFINITY ? 0.0f : -mrow[g][rb], pv);
        lrow[g][rb] = row_weights(pv, lrow[g][rb]);
        products(rb, pv);
      }
    }
  };
  using One = std::integral_constant<int, 1>;
  using Two = std::integral_constant<int, 2>;

  // One block on its own: its scores, running max, P and PV; `next` runs once
  // the block's operands are out of `buf` (it may load the next block there).
  auto one_block = [&](KvBlock<NG>& buf, const int kb, const int kend, auto next) {
    substitute(buf, kb);
    // PG: a block that runs past the chunk's end zeroes the V bytes of its
    // keys there.
    if constexpr (PG)
      if (kb + kKeyBlock > kend) zero_v_past(buf, kend - 1 - kb, q4);
    float z[1][NG][NRB][8];
    qk(buf, z[0]);
    v8h va[1][NG][4];
    v_operand(buf, va[0]);
    // The operand is formed before `next` refills `buf`, so that the new rows
    // land in the registers the old ones leave (else every block pays copies).
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) asm volatile("" ::"v"(va[0][g][c]) : "memory");
    next();
    mask(kb, z[0], kend);
#pragma unroll
    for (int g = 0; g < NG; ++g) softmax_pv(g, z, va, One{});
  };
  auto nothing = [] {};
  // Units of a whole verify block (four 16-row blocks per wave) take their
  // blocks one at a time: a pair's scores and operands would not fit the
  // registers of two waves per SIMD.
  constexpr bool kSingle = NRB >= 4;

  // kNewApart: the request's new keys p0 .. cs - 1 as one block, K and V from
  // the prologue's LDS codes (substitute fills every key of a block at p0),
  // masked by the rows' own ranges; the last split's last wave of each head
  // takes it, so it is counted once.  It goes first, while the wave's first
  // cached blocks are still arriving (B 32, L 8, W 2048: 16.7 us, against
  // 17.8 with it after the cached blocks).
  if constexpr (kNewApart)
    if (kc == nsp - 1 && kw == KW - 1 && cs > max(p0, 0)) {
      KvBlock<NG> nbk{};
      one_block(nbk, p0, cs, nothing);
    }

  if (kLateB && nb <= 2) {
    // A short chunk (at most one pair per wave): block A is processed while
    // block B's rows are still arriving.
    const int kb0 = start + kw * kKeyBlock;
    if (nb > 0) one_block(bufA, kb0, end, nothing);
    if (nb > 1) one_block(bufB, kb0 + KW * kKeyBlock, end, nothing);
  } else if constexpr (kSingle) {
    // Blocks A and B alternate; each block's successor (two blocks on) is
    // requested as soon as its operands are out of the buffer.  The two waves
    // of a block (one per KV head) read the two halves of its rows: a
    // workgroup barrier every second pair keeps them close enough that the
    // second half finds the row still in L2 (every wave runs the first wave's
    // block count).  B = 8, L = 8, 64k-128k keys: HBM fetch 336 -> 208 MB per
    // step (the algorithmic bytes: 206 MB), 73.7 -> 70.9 us; a barrier every
    // pair 72.5 us, every block 78.9, every fourth pair 70.6 with 225 MB.
    // (Refilling every buffer on every pass, with masked filler blocks for the
    // waves past their own count, makes the compiler's memory-counter waits
    // exact, but measured slower: B 8, L 8, 64k-128k keys, pages of 64: 60.7
    // against 57.4-58.3 us.)
    const int nb_all = nblk > 0 ? (nblk + KW - 1) / KW : 0;
    for (int bi = 0; bi < nb_all; bi += 2) {
      const int kb0 = start + (kw + KW * bi) * kKeyBlock;
      if ((bi & 3) == 0) __builtin_amdgcn_s_barrier();
      if (bi < nb)
        one_block(bufA, kb0, end, [&] {
          if (bi + 2 < nb) {
            bufA = load_block(pa, bi + 2);
            pa = load_pte(bi + 4);
          }
        });
      if (bi + 1 < nb)
        one_block(bufB, kb0 + KW * kKeyBlock, end, [&] {
          if (bi + 3 < nb) {
            bufB = load_block(pb, bi + 3);
            pb = load_pte(bi + 5);
          }
        });
    }
  } else {
    // Blocks are taken in pairs: the scores and V^T operands of both, then the
    // next pair's loads are issued, then per KV head one running-max decision for
    // the pair and P / PV for both.  Scores stay raw (q.k): the scale (> 0) goes
    // into the exponent's fma, so the maximum is taken on raw scores.
    // Units of three or more tokens take an odd last block on its own (below);
    // the one- and two-token kernels pair it with an empty second block, past
    // the chunk (every key masked, no codes substituted), which measured faster
    // for them.
    constexpr bool kOddAlone = !kLateB;
    int bi = 0;
    for (; kOddAlone ? bi + 1 < nb : bi < nb; bi += 2) {
      const bool has_b = kOddAlone || bi + 1 < nb;
      const int kb0 = start + (kw + KW * bi) * kKeyBlock;
      const int kb1 = has_b ? kb0 + KW * kKeyBlock : end;
      substitute(bufA, kb0);
      if (has_b) substitute(bufB, kb1);
      float z0[NG][NRB][8], z1[NG][NRB][8];
      qk(bufA, z0);
      qk(bufB, z1);
      v8h va0[NG][4], va1[NG][4];
      v_operand(bufA, va0);
      v_operand(bufB, va1);
      // The next pair's loads (wave-uniform branch): a wave's last pair issues
      // none, which spares a short chunk (a decode window: one pair per wave)
      // re-reading its blocks behind the softmax in issue order.
      if (bi + 2 < nb) {
        bufA = load_block(pa, bi + 2);
        bufB = load_block(pb, bi + 3);
        pa = load_pte(bi + 4);
        pb = load_pte(bi + 5);
      }
      mask(kb0, z0, end);
      mask(kb1, z1, end);
  #pragma unroll
      for (int g = 0; g < NG; ++g) {
        float lmx[NRB];     // this lane's scaled maximum over its 16 keys of the pair
        bool grow = false;  // some lane's maximum passes its row's lazy bound
  #pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float* u = z0[g][rb];
          const float* v = z1[g][rb];
          float m = fmax3(fmax3(u[0], u[1], u[2]), fmax3(u[3], u[4], u[5]), fmax3(u[6], u[7], v[0]));
          m = fmax3(m, fmax3(v[1], v[2], v[3]), fmax3(v[4], v[5], v[6]));
          lmx[rb] = fmax3(m, v[7], -INFINITY) * scale;
          grow |= lmx[rb] > mrow[g][rb] + kLazyRescale;
        }
        // A row's maximum moves only when its full maximum (over the four lane
        // groups) passes the bound, which no lane's own maximum does in the common
        // case: then nothing moves and the cross-lane reduction is skipped.
        if (__any(grow)) {
  #pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const float mx = rows_max(lmx[rb]);
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
          const float nmuse = mrow[g][rb] == -INFINITY ? 0.0f : -mrow[g][rb];
          v8h pp[2];
  #pragma unroll
          for (int k = 0; k < 8; ++k) {
            pp[0][k] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(z0[g][rb][k], scale, nmuse));
            pp[1][k] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(z1[g][rb][k], scale, nmuse));
          }
          lrow[g][rb] = row_weights(pp, lrow[g][rb]);
          const v8h p0v = pp[0], p1v = pp[1];
  #pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[g][rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va0[g][c], p0v, acc[g][rb][c], 0, 0, 0);
            acc[g][rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va1[g][c], p1v, acc[g][rb][c], 0, 0, 0);
          }
        }
      }
    }
    // An odd block count leaves one block (already in bufA), taken on its own
    // rather than as a pair with an empty second block: with 65 blocks over
    // 16 waves (a window of 2048 plus the verify block's keys) one wave of most
    // units holds five (B 32, L 8, W 2048: 18.5 -> 17.5 us).
    if constexpr (kOddAlone)
      if (bi < nb) one_block(bufA, start + (kw + KW * bi) * kKeyBlock, end, nothing);
  }

  // Row sums: each lane summed its own keys; add the four lane groups of a row.
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) lrow[g][rb] = rows_sum(lrow[g][rb]);

  // ---------------- C. merge the waves, publish the partial ----------------
  // Every wave parks (m, l, o) of its valid rows in the LDS slot of its place
  // among its head's waves; after one barrier all threads merge 4 columns of a
  // row each and publish the unit's partial.
  // LDS row of the group's token ti, query head h (compact row ti * 16 + h).
  auto lds_row = [](int cr) { return ((cr & 15) >> 3) * (LU * kGroup) + (cr >> 4) * kGroup + (cr & 7); };
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = 16 * rb + j;
      const int ti = r >> 3;
      if (ti >= t_n) continue;
      const int cr = (g0 + g) * (LU * kGroup) + r;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        *reinterpret_cast<float4*>(&s_mo[kw][cr][16 * q4 + 4 * ii]) =
            make_float4(acc[g][rb][0][ii], acc[g][rb][1][ii], acc[g][rb][2][ii], acc[g][rb][3][ii]);
      if (q4 == 0) *reinterpret_cast<float2*>(&s_ml[kw][cr][0]) = make_float2(mrow[g][rb], lrow[g][rb]);
    }
  lds_barrier();
  // Merge of one (row, 4 columns) over the waves' LDS slots.
  auto merge = [&](int cr, int c4, float& m_out, float& l_out, float4& o_out) {
    float mw[KW], lw[KW];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const float2 ml = *reinterpret_cast<const float2*>(&s_ml[w][lds_row(cr)][0]);
      mw[w] = ml.x;
      lw[w] = ml.y;
      mx = fmaxf(mx, ml.x);
    }
    const float muse = mx == -INFINITY ? 0.0f : mx;
    float lsum = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const float a = __builtin_amdgcn_exp2f(mw[w] - muse);
      const float4 v = *reinterpret_cast<const float4*>(&s_mo[w][lds_row(cr)][c4]);
      lsum += a * lw[w];
      o.x += a * v.x;
      o.y += a * v.y;
      o.z += a * v.z;
      o.w += a * v.w;
    }
    m_out = mx;
    l_out = lsum;
    o_out = o;
  };
  // Token ti of the group is merged by split ti % nsp of its request (its
  // combiner), so a group's combines are spread over its splits; every other
  // split publishes its partial rows of that token.
  // The combine's thread mapping: thread (th, h, c4) takes columns c4..c4+3 of
  // head h for the combiner's tokens kc + nsp * (th + TS * k), k = 0, 1, ...
  // (TS = threads / 256), one token per thread at a time.
  constexpr int TS = kThreads / 256;            // thread groups, 256 threads each
  const int c4 = (tid & 15) * 4;
  const int h = (tid >> 4) & (kQHeads - 1);
  const int th = tid >> 8;
  // Partial rows are ((sbase + kc) * L + token) * 16 + head.
  const int64_t stride = (int64_t)L * kQHeads;  // partial rows per split
  const int64_t base = (int64_t)sbase * stride + (int64_t)t_lo * kQHeads + h;
  if (p.sep_combine || nsp > 1) {
    // A producer of the tokens it does not merge: merge the waves and publish
    // the unit's partial rows, each 8-byte word one device-coherent store
    // (never the sentinel pattern); no wait.  With the separate combine every
    // unit publishes every token (combine_kernel merges after this launch).
    const int64_t prow0 = ((int64_t)ru * L + t_lo) * kQHeads;
    for (int idx = tid; idx < t_n * kQHeads * 16; idx += kThreads) {
      const int cr = idx >> 4, cc = (idx & 15) * 4;
      if (!p.sep_combine && (cr >> 4) % nsp == kc) continue;  // merged here
      float mx, lsum;
      float4 o;
      merge(cr, cc, mx, lsum, o);
      // o / l is a weighted mean of V codes (|.| <= 448): f16 holds it.
      const float rl = lsum > 0.0f ? __builtin_amdgcn_rcpf(lsum) : 0.0f;
      if (p.sep_combine) {
        // Read by the next launch: plain stores (the kernel boundary makes
        // them visible), no write-through.
        const v2h lo = {(_Float16)(o.x * rl), (_Float16)(o.y * rl)}, hi = {(_Float16)(o.z * rl), (_Float16)(o.w * rl)};
        *reinterpret_cast<uint2*>(p.part_o + (prow0 + cr) * kHeadDim + cc) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        if (cc == 0) *reinterpret_cast<float2*>(p.part_ml + (prow0 + cr) * 2) = make_float2(mx, lsum);
      } else {
        publish_h4(p.part_o + (prow0 + cr) * kHeadDim + cc, o.x * rl, o.y * rl, o.z * rl, o.w * rl);
        if (cc == 0) publish_ml(p.part_ml + (prow0 + cr) * 2, mx, lsum);
      }
    }
    if (p.sep_combine || kc >= t_n) return;
  }

  // ---------------- D. combine + gated epilogue (the token's combiner) ----------------
  // The unit's own partial comes from its waves' LDS slots; the other splits'
  // (kc + 1, kc + 2, ... modulo nsp) are polled until none of their words
  // holds the sentinel (a producer publishes without waiting, so the first
  // poll usually finds them), KS splits at a time, then merged.  The consumed
  // words are set back to the sentinel for the next step.
  constexpr int KS = 16;
  bool lost = false;  // a split never arrived within the wait bound
  const uint64_t t_wait0 = wall_clock64();
  for (int k = 0; kc + nsp * TS * k < t_n; ++k) {
    const int ti = kc + nsp * (th + TS * k);
    if (ti >= t_n) break;  // whole waves: th is uniform in a wave
    const uint2 graw = *reinterpret_cast<const uint2*>(p.qkv + (tok0 + t_lo + ti) * kWidth + kGateOffset +
                                                        h * kHeadDim + c4);
    float mrun, lrun, o[4];
    {
      float4 ov;
      merge(ti * kQHeads + h, c4, mrun, lrun, ov);
      o[0] = ov.x;
      o[1] = ov.y;
      o[2] = ov.z;
      o[3] = ov.w;
    }
    for (int s0 = 1; s0 < nsp; s0 += KS) {
      uint64_t mlw[KS], ow[KS];
      auto split_of = [&](int q) {  // the (s0 + q)-th split after this one
        const int sq = kc + s0 + q;
        return sq >= nsp ? sq - nsp : sq;
      };
      auto ml_at = [&](int q) { return p.part_ml + (base + (int64_t)split_of(q) * stride + ti * kQHeads) * 2; };
      auto o_at = [&](int q) { return p.part_o + (base + (int64_t)split_of(q) * stride + ti * kQHeads) * kHeadDim + c4; };
      auto used = [&](int q) { return s0 + q < nsp; };
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        mlw[q] = kEmptyPartialMl;
        ow[q] = 0;
        if (used(q)) {
          mlw[q] = poll_word(ml_at(q));
          ow[q] = poll_word(o_at(q));
        }
      }
      // Every lane waits for its own words; the wait is bounded.
      for (;;) {
        bool pending = false;
#pragma unroll
        for (int q = 0; q < KS; ++q) pending |= mlw[q] == kPartialSentinel || ow[q] == kPartialSentinel;
        if (!pending) break;
        if (wall_clock64() - t_wait0 > kPartialWaitTicks) {
          lost = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          if (mlw[q] == kPartialSentinel) mlw[q] = poll_word(ml_at(q));
          if (ow[q] == kPartialSentinel) ow[q] = poll_word(o_at(q));
        }
      }
      // The words are consumed: back to the sentinel for the next step.
#pragma unroll
      for (int q = 0; q < KS; ++q)
        if (used(q)) {
          reset_word(ml_at(q));
          reset_word(o_at(q));
        }
      float mc = mrun;
#pragma unroll
      for (int q = 0; q < KS; ++q) mc = fmaxf(mc, __uint_as_float((uint32_t)mlw[q]));
      const float muse = mc == -INFINITY ? 0.0f : mc;
      const float a = __builtin_amdgcn_exp2f(mrun - muse);
      lrun *= a;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] *= a;
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        // A split's weight is its l times 2^(m - max); its partial is o / l.
        const float wk = __builtin_amdgcn_exp2f(__uint_as_float((uint32_t)mlw[q]) - muse) *
                         __uint_as_float((uint32_t)(mlw[q] >> 32));
        lrun += wk;
        o[0] += wk * h_lo((uint32_t)ow[q]);
        o[1] += wk * h_hi((uint32_t)ow[q]);
        o[2] += wk * h_lo((uint32_t)(ow[q] >> 32));
        o[3] += wk * h_hi((uint32_t)(ow[q] >> 32));
      }
      mrun = mc;
    }
    *reinterpret_cast<uint2*>(p.out + (tok0 + t_lo + ti) * (kQHeads * kHeadDim) + h * kHeadDim + c4) =
        gated_epilogue(o, lrun, vs, graw, lost);
  }
}

// The separate combine (q_len <= kMaxQLen, when the plan moves the merge of
// the partials out of the attention launch): one 64-thread workgroup per
// (token, head), lane (q, c4) merging columns c4..c4+3 over the splits
// q, q + 4, q + 8, ... of the token's request (up to 8 loads in flight per
// round), the four lanes of a column then merging their states with lane
// swaps.  The request has nsp partial rows per (token, head), split kc's at
// ((sbase + kc) * L + t) * 16 + h, merged by log-sum-exp (split weight
// l * 2^(m - max), partial o / l) and followed by the gated epilogue, exactly
// as a combining unit would.  The partials come from the previous launch, so
// plain loads see them.
__global__ __launch_bounds__(64) void combine_kernel(StepParams p) {
  constexpr int KQ = 4;   // split classes (lanes per column)
  constexpr int KS = 8;   // splits per lane per round of loads
  const int tok = (int)(blockIdx.x >> 4), h = (int)(blockIdx.x & 15);
  const int L = p.q_len;
  const int b = tok / L, t = tok - b * L;
  const int lane = threadIdx.x;
  const int c4 = (lane & 15) * 4, q = lane >> 4;
  int sbase = b * p.splits, nsp = p.splits;
  if (p.balanced) {
    int csl;
    const int rl = balanced_first_unit(p, L, lane, csl);
    sbase = __builtin_amdgcn_readlane(rl, b);
    nsp = (b + 1 < p.batch ? __builtin_amdgcn_readlane(rl, b + 1) : p.batch * p.splits) - sbase;
  }
  const float vs = p.scaled ? *p.v_scale : 1.0f;
  const uint2 graw =
      *reinterpret_cast<const uint2*>(p.qkv + (int64_t)tok * kWidth + kGateOffset + h * kHeadDim + c4);
  const int64_t stride = (int64_t)L * kQHeads;  // partial rows per split
  const int64_t base = ((int64_t)sbase * L + t) * kQHeads + h;
  float mrun = -INFINITY, lrun = 0.0f, o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = q; s0 < nsp; s0 += KQ * KS) {
    float2 ml[KS];
    uint2 oh[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int s = s0 + KQ * k;
      ml[k] = make_float2(-INFINITY, 0.0f);
      oh[k] = make_uint2(0, 0);
      if (s < nsp) {
        const int64_t r = base + (int64_t)s * stride;
        ml[k] = *reinterpret_cast<const float2*>(p.part_ml + r * 2);
        oh[k] = *reinterpret_cast<const uint2*>(p.part_o + r * kHeadDim + c4);
      }
    }
    float mc = mrun;
#pragma unroll
    for (int k = 0; k < KS; ++k) mc = fmaxf(mc, ml[k].x);
    const float muse = mc == -INFINITY ? 0.0f : mc;
    const float a = __builtin_amdgcn_exp2f(mrun - muse);
    lrun *= a;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] *= a;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const float wk = __builtin_amdgcn_exp2f(ml[k].x - muse) * ml[k].y;
      lrun += wk;
      o[0] += wk * h_lo(oh[k].x);
      o[1] += wk * h_hi(oh[k].x);
      o[2] += wk * h_lo(oh[k].y);
      o[3] += wk * h_hi(oh[k].y);
    }
    mrun = mc;
  }
  // The four split classes of a column (lanes 16 apart): two swap rounds.
#pragma unroll
  for (int d = 16; d < 64; d <<= 1) {
    const float mo = __shfl_xor(mrun, d), lo = __shfl_xor(lrun, d);
    float oo[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) oo[c] = __shfl_xor(o[c], d);
    const float mc = fmaxf(mrun, mo);
    const float muse = mc == -INFINITY ? 0.0f : mc;
    const float a0 = __builtin_amdgcn_exp2f(mrun - muse), a1 = __builtin_amdgcn_exp2f(mo - muse);
    lrun = lrun * a0 + lo * a1;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = o[c] * a0 + oo[c] * a1;
    mrun = mc;
  }
  const uint2 ov = gated_epilogue(o, lrun, vs, graw, false);
  if (q == 0) *reinterpret_cast<uint2*>(p.out + (int64_t)tok * (kQHeads * kHeadDim) + h * kHeadDim + c4) = ov;
}

template <int LU, bool HS, int KW, bool SP = false, bool BAL = false, bool PG = false>
hipError_t launch_lu(const StepParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.batch * (unsigned)p.tgroups * (unsigned)p.splits;
  hipLaunchKernelGGL((fused_step_kernel<LU, HS, KW, SP, BAL, PG>), dim3(grid), dim3(64 * (HS ? 2 : 1) * KW), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.sep_combine) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(p.batch * p.q_len * kQHeads)), dim3(64), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

template <int LU>
hipError_t launch_served(const StepParams& p, hipStream_t stream) {
  if constexpr (LU == kMaxQLen) {
    // A whole verify block per unit: one KV head per wave only.
    if (!p.head_split) return hipErrorInvalidValue;
    if (p.balanced && p.page_shift >= 5) return launch_lu<LU, true, kAttnWaves, false, true, true>(p, stream);
    return p.balanced ? launch_lu<LU, true, kAttnWaves, false, true>(p, stream)
                      : launch_lu<LU, true, kAttnWaves>(p, stream);
  } else if constexpr (max_q_len_for(LU) >= LU) {
    if (p.head_split) return launch_lu<LU, true, kAttnWaves>(p, stream);
    // Balanced splits (the plan sets them only with both KV heads per wave).
    if constexpr (LU == 1)
      if (p.key_waves == 2 * kAttnWaves)
        return p.balanced ? launch_lu<LU, false, 2 * kAttnWaves, false, true>(p, stream)
                          : launch_lu<LU, false, 2 * kAttnWaves>(p, stream);
    return p.balanced ? launch_lu<LU, false, kAttnWaves, false, true>(p, stream)
                      : launch_lu<LU, false, kAttnWaves>(p, stream);
  }
  return hipErrorInvalidValue;
}

__global__ void zero_counters_kernel(int32_t* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0;
}

__global__ void fill_sentinel_kernel(uint64_t* w, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    w[i] = kPartialSentinel;
}

}  // namespace

hipError_t launch_step(const StepParams& p, hipStream_t stream, hipEvent_t attn_start) {
  if (p.batch == 0) return hipSuccess;
  if (p.q_len > kMaxQLen) return launch_extend(p, stream, attn_start);  // extend / prefill
  if (p.sparse_block > 0) {
    // Page-list-driven decode: q_len 1, one KV head per wave (each head has its
    // own list), blocks of a multiple of 32 keys, at most kMaxSparseTopk slots.
    if (p.q_len != 1 || p.tgroups != 1 || !p.head_split || p.key_waves != kAttnWaves ||
        p.sparse_block % kKeyBlock || p.sparse_topk < 1 || p.sparse_topk > kMaxSparseTopk ||
        !p.block_idx)
      return hipErrorInvalidValue;
    return launch_lu<1, true, kAttnWaves, true>(p, stream);
  }
  if (p.q_len < 1 || p.q_len > kMaxQLen ||
      (p.tgroups != token_groups(p.q_len, false) && p.tgroups != token_groups(p.q_len, true)))
    return hipErrorInvalidValue;
  switch (unit_tokens(p.q_len, p.tgroups)) {
    case 1: return launch_served<1>(p, stream);
    case 2: return launch_served<2>(p, stream);
    case 3: return launch_served<3>(p, stream);
    case 4: return launch_served<4>(p, stream);
    case kMaxQLen: return launch_served<kMaxQLen>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_sentinel(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / sizeof(uint64_t));
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_sentinel_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint64_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_zero_counters(int32_t* counters, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, counters, n);
  return hipGetLastError();
}

}  // namespace mi355x_ga
