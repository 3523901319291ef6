// extend_kernel.hip -- the gated-attention layer-step for blocks of more than
// kMaxQLen new tokens per request (extend / prefill) as two gfx950 launches.
//
// Definition: the same step as for decode (page "012-attention-local-splits.py":
// `_prepare_qkv`, `_cos_sin`, kernel_fn's flash_attn_with_kvcache call and its
// rms_norm_gate epilogue) at a larger q_len: query i of request b sits at
// position cache_seqlens[b] - q_len + i and sees the keys up to its own position
// within its window.  Page "msa.py" (msa_sparse_prefill_main) states a prefill
// the same way: causal attention with the query offset equal to the prefix length.
#include "kernels.h"
#include "numerics.h"
#include "step_device.h"

namespace mi355x_ga {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------- Extend / prefill: q_len > kMaxQLen ----------------
// Two launches.  The prologue normalises, rotates and encodes every new token
// (q to the workspace, K/V rows to the cache); the launch boundary orders all
// those stores before any attention read, so the attention kernel reads the
// new keys from the cache like every other key.
//
// Attention unit = (request, tile of kExtTile new tokens, KV head): 128 query
// rows (token, q head of the KV head), one workgroup of eight waves in two
// groups of four.  Each wave holds 32 rows (two 16-row MFMA blocks) and the
// two groups split the tile's key range: every barrier stages 64 keys (two
// 32-key blocks) in LDS, group 0 takes the first block and group 1 the
// second, and at the end group 0 merges group 1's (max, sum, output) through
// LDS.  Staging is one 16-byte load per thread: waves 0-3 stage K rows as they
// are (the fp8 QK^T operand), waves 4-7 widen V to f16 exactly and store its
// rows as they are ([key][dim]); the PV operand (V^T: four consecutive keys of
// one dim per lane and half) comes from two transposing LDS reads per MFMA.
// fp8 QK^T and f16 PV on the matrix cores, base-2 online softmax in fp32 with
// a lazily moved running max; the unit ends with the gated epilogue of its rows.
constexpr int kExtTile = 16;                    // new tokens per attention unit
constexpr int kExtRows = kExtTile * kGroup;     // 128 query rows
constexpr int kExtWaves = 8;                    // two key groups of four waves
constexpr int kExtStageKeys = 2 * kKeyBlock;    // keys staged per barrier (one block per group)
constexpr int kExtKStride = kHeadDim + 16;      // LDS bytes per staged K row (fp8; bank spread)
// LDS bytes per staged V row (f16 x 64 dims + 48 bytes of pad): an odd number
// of 16-byte units, so the staging stores of consecutive keys (one key per
// lane, 16 bytes each) start in different banks.  Measured against 160- and
// 192-byte rows, whose transposing reads conflict less but whose stores
// conflict more, the fastest.
constexpr int kExtVStride = 2 * kHeadDim + 48;
constexpr int kExtVBlock = kKeyBlock * kExtVStride;                   // one block's 32 rows
constexpr int kExtKBytes = 2 * kExtStageKeys * kExtKStride;           // double-buffered K
constexpr int kExtVBytes = 2 * 2 * kExtVBlock;                        // double-buffered V, 2 blocks
constexpr int kExtOBytes = kExtRows * (kHeadDim + 4) * 4 + kExtRows * 8;  // merge / epilogue rows + (m, l)
constexpr int kExtSmem = (kExtKBytes + kExtVBytes) > kExtOBytes ? (kExtKBytes + kExtVBytes) : kExtOBytes;
constexpr int kXcds = 8;                        // MI355X: accelerator complex dies, one L2 each

// Prologue: kExtPrologueTokens new tokens per workgroup, their 160 items each
// ((16 q, 2 k, 2 v head rows) x 8 column slices, eight lanes per head row) dealt
// over the 256 threads, three per thread at most.  The sincos table's positions
// are requested first, then every item's load; the threads holding two items
// compute the tokens' RoPE sincos table while the rows arrive, then their
// norms, and the others their three norms; RoPE, the e4m3 codes and the stores
// follow the barrier.
constexpr int kExtPrologueTokens = 4;
constexpr int kExtItems = (kQHeads + 2 * kKvHeads) * 8;                              // per token
constexpr int kExtPrologueIters = (kExtPrologueTokens * kExtItems + 255) / 256;      // 3
constexpr int kExtCsBase = 256 - 32 * kExtPrologueTokens;                            // sincos threads
static_assert(kExtPrologueTokens * kExtItems - 256 * (kExtPrologueIters - 1) <= kExtCsBase,
              "the sincos threads hold no third item");

__global__ __launch_bounds__(256) void extend_prologue_kernel(StepParams p) {
  __shared__ float s_cs[kExtPrologueTokens][kHeadDim / 2][2];
  const int64_t T = p.total_q;
  const int64_t t0 = (int64_t)blockIdx.x * kExtPrologueTokens;
  const int tid = threadIdx.x;
  // The sincos table's inputs are requested first, so that its fp64 sincos
  // runs while the projection rows are still arriving (loads return in issue
  // order).  Without RoPE, positions may be absent: a cache row index is read
  // instead (same type, always present) and ignored.
  const int cs_tok = max(tid - kExtCsBase, 0) >> 5;
  const int64_t cs_pos = (p.rope ? p.positions : p.cache_loc)[min(t0 + cs_tok, T - 1)];
  // (read through the argument segment as volatile: a plain load of the
  // argument's table may be scheduled after the rows', and then waits for them)
  const float freq = reinterpret_cast<const volatile __attribute__((address_space(4))) float*>(
      (const __attribute__((address_space(4))) uint8_t*)__builtin_amdgcn_kernarg_segment_ptr() +
      offsetof(StepParams, inv_freq))[tid & 31];
  asm volatile("" ::: "memory");
  uint4 xv[kExtPrologueIters];
#pragma unroll
  for (int it = 0; it < kExtPrologueIters; ++it) {
    const int item = min(tid + 256 * it, kExtPrologueTokens * kExtItems - 1);
    const int64_t tk = min(t0 + item / kExtItems, T - 1);
    const int rem = item % kExtItems;
    xv[it] = *reinterpret_cast<const uint4*>(p.qkv + tk * kWidth + (rem >> 3) * kHeadDim + (rem & 7) * 8);
  }
  if (p.rope && tid >= kExtCsBase) {
    const float ang = (float)cs_pos * freq;
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    s_cs[cs_tok][tid & 31][0] = (float)cd;
    s_cs[cs_tok][tid & 31][1] = (float)sd;
  }
  const float ks = p.scaled ? *p.k_scale : 1.0f;
  const float vs = p.scaled ? *p.v_scale : 1.0f;

  float y[kExtPrologueIters][8];
#pragma unroll
  for (int it = 0; it < kExtPrologueIters; ++it) {
    const int item = tid + 256 * it;
    const int hr = (item % kExtItems) >> 3;
    // Whole 8-lane groups are active or not together (a group is one head row).
    if (item < kExtPrologueTokens * kExtItems && t0 + item / kExtItems < T) {
      float x[8];
      const uint32_t w[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_value(w[k] & 0xffffu);
        x[2 * k + 1] = bf16_value(w[k] >> 16);
      }
      if (hr < kQHeads + kKvHeads) {
        norm8(x, hr < kQHeads ? p.q_scale : 1.0f, y[it]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[it][k] = p.scaled ? round_bf16(x[k] / vs) : x[k];  // raw value
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int it = 0; it < kExtPrologueIters; ++it) {
    const int item = tid + 256 * it;
    const int tl = item / kExtItems, rem = item % kExtItems;
    const int hr = rem >> 3, c8 = rem & 7;
    const int64_t t = t0 + tl;
    if (item >= kExtPrologueTokens * kExtItems || t >= T) continue;
    if (hr < kQHeads + kKvHeads) {
      if (p.rope) rope8(s_cs[tl], c8, y[it]);
      if (hr >= kQHeads && p.scaled) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[it][k] = round_bf16(y[it][k] / ks);
      }
    }
    const uint2 codes = pack_e4m3x8(y[it]);
    if (hr < kQHeads) {
      *reinterpret_cast<uint2*>(p.q_out + (t * kQHeads + hr) * kHeadDim + c8 * 8) = codes;
    } else {
      const int64_t slot = p.cache_loc[t];
      if (slot >= 0 && slot < p.num_rows) {
        uint8_t* base = hr < kQHeads + kKvHeads ? p.k_cache + (hr - kQHeads) * kHeadDim
                                                : p.v_cache + (hr - kQHeads - kKvHeads) * kHeadDim;
        *reinterpret_cast<uint2*>(base + slot * kRowBytes + c8 * 8) = codes;
      }
    }
  }
}

__global__ __launch_bounds__(64 * kExtWaves, 4) void extend_attn_kernel(StepParams p) {
  // Staging buffers during the key loop; merge rows and (m, l) after it.
  __shared__ __align__(16) uint8_t smem[kExtSmem];
  auto s_k = reinterpret_cast<uint8_t(*)[kExtStageKeys][kExtKStride]>(smem);                  // [2][64][80]
  auto s_v = reinterpret_cast<uint8_t(*)[2][kExtVBlock]>(smem + kExtKBytes);                  // [2][2][5632]
  auto s_o = reinterpret_cast<float(*)[kHeadDim + 4]>(smem);                                  // [128][68]
  auto s_ml = reinterpret_cast<float2*>(smem + kExtRows * (kHeadDim + 4) * 4);                // [128]

  const int L = p.q_len;
  const int n_tiles = (L + kExtTile - 1) / kExtTile;
  // Units in (request, tile, KV head) order, a contiguous range of them per
  // XCD (workgroups reach the XCDs round-robin): one L2 then holds a request's
  // keys for its neighbouring tiles and both KV heads, which share each cache
  // row.  The grid is padded to a multiple of kXcds; the padding exits.
  // With S key splits (the plan's choice when the units alone do not fill the
  // chip) the order is (request, split, tile, KV head); split ks of a unit
  // walks its share of the unit's 64-key stages.
  const int S = p.splits;
  const int tid = threadIdx.x, lane = tid & 63;
  int g, tile, ks, b;
  if (p.cu_seqlens_q && p.batch <= 64) {
    // A ragged batch of at most 64 requests: only the tiles that hold rows get
    // workgroups, in the same order, so every XCD takes an equal share of them
    // whatever the segments' lengths (in the padded order a request's tiles,
    // rows or not, fill one XCD).  Two scalar passes over the segments: their
    // tile count, then the request holding workgroup li (empty segments hold
    // none and are passed over).
    auto seg_tiles = [&](int r) {
      const int n = p.cu_seqlens_q[r + 1] - p.cu_seqlens_q[r];
      return (max(0, min(n, L)) + kExtTile - 1) / kExtTile;
    };
    int tot = 0;
    for (int r = 0; r < p.batch; ++r) tot += seg_tiles(r);
    const int n_wg = tot * kKvHeads * S;
    const int per_xcd = (n_wg + kXcds - 1) / kXcds;
    const int kx = (int)(blockIdx.x / kXcds);  // the grid holds the padded order's count
    if (kx >= per_xcd) return;
    const int li = (int)(blockIdx.x % kXcds) * per_xcd + kx;
    if (li >= n_wg) return;
    int first = 0, tb = 0;
    b = 0;
    for (int r = 0; r < p.batch; ++r) {
      tb = seg_tiles(r);
      const int u = tb * kKvHeads * S;
      if (li < first + u) {
        b = r;
        break;
      }
      first += u;
    }
    const int rr = li - first;
    g = rr % kKvHeads;
    tile = (rr / kKvHeads) % tb;
    ks = rr / (kKvHeads * tb);
  } else if (S == 1 && p.window == 0 && p.batch * n_tiles >= 128 && p.batch * n_tiles <= 256) {
    // Without a window a tile's keys grow with its position and with its
    // request's prefix.  Every workgroup is resident at once (two per compute
    // unit), and workgroups b and b + 256 share a unit: the first 128 tile
    // pairs (both KV heads, adjacent workgroups) take the tiles longest first,
    // requests interleaved, and the rest the same ranks mirrored, so each unit
    // holds a long tile and a short one of the opposite rank.
    const int q = (int)(blockIdx.x >> 1);
    const int T = p.batch * n_tiles;
    if (q >= T) return;
    g = (int)(blockIdx.x & 1);
    const int rank = q < 128 ? q : T - 1 - (q - 128);
    b = rank % p.batch;
    tile = n_tiles - 1 - rank / p.batch;
    ks = 0;
  } else {
    const int n_wg = p.batch * n_tiles * kKvHeads * S;
    const int per_xcd = (n_wg + kXcds - 1) / kXcds;
    const int li = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (li >= n_wg) return;
    g = li % kKvHeads;
    tile = (li / kKvHeads) % n_tiles;
    ks = (li / (kKvHeads * n_tiles)) % S;
    b = li / (kKvHeads * n_tiles * S);
  }
  const int unit = (b * n_tiles + tile) * kKvHeads + g;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  const int kg = wave >> 2, wq = wave & 3;  // key group; the wave's rows within the tile

  const int cs = p.cache_seqlens[b];
  // Ragged batches: request b's segment is tokens cu[b] .. cu[b+1]-1 (clamped
  // to q_len and to the step's tokens); a tile past its segment has no rows
  // and its workgroups leave before any shared state is touched.
  int Lb = L;
  int64_t base = (int64_t)b * L;
  if (p.cu_seqlens_q) {
    const int c0 = p.cu_seqlens_q[b], c1 = p.cu_seqlens_q[b + 1];
    Lb = max(0, min(c1 - c0, L));
    base = max<int64_t>(0, min<int64_t>(c0, p.total_q - Lb));
  }
  const int i_lo = tile * kExtTile;             // the tile's first token (request-local)
  if (i_lo >= Lb) return;
  const int n_tok = min(kExtTile, Lb - i_lo);
  const int p_first = cs - Lb + i_lo;           // its position
  const int hi = p_first + n_tok - 1;           // keys lo..hi (the last token's position)
  const int lo = p.window > 0 ? max(0, p_first - p.window + 1) : 0;
  const int nblk = hi >= lo ? (hi - lo) / kKeyBlock + 1 : 0;
  const int n_stage_all = (nblk + 1) / 2;
  const int per_split = (n_stage_all + S - 1) / S;
  const int s_first = ks * per_split;                                    // this split's stages
  const int n_stage = max(0, min(n_stage_all - s_first, per_split));
  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int64_t tok0 = base + i_lo;             // the tile's first token (global)
  const float kscale = p.scaled ? *p.k_scale : 1.0f;
  const float vs = p.scaled ? *p.v_scale : 1.0f;
  const float scale = p.sm_scale_log2 * kscale;
  // The matrix cores' block scales (E8M0 127 = 2^0), one opaque register held
  // for the whole kernel, so no product's result is ever allocated over it.
  int unit_scale;
  asm volatile("v_mov_b32 %0, 127" : "=v"(unit_scale));

  // The wave's 32 rows, one per lane pair: lane l holds row n = l % 32 (tile
  // row r = 32 wq + n: token r / 8 of the tile, q head 8 g + r % 8; both key
  // groups hold the same rows) and, as the QK^T operand, its 32 q bytes of
  // head-dim half l / 32.
  const int n32 = lane & 31, hf = lane >> 5;
  v8i qB;
  int prow, plo;
  bool valid;
  {
    const int r = 32 * wq + n32;
    const int ti = r >> 3;
    valid = ti < n_tok;
    const uint4* qs = reinterpret_cast<const uint4*>(
        p.q_out + ((tok0 + min(ti, n_tok - 1)) * kQHeads + kGroup * g + (r & 7)) * kHeadDim + 32 * hf);
    const uint4 q0 = qs[0], q1 = qs[1];
    qB = valid ? v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w}
               : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    prow = valid ? p_first + ti : -1;  // an invalid row sees no key
    plo = p.window > 0 ? p_first + ti - p.window + 1 : 0;
  }

  // Staging: thread -> (K for waves 0-3 / V for waves 4-7, key of the 64-key
  // stage, 16-byte quarter of the head's row).  A K wave's lanes take 16 keys'
  // rows, four lanes per key; V wave 4 + c takes quarter c of all 64 keys, one
  // key per lane.
  const int st_v = wave >> 2;
  const int st_key = st_v ? lane : (tid >> 2) & (kExtStageKeys - 1);
  const int st_c = st_v ? wave & 3 : tid & 3;
  // Keys past hi reload key hi (masked); with no key at all (hi < lo, hi maybe
  // negative) key 0, in bounds and unused.
  auto st_keyof = [&](int s) { return max(min(lo + (s_first + s) * kExtStageKeys + st_key, hi), 0); };
  auto st_entry = [&](int s) { return page_entry(p, pt, st_keyof(s)); };
  auto st_load = [&](int entry, int s) {
    const int row = key_row(p, entry, st_keyof(s));
    const uint8_t* src = (st_v ? p.v_cache : p.k_cache) + (int64_t)row * kRowBytes + g * kHeadDim + st_c * 16;
    return *reinterpret_cast<const uint4*>(src);
  };
  // V: 16 e4m3 values (dims 16 c .. 16 c + 15 of one key) widened to f16
  // exactly, 32 bytes of the key's row.
  auto stage_v = [&](const int buf, const uint4 d) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
    uint32_t h[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], 1.0f, false));
      h[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], 1.0f, true));
    }
    uint4* dst = reinterpret_cast<uint4*>(
        &s_v[buf][st_key >> 5][(st_key & (kKeyBlock - 1)) * kExtVStride + 32 * st_c]);
    dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
    dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
  };
  // Transposing read of the PV operand (ds_read_b64_tr_b16): within each
  // 16-lane group, lane 4 j + q names 8 bytes (four f16) and lane i receives
  // element i % 4 of the piece lane 4 j + i / 4 named, for j = 0..3.  Lane i
  // of a group naming key kb + i / 4, dims D0 + 4 (i % 4) .. + 3 thus
  // receives keys kb .. kb + 3 of dim D0 + i.  Lane l's group covers dims
  // 32 d + 16 ((l / 16) % 2) + {0..15} and key offset 4 (l / 32) (its half hf).
  const int tr_off = ((lane & 15) >> 2) * kExtVStride + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  auto tr_read = [&](const uint8_t* blk, int key0, int dim0) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(blk + key0 * kExtVStride + 2 * dim0 + tr_off));
    return __builtin_bit_cast(uint2, r);
  };

  // Per row (both lanes of the row hold the same values): the reference max
  // mref (log2 units; P = 2^(score * scale - mref)) and nm = -mref; `seen`
  // once the reference comes from the row's own keys (before, it is 0 and every
  // block takes the exact path below; padding rows never see a key and keep
  // it).  Per lane: the output accumulators (its row, 16 dims of each 32-dim
  // half) and the sum of the f16 weights of its keys.
  float mref = 0.0f, nm = 0.0f, lpart = 0.0f;
  bool seen = !valid;
  v16f acc[2] = {};
  const v2h ones2 = {1.0f16, 1.0f16};

  // One 32-key block of the wave's key group from stage buffer buf, as 32 x 32
  // matrix-core tiles: QK^T on one v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3,
  // unit scales), PV on four v_mfma_f32_32x32x16_f16.  Lane l's scores are
  // row l % 32's keys 8 (i / 4) + 4 (l / 32) + i % 4, i = 0..15; its f16
  // weights are directly the PV operand for the key order {0-3, 8-11 | 4-7,
  // 12-15} (and + 16), which the V^T operand follows.
  //
  // Lazy reference: a lane whose 16 weights sum to at most 16 * 2^8 keeps the
  // reference (its weights stay below 2^12, exact enough in f16 and far from
  // overflow) and no maximum is taken.  A larger sum (or a row without a
  // reference yet) sends the wave to the exact path: the row's block maximum,
  // and when it passes the reference by more than the lazy bound (or gives the
  // row its first reference) the reference moves to it and the row's
  // accumulators and sum are rescaled before the weights are formed again.
  auto compute = [&](const int buf, const int blk) {
    const int kbase = lo + blk * kKeyBlock;
    // Interior: every key <= the first row's position (so <= hi) and inside the
    // last real row's window.
    const bool edge = !(kbase + kKeyBlock - 1 <= p_first && (p.window == 0 || kbase >= hi - p.window + 1));
    const uint4* kr = reinterpret_cast<const uint4*>(&s_k[buf][kKeyBlock * kg + n32][32 * hf]);
    const uint4 k0 = kr[0], k1 = kr[1];
    const v8i kA = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
    v16f z = {};
    z = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kA, qB, z, 0, 0, 0, unit_scale, 0, unit_scale);
    // Causal and window mask of the row, on edge blocks only (an interior
    // block is visible to every real row; padding rows are never stored).
    if (edge) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + 8 * (i >> 2) + 4 * hf + (i & 3);
        z[i] = (key <= prow && key >= plo) ? z[i] : -INFINITY;
      }
    }
    v8h pv[2];
    float bs;
    auto weights = [&]() {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pv[i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(z[i], scale, nm));
      bs = 0.0f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bs = __builtin_amdgcn_fdot2(v2h{pv[kh][2 * i], pv[kh][2 * i + 1]}, ones2, bs, false);
    };
    weights();
    // The K operand stays live past the product (to here, after its result is
    // read): a 16-pass MFMA must not write registers it is still reading, and
    // the allocator would otherwise give the result kA's registers (the zero
    // accumulator being an inline constant).
    asm volatile("" ::"v"(kA), "v"(bs));
    if (__any(!(bs <= 16.0f * (float)(1 << (int)kLazyRescale)) || !seen)) {
      float m = fmax3(fmax3(z[0], z[1], z[2]), fmax3(z[3], z[4], z[5]), fmax3(z[6], z[7], z[8]));
      m = fmax3(m, fmax3(z[9], z[10], z[11]), fmax3(z[12], z[13], z[14]));
      m = __builtin_elementwise_maximum(m, z[15]);
      m = __builtin_elementwise_maximum(m, __shfl_xor(m, 32)) * scale;  // the row's other half
      const bool mv = m > -INFINITY && (m - mref > kLazyRescale || !seen);
      const float sh = mv ? m - mref : 0.0f;
      mref += sh;
      nm = -mref;
      seen = seen || mv;
      const float alpha = __builtin_amdgcn_exp2f(-sh);
      lpart *= alpha;
#pragma unroll
      for (int d = 0; d < 2; ++d) acc[d] *= alpha;
      weights();
    }
    lpart += bs;
    // V^T operand of dims 32 d + l % 32: keys 16 kh + 4 (l / 32) + {0..3} and
    // 16 kh + 8 + 4 (l / 32) + {0..3}, one transposing read each.
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const uint2 a0 = tr_read(s_v[buf][kg], 16 * kh + 4 * hf, 32 * d);
        const uint2 a1 = tr_read(s_v[buf][kg], 16 * kh + 8 + 4 * hf, 32 * d);
        const v8h va = __builtin_bit_cast(v8h, make_uint4(a0.x, a0.y, a1.x, a1.y));
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pv[kh], acc[d], 0, 0, 0);
      }
    }
  };

  // Loads run two stages ahead of the compute (a gather's latency exceeds one
  // stage's compute), page-table entries two stages ahead of the loads; the
  // two register sets alternate, so each wait is for the oldest load only.
  // Primed unconditionally and in the loop's own issue order (data, entry,
  // data, entry), so the compiler's wait counts at the loop head stay exact.
  const int last = max(n_stage - 1, 0);
  const int e0 = st_entry(0), e1 = st_entry(min(1, last));
  uint4 dA = st_load(e0, 0);
  int eA = st_entry(min(2, last));
  uint4 dB = st_load(e1, min(1, last));
  int eB = st_entry(min(3, last));
  // The q operands are taken here, once (issued first, they are in by now):
  // a first use inside the loop would make every iteration wait for all loads.
  asm volatile("" ::"v"(qB));

  auto stage_step = [&](const int s, uint4& data, int& e_next) {
    const int buf = s & 1;
    if (st_v)
      stage_v(buf, data);
    else
      *reinterpret_cast<uint4*>(&s_k[buf][st_key][st_c * 16]) = data;
    lds_barrier();  // stage s in LDS; stage s-2's reads of this buffer are behind every wave
    // Unconditional (the last stages reload stage n_stage - 1, in bounds and
    // unused), so the loop has no branch around its loads.
    data = st_load(e_next, min(s + 2, last));
    e_next = st_entry(min(s + 4, last));
    if (2 * (s_first + s) + kg < nblk) compute(buf, 2 * (s_first + s) + kg);
  };
  // Whole stage pairs in the loop (its back edge always follows the second
  // half, so the loads are always in the same order there), an odd last stage
  // after it.
  int s = 0;
  for (; s + 1 < n_stage; s += 2) {
    stage_step(s, dA, eA);
    stage_step(s + 1, dB, eB);
  }
  if (s < n_stage) stage_step(s, dA, eA);

  // Merge: group 1 leaves its rows' raw accumulators and (m, l) in LDS (the
  // staging buffers are free once every wave is past the loop); group 0 adds
  // them at a common reference max and leaves o / l (times the V descale when
  // the unit is whole) and its (m, l).  A row's sum is its two lanes' parts;
  // lane l holds dims 32 d + 8 (i / 4) + 4 (l / 32) + {0..3} of row l % 32.
  const float l_own = lpart + __shfl_xor(lpart, 32);
  // A row without a reference of its own has no weight (l = 0, max -inf).
  const float mrow = seen ? mref : -INFINITY;
  const int rr = 32 * wq + n32;
  lds_barrier();
  if (kg == 1) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(&s_o[rr][32 * d + 8 * i4 + 4 * hf]) =
            make_float4(acc[d][4 * i4], acc[d][4 * i4 + 1], acc[d][4 * i4 + 2], acc[d][4 * i4 + 3]);
    if (hf == 0) s_ml[rr] = make_float2(mrow, l_own);
  }
  lds_barrier();
  if (kg == 0) {
    const float2 ml = s_ml[rr];
    const float mt = fmaxf(mrow, ml.x);
    const float mc = mt == -INFINITY ? 0.0f : mt;
    const float a0 = __builtin_amdgcn_exp2f(mrow - mc), a1 = __builtin_amdgcn_exp2f(ml.x - mc);
    const float l = l_own * a0 + ml.y * a1;
    const float inv = l > 0.0f ? (S == 1 ? vs : 1.0f) * __builtin_amdgcn_rcpf(l) : 0.0f;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4* o = reinterpret_cast<float4*>(&s_o[rr][32 * d + 8 * i4 + 4 * hf]);
        const float4 u = *o;
        *o = make_float4((acc[d][4 * i4] * a0 + u.x * a1) * inv, (acc[d][4 * i4 + 1] * a0 + u.y * a1) * inv,
                         (acc[d][4 * i4 + 2] * a0 + u.z * a1) * inv, (acc[d][4 * i4 + 3] * a0 + u.w * a1) * inv);
      }
    // Both lanes of the row have read s_ml[rr] (one wave, in order) before this.
    if (hf == 0) s_ml[rr] = make_float2(mt, l);
  }
  lds_barrier();

  // Key splits: publish this split's rows (o / l in f16, a weighted mean of V
  // codes; m and l in fp32) with device-coherent stores; the last split of the
  // unit (an atomic counter per unit) merges them all, as the decode step's
  // combine does, and runs the epilogue.
  if (S > 1) {
    __shared__ int s_last;
    const int r = tid >> 2, d0 = (tid & 3) * 16;  // 4 threads per row, 16 columns each
    const int64_t prow = ((int64_t)unit * S + ks) * kExtRows + r;
    {
      const float4* o = reinterpret_cast<const float4*>(&s_o[r][d0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = o[c];
        store_coherent_h4(p.part_o + prow * kHeadDim + d0 + 4 * c, v.x, v.y, v.z, v.w);
      }
      if ((tid & 3) == 0) store_coherent(p.part_ml + prow * 2, s_ml[r].x, s_ml[r].y);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
    __syncthreads();
    int32_t* counter = p.counters + unit;
    if (tid == 0) s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (!s_last) return;
    // Eight splits' loads are issued together, then merged at a running max.
    constexpr int KB = 8;
    const int64_t prow0 = (int64_t)unit * S * kExtRows + r;
    float mrun = -INFINITY, lt = 0.0f, o[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] = 0.0f;
    for (int q0 = 0; q0 < S; q0 += KB) {
      float2 ml[KB];
      uint2 oh[KB][4];
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        const int64_t pr = prow0 + (int64_t)min(q0 + q, S - 1) * kExtRows;
        ml[q] = load_coherent(p.part_ml + pr * 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) oh[q][c] = load_coherent_h4(p.part_o + pr * kHeadDim + d0 + 4 * c);
        if (q0 + q >= S) ml[q] = make_float2(-INFINITY, 0.0f);  // past the last split: no weight
      }
      float mc = mrun;
#pragma unroll
      for (int q = 0; q < KB; ++q) mc = fmaxf(mc, ml[q].x);
      const float mref = mc == -INFINITY ? 0.0f : mc;
      const float a = __builtin_amdgcn_exp2f(mrun - mref);
      lt *= a;
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c] *= a;
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        const float w = __builtin_amdgcn_exp2f(ml[q].x - mref) * ml[q].y;  // the split's weight
        lt += w;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          o[4 * c + 0] += w * h_lo(oh[q][c].x);
          o[4 * c + 1] += w * h_hi(oh[q][c].x);
          o[4 * c + 2] += w * h_lo(oh[q][c].y);
          o[4 * c + 3] += w * h_hi(oh[q][c].y);
        }
      }
      mrun = mc;
    }
    const float inv = lt > 0.0f ? vs * __builtin_amdgcn_rcpf(lt) : 0.0f;
    float4* so = reinterpret_cast<float4*>(&s_o[r][d0]);
#pragma unroll
    for (int c = 0; c < 4; ++c) so[c] = make_float4(o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv, o[4 * c + 3] * inv);
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // re-armed
    lds_barrier();
  }
  // Gated epilogue: 16 threads per row, 4 columns each, 32 rows per pass.
  const int c4 = (tid & 15) * 4;
#pragma unroll
  for (int pass = 0; pass < kExtRows / (4 * kExtWaves); ++pass) {
    const int r = pass * (4 * kExtWaves) + (tid >> 4);
    const int ti = r >> 3, h = kGroup * g + (r & 7);
    const bool valid = ti < n_tok;
    const int64_t tok = tok0 + min(ti, n_tok - 1);
    const uint2 graw = *reinterpret_cast<const uint2*>(p.qkv + tok * kWidth + kGateOffset + h * kHeadDim + c4);
    const float4 o = *reinterpret_cast<const float4*>(&s_o[r][c4]);
    float y[4] = {round_bf16(o.x), round_bf16(o.y), round_bf16(o.z), round_bf16(o.w)};
    float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
    ss = sum16(ss);
    const float rr = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + 1.0e-5f);
    const float gate[4] = {bf16_value(graw.x & 0xffffu), bf16_value(graw.x >> 16),
                           bf16_value(graw.y & 0xffffu), bf16_value(graw.y >> 16)};
    uint32_t ob[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ob[c] = bf16_bits(y[c] * rr * __builtin_amdgcn_rcpf(1.0f + __expf(-gate[c])));
    if (valid)
      *reinterpret_cast<uint2*>(p.out + tok * (kQHeads * kHeadDim) + h * kHeadDim + c4) =
          make_uint2(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16));
  }
}

}  // namespace

hipError_t launch_extend_prologue(const StepParams& p, hipStream_t stream) {
  if (p.total_q <= 0) return hipSuccess;
  const unsigned pro_grid = (unsigned)((p.total_q + kExtPrologueTokens - 1) / kExtPrologueTokens);
  hipLaunchKernelGGL(extend_prologue_kernel, dim3(pro_grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_extend(const StepParams& p, hipStream_t stream, hipEvent_t attn_start) {
  if (p.batch == 0) return hipSuccess;
  if (p.sparse_block > 0 || p.q_len <= kMaxQLen || p.q_len > kMaxExtendLen ||
      p.total_q < 0 || p.total_q > (int64_t)p.batch * p.q_len)
    return hipErrorInvalidValue;
  if (p.total_q == 0) return hipSuccess;  // a ragged batch without new tokens
  const unsigned tokens = (unsigned)p.total_q;
  const unsigned pro_grid = (tokens + kExtPrologueTokens - 1) / kExtPrologueTokens;
  hipLaunchKernelGGL(extend_prologue_kernel, dim3(pro_grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && attn_start) e = hipEventRecord(attn_start, stream);
  if (e != hipSuccess) return e;
  if (p.splits < 1) return hipErrorInvalidValue;
  const unsigned units = (unsigned)p.batch * kKvHeads * (unsigned)((p.q_len + kExtTile - 1) / kExtTile);
  const unsigned wgs = units * (unsigned)p.splits;
  const unsigned grid = (wgs + kXcds - 1) / kXcds * kXcds;  // the kernel's XCD-aware order
  hipLaunchKernelGGL(extend_attn_kernel, dim3(grid), dim3(64 * kExtWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mi355x_ga
