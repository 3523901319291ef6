// api.cpp -- the C ABI declared in include/mi355x_gated_attn.h: validation,
// the split-KV plan, the workspace layout, the launch of a step and the
// optional timing hook.
//
// The plan replaces the page's FA3 scheduler metadata and its H200 split
// heuristic max(1, min(16, cdiv(132, B*Hkv))) ("012-attention-local-splits.py",
// kernel_fn): on gfx950 a work unit covers both KV heads of a request (every
// 128-byte cache row is used whole), so the split count is chosen from the
// batch and the key bound against 256 compute units.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mi355x_gated_attn.h"
#include "kernels.h"

using namespace mi355x_ga;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MI355X_GA_OK;
}

constexpr int kComputeUnits = 256;   // MI355X: 8 XCDs x 32 CUs; the plan aims at one unit per CU
constexpr int kMaxSplits = 256;
constexpr int64_t kPartialRowBytes = kHeadDim * 2 + 8;  // f16 o / l + fp32 (m, l)
constexpr int64_t kSepCombineBytes = 32 << 10;
constexpr int64_t kShortKeys = 4096;  // key ranges up to this: pairs (L <= 4), one KV head per wave

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }


}  // namespace

struct mi355x_gated_attn_ctx {
  mi355x_gated_attn_config cfg;
  int device;
  float inv_freq[kHeadDim / 2];
  bool planned = false;
  int32_t splits = 0;
  int32_t groups = 1;  // token groups per request
  bool head_split = false;
  int32_t key_waves = kAttnWaves;
  bool balanced = false;  // splits per request by key count
  bool sep_combine = false;  // partials merged by a second launch
  size_t q_bytes = 0, po_off = 0, pml_off = 0, cnt_off = 0, ws_bytes = 0;
  size_t po_bytes = 0, pml_bytes = 0;  // partial o / l and (m, l) region sizes
  int64_t n_counters = 0;              // int32 counters (B x groups)
  bool timing = false;
  std::vector<hipEvent_t> events;  // 2 per timed step, reused
  size_t events_used = 0;
};

namespace {

int check_workspace(const mi355x_gated_attn_ctx* ctx, const void* workspace, size_t bytes) {
  if (!workspace) return fail(MI355X_GA_INVALID_ARGUMENT, "workspace is NULL");
  if (bytes < ctx->ws_bytes)
    return fail(MI355X_GA_WORKSPACE_TOO_SMALL, "workspace %zu bytes < planned %zu", bytes,
                ctx->ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MI355X_GA_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  return MI355X_GA_OK;
}

int check_device(const mi355x_gated_attn_ctx* ctx) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device)
    return fail(MI355X_GA_INVALID_ARGUMENT, "current device %d is not the ctx device %d", cur,
                ctx->device);
  return MI355X_GA_OK;
}

}  // namespace

extern "C" {

const char* mi355x_gated_attn_last_error(void) { return g_last_error.c_str(); }

int mi355x_gated_attn_supports(const mi355x_gated_attn_config* c) {
  if (!c) return fail(MI355X_GA_INVALID_ARGUMENT, "config is NULL");
  if (c->batch < 0) return fail(MI355X_GA_INVALID_ARGUMENT, "batch %d < 0", c->batch);
  if (c->q_len < 1) return fail(MI355X_GA_INVALID_ARGUMENT, "q_len %d < 1", c->q_len);
  if (c->num_q_heads < 1 || c->num_kv_heads < 1 || c->head_dim < 1)
    return fail(MI355X_GA_INVALID_ARGUMENT, "head counts and head_dim must be positive");
  if (c->page_size < 1) return fail(MI355X_GA_INVALID_ARGUMENT, "page_size %d < 1", c->page_size);
  if (c->window < 0) return fail(MI355X_GA_INVALID_ARGUMENT, "window %d < 0", c->window);
  if (c->max_pages < 1) return fail(MI355X_GA_INVALID_ARGUMENT, "max_pages %d < 1", c->max_pages);
  if (c->num_pages < 1) return fail(MI355X_GA_INVALID_ARGUMENT, "num_pages < 1");
  if (!(c->rope_theta >= 0.0f) || std::isinf(c->rope_theta))
    return fail(MI355X_GA_INVALID_ARGUMENT, "rope_theta must be 0 or a finite positive value");
  if (!(c->sm_scale > 0.0f) || std::isinf(c->sm_scale))
    return fail(MI355X_GA_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  if (!(c->kv_scale > 0.0f) || std::isinf(c->kv_scale))
    return fail(MI355X_GA_INVALID_ARGUMENT, "kv_scale must be finite and positive");
  if (!(c->q_scale > 0.0f) || std::isinf(c->q_scale))
    return fail(MI355X_GA_INVALID_ARGUMENT, "q_scale must be finite and positive (1: none)");
  if (c->sparse_block < 0 || c->sparse_topk < 0)
    return fail(MI355X_GA_INVALID_ARGUMENT, "sparse_block and sparse_topk must be >= 0");
  if (c->sparse_block > 0) {
    if (c->sparse_topk < 1) return fail(MI355X_GA_INVALID_ARGUMENT, "sparse_topk must be >= 1");
    if (c->sparse_block % kKeyBlock)
      return fail(MI355X_GA_UNSUPPORTED, "sparse_block %d: this build serves multiples of %d",
                  c->sparse_block, kKeyBlock);
    if (c->sparse_topk > kMaxSparseTopk)
      return fail(MI355X_GA_UNSUPPORTED, "sparse_topk %d: this build serves up to %d", c->sparse_topk,
                  kMaxSparseTopk);
    if (c->q_len != 1 || c->window != 0)
      return fail(MI355X_GA_UNSUPPORTED, "page-list-driven decode serves q_len 1 without a window");
    if ((int64_t)c->sparse_block * c->sparse_topk > (int64_t)1 << 30)
      return fail(MI355X_GA_UNSUPPORTED, "sparse_block * sparse_topk exceeds 2^30 keys");
  }
  if (c->num_q_heads % c->num_kv_heads)
    return fail(MI355X_GA_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d",
                c->num_q_heads, c->num_kv_heads);
  if (c->head_dim != kHeadDim)
    return fail(MI355X_GA_UNSUPPORTED, "head_dim %d: this build serves %d", c->head_dim, kHeadDim);
  if (c->num_q_heads != kQHeads || c->num_kv_heads != kKvHeads)
    return fail(MI355X_GA_UNSUPPORTED, "heads %d/%d: this build serves %d query / %d KV heads",
                c->num_q_heads, c->num_kv_heads, kQHeads, kKvHeads);
  if (c->q_len > kMaxExtendLen)
    return fail(MI355X_GA_UNSUPPORTED, "q_len %d: this build serves 1..%d", c->q_len, kMaxExtendLen);
  if (c->q_len > kMaxQLen && (int64_t)c->batch * c->q_len > (int64_t)INT32_MAX)
    return fail(MI355X_GA_UNSUPPORTED, "extend: batch * q_len exceeds one launch's 2^31 - 1 workgroups");
  if ((int64_t)c->max_pages * c->page_size > (int64_t)1 << 30)
    return fail(MI355X_GA_UNSUPPORTED, "max_pages * page_size exceeds 2^30 keys per request");
  if (c->num_pages * (int64_t)c->page_size >= (int64_t)1 << 31)
    return fail(MI355X_GA_UNSUPPORTED, "num_pages * page_size exceeds 2^31 - 1 cache rows");
  return ok();
}

int mi355x_gated_attn_prepare(const mi355x_gated_attn_config* cfg, int device,
                              mi355x_gated_attn_ctx** out_ctx) {
  if (!out_ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "out_ctx is NULL");
  *out_ctx = nullptr;
  int rc = mi355x_gated_attn_supports(cfg);
  if (rc) return rc;
  if (device < 0) return fail(MI355X_GA_INVALID_ARGUMENT, "device %d < 0", device);
  auto* ctx = new (std::nothrow) mi355x_gated_attn_ctx();
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "out of host memory");
  ctx->cfg = *cfg;
  ctx->device = device;
  // inv_freq[i] = 1 / theta^(2i/D): the exponent is exact in fp32, the power is
  // rounded once to fp32, then the fp32 reciprocal (the page's fp32 recipe).
  for (int i = 0; i < kHeadDim / 2; ++i) {
    ctx->inv_freq[i] = 0.0f;
    if (cfg->rope_theta != 0.0f) {
      const float ex = (float)(2 * i) / (float)kHeadDim;
      const float pw = (float)std::pow((double)cfg->rope_theta, (double)ex);
      ctx->inv_freq[i] = 1.0f / pw;
    }
  }
  *out_ctx = ctx;
  return ok();
}

int mi355x_gated_attn_plan(mi355x_gated_attn_ctx* ctx, int32_t max_context, int32_t num_splits,
                           size_t* workspace_bytes, int32_t* num_splits_out) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  if (max_context < 0) return fail(MI355X_GA_INVALID_ARGUMENT, "max_context %d < 0", max_context);
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(MI355X_GA_INVALID_ARGUMENT, "num_splits %d outside 0..%d", num_splits, kMaxSplits);
  const auto& c = ctx->cfg;
  const size_t T = (size_t)c.batch * c.q_len;
  if (c.q_len > kMaxQLen) {
    // Extend / prefill: a unit per (request, 16-token tile, KV head) walks its
    // key range in 64-key stages.  Units that fill the chip need no split;
    // fewer units split their stages S ways (a workgroup per CU, at least four
    // stages per split, at most 32 splits: the last split of each unit merges
    // the others' partials, and that merge grows with S).  Measured (B = 4,
    // L = 16, 32k keys, 8 units): S = 1 410 us, 8 70.5, 16 51.1, 32 49.0,
    // 64 65.9.  The workspace holds q, the partials (S > 1) and one counter
    // per unit.
    const int64_t tiles = (c.q_len + 15) / 16;
    const int64_t units = (int64_t)c.batch * kKvHeads * tiles;
    int64_t keys = max_context;
    if (c.window > 0) keys = std::min<int64_t>(keys, (int64_t)c.window + c.q_len - 1);
    int32_t s = num_splits;
    if (s == 0) {
      const int64_t stages = std::max<int64_t>(1, (keys + 63) / 64);
      const int64_t target = kComputeUnits;
      const int64_t by_batch = units > 0 ? (target + units - 1) / units : 1;
      s = (int32_t)std::max<int64_t>(1, std::min<int64_t>({by_batch, stages / 4, (int64_t)32}));
    }
    if (units * s + 7 > (int64_t)INT32_MAX)
      return fail(MI355X_GA_UNSUPPORTED, "batch %d x %lld tiles x %d splits exceeds one launch's workgroups",
                  c.batch, (long long)tiles, s);
    const size_t rows = (size_t)units * 128;  // (tile token, q head) rows of every unit
    ctx->q_bytes = T * kQHeads * kHeadDim;
    ctx->po_bytes = s > 1 ? (size_t)s * rows * kHeadDim * sizeof(uint16_t) : 0;
    ctx->pml_bytes = s > 1 ? (size_t)s * rows * 2 * sizeof(float) : 0;
    ctx->n_counters = units;
    ctx->po_off = align_up(ctx->q_bytes, 256);
    ctx->pml_off = align_up(ctx->po_off + ctx->po_bytes, 256);
    ctx->cnt_off = align_up(ctx->pml_off + ctx->pml_bytes, 256);
    ctx->ws_bytes = align_up(ctx->cnt_off + (size_t)units * sizeof(int32_t), 256);
    if (ctx->ws_bytes == 0) ctx->ws_bytes = 256;
    ctx->splits = s;
    ctx->groups = (int32_t)(kKvHeads * tiles);  // counters per request (workspace_init clears B x groups)
    ctx->head_split = false;
    ctx->key_waves = kAttnWaves;
    ctx->balanced = false;
    ctx->planned = true;
    if (workspace_bytes) *workspace_bytes = ctx->ws_bytes;
    if (num_splits_out) *num_splits_out = s;
    return ok();
  }
  const bool sparse = c.sparse_block > 0;
  int64_t keys = max_context;  // union of a request's visible keys
  if (c.window > 0) keys = std::min<int64_t>(keys, (int64_t)c.window + c.q_len - 1);
  // Page-list-driven decode walks topk * block_size list positions per KV head.
  if (sparse) keys = (int64_t)c.sparse_topk * c.sparse_block;
  // Token groups: a unit's prologue (q of its tokens, every unit of a group
  // computing the same) grows with its tokens and each group walks the keys
  // again (the combine is spread over the splits, one token per combining
  // unit, whatever the grouping).  Over a sliding window (B = 32, L = 8,
  // W = 2048) two groups of four at S = 4 take 19.1 us, four pairs at S = 2
  // 19.45, one group of eight at S = 8 20.0 (its prologue alone 5 us); over
  // long ranges the key loop dominates and one group reads every key once
  // (B = 8, L = 8, 64k-128k keys, balanced: one group of eight at S = 32,
  // 75.0 us; two groups of four at S = 16, 83.2; four pairs, 116).  Pairs keep
  // L <= 4 over short ranges.
  const bool short_keys = keys <= kShortKeys;
  const int groups = token_groups(c.q_len, short_keys);
  const int unit_size = unit_tokens(c.q_len, groups);
  // Eight waves per unit (one KV head each, two waves per SIMD) pay where the
  // key loop is short and compute-heavy (q_len > 1 over a short key range:
  // 19.2 against 20.7 us at B = 32, L = 8, W = 2048), and a unit of a whole
  // verify block needs them (its rows would not fit the registers of four
  // waves).  Elsewhere the two halves of a cache row, fetched by different
  // waves, cost HBM efficiency (B = 64, L = 1, 32k keys: 160 against 113 us;
  // B = 32, L = 1, W = 2048: 13.0 against 12.5 us), so four waves keep both
  // heads.
  // (Page-list-driven decode: each KV head has its own list, so one head per wave.)
  const bool head_split = sparse || (short_keys && c.q_len > 1) || unit_size == kMaxQLen;
  // Decode over long key ranges keeps more K/V blocks in flight with eight
  // waves per unit, both heads each (B = 64, 32k keys: 106 against 113 us); over
  // a window the extra merge and barrier cost more (B = 32, W = 2048: 15.7
  // against 12.5 us).
  const int key_waves = (!sparse && c.q_len == 1 && keys > kShortKeys) ? 2 * kAttnWaves : kAttnWaves;
  int32_t s = num_splits;
  if (s == 0) {
    const int64_t min_keys_per_split = (int64_t)key_waves * kKeyBlock;  // a block per wave
    const int64_t by_len = std::max<int64_t>(1, (keys + min_keys_per_split - 1) / min_keys_per_split);
    const int64_t target = kComputeUnits;
    const int64_t units = (int64_t)c.batch * groups;  // units per split
    const int64_t by_batch = units > 0 ? (target + units - 1) / units : 1;
    s = (int32_t)std::max<int64_t>(1, std::min<int64_t>({by_len, by_batch, (int64_t)kMaxSplits}));
  }
  if ((int64_t)c.batch * groups * s > (int64_t)INT32_MAX)
    return fail(MI355X_GA_UNSUPPORTED, "batch %d x %d splits exceeds one launch's workgroups", c.batch, s);
  const size_t rows = T * kQHeads;  // (token, q head) rows
  ctx->q_bytes = T * kQHeads * kHeadDim;
  ctx->po_bytes = (size_t)s * rows * kHeadDim * sizeof(uint16_t);
  ctx->pml_bytes = (size_t)s * rows * 2 * sizeof(float);
  ctx->n_counters = (int64_t)c.batch * groups;
  ctx->po_off = align_up(ctx->q_bytes, 256);
  ctx->pml_off = align_up(ctx->po_off + ctx->po_bytes, 256);
  ctx->cnt_off = align_up(ctx->pml_off + ctx->pml_bytes, 256);
  ctx->ws_bytes = align_up(ctx->cnt_off + (size_t)c.batch * groups * sizeof(int32_t), 256);
  if (ctx->ws_bytes == 0) ctx->ws_bytes = 256;
  ctx->splits = s;
  ctx->groups = groups;
  ctx->head_split = head_split;
  ctx->key_waves = key_waves;
  // Without a window, requests' key counts differ as their lengths do, and the
  // uniform S splits each leave the step as long as its longest request; the
  // kernel then deals the B * S units out in proportion to each request's keys
  // (every unit reads the batch's cached lengths, one per lane: B <= 64; the
  // units with both KV heads per wave, and those of a whole verify block).
  // Measured (B = 8, L = 8, 64k-128k keys, two groups of four, S = 16): 94.1
  // against 84.6 us per step.
  ctx->balanced = !sparse && (!head_split || unit_size == kMaxQLen) && c.window == 0 && c.batch > 1 &&
                  c.batch <= 64 && s > 1;
  // Token t of a request-group is merged by split t mod S, which reads the
  // other splits' (S - 1) * 16 partial rows of 136 bytes per token it merges
  // through one compute unit with device-coherent loads; beyond
  // kSepCombineBytes per unit a second launch merges them over the whole chip
  // with plain loads instead (one more launch, ~1.6 us).
  const int64_t lu = tokens_per_unit(c.q_len, groups);
  const int64_t merged_per_unit = (lu + s - 1) / s;  // tokens a combining unit merges
  ctx->sep_combine =
      s > 1 && (int64_t)(s - 1) * merged_per_unit * kQHeads * kPartialRowBytes > kSepCombineBytes;
  ctx->planned = true;
  if (workspace_bytes) *workspace_bytes = ctx->ws_bytes;
  if (num_splits_out) *num_splits_out = s;
  return ok();
}

int mi355x_gated_attn_workspace_init(mi355x_gated_attn_ctx* ctx, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  if (!ctx->planned) return fail(MI355X_GA_INVALID_ARGUMENT, "workspace_init before plan");
  if (ctx->cfg.batch == 0) return ok();
  int rc = check_workspace(ctx, workspace, workspace_bytes);
  if (rc) return rc;
  rc = check_device(ctx);
  if (rc) return rc;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_zero_counters(reinterpret_cast<int32_t*>(ws + ctx->cnt_off),
                                      (int)ctx->n_counters, st);
  // The decode step's partial slots start empty (every word the sentinel).
  if (e == hipSuccess && ctx->cfg.q_len <= kMaxQLen)
    e = launch_fill_sentinel(ws + ctx->po_off, ctx->pml_off + ctx->pml_bytes - ctx->po_off, st);
  if (e != hipSuccess) return fail(MI355X_GA_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int mi355x_gated_attn_step_meta(mi355x_gated_attn_ctx* ctx, const int32_t* seq_lens,
                                const int32_t* page_table, int64_t* positions, int64_t* cache_loc,
                                int32_t* cache_seqlens, void* stream) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  const auto& c = ctx->cfg;
  if (c.batch == 0) return ok();
  if (!seq_lens || !page_table || !positions || !cache_loc || !cache_seqlens)
    return fail(MI355X_GA_INVALID_ARGUMENT, "a required pointer is NULL");
  int rc = check_device(ctx);
  if (rc) return rc;
  MetaParams m{};
  m.seq_lens = seq_lens;
  m.page_table = page_table;
  m.positions = positions;
  m.cache_loc = cache_loc;
  m.cache_seqlens = cache_seqlens;
  m.batch = c.batch;
  m.q_len = c.q_len;
  m.max_pages = c.max_pages;
  m.page_size = c.page_size;
  m.page_shift = (c.page_size & (c.page_size - 1)) == 0 ? __builtin_ctz((unsigned)c.page_size) : -1;
  const hipError_t e = launch_step_meta(m, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI355X_GA_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int mi355x_gated_attn_page_table(mi355x_gated_attn_ctx* ctx, const int32_t* req_to_token,
                                 int64_t req_stride, int64_t max_reqs, const int32_t* slot_ids,
                                 const int32_t* kv_lens, int32_t* page_table, int32_t* kv_indices,
                                 int32_t* kv_indptr, void* stream) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  const auto& c = ctx->cfg;
  if (c.batch == 0) return ok();
  if (!req_to_token || !slot_ids || !kv_lens)
    return fail(MI355X_GA_INVALID_ARGUMENT, "req_to_token, slot_ids and kv_lens are required");
  if (!page_table && !kv_indices)
    return fail(MI355X_GA_INVALID_ARGUMENT, "neither page_table nor kv_indices is given");
  if (kv_indices && !kv_indptr)
    return fail(MI355X_GA_INVALID_ARGUMENT, "kv_indices needs kv_indptr");
  if (req_stride < 1 || max_reqs < 1)
    return fail(MI355X_GA_INVALID_ARGUMENT, "req_stride and max_reqs must be >= 1");
  int rc = check_device(ctx);
  if (rc) return rc;
  PageTableParams q{};
  q.req_to_token = req_to_token;
  q.req_stride = req_stride;
  q.max_reqs = max_reqs;
  q.slot_ids = slot_ids;
  q.kv_lens = kv_lens;
  q.batch = c.batch;
  q.page_size = c.page_size;
  q.page_shift = (c.page_size & (c.page_size - 1)) == 0 ? __builtin_ctz((unsigned)c.page_size) : -1;
  q.max_pages = c.max_pages;
  q.page_table = page_table;
  q.kv_indices = kv_indices;
  q.kv_indptr = kv_indices ? kv_indptr : nullptr;
  const hipError_t e = launch_page_table(q, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI355X_GA_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Where a step keeps q, the split partials and the counters: the caller's
// workspace (at the plan's offsets) or the library's static scratch.
struct Regions {
  uint8_t* q = nullptr;
  uint8_t* po = nullptr;
  uint8_t* pml = nullptr;
  int32_t* counters = nullptr;
};

Regions workspace_regions(const mi355x_gated_attn_ctx* ctx, void* workspace) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  Regions r;
  r.q = ws;
  r.po = ws + ctx->po_off;
  r.pml = ws + ctx->pml_off;
  r.counters = reinterpret_cast<int32_t*>(ws + ctx->cnt_off);
  return r;
}

int run_step(mi355x_gated_attn_ctx* ctx, const void* qkv, const int64_t* positions,
             const int64_t* cache_loc, const int32_t* cache_seqlens, const int32_t* page_table,
             const int32_t* block_idx, void* k_cache, void* v_cache, const float* k_scale,
             const float* v_scale, void* out, void* workspace, size_t workspace_bytes, void* stream,
             const int32_t* cu_seqlens_q = nullptr, int64_t total_q = -1,
             const int32_t* token_req = nullptr, int32_t pt_rows = 0,
             const Regions* fixed = nullptr) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  if (!ctx->planned) return fail(MI355X_GA_INVALID_ARGUMENT, "step before plan");
  const auto& c = ctx->cfg;
  if (c.batch == 0) return ok();
  if ((c.sparse_block > 0) != (block_idx != nullptr))
    return fail(MI355X_GA_INVALID_ARGUMENT,
                c.sparse_block > 0 ? "a page-list-driven config needs block_idx (sparse_step)"
                                   : "block_idx given for a dense config (use step)");
  if (c.batch == 0) return ok();
  const bool scaled = c.kv_scale != 1.0f;
  const bool rope = c.rope_theta != 0.0f;
  if (!qkv || !cache_loc || !cache_seqlens || !page_table || !k_cache || !v_cache || !out ||
      (!fixed && !workspace))
    return fail(MI355X_GA_INVALID_ARGUMENT, "a required pointer is NULL");
  if (rope && !positions) return fail(MI355X_GA_INVALID_ARGUMENT, "positions is NULL with RoPE on");
  if (scaled && (!k_scale || !v_scale))
    return fail(MI355X_GA_INVALID_ARGUMENT, "k_scale/v_scale are NULL on the scaled path");
  int rc = fixed ? MI355X_GA_OK : check_workspace(ctx, workspace, workspace_bytes);
  if (rc) return rc;
  if (reinterpret_cast<uintptr_t>(qkv) % 16 || reinterpret_cast<uintptr_t>(k_cache) % 16 ||
      reinterpret_cast<uintptr_t>(v_cache) % 16 || reinterpret_cast<uintptr_t>(out) % 8)
    return fail(MI355X_GA_INVALID_ARGUMENT, "qkv/cache/out pointers are misaligned");
  rc = check_device(ctx);
  if (rc) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Regions reg = fixed ? *fixed : workspace_regions(ctx, workspace);

  StepParams sp{};
  sp.qkv = reinterpret_cast<const uint16_t*>(qkv);
  sp.positions = positions;
  sp.cache_loc = cache_loc;
  sp.cache_seqlens = cache_seqlens;
  sp.page_table = page_table;
  sp.k_cache = reinterpret_cast<uint8_t*>(k_cache);
  sp.v_cache = reinterpret_cast<uint8_t*>(v_cache);
  sp.k_scale = k_scale;
  sp.v_scale = v_scale;
  sp.out = reinterpret_cast<uint16_t*>(out);
  sp.q_out = reg.q;
  sp.part_o = reinterpret_cast<_Float16*>(reg.po);
  sp.part_ml = reinterpret_cast<float*>(reg.pml);
  sp.counters = reg.counters;
  sp.num_pages = c.num_pages;
  sp.num_rows = c.num_pages * (int64_t)c.page_size;
  sp.batch = c.batch;
  sp.q_len = c.q_len;
  sp.tgroups = ctx->groups;
  sp.splits = ctx->splits;
  sp.balanced = ctx->balanced ? 1 : 0;
  sp.head_split = ctx->head_split ? 1 : 0;
  sp.key_waves = ctx->key_waves;
  sp.sep_combine = ctx->sep_combine ? 1 : 0;
  sp.max_pages = c.max_pages;
  sp.page_size = c.page_size;
  sp.page_shift = (c.page_size & (c.page_size - 1)) == 0 ? __builtin_ctz((unsigned)c.page_size) : -1;
  sp.window = c.window;
  sp.scaled = scaled ? 1 : 0;
  sp.rope = rope ? 1 : 0;
  sp.sm_scale_log2 = c.sm_scale * 1.4426950408889634f;
  sp.q_scale = c.q_scale;
  sp.block_idx = block_idx;
  sp.sparse_block = c.sparse_block;
  sp.sparse_topk = c.sparse_topk;
  sp.sparse_shift = c.sparse_block > 0 && (c.sparse_block & (c.sparse_block - 1)) == 0
                        ? __builtin_ctz((unsigned)c.sparse_block)
                        : -1;
  sp.cu_seqlens_q = cu_seqlens_q;
  sp.total_q = cu_seqlens_q ? total_q : (int64_t)c.batch * c.q_len;
  sp.token_req = token_req;
  sp.pt_rows = pt_rows;
  std::memcpy(sp.inv_freq, ctx->inv_freq, sizeof sp.inv_freq);

  hipEvent_t* ev = nullptr;
  if (ctx->timing && !fixed) {  // the no-allocation entry point creates no events
    if (ctx->events_used + 2 > ctx->events.size()) {
      for (int k = 0; k < 2; ++k) {
        hipEvent_t e;
        // Timing-only events: no system-scope fence (cache write-back and
        // invalidate) when they are recorded, which would stretch the interval.
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
          return fail(MI355X_GA_HIP_ERROR, "hipEventCreate failed");
        ctx->events.push_back(e);
      }
    }
    ev = &ctx->events[ctx->events_used];
    ctx->events_used += 2;
  }
  hipError_t e = hipSuccess;
  // The hook times the attention kernel: the whole step for q_len <= 8, the
  // second launch of an extend step.
  const bool extend = c.q_len > kMaxQLen;
  if (ev && !extend) e = hipEventRecord(ev[0], st);
  // Sparse prefill: every query's K/V row is stored before any query reads
  // the cache (its own row included), as the extend path does.
  if (e == hipSuccess && token_req) e = launch_extend_prologue(sp, st);
  if (e == hipSuccess) e = launch_step(sp, st, ev && extend ? ev[0] : nullptr);
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
  if (e != hipSuccess) return fail(MI355X_GA_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int mi355x_gated_attn_step(mi355x_gated_attn_ctx* ctx, const void* qkv, const int64_t* positions,
                           const int64_t* cache_loc, const int32_t* cache_seqlens,
                           const int32_t* page_table, const int32_t* seq_lens, void* k_cache,
                           void* v_cache, const float* k_scale, const float* v_scale, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  (void)seq_lens;  // the page's attention call takes cache_seqlens only
  return run_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table, nullptr, k_cache,
                  v_cache, k_scale, v_scale, out, workspace, workspace_bytes, stream);
}

int mi355x_gated_attn_ragged_step(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                  const int64_t* positions, const int64_t* cache_loc,
                                  const int32_t* cu_seqlens_q, int64_t total_q,
                                  const int32_t* cache_seqlens, const int32_t* page_table,
                                  void* k_cache, void* v_cache, const float* k_scale,
                                  const float* v_scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  const auto& c = ctx->cfg;
  if (c.batch == 0) return ok();
  if (c.q_len <= kMaxQLen || c.sparse_block > 0)
    return fail(MI355X_GA_INVALID_ARGUMENT,
                "ragged_step needs a dense extend config: q_len (the bound on every segment) > %d",
                kMaxQLen);
  if (!cu_seqlens_q) return fail(MI355X_GA_INVALID_ARGUMENT, "cu_seqlens_q is NULL");
  if (total_q < 0 || total_q > (int64_t)c.batch * c.q_len)
    return fail(MI355X_GA_INVALID_ARGUMENT, "total_q %lld outside 0..batch * q_len = %lld",
                (long long)total_q, (long long)c.batch * c.q_len);
  return run_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table, nullptr, k_cache,
                  v_cache, k_scale, v_scale, out, workspace, workspace_bytes, stream, cu_seqlens_q,
                  total_q);
}

int mi355x_gated_attn_sparse_prefill_step(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                          const int64_t* positions, const int64_t* cache_loc,
                                          const int32_t* token_req, int32_t num_requests,
                                          const int32_t* cache_seqlens, const int32_t* page_table,
                                          const int32_t* block_idx, void* k_cache, void* v_cache,
                                          const float* k_scale, const float* v_scale, void* out,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  const auto& c = ctx->cfg;
  if (c.batch == 0) return ok();
  if (c.sparse_block == 0)
    return fail(MI355X_GA_INVALID_ARGUMENT, "sparse_prefill_step on a dense config (sparse_block 0)");
  if (!token_req || !block_idx)
    return fail(MI355X_GA_INVALID_ARGUMENT, "token_req or block_idx is NULL");
  if (num_requests < 1)
    return fail(MI355X_GA_INVALID_ARGUMENT, "num_requests %d < 1", num_requests);
  return run_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table, block_idx, k_cache,
                  v_cache, k_scale, v_scale, out, workspace, workspace_bytes, stream, nullptr, -1,
                  token_req, num_requests);
}

int mi355x_gated_attn_sparse_step(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                  const int64_t* positions, const int64_t* cache_loc,
                                  const int32_t* cache_seqlens, const int32_t* page_table,
                                  const int32_t* block_idx, void* k_cache, void* v_cache,
                                  const float* k_scale, const float* v_scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (ctx && ctx->cfg.batch > 0 && !block_idx)
    return fail(MI355X_GA_INVALID_ARGUMENT, "block_idx is NULL");
  if (ctx && ctx->cfg.sparse_block == 0)
    return fail(MI355X_GA_INVALID_ARGUMENT, "sparse_step on a dense config (sparse_block 0)");
  return run_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table, block_idx, k_cache,
                  v_cache, k_scale, v_scale, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- The step without allocation: a static scratch array per GPU ----------
// For callers that cannot call hipMalloc (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  `scratch` is this
// module's device global, so every GPU the library runs on holds its own copy,
// at its own address, until the process ends.  Host code never passes the
// array's name to a kernel or a copy: the address hipGetSymbolAddress returns
// on each device is used instead.  Layout: the counters first (zeroed once
// per device; every completed step leaves them at zero again), then the
// decode steps' partial slots (set to the empty-slot sentinel once per
// device; every completed decode step leaves them so again), then the extend
// steps' partials and q, each 256-byte aligned.
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;          // 32 MiB per GPU
constexpr size_t kScratchCounterBytes = size_t(64) << 10;   // 16,384 int32 counters
constexpr size_t kScratchSlotBytes = size_t(8) << 20;       // decode partial slots
constexpr int kMaxScratchDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxScratchDevices];  // device address of `scratch` per device; null until set up

// The calling thread's current device must be `device`.  The first call on a
// device takes the array's address there and zeroes its counters with a
// kernel on `stream` (stream-ordered before the step that follows).
int scratch_on(int device, hipStream_t stream, uint8_t** out) {
  if (device < 0 || device >= kMaxScratchDevices)
    return fail(MI355X_GA_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", device,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MI355X_GA_HIP_ERROR, "hipGetSymbolAddress(scratch) on device %d: %s", device,
                  hipGetErrorString(e));
    hipError_t z = launch_zero_counters(reinterpret_cast<int32_t*>(ptr),
                                        (int)(kScratchCounterBytes / sizeof(int32_t)), stream);
    if (z == hipSuccess)
      z = launch_fill_sentinel(reinterpret_cast<uint8_t*>(ptr) + kScratchCounterBytes, kScratchSlotBytes,
                               stream);
    if (z != hipSuccess)
      return fail(MI355X_GA_HIP_ERROR, "preparing the scratch: %s", hipGetErrorString(z));
    g_scratch[device] = reinterpret_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[device];
  return MI355X_GA_OK;
}

}  // namespace

extern "C" {

int mi355x_gated_attn_step_noalloc(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                   const int64_t* positions, const int64_t* cache_loc,
                                   const int32_t* cache_seqlens, const int32_t* page_table,
                                   const int32_t* seq_lens, void* k_cache, void* v_cache,
                                   const float* k_scale, const float* v_scale, void* out,
                                   void* stream) {
  (void)seq_lens;
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  if (!ctx->planned) return fail(MI355X_GA_INVALID_ARGUMENT, "step before plan");
  if (ctx->cfg.batch == 0) return ok();
  // Partials exchanged within the decode launch live in the sentinel slot
  // region; extend partials and separately combined ones after it.
  const bool decode = ctx->cfg.q_len <= kMaxQLen && !ctx->sep_combine;
  const size_t parts = align_up(ctx->po_bytes, 256) + align_up(ctx->pml_bytes, 256);
  const size_t slot_need = decode ? parts : 0;
  const size_t rest_need = (decode ? 0 : parts) + align_up(ctx->q_bytes, 256);
  const size_t rest_have = kScratchBytes - kScratchCounterBytes - kScratchSlotBytes;
  if ((size_t)ctx->n_counters * sizeof(int32_t) > kScratchCounterBytes || slot_need > kScratchSlotBytes ||
      rest_need > rest_have)
    return fail(MI355X_GA_WORKSPACE_TOO_SMALL,
                "the plan needs %zu bytes of decode partial slots, %zu bytes of other scratch and "
                "%lld counters; the static scratch holds %zu, %zu and %zu (use "
                "mi355x_gated_attn_step with a workspace)",
                slot_need, rest_need, (long long)ctx->n_counters, kScratchSlotBytes, rest_have,
                kScratchCounterBytes / sizeof(int32_t));
  int rc = check_device(ctx);
  if (rc) return rc;
  uint8_t* base = nullptr;
  rc = scratch_on(ctx->device, reinterpret_cast<hipStream_t>(stream), &base);
  if (rc) return rc;
  Regions r;
  r.counters = reinterpret_cast<int32_t*>(base);
  uint8_t* const slots = base + kScratchCounterBytes;
  uint8_t* const rest = slots + kScratchSlotBytes;
  r.po = decode ? slots : rest;
  r.pml = r.po + align_up(ctx->po_bytes, 256);
  r.q = decode ? rest : r.pml + align_up(ctx->pml_bytes, 256);
  return run_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table, nullptr, k_cache,
                  v_cache, k_scale, v_scale, out, nullptr, 0, stream, nullptr, -1, nullptr, 0, &r);
}

void mi355x_gated_attn_destroy(mi355x_gated_attn_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
  delete ctx;
}

int mi355x_gated_attn_timing(mi355x_gated_attn_ctx* ctx, int enable) {
  if (!ctx) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx is NULL");
  ctx->timing = enable != 0;
  if (ctx->timing) ctx->events_used = 0;
  return ok();
}

int mi355x_gated_attn_timing_read(mi355x_gated_attn_ctx* ctx, double* kernel_ms, int64_t* steps) {
  if (!ctx || !kernel_ms) return fail(MI355X_GA_INVALID_ARGUMENT, "ctx or kernel_ms is NULL");
  double acc = 0.0;
  const size_t n = ctx->events_used / 2;
  if (n) {
    if (hipEventSynchronize(ctx->events[ctx->events_used - 1]) != hipSuccess)
      return fail(MI355X_GA_HIP_ERROR, "hipEventSynchronize failed");
  }
  for (size_t i = 0; i < n; ++i) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, ctx->events[2 * i], ctx->events[2 * i + 1]) != hipSuccess)
      return fail(MI355X_GA_HIP_ERROR, "hipEventElapsedTime failed");
    acc += ms;
  }
  *kernel_ms = acc;
  if (steps) *steps = (int64_t)n;
  ctx->events_used = 0;
  return ok();
}

}  // extern "C"

extern "C" int mi355x_qk_norm_supports(int32_t dtype, int32_t head_dim) {
  // The page's launch-shape table gives 8, 16 or 32 threads of eight 16-bit
  // values per head for head_dim up to 64, 128 and 3072, and more threads
  // (never matching) beyond: with no tail path, 64, 128 and 256 are served.
  if (dtype != MI355X_QKN_BF16 && dtype != MI355X_QKN_FP16) return 0;
  return head_dim == 64 || head_dim == 128 || head_dim == 256;
}

extern "C" int mi355x_qk_norm(const void* x, void* out, int64_t M, int32_t num_heads,
                              int32_t head_dim, int64_t x_row_stride, int32_t dtype, float eps,
                              float scale, void* stream) {
  if (!mi355x_qk_norm_supports(dtype, head_dim))
    return fail(MI355X_GA_UNSUPPORTED, "qk_norm serves bf16/fp16 with head_dim 64, 128 or 256 (got dtype %d, head_dim %d)",
                dtype, head_dim);
  if (M < 0) return fail(MI355X_GA_INVALID_ARGUMENT, "M = %lld < 0", (long long)M);
  if (num_heads < 1) return fail(MI355X_GA_INVALID_ARGUMENT, "num_heads = %d < 1", num_heads);
  const int64_t n = (int64_t)num_heads * head_dim;
  if (x_row_stride < n || x_row_stride % 8)
    return fail(MI355X_GA_INVALID_ARGUMENT, "x_row_stride %lld: must be a multiple of 8 and >= %lld",
                (long long)x_row_stride, (long long)n);
  if (M == 0) return ok();
  if (!x || !out) return fail(MI355X_GA_INVALID_ARGUMENT, "x or out is NULL");
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
    return fail(MI355X_GA_INVALID_ARGUMENT, "x and out must be 16-byte aligned");
  QkNormParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.out = static_cast<uint16_t*>(out);
  p.rows = M;
  p.row_stride = x_row_stride;
  p.heads = num_heads;
  p.head_dim = head_dim;
  p.fp16 = dtype == MI355X_QKN_FP16;
  p.eps = eps;
  p.scale = scale;
  const hipError_t e = launch_qk_norm(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI355X_GA_HIP_ERROR, "qk_norm launch: %s", hipGetErrorString(e));
  return ok();
}
