// kernels.h -- internal interface between the C-ABI host code and the gfx950
// kernel of the gated-attention step.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355x_ga {

// Shapes this build serves: one GPU's head share of the page's model
// (16 query heads, 2 KV heads, head_dim 64; 8 query heads per KV head).
constexpr int kHeadDim = 64;
constexpr int kQHeads = 16;
constexpr int kKvHeads = 2;
constexpr int kGroup = kQHeads / kKvHeads;           // 8
constexpr int kRowBytes = kKvHeads * kHeadDim;       // 128 B: one cache row, both KV heads
constexpr int kMaxQLen = 8;
constexpr int kWidth = (2 * kQHeads + 2 * kKvHeads) * kHeadDim;  // 2304 projection columns
constexpr int kGateOffset = (kQHeads + 2 * kKvHeads) * kHeadDim; // 1280

// Work unit = (request, token group, split): a workgroup of kAttnWaves waves
// (or twice that, one KV head each) walks the split's key chunk in blocks of
// kKeyBlock keys, one block per wave at a time, for the query rows of the
// group's tokens.  A request's q_len tokens form G groups of consecutive
// tokens (the plan's choice): over a short key range G = ceil(q_len / 2) up to
// q_len 4 and ceil(q_len / 4) beyond; over a long one a single group.  A unit
// carries ceil(q_len / G) tokens, served by the kernel of unit size
// unit_tokens(q_len, G): 1..4, or kMaxQLen for one group of five to eight.
constexpr int kAttnWaves = 4;
constexpr int kKeyBlock = 32;
constexpr int kMaxTokensPerUnit = 4;
constexpr int kMaxSparseTopk = 256;  // list slots per (KV head, request) of page-list-driven decode
constexpr int kMaxExtendLen = 65536;  // longest extend / prefill block (q_len > kMaxQLen) served
constexpr int token_groups(int q_len, bool short_keys) {
  return !short_keys ? 1
                     : (q_len <= kMaxTokensPerUnit ? (q_len + 1) / 2
                                                   : (q_len + kMaxTokensPerUnit - 1) / kMaxTokensPerUnit);
}
constexpr int tokens_per_unit(int q_len, int groups) { return (q_len + groups - 1) / groups; }
// Kernel unit size for q_len tokens in `groups` groups: 1..4, or kMaxQLen for
// one group of five to eight tokens.
constexpr int unit_tokens(int q_len, int groups) {
  return tokens_per_unit(q_len, groups) > kMaxTokensPerUnit ? kMaxQLen : tokens_per_unit(q_len, groups);
}
// The longest q_len served by units of lu tokens under either grouping (0 if none).
constexpr int max_q_len_for(int lu) {
  if (lu == kMaxQLen) return kMaxQLen;
  int m = 0;
  for (int l = 1; l <= kMaxQLen; ++l)
    if (tokens_per_unit(l, token_groups(l, false)) == lu || tokens_per_unit(l, token_groups(l, true)) == lu)
      m = l;
  return m;
}

struct StepParams {
  const uint16_t* qkv;           // bf16 [T, kWidth]
  const int64_t* positions;      // [T] (read iff rope)
  const int64_t* cache_loc;      // [T]
  const int32_t* cache_seqlens;  // [B]
  const int32_t* page_table;     // [B, max_pages]
  uint8_t* k_cache;              // e4m3 [rows, kKvHeads, kHeadDim]
  uint8_t* v_cache;
  const float* k_scale;          // device scalars, read iff scaled
  const float* v_scale;
  uint16_t* out;                 // bf16 [T, kQHeads * kHeadDim]
  uint8_t* q_out;                // e4m3 [T, kQHeads, kHeadDim] (workspace)
  _Float16* part_o;              // f16 [B, S, L*kQHeads, kHeadDim]: o / l of the split
  float* part_ml;                // fp32 [B, S, L*kQHeads, 2]: running max (log2 units), sum
                                 // (q_len <= kMaxQLen: every 8-byte word of both is the empty-slot
                                 // sentinel between steps)
  int32_t* counters;             // extend: one per unit, finished splits, 0 between steps
  int64_t num_pages;
  int64_t num_rows;              // num_pages * page_size (< 2^31)
  int32_t batch;
  int32_t q_len;                 // L
  int32_t tgroups;               // G: token_groups(L, short or not)
  int32_t splits;                // S
  int32_t balanced;              // 1: splits per request by key count (batch <= 64), else S each
  int32_t head_split;            // 1: eight waves per unit, one KV head each
  int32_t key_waves;             // waves per KV head taking blocks round-robin (4, or 8 at q_len 1)
  int32_t sep_combine;           // 1: every unit publishes its partial and a second launch
                                 // (combine_kernel) merges them and runs the epilogue
  int32_t max_pages;
  int32_t page_size;
  int32_t page_shift;            // log2(page_size) if a power of two, else -1
  int32_t window;
  int32_t scaled;                // 1 iff kv_scale != 1
  int32_t rope;                  // 1 iff rope_theta != 0
  float sm_scale_log2;           // sm_scale * log2(e)
  float q_scale;                 // q's norm output scale before its bf16 rounding (1: none)
  const int32_t* block_idx;      // page-list-driven decode: int32 [Hkv, B, topk] block lists (-1 pad)
  int32_t sparse_block;          // keys per listed block (a multiple of 32); 0: dense step
  int32_t sparse_topk;           // list slots per (KV head, request), <= kMaxSparseTopk
  const int32_t* cu_seqlens_q;   // ragged extend: [B+1], request b's tokens cu[b] .. cu[b+1]-1 (at most
                                 // q_len each); null: b*q_len .. (b+1)*q_len-1
  int64_t total_q;               // tokens of the step: cu[B] when ragged, else B*q_len
  const int32_t* token_req;      // sparse prefill: [B] page-table row of each query (its request);
                                 // null: query b uses row b
  int32_t pt_rows;               // sparse prefill: rows of page_table (token_req is clamped to them)
  float inv_freq[kHeadDim / 2];
  int32_t sparse_shift;          // log2(sparse_block) if a power of two, else -1
};

// attn_start (may be null): for q_len > kMaxQLen, an event recorded between
// the prologue launch and the attention launch.
hipError_t launch_step(const StepParams& p, hipStream_t stream, hipEvent_t attn_start = nullptr);
// The q_len > kMaxQLen path of launch_step (two launches: prologue, then
// attention and epilogue; attn_start as above).
hipError_t launch_extend(const StepParams& p, hipStream_t stream, hipEvent_t attn_start);
// The extend path's prologue alone over p.total_q tokens: norm, RoPE, q e4m3 to
// the workspace, the new K/V rows stored at cache_loc.
hipError_t launch_extend_prologue(const StepParams& p, hipStream_t stream);

// Per-head RMSNorm with an output scale (qk_norm_kernel.hip).
struct QkNormParams {
  const uint16_t* x;   // bf16 or fp16 [rows, row_stride], 16-byte aligned rows
  uint16_t* out;       // same type [rows, heads * head_dim]
  int64_t rows;
  int64_t row_stride;  // elements between rows of x (a multiple of 8)
  int32_t heads;
  int32_t head_dim;    // 64, 128 or 256
  int32_t fp16;        // 1: binary16, 0: bfloat16
  float eps;
  float scale;         // the product is skipped when 1
};

hipError_t launch_qk_norm(const QkNormParams& p, hipStream_t stream);

// Per-step metadata shared by every layer (meta_kernel.hip).
struct MetaParams {
  const int32_t* seq_lens;       // [B]
  const int32_t* page_table;     // [B, max_pages]
  int64_t* positions;            // [B*L] out
  int64_t* cache_loc;            // [B*L] out
  int32_t* cache_seqlens;        // [B] out
  int32_t batch;
  int32_t q_len;
  int32_t max_pages;
  int32_t page_size;
  int32_t page_shift;            // log2(page_size) if a power of two, else -1
};
hipError_t launch_step_meta(const MetaParams& m, hipStream_t stream);

// The step's physical page table from the allocator's map (meta_kernel.hip).
struct PageTableParams {
  const int32_t* req_to_token;   // [max_reqs, req_stride] physical slot per logical position
  int64_t req_stride;
  int64_t max_reqs;
  const int32_t* slot_ids;       // [B] map row of each request
  const int32_t* kv_lens;        // [B] logical positions to cover
  int32_t batch;
  int32_t page_size;
  int32_t page_shift;            // log2(page_size) if a power of two, else -1
  int32_t max_pages;
  int32_t* page_table;           // [B, max_pages] padded with -1, or null
  int32_t* kv_indices;           // packed pages, or null
  int32_t* kv_indptr;            // [B+1] exclusive prefix sums (written when kv_indices is)
};
hipError_t launch_page_table(const PageTableParams& q, hipStream_t stream);
hipError_t launch_zero_counters(int32_t* counters, int n, hipStream_t stream);
// Set every 8-byte word of [p, p + bytes) to the decode step's empty-slot
// sentinel (all bits set); bytes is a multiple of 8.
hipError_t launch_fill_sentinel(void* p, size_t bytes, hipStream_t stream);

}  // namespace mi355x_ga
