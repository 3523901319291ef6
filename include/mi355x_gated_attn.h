/*
 * mi355x_gated_attn.h -- C ABI of the MI355X (gfx950) gated-attention step.
 *
 * One decoder layer's attention step for a decode (q_len 1), speculative
 * verify (q_len up to 8) or extend / prefill (a block of up to 65536 new
 * tokens per request) batch, at one GPU's head share, as defined on the
 * page "012-attention-local-splits.py" (SGLang's Muse Spark Open gated
 * attention, FP8 e4m3 KV cache).  In the page's order (module docstring):
 *
 *   1. per-head unweighted RMSNorm (eps 1e-5) of the q and k heads of the
 *      fused bf16 projection row, with interleaved RoPE on sliding-window
 *      layers (`_prepare_qkv`, `_cos_sin`);
 *   2. k and v stored as float8 e4m3 at each new token's flat cache row,
 *      divided by the cache scales when they are not 1 (`set_kv_buffer`);
 *      q cast to e4m3 (`prepare_paged_mha_query`);
 *   3. paged, causal, sliding-window grouped-query attention over the e4m3
 *      cache (the `flash_attn_with_kvcache` call in `kernel_fn`);
 *   4. per-head RMSNorm of the bf16 attention output times sigmoid(gate)
 *      (`rms_norm_gate`).
 *
 * Conventions.  Every buffer is caller-owned device memory unless stated;
 * the library never allocates, frees or retains a caller buffer.  Every
 * entry point returns an int status (MI355X_GA_*); nothing throws across the
 * ABI and mi355x_gated_attn_last_error() gives the calling thread's last
 * message.  Validation is host-side and reads scalars only: device-resident
 * values (lengths, rows, positions) are never read on the host, so a step can
 * be captured in a HIP graph.  Out-of-range device values are clamped where a
 * memory access depends on them (no fault), but their results are undefined.
 */
#ifndef MI355X_GATED_ATTN_H
#define MI355X_GATED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MI355X_GA_OK = 0,
  MI355X_GA_UNSUPPORTED = 1,          /* a shape this build does not serve      */
  MI355X_GA_INVALID_ARGUMENT = 2,     /* bad scalar, null pointer, unplanned ctx */
  MI355X_GA_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the plan's size  */
  MI355X_GA_HIP_ERROR = 4             /* a HIP runtime call or launch failed    */
};

/*
 * Step configuration: the page's Config (batch, q_len, num_q_heads,
 * num_kv_heads, head_dim, page_size, window, rope_theta, sm_scale, kv_scale)
 * plus the two bounds the library needs to keep every access in range, and
 * q_scale, the output scale of page "qk_norm" applied to q's norm.
 */
typedef struct mi355x_gated_attn_config {
  int32_t batch;        /* B >= 0 requests; B == 0 makes every step a no-op     */
  int32_t q_len;        /* L new tokens per request, 1..65536 (causal in the block) */
  int32_t num_q_heads;  /* Hq; this build serves 16 (one GPU's share under TP8) */
  int32_t num_kv_heads; /* Hkv; this build serves 2; q head h reads h/(Hq/Hkv)  */
  int32_t head_dim;     /* D; 64                                                */
  int32_t page_size;    /* P >= 1 cache rows per page                           */
  int32_t window;       /* W >= 0: a query at p sees keys p-W+1..p; 0 = all     */
  int32_t max_pages;    /* >= 1, row stride of page_table                       */
  int64_t num_pages;    /* >= 1, pages in the cache pool (rows = num_pages * P) */
  float rope_theta;     /* 0 = no RoPE; > 0 = interleaved RoPE base             */
  float sm_scale;       /* the softmax scale applied to q.k (the page folds its */
                        /* query factor in: sm_scale * qk_scale_factor)        */
  float kv_scale;       /* != 1 selects the scaled store (divide by k_scale /   */
                        /* v_scale) and the descaled read; == 1 ignores them    */
  float q_scale;        /* > 0: q's normed fp32 product is multiplied by it     */
                        /* before its one bf16 rounding (page "qk_norm",        */
                        /* QKNormDirectKernel's output scale: a query factor    */
                        /* carried by q, not by sm_scale); 1 = page 1's norm    */
  int32_t sparse_block; /* 0: dense (window) step.  > 0: page-list-driven decode */
                        /* (mi355x_gated_attn_sparse_step) over blocks of this   */
                        /* many keys, a multiple of 32; needs q_len 1, window 0 */
  int32_t sparse_topk;  /* list slots per (KV head, request), 1..256 when sparse */
} mi355x_gated_attn_config;

/* Opaque per-configuration context (host memory only). */
typedef struct mi355x_gated_attn_ctx mi355x_gated_attn_ctx;

/*
 * Whether this build serves cfg (the query page "qk_norm" gives its kernel,
 * supports_qk_norm: a shape a kernel does not serve is reported, not
 * attempted): returns MI355X_GA_OK, MI355X_GA_UNSUPPORTED (head_dim != 64,
 * Hq != 16, Hkv != 2, q_len outside 1..65536, B * q_len beyond 2^31 - 1 for
 * q_len > 8) or MI355X_GA_INVALID_ARGUMENT (negative or zero sizes, window <
 * 0, rope_theta < 0, non-finite or non-positive scales).  Pure host code.
 */
int mi355x_gated_attn_supports(const mi355x_gated_attn_config* cfg);

/*
 * Validate cfg and create a context bound to HIP device `device`.
 * Host-only: computes the RoPE inverse frequencies, 1 / theta^(2i/D) with the
 * power and the reciprocal each rounded to fp32 (the page's `_cos_sin`
 * recipe), and touches no device memory.  *out_ctx receives the context;
 * release it with mi355x_gated_attn_destroy.
 */
int mi355x_gated_attn_prepare(const mi355x_gated_attn_config* cfg, int device,
                              mi355x_gated_attn_ctx** out_ctx);

/*
 * Plan the split-KV schedule for every step (and layer) that uses this ctx,
 * outside any graph capture; it replaces the page's per-step FA3 scheduler
 * metadata and its split-count heuristic.  max_context bounds
 * cache_seqlens[b] (keys per request including the new tokens) and only steers
 * the split count; num_splits > 0 forces the count (1..256), 0 chooses it.
 * The plan also groups each request's L tokens into G token groups, one work
 * unit per (request, group, split): G = ceil(L/2) when the key range (the
 * window + L - 1, or max_context) is at most 4096 keys, else ceil(L/4).  A step
 * launches B * G * splits workgroups (UNSUPPORTED beyond 2^31-1).
 * q_len > 8 (extend / prefill; page "msa.py", msa_sparse_prefill_main: causal
 * attention with the query offset = the prefix length, here dense) has one
 * work unit per (request, 16-token tile, KV head); 0 chooses a key split only
 * when the B * 2 * ceil(L/16) units do not fill the chip (S = min(ceil(256 /
 * units), stages / 4, 32) over 64-key stages of the key bound), and
 * num_splits > 0 forces it (1..256).  UNSUPPORTED when units * S exceeds one
 * launch's workgroups.
 * Outputs (either may be NULL): *workspace_bytes = the workspace a step needs,
 * *num_splits_out = the chosen split count.  Host-only.
 */
int mi355x_gated_attn_plan(mi355x_gated_attn_ctx* ctx, int32_t max_context, int32_t num_splits,
                           size_t* workspace_bytes, int32_t* num_splits_out);

/*
 * Prepare a freshly allocated workspace for the ctx's plan: zero its
 * cross-workgroup counters (q_len > 8) and set every word of its split-partial
 * slots to the empty pattern (q_len <= 8).  Call once per workspace (per ctx
 * plan) before its first step, and again before a workspace serves another
 * plan; every completed step leaves the workspace ready for the next one.
 * Asynchronous on `stream`; kernel launches, never a memset, so it may also be
 * captured in a HIP graph.
 */
int mi355x_gated_attn_workspace_init(mi355x_gated_attn_ctx* ctx, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * The step metadata every layer of a step shares, built on the device once per
 * step (page "012-attention-local-splits.py", `Inputs`: token t = b*L + i sits
 * at position seq_lens[b] + i, its cache row is the flat row the page table
 * gives that position, cache_seqlens = seq_lens + L; page "msa.py",
 * update_msa_decode_cg_meta: graph replay pads the batch with seq_len == 0
 * slots).  Asynchronous on `stream`; no host synchronisation or allocation, so
 * capturable; the calling thread's current device must be the ctx's device.
 *
 *   seq_lens       int32 [B]    cached tokens per request; a slot with
 *                  seq_lens[b] <= 0 is padding when q_len <= 8 (a decode
 *                  request always has cached tokens), seq_lens[b] < 0 when
 *                  q_len > 8 (0 is a new request with an empty prefix)
 *   page_table     int32 [B, max_pages]  physical page of each logical page,
 *                  already covering the step's new positions (-1 unused)
 *   positions      int64 [B*L]  out: seq_lens[b] + i (0 in a padded slot)
 *   cache_loc      int64 [B*L]  out: page_table[b, p / P] * P + p % P, or -1
 *                  for a padded slot or a position whose page entry is
 *                  negative or beyond max_pages (the step then stores nothing)
 *   cache_seqlens  int32 [B]    out: seq_lens[b] + L (0 in a padded slot: the
 *                  step then outputs zeros for it)
 * Needs only `prepare` (B, L, page_size, max_pages of the ctx's config).
 * Returns MI355X_GA_OK with no launch when B == 0; INVALID_ARGUMENT for a NULL
 * pointer.
 */
int mi355x_gated_attn_step_meta(mi355x_gated_attn_ctx* ctx, const int32_t* seq_lens,
                                const int32_t* page_table, int64_t* positions, int64_t* cache_loc,
                                int32_t* cache_seqlens, void* stream);

/*
 * The step's physical page table from the allocator's map, built on the device
 * once per step for every layer (page "msa.py", _build_page_table: a page holds
 * page_size contiguous slots, so the physical page of logical page i of request
 * b is req_to_token[slot_ids[b], i * P] / P, for i < ceil(kv_lens[b] / P); the
 * page replaces its host-side .item() by a device scan, so the call needs no
 * host synchronisation and may be captured in a HIP graph).
 *
 *   req_to_token  int32 [max_reqs, req_stride]  physical slot of each logical
 *                 position of each allocator row (caller-owned, read only)
 *   slot_ids      int32 [B]  allocator row of each request (clamped to
 *                 0..max_reqs-1)
 *   kv_lens       int32 [B]  logical positions to cover per request (for a
 *                 step: its cache_seqlens, which include the new tokens); <= 0
 *                 gives no page (a padded slot)
 *   page_table    int32 [B, max_pages] out, or NULL: those pages, -1 after
 *                 them (page 1's layout, the step's page_table argument)
 *   kv_indices    int32 out, or NULL: the same pages packed request after
 *                 request (page 2's kv_indices); request b's start at
 *   kv_indptr     int32 [B+1] out (needed with kv_indices): exclusive prefix
 *                 sums of the page counts
 * A negative map entry gives -1.  Pages starting past a map row or beyond
 * max_pages are a caller error: the kernels clamp the count to stay in bounds.
 * B, P and max_pages come from the ctx's config (only `prepare` is needed).
 * Returns MI355X_GA_OK with no launch when B == 0; INVALID_ARGUMENT for a NULL
 * required pointer, no output, or req_stride / max_reqs < 1.
 */
int mi355x_gated_attn_page_table(mi355x_gated_attn_ctx* ctx, const int32_t* req_to_token,
                                 int64_t req_stride, int64_t max_reqs, const int32_t* slot_ids,
                                 const int32_t* kv_lens, int32_t* page_table, int32_t* kv_indices,
                                 int32_t* kv_indptr, void* stream);

/*
 * One layer-step, asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream); the calling thread's current device must be the ctx's device.
 * No host synchronisation, allocation or device-value read: capturable.
 * The whole step is one kernel launch for q_len <= 8; for q_len > 8 it is two
 * (the prologue of every new token, then attention and epilogue, which reads
 * the new keys back from the cache rows the first launch stored).
 *
 *   qkv            bf16 [B, L, (2Hq + 2Hkv) * D], rows contiguous: q heads |
 *                  k heads | v heads | gate logits (Hq*D); 16-byte aligned
 *   positions      int64 [B*L]  RoPE position of each new token (read iff
 *                  rope_theta != 0; must be < 2^21 as on the page)
 *   cache_loc      int64 [B*L]  flat cache row of each new token; rows outside
 *                  [0, num_pages*P) are not written
 *   cache_seqlens  int32 [B]    keys per request including the L new tokens;
 *                  query i of request b sits at p = cache_seqlens[b] - L + i
 *   page_table     int32 [B, max_pages]  physical page of each logical page,
 *                  -1 where unused (never read beyond a request's keys).  The
 *                  rows it gives for the new tokens' positions must be their
 *                  cache_loc rows (as when both come from one allocator): the
 *                  step attends to the new keys and values it computes, and
 *                  stores them at cache_loc
 *   seq_lens       int32 [B]    cached tokens per request; accepted for parity
 *                  with the page's inputs and not read (the page's attention
 *                  call takes cache_seqlens); may be NULL
 *   k_cache, v_cache  float8 e4m3 (OCP) [num_pages, P, Hkv, D], written in
 *                  place at the cache_loc rows only; 16-byte aligned
 *   k_scale, v_scale  device float32 scalars (read iff kv_scale != 1; may be
 *                  NULL otherwise)
 *   out            bf16 [B, L, Hq * D]; 8-byte aligned
 *   workspace      device memory of at least the planned size, 256-byte
 *                  aligned, initialised once by mi355x_gated_attn_workspace_init.
 *                  Layout after a step: bytes [0, B*L*Hq*D) hold q as e4m3
 *                  [B*L, Hq, D]; then split partials and B*G int32
 *                  counters (G token groups per request, from the plan; for
 *                  q_len > 8 partials only when split, and one counter per
 *                  (request, 16-token tile, KV head); q_len <= 8 uses no
 *                  counter: its partial slots are empty between steps).
 * Calls that share a workspace, or write the same cache rows, must be ordered
 * on one stream.  Returns MI355X_GA_OK with no launch when B == 0.
 * With q_len <= 8 and more than one split, the first split of each request
 * (and token group) waits for the others' partials: the launch's B*G*S
 * workgroups (at most a few hundred whenever S > 1) must be able to run
 * together, as they do on an MI355X unless other work holds every compute
 * unit; a split that has not arrived after 100 ms makes that group's output
 * NaN rather than hang the device.
 */
int mi355x_gated_attn_step(mi355x_gated_attn_ctx* ctx, const void* qkv, const int64_t* positions,
                           const int64_t* cache_loc, const int32_t* cache_seqlens,
                           const int32_t* page_table, const int32_t* seq_lens, void* k_cache,
                           void* v_cache, const float* k_scale, const float* v_scale, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * mi355x_gated_attn_step without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing and calls no
 * allocating routine.  q, the split partials and the counters live in a
 * static device array of the library, 32 MiB per GPU (the counters in its
 * first 64 KiB), held by each GPU the library runs on until the process
 * ends.  The first call on a device takes the array's address there and
 * zeroes its counters with one extra small kernel on `stream`; every
 * completed step leaves them at zero.  Every call on a GPU shares that GPU's
 * array and finds the last call's contents in it: calls that overlap on one
 * GPU (other streams, other threads, other contexts) race and must be
 * ordered by the caller.  The timing hook does not record these calls.
 * Arguments, effects and results are those of mi355x_gated_attn_step (same
 * kernels, same outputs and cache writes) without workspace and
 * workspace_bytes; the config must be dense (sparse_block 0).
 * MI355X_GA_WORKSPACE_TOO_SMALL when the plan needs more than the array holds
 * (32 MiB - 64 KiB of partials and q, 16,384 counters: e.g. an extend block
 * of more than about 31k new tokens); MI355X_GA_UNSUPPORTED for a device
 * index above 63; otherwise as mi355x_gated_attn_step.
 */
int mi355x_gated_attn_step_noalloc(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                   const int64_t* positions, const int64_t* cache_loc,
                                   const int32_t* cache_seqlens, const int32_t* page_table,
                                   const int32_t* seq_lens, void* k_cache, void* v_cache,
                                   const float* k_scale, const float* v_scale, void* out,
                                   void* stream);

/*
 * Release a context made by mi355x_gated_attn_prepare (NULL is ignored): its
 * host memory and the timing hook's events.  Does not synchronise; steps
 * already enqueued keep running (they read nothing from the ctx).
 */
void mi355x_gated_attn_destroy(mi355x_gated_attn_ctx* ctx);

/*
 * The calling thread's last error message ("" after a call that succeeded).
 * Every failure is a returned status with this text, never a crash or an
 * exception across the ABI: page "msa.py" makes an unavailable kernel a
 * raised, catchable error (MSAUnavailableError) that callers test for, and
 * this library reports every unserved shape, bad argument and HIP failure the
 * same way.
 */
const char* mi355x_gated_attn_last_error(void);

/*
 * Page-list-driven (top-k block-sparse) decode step: page "msa.py"
 * (msa_sparse_decode_main; build_msa_decode_meta places each request's one
 * query at its last cached position).  The same prologue, combine and gated
 * epilogue as mi355x_gated_attn_step, with attention restricted per KV head to
 * the keys of the blocks its list selects: for KV head g and request b,
 *   keys = union over i < sparse_topk with j = block_idx[(g * B + b) *
 *          sparse_topk + i] >= 0 of  j*sparse_block .. (j+1)*sparse_block - 1,
 *          those below cache_seqlens[b] (the new token's key included when its
 *          block is listed; no window);
 * query head h uses KV head h / (Hq/Hkv).  An empty set gives output 0.
 *   block_idx  device int32 [Hkv, B, sparse_topk], -1 for unused slots; block
 *              indices are logical (key / sparse_block) and distinct within a
 *              list (a repeated index is a caller error)
 * Other arguments as mi355x_gated_attn_step (seq_lens is not taken).  The
 * config must have sparse_block > 0 (INVALID_ARGUMENT otherwise, and
 * mi355x_gated_attn_step rejects such a config); the plan sizes splits for
 * sparse_topk * sparse_block keys per head.
 */
int mi355x_gated_attn_sparse_step(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                  const int64_t* positions, const int64_t* cache_loc,
                                  const int32_t* cache_seqlens, const int32_t* page_table,
                                  const int32_t* block_idx, void* k_cache, void* v_cache,
                                  const float* k_scale, const float* v_scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Page-list-driven (top-k block-sparse) prefill: page "msa.py"
 * (msa_sparse_prefill_main: every new token of a chunk is a query with its
 * own per-KV-head block list, topk_idx [Hkv, total_q, topk], causal with the
 * prefix as query offset; block_size_k == page_size there).  Each of the
 * config's `batch` queries is served as its own one-token step of
 * mi355x_gated_attn_sparse_step, after every query's K/V row has been stored
 * (a first launch runs the extend path's prologue over all of them):
 *   query t of request r = token_req[t] sits at position positions[t] =
 *   cache_seqlens[t] - 1, reads page_table row r, and attends, per KV head g,
 *   to the keys of the blocks block_idx[(g * batch + t) * sparse_topk + i]
 *   (-1 unused) below cache_seqlens[t]: the new tokens of the same chunk
 *   before it included, those after it not (no window).
 *   token_req      device int32 [batch], the page-table row of each query
 *                  (clamped to 0..num_requests-1)
 *   num_requests   host int32 >= 1, rows of page_table
 *   cache_seqlens  device int32 [batch], per query: its position + 1
 *   qkv, positions, cache_loc, out: per query ([batch, 1, ...]), as
 *                  mi355x_gated_attn_step at q_len 1
 * The config is a page-list-driven decode config (q_len 1, window 0,
 * sparse_block > 0) whose batch is the number of queries.  INVALID_ARGUMENT
 * for a dense config, a NULL token_req or block_idx, or num_requests < 1.
 * Other arguments, ownership and effects as mi355x_gated_attn_sparse_step.
 */
int mi355x_gated_attn_sparse_prefill_step(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                          const int64_t* positions, const int64_t* cache_loc,
                                          const int32_t* token_req, int32_t num_requests,
                                          const int32_t* cache_seqlens, const int32_t* page_table,
                                          const int32_t* block_idx, void* k_cache, void* v_cache,
                                          const float* k_scale, const float* v_scale, void* out,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged extend / prefill batch: page "msa.py" (msa_sparse_prefill_main:
 * per-request query segments given by cumulative lengths cu_seqlens,
 * qo_segment_lens = cu_seqlens[1:] - cu_seqlens[:-1], causal with the query
 * offset qo_offset = the prefix length; here with dense keys and page 1's
 * window).  The step of mi355x_gated_attn_step for q_len > 8, with request b's
 * new tokens being rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of a packed
 * batch instead of b*L .. (b+1)*L-1:
 *   segment length L_b = cu_seqlens_q[b+1] - cu_seqlens_q[b], 0 <= L_b <= the
 *   config's q_len (which must be > 8: the bound on every segment, sizing the
 *   plan and workspace); token i < L_b of request b sits at position
 *   cache_seqlens[b] - L_b + i (its own key is cache row cache_loc of that
 *   token) and sees the keys up to that position (within the window).
 *   cu_seqlens_q  device int32 [B+1], nondecreasing from 0 to total_q
 *   total_q       host int64, the batch's new tokens, 0..B*q_len
 *   qkv           bf16 [total_q, (2Hq + 2Hkv) * D]; positions and cache_loc
 *                 int64 [total_q]; out bf16 [total_q, Hq * D]
 * Other arguments, ownership and effects as mi355x_gated_attn_step (seq_lens
 * is not taken).  INVALID_ARGUMENT for a config with q_len <= 8 or
 * sparse_block > 0, a NULL cu_seqlens_q, or total_q outside 0..B*q_len;
 * device values that break the layout above (a segment longer than q_len,
 * offsets past total_q) are a caller error: the kernels clamp them to stay
 * in bounds, with undefined results.  A segment of length 0 writes nothing.
 */
int mi355x_gated_attn_ragged_step(mi355x_gated_attn_ctx* ctx, const void* qkv,
                                  const int64_t* positions, const int64_t* cache_loc,
                                  const int32_t* cu_seqlens_q, int64_t total_q,
                                  const int32_t* cache_seqlens, const int32_t* page_table,
                                  void* k_cache, void* v_cache, const float* k_scale,
                                  const float* v_scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Measurement hook (not part of the page's interface): while enabled, each
 * step records a HIP event pair on its stream around its attention kernel
 * (the step's one launch for q_len <= 8; the second of its two, attention and
 * epilogue, for q_len > 8).  `enable`
 * != 0 starts a fresh accumulation, 0 stops recording.  Not for use under
 * graph capture.
 */
int mi355x_gated_attn_timing(mi355x_gated_attn_ctx* ctx, int enable);

/*
 * Wait for the recorded events and return the summed kernel duration in
 * milliseconds (*kernel_ms) and the number of timed steps; then clear the
 * accumulation.
 */
int mi355x_gated_attn_timing_read(mi355x_gated_attn_ctx* ctx, double* kernel_ms,
                                  int64_t* steps);

/* ---- Per-head QK-norm with an output scale --------------------------------
 * The operation of the page "qk_norm" (vLLM's CuTeDSL fused QK-norm for
 * MuseSpark1x attention: the qk_norm function, QKNormDirectKernel's kernel and
 * supports_qk_norm).  Independent of any ctx. */

/* Element types of the QK-norm input and output. */
enum { MI355X_QKN_BF16 = 0, MI355X_QKN_FP16 = 1 };

/*
 * Whether mi355x_qk_norm serves (dtype, head_dim): 1 if it does, 0 if not.
 * On the page a head is covered by a fixed number of threads per row (chosen
 * from head_dim by the launch-shape table of _DirectConfig) holding eight
 * 16-bit values each, with no tail path; for 16-bit types that leaves
 * head_dim 64, 128 and 256.  This build serves the same set, for bfloat16 and
 * binary16.
 */
int mi355x_qk_norm_supports(int32_t dtype, int32_t head_dim);

/*
 * Unweighted RMSNorm of every head_dim-wide group plus an output scale.  For
 * row r < M and head h < num_heads, with v[c] = x[r * x_row_stride +
 * h * head_dim + c], c < head_dim:
 *   rstd = 1 / sqrt(sum_c v[c]^2 / head_dim + eps)
 *   out[r * num_heads * head_dim + h * head_dim + c] = round(v[c] * rstd * scale)
 * rstd is fp32 (the sum of squares formed exactly and rounded once, the
 * quotient and + eps in fp32, rsqrt correctly rounded); the products are fp32,
 * the one by scale only when scale != 1; round is to nearest even in dtype and
 * is the only rounding.
 *   x             device, dtype [M, x_row_stride]: only the first
 *                 num_heads * head_dim columns of each row are read; 16-byte
 *                 aligned, x_row_stride (elements) a multiple of 8 and
 *                 >= num_heads * head_dim (a strided view of a wider row, such
 *                 as the q columns of a fused projection, is served as is)
 *   out           device, dtype [M, num_heads * head_dim], 16-byte aligned;
 *                 must not overlap x
 *   M             rows >= 0; M == 0 returns MI355X_GA_OK with no launch
 *   stream        hipStream_t (NULL: the null stream); the call is asynchronous
 *                 on it and allocates nothing
 * Caller-owned memory throughout.  Returns MI355X_GA_UNSUPPORTED when
 * mi355x_qk_norm_supports(dtype, head_dim) is 0; MI355X_GA_INVALID_ARGUMENT
 * for M < 0, num_heads < 1, a short or unaligned row stride, or (M > 0) a NULL
 * or misaligned pointer; MI355X_GA_HIP_ERROR when the launch fails.
 */
int mi355x_qk_norm(const void* x, void* out, int64_t M, int32_t num_heads, int32_t head_dim,
                   int64_t x_row_stride, int32_t dtype, float eps, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355X_GATED_ATTN_H */
