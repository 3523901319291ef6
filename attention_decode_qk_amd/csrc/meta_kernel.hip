// meta_kernel.hip -- the per-step metadata every layer of a step shares: each
// new token's position and cache row, and each request's key count, from the
// cached lengths and the page table.
//
// Definition: page "012-attention-local-splits.py", `Inputs` (token b*L + i
// sits at position seq_lens[b] + i; cache_loc is the flat row the page table
// gives that position; cache_seqlens = seq_lens + L); page "msa.py",
// update_msa_decode_cg_meta (graph replay pads the batch with seq_len == 0
// slots).  In a decode or verify step (q_len <= 8) a slot with seq_lens[b] <=
// 0 is padding; in an extend step seq_lens[b] == 0 is a new request with an
// empty prefix and only seq_lens[b] < 0 is padding.  A padded slot gets
// position 0, row -1 (the step stores nothing) and key count 0 (the step
// outputs zeros).  A position whose page-table entry is negative or beyond
// max_pages gets row -1.
//
// Also the step's physical page table from the allocator's map (page
// "msa.py", _build_page_table): the physical page of logical page i of request
// b is req_to_token[slot_ids[b], i * P] / P for i < ceil(kv_lens[b] / P),
// written as page 1's padded table and/or page 2's packed one.
//
// One thread per token or per page entry; integer work only, so results are
// exact.
#include <algorithm>

#include "kernels.h"

namespace mi355x_ga {
namespace {

__global__ __launch_bounds__(256) void step_meta_kernel(MetaParams m) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)m.batch * m.q_len) return;
  const int64_t b = t / m.q_len;
  const int i = (int)(t - b * m.q_len);
  const int32_t len = m.seq_lens[b];
  const bool pad = m.q_len <= kMaxQLen ? len <= 0 : len < 0;
  if (i == 0) m.cache_seqlens[b] = pad ? 0 : len + m.q_len;
  if (pad) {
    m.positions[t] = 0;
    m.cache_loc[t] = -1;
    return;
  }
  const int64_t p = (int64_t)len + i;
  m.positions[t] = p;
  const int64_t page = m.page_shift >= 0 ? p >> m.page_shift : p / m.page_size;
  const int64_t off = p - page * m.page_size;
  const int32_t entry = page < m.max_pages ? m.page_table[b * m.max_pages + page] : -1;
  m.cache_loc[t] = entry < 0 ? -1 : (int64_t)entry * m.page_size + off;
}

// Pages of request b: ceil(kv_lens[b] / P), 0 for a padded slot, clamped so
// that every page starts inside the map's row and fits the padded table.
__device__ inline int pages_of(const PageTableParams& q, int b) {
  const int64_t len = q.kv_lens[b];
  int64_t n = len > 0 ? (len + q.page_size - 1) / q.page_size : 0;
  n = min(n, (q.req_stride + q.page_size - 1) / q.page_size);
  return (int)min(n, (int64_t)q.max_pages);
}

// Exclusive prefix sums of the page counts into kv_indptr[0 .. B]: one
// workgroup of 1024 threads, 1024 requests per round (a wave's sum by lane
// shifts, the waves' by LDS, a running total between rounds).
__global__ __launch_bounds__(1024) void page_scan_kernel(PageTableParams q) {
  __shared__ int s_wave[16];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < q.batch; base += 1024) {
    const int b = base + tid;
    const int n = b < q.batch ? pages_of(q, b) : 0;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (b < q.batch) q.kv_indptr[b] = before + incl - n;
    __syncthreads();
    if (tid == 1023) s_carry = before + incl;
    __syncthreads();
  }
  if (tid == 0) q.kv_indptr[q.batch] = s_carry;
}

// One thread per (request, page slot) of the padded table.
__global__ __launch_bounds__(256) void page_fill_kernel(PageTableParams q) {
  const int64_t total = (int64_t)q.batch * q.max_pages;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(e / q.max_pages);
    const int i = (int)(e - (int64_t)b * q.max_pages);
    const int n = pages_of(q, b);
    int32_t page = -1;
    if (i < n) {
      const int64_t r = min(max((int64_t)q.slot_ids[b], (int64_t)0), q.max_reqs - 1);
      const int32_t slot = q.req_to_token[r * q.req_stride + (int64_t)i * q.page_size];
      page = slot < 0 ? -1 : (q.page_shift >= 0 ? slot >> q.page_shift : slot / q.page_size);
      if (q.kv_indices) q.kv_indices[q.kv_indptr[b] + i] = page;
    }
    if (q.page_table) q.page_table[e] = page;
  }
}

}  // namespace

hipError_t launch_page_table(const PageTableParams& q, hipStream_t stream) {
  if (q.batch == 0) return hipSuccess;
  if (q.kv_indices) {
    hipLaunchKernelGGL(page_scan_kernel, dim3(1), dim3(1024), 0, stream, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = (int64_t)q.batch * q.max_pages;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(page_fill_kernel, dim3(grid), dim3(256), 0, stream, q);
  return hipGetLastError();
}

hipError_t launch_step_meta(const MetaParams& m, hipStream_t stream) {
  const int64_t tokens = (int64_t)m.batch * m.q_len;
  if (tokens == 0) return hipSuccess;
  const unsigned grid = (unsigned)((tokens + 255) / 256);
  hipLaunchKernelGGL(step_meta_kernel, dim3(grid), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace mi355x_ga
