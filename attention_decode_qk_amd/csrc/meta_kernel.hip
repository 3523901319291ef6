// meta_kernel.hip -- the per-step metadata every layer of a step shares: each
// new token's position and cache row, and each request's key count, from the
// cached lengths and the page table.
//
// Definition: page "012-attention-local-splits.py", `Inputs` (token b*L + i
// sits at position seq_lens[b] + i; cache_loc is the flat row the page table
// gives that position; cache_seqlens = seq_lens + L); page "msa.py",
// update_msa_decode_cg_meta (graph replay pads the batch with seq_len == 0
// slots).  A slot with seq_lens[b] <= 0 is padding: position 0, row -1 (the
// step stores nothing) and key count 0 (the step outputs zeros).  A position
// whose page-table entry is negative or beyond max_pages gets row -1.
//
// One thread per token; integer work only, so results are exact.
#include "kernels.h"

namespace mi355x_ga {
namespace {

__global__ __launch_bounds__(256) void step_meta_kernel(MetaParams m) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)m.batch * m.q_len) return;
  const int64_t b = t / m.q_len;
  const int i = (int)(t - b * m.q_len);
  const int32_t len = m.seq_lens[b];
  const bool pad = len <= 0;
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

}  // namespace

hipError_t launch_step_meta(const MetaParams& m, hipStream_t stream) {
  const int64_t tokens = (int64_t)m.batch * m.q_len;
  if (tokens == 0) return hipSuccess;
  const unsigned grid = (unsigned)((tokens + 255) / 256);
  hipLaunchKernelGGL(step_meta_kernel, dim3(grid), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace mi355x_ga
