"""Python binding of the MI355X (gfx950) gated-attention step library.

Thin ctypes marshalling over ``libmi355x_gated_attn.so`` (C ABI in
``include/mi355x_gated_attn.h``): the functions keep the C names, turn torch
tensors into device pointers and raise :class:`GatedAttnError` on a non-zero
status.  Every step of the computation runs in the library's HIP kernels;
torch only provides device memory and streams.  There is no fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmi355x_gated_attn.so")

MI355X_GA_OK = 0
MI355X_GA_UNSUPPORTED = 1
MI355X_GA_INVALID_ARGUMENT = 2
MI355X_GA_WORKSPACE_TOO_SMALL = 3
MI355X_GA_HIP_ERROR = 4

EXPORTED = ["mi355x_gated_attn_supports", "mi355x_gated_attn_prepare", "mi355x_gated_attn_plan",
            "mi355x_gated_attn_workspace_init", "mi355x_gated_attn_step", "mi355x_gated_attn_destroy",
            "mi355x_gated_attn_last_error", "mi355x_gated_attn_timing",
            "mi355x_gated_attn_timing_read", "mi355x_gated_attn_step_meta",
            "mi355x_qk_norm_supports", "mi355x_qk_norm", "mi355x_gated_attn_sparse_step",
            "mi355x_gated_attn_ragged_step", "mi355x_gated_attn_sparse_prefill_step"]

MI355X_QKN_BF16 = 0
MI355X_QKN_FP16 = 1


class GatedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class Config(ctypes.Structure):
    """mi355x_gated_attn_config."""
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("rope_theta", ctypes.c_float),
                ("sm_scale", ctypes.c_float), ("kv_scale", ctypes.c_float),
                ("q_scale", ctypes.c_float), ("sparse_block", ctypes.c_int32),
                ("sparse_topk", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m attention_decode_qk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.mi355x_gated_attn_supports.argtypes = [ctypes.POINTER(Config)]
        L.mi355x_gated_attn_prepare.argtypes = [ctypes.POINTER(Config), ctypes.c_int,
                                                ctypes.POINTER(P)]
        L.mi355x_gated_attn_plan.argtypes = [P, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_int32)]
        L.mi355x_gated_attn_workspace_init.argtypes = [P, P, ctypes.c_size_t, P]
        L.mi355x_gated_attn_step.argtypes = [P] * 13 + [ctypes.c_size_t, P]
        L.mi355x_gated_attn_step_meta.argtypes = [P] * 7
        L.mi355x_gated_attn_sparse_step.argtypes = [P] * 13 + [ctypes.c_size_t, P]
        L.mi355x_gated_attn_sparse_prefill_step.argtypes = [P] * 5 + [ctypes.c_int32] + \
            [P] * 9 + [ctypes.c_size_t, P]
        L.mi355x_gated_attn_ragged_step.argtypes = [P] * 5 + [ctypes.c_int64] + [P] * 8 + \
            [ctypes.c_size_t, P]
        L.mi355x_gated_attn_destroy.argtypes = [P]
        L.mi355x_gated_attn_destroy.restype = None
        L.mi355x_gated_attn_last_error.argtypes = []
        L.mi355x_gated_attn_last_error.restype = ctypes.c_char_p
        L.mi355x_gated_attn_timing.argtypes = [P, ctypes.c_int]
        L.mi355x_gated_attn_timing_read.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                                    ctypes.POINTER(ctypes.c_int64)]
        L.mi355x_qk_norm_supports.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.mi355x_qk_norm.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_float, P]
        for name in EXPORTED:
            if name not in ("mi355x_gated_attn_destroy", "mi355x_gated_attn_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def mi355x_gated_attn_last_error() -> str:
    return lib().mi355x_gated_attn_last_error().decode()


def _check(rc: int):
    if rc != MI355X_GA_OK:
        raise GatedAttnError(rc, mi355x_gated_attn_last_error())


def make_config(batch, q_len, page_size, window, max_pages, num_pages, rope_theta=0.0,
                sm_scale=0.125, kv_scale=1.0, num_q_heads=16, num_kv_heads=2,
                head_dim=64, q_scale=1.0, sparse_block=0, sparse_topk=0) -> Config:
    return Config(batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, window,
                  max_pages, num_pages, rope_theta, sm_scale, kv_scale, q_scale, sparse_block,
                  sparse_topk)


def mi355x_gated_attn_supports(cfg: Config) -> int:
    """Status code (0 = served); does not raise."""
    return lib().mi355x_gated_attn_supports(ctypes.byref(cfg))


def mi355x_gated_attn_prepare(cfg: Config, device: int = 0) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    _check(lib().mi355x_gated_attn_prepare(ctypes.byref(cfg), device, ctypes.byref(ctx)))
    return ctx


def mi355x_gated_attn_plan(ctx, max_context: int, num_splits: int = 0):
    """Returns (workspace_bytes, num_splits)."""
    ws = ctypes.c_size_t()
    s = ctypes.c_int32()
    _check(lib().mi355x_gated_attn_plan(ctx, int(max_context), int(num_splits), ctypes.byref(ws),
                                        ctypes.byref(s)))
    return ws.value, s.value


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    return ctypes.c_void_p(x.data_ptr())


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def mi355x_gated_attn_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table, seq_lens,
                           k_cache, v_cache, k_scale, v_scale, out, workspace, stream=None):
    """Launch one step.  Tensor arguments must be contiguous device tensors of the
    dtypes the C ABI names (bf16 qkv/out, int64 positions/cache_loc, int32
    lengths/page_table, uint8 or float8_e4m3fn caches, float32 scales, a byte
    workspace); `stream` is a torch stream, a raw handle, or None for torch's
    current stream."""
    import torch
    tensors = dict(qkv=qkv, positions=positions, cache_loc=cache_loc, cache_seqlens=cache_seqlens,
                   page_table=page_table, k_cache=k_cache, v_cache=v_cache, out=out,
                   workspace=workspace)
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_step(
        ctx, _ptr(qkv), _ptr(positions), _ptr(cache_loc), _ptr(cache_seqlens), _ptr(page_table),
        _ptr(seq_lens), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        _ptr(workspace), _nbytes(workspace), ctypes.c_void_p(handle)))


def mi355x_gated_attn_sparse_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table,
                                  block_idx, k_cache, v_cache, k_scale, v_scale, out, workspace,
                                  stream=None):
    """Launch one page-list-driven decode step (block_idx: contiguous int32
    device tensor [Hkv, B, topk], -1 padded); otherwise as mi355x_gated_attn_step."""
    import torch
    tensors = dict(qkv=qkv, positions=positions, cache_loc=cache_loc, cache_seqlens=cache_seqlens,
                   page_table=page_table, block_idx=block_idx, k_cache=k_cache, v_cache=v_cache,
                   out=out, workspace=workspace)
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_sparse_step(
        ctx, _ptr(qkv), _ptr(positions), _ptr(cache_loc), _ptr(cache_seqlens), _ptr(page_table),
        _ptr(block_idx), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        _ptr(workspace), _nbytes(workspace), ctypes.c_void_p(handle)))


def mi355x_gated_attn_ragged_step(ctx, qkv, positions, cache_loc, cu_seqlens_q, total_q: int,
                                  cache_seqlens, page_table, k_cache, v_cache, k_scale, v_scale,
                                  out, workspace, stream=None):
    """Launch one ragged extend step: request b's new tokens are rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (contiguous int32 device tensor
    [B+1]) of the packed qkv / positions / cache_loc / out, total_q of them;
    otherwise as mi355x_gated_attn_step."""
    import torch
    tensors = dict(qkv=qkv, positions=positions, cache_loc=cache_loc, cu_seqlens_q=cu_seqlens_q,
                   cache_seqlens=cache_seqlens, page_table=page_table, k_cache=k_cache,
                   v_cache=v_cache, out=out, workspace=workspace)
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_ragged_step(
        ctx, _ptr(qkv), _ptr(positions), _ptr(cache_loc), _ptr(cu_seqlens_q), int(total_q),
        _ptr(cache_seqlens), _ptr(page_table), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(out), _ptr(workspace), _nbytes(workspace), ctypes.c_void_p(handle)))


def mi355x_gated_attn_sparse_prefill_step(ctx, qkv, positions, cache_loc, token_req,
                                          num_requests: int, cache_seqlens, page_table,
                                          block_idx, k_cache, v_cache, k_scale, v_scale, out,
                                          workspace, stream=None):
    """Launch one page-list-driven prefill: the config's batch is the number of
    queries; token_req (int32 [batch]) names each query's page-table row,
    cache_seqlens (int32 [batch]) is each query's position + 1, block_idx is
    int32 [Hkv, batch, topk]; otherwise as mi355x_gated_attn_sparse_step."""
    import torch
    tensors = dict(qkv=qkv, positions=positions, cache_loc=cache_loc, token_req=token_req,
                   cache_seqlens=cache_seqlens, page_table=page_table, block_idx=block_idx,
                   k_cache=k_cache, v_cache=v_cache, out=out, workspace=workspace)
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_sparse_prefill_step(
        ctx, _ptr(qkv), _ptr(positions), _ptr(cache_loc), _ptr(token_req), int(num_requests),
        _ptr(cache_seqlens), _ptr(page_table), _ptr(block_idx), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(out), _ptr(workspace), _nbytes(workspace),
        ctypes.c_void_p(handle)))


def mi355x_gated_attn_step_meta(ctx, seq_lens, page_table, positions, cache_loc, cache_seqlens,
                                stream=None):
    """Build a step's positions, cache rows and key counts on the device (int32
    seq_lens [B] and page_table [B, max_pages] in; int64 positions and cache_loc
    [B*L], int32 cache_seqlens [B] out)."""
    import torch
    for name, t in dict(seq_lens=seq_lens, page_table=page_table, positions=positions,
                        cache_loc=cache_loc, cache_seqlens=cache_seqlens).items():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(seq_lens.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_step_meta(ctx, _ptr(seq_lens), _ptr(page_table), _ptr(positions),
                                             _ptr(cache_loc), _ptr(cache_seqlens),
                                             ctypes.c_void_p(handle)))


def mi355x_gated_attn_workspace_init(ctx, workspace, stream=None):
    """Zero a new workspace's counters (once, before its first step)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_workspace_init(ctx, _ptr(workspace), _nbytes(workspace),
                                                  ctypes.c_void_p(handle)))


def mi355x_gated_attn_destroy(ctx):
    lib().mi355x_gated_attn_destroy(ctx)


def mi355x_gated_attn_timing(ctx, enable: bool):
    _check(lib().mi355x_gated_attn_timing(ctx, 1 if enable else 0))


def mi355x_gated_attn_timing_read(ctx):
    """Returns (summed kernel milliseconds, timed steps)."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().mi355x_gated_attn_timing_read(ctx, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class GatedAttnStep:
    """A prepared and planned context plus its device workspace (torch memory)."""

    def __init__(self, cfg: Config, max_context: int, num_splits: int = 0, device: int = 0):
        import torch
        self.cfg = cfg
        self.ctx = mi355x_gated_attn_prepare(cfg, device)
        self.workspace_bytes, self.splits = mi355x_gated_attn_plan(self.ctx, max_context,
                                                                   num_splits)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8,
                                     device=f"cuda:{device}")
        mi355x_gated_attn_workspace_init(self.ctx, self.workspace)

    def q_bytes(self):
        """The q e4m3 codes a step left in the workspace, [B*L, Hq, D]."""
        c = self.cfg
        n = c.batch * c.q_len * c.num_q_heads * c.head_dim
        return self.workspace[:n].view(c.batch * c.q_len, c.num_q_heads, c.head_dim)

    def __call__(self, qkv, positions, cache_loc, cache_seqlens, page_table, seq_lens, k_cache,
                 v_cache, k_scale, v_scale, out, stream=None):
        mi355x_gated_attn_step(self.ctx, qkv, positions, cache_loc, cache_seqlens, page_table,
                               seq_lens, k_cache, v_cache, k_scale, v_scale, out, self.workspace,
                               stream)
        return out

    def sparse(self, qkv, positions, cache_loc, cache_seqlens, page_table, block_idx, k_cache,
               v_cache, k_scale, v_scale, out, stream=None):
        """One page-list-driven decode step (a config with sparse_block > 0)."""
        mi355x_gated_attn_sparse_step(self.ctx, qkv, positions, cache_loc, cache_seqlens,
                                      page_table, block_idx, k_cache, v_cache, k_scale, v_scale,
                                      out, self.workspace, stream)
        return out

    def sparse_prefill(self, qkv, positions, cache_loc, token_req, num_requests, cache_seqlens,
                       page_table, block_idx, k_cache, v_cache, k_scale, v_scale, out,
                       stream=None):
        """One page-list-driven prefill (a sparse config whose batch counts queries)."""
        mi355x_gated_attn_sparse_prefill_step(self.ctx, qkv, positions, cache_loc, token_req,
                                              num_requests, cache_seqlens, page_table, block_idx,
                                              k_cache, v_cache, k_scale, v_scale, out,
                                              self.workspace, stream)
        return out

    def ragged(self, qkv, positions, cache_loc, cu_seqlens_q, total_q, cache_seqlens, page_table,
               k_cache, v_cache, k_scale, v_scale, out, stream=None):
        """One ragged extend step (a config with q_len > 8 bounding every segment)."""
        mi355x_gated_attn_ragged_step(self.ctx, qkv, positions, cache_loc, cu_seqlens_q, total_q,
                                      cache_seqlens, page_table, k_cache, v_cache, k_scale,
                                      v_scale, out, self.workspace, stream)
        return out

    def meta(self, seq_lens, page_table, positions, cache_loc, cache_seqlens, stream=None):
        """Build the step's positions, cache rows and key counts on the device."""
        mi355x_gated_attn_step_meta(self.ctx, seq_lens, page_table, positions, cache_loc,
                                    cache_seqlens, stream)

    def close(self):
        if self.ctx is not None:
            mi355x_gated_attn_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- per-head QK-norm with an output scale (page "qk_norm") ----------------

def mi355x_qk_norm_supports(dtype: int, head_dim: int) -> bool:
    return bool(lib().mi355x_qk_norm_supports(int(dtype), int(head_dim)))


def mi355x_qk_norm(x, out, M: int, num_heads: int, head_dim: int, x_row_stride: int, dtype: int,
                   eps: float = 1e-5, scale: float = 1.0, stream=None):
    """Raw entry point: x and out are device pointers (ints) or None."""
    _check(lib().mi355x_qk_norm(x, out, int(M), int(num_heads), int(head_dim), int(x_row_stride),
                                int(dtype), ctypes.c_float(eps), ctypes.c_float(scale), stream))


def _qk_dtype(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return MI355X_QKN_BF16
    if dtype == torch.float16:
        return MI355X_QKN_FP16
    return -1


def supports_qk_norm(dtype, head_dim: int) -> bool:
    """Whether qk_norm serves a torch dtype and head_dim (the page's
    supports_qk_norm)."""
    d = _qk_dtype(dtype)
    return d >= 0 and mi355x_qk_norm_supports(d, head_dim)


def qk_norm(x, head_dim: int, eps: float = 1e-5, scale: float = 1.0, out=None, stream=None):
    """The page's qk_norm(x, head_dim, eps, scale): x is [num_tokens,
    num_heads * head_dim] (bf16 or fp16, last dimension contiguous, rows may be
    strided); returns a new contiguous tensor of the same shape and type."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [num_tokens, num_heads * head_dim]")
    if x.stride(1) != 1:
        raise ValueError("x must be contiguous along its last dim")
    M, N = x.shape
    if N % head_dim:
        raise ValueError(f"{N} is not a multiple of head_dim={head_dim}")
    d = _qk_dtype(x.dtype)
    if d < 0 or not mi355x_qk_norm_supports(d, head_dim):
        raise GatedAttnError(MI355X_GA_UNSUPPORTED, f"qk_norm does not serve {x.dtype} with head_dim {head_dim}")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if M == 0:
        return out
    s = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    mi355x_qk_norm(x.data_ptr(), out.data_ptr(), M, N // head_dim, head_dim, x.stride(0), d, eps,
                   scale, s)
    return out
