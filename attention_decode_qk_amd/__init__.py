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
# MI355X_GA_LIB may name another build of the same library (the host-sanitized
# one of the sanitizer tests); by default the in-tree product library.
LIB_PATH = os.environ.get("MI355X_GA_LIB") or os.path.join(HERE, "libmi355x_gated_attn.so")

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
            "mi355x_gated_attn_ragged_step", "mi355x_gated_attn_sparse_prefill_step",
            "mi355x_gated_attn_step_noalloc", "mi355x_gated_attn_page_table"]

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
        L.mi355x_gated_attn_step_noalloc.argtypes = [P] * 13
        L.mi355x_gated_attn_step_meta.argtypes = [P] * 7
        L.mi355x_gated_attn_page_table.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64] + [P] * 6
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


# The configuration and device of every live context, so that the launch
# wrappers can check each tensor against them before the C ABI sees a pointer.
_CTX = {}


def mi355x_gated_attn_prepare(cfg: Config, device: int = 0) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    _check(lib().mi355x_gated_attn_prepare(ctypes.byref(cfg), device, ctypes.byref(ctx)))
    _CTX[ctx.value] = (Config.from_buffer_copy(cfg), int(device))
    return ctx


def _ctx_key(ctx):
    return ctx.value if isinstance(ctx, ctypes.c_void_p) else ctx


def _dt(*names):
    import torch
    return tuple(getattr(torch, n) for n in names if hasattr(torch, n))


def _check_tensors(specs, device):
    """specs: (name, tensor, dtypes, numel, min_numel, required) per argument.
    Presence, dtype and size of every tensor are checked first, then device
    and layout (so that a wrong dtype or size is named even on the host);
    raises ValueError naming the argument."""
    for name, t, dtypes, numel, min_numel, required in specs:
        if t is None:
            if required:
                raise ValueError(f"{name} is required")
            continue
        if t.dtype not in dtypes:
            raise ValueError(f"{name}: dtype {t.dtype} is not one of "
                             f"{', '.join(str(d) for d in dtypes)}")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{name}: {t.numel()} elements, the configuration needs {numel}")
        if min_numel is not None and t.numel() < min_numel:
            raise ValueError(f"{name}: {t.numel()} elements, the configuration needs at least "
                             f"{min_numel}")
    for name, t, *_ in specs:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if device is not None and t.device.index != device:
            raise ValueError(f"{name} is on cuda:{t.device.index}, the context on cuda:{device}")


def _ctx_entry(ctx):
    entry = _CTX.get(_ctx_key(ctx))
    if entry is None:
        raise ValueError("unknown or destroyed context")
    return entry


def _step_specs(c, tokens, qkv, positions, cache_loc, cache_seqlens, page_table, k_cache, v_cache,
                k_scale, v_scale, out, workspace, page_rows=None, seq_lens=None):
    """Specs of the tensors every step variant takes, against config c: tokens =
    the step's new tokens (B*L, or total_q for a ragged batch), page_rows = rows
    of page_table (B unless stated)."""
    two = _dt("bfloat16", "int16", "uint16")
    one = _dt("uint8", "int8", "float8_e4m3fn")
    i32, i64, f32 = _dt("int32"), _dt("int64"), _dt("float32")
    width = (2 * c.num_q_heads + 2 * c.num_kv_heads) * c.head_dim
    rows = c.batch if page_rows is None else page_rows
    cache = c.num_pages * c.page_size * c.num_kv_heads * c.head_dim
    scaled = c.kv_scale != 1.0
    per_tok = (lambda n: n * tokens) if tokens else (lambda n: None)  # no token: none is read
    return [("qkv", qkv, two, per_tok(width), None, True),
            ("positions", positions, i64, per_tok(1), None, c.rope_theta != 0.0),
            ("cache_loc", cache_loc, i64, per_tok(1), None, True),
            ("cache_seqlens", cache_seqlens, i32, c.batch, None, True),
            ("page_table", page_table, i32, rows * c.max_pages, None, True),
            ("seq_lens", seq_lens, i32, c.batch, None, False),
            ("k_cache", k_cache, one, None, cache, True),
            ("v_cache", v_cache, one, None, cache, True),
            ("k_scale", k_scale, f32, 1, None, scaled),
            ("v_scale", v_scale, f32, 1, None, scaled),
            ("out", out, two, per_tok(c.num_q_heads * c.head_dim), None, True),
            ("workspace", workspace, _dt("uint8", "int8"), None, None, True)]


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
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    _check_tensors(_step_specs(c, c.batch * c.q_len, qkv, positions, cache_loc, cache_seqlens,
                               page_table, k_cache, v_cache, k_scale, v_scale, out, workspace,
                               seq_lens=seq_lens), dev)
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_step(
        ctx, _ptr(qkv), _ptr(positions), _ptr(cache_loc), _ptr(cache_seqlens), _ptr(page_table),
        _ptr(seq_lens), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        _ptr(workspace), _nbytes(workspace), ctypes.c_void_p(handle)))


def mi355x_gated_attn_step_noalloc(ctx, qkv, positions, cache_loc, cache_seqlens, page_table,
                                   seq_lens, k_cache, v_cache, k_scale, v_scale, out, stream=None):
    """Launch one step without a workspace (the library's static per-GPU scratch
    holds q, the partials and the counters); otherwise as mi355x_gated_attn_step."""
    import torch
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    specs = _step_specs(c, c.batch * c.q_len, qkv, positions, cache_loc, cache_seqlens,
                        page_table, k_cache, v_cache, k_scale, v_scale, out, None,
                        seq_lens=seq_lens)
    _check_tensors([sp for sp in specs if sp[0] != "workspace"], dev)
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_step_noalloc(
        ctx, _ptr(qkv), _ptr(positions), _ptr(cache_loc), _ptr(cache_seqlens), _ptr(page_table),
        _ptr(seq_lens), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        ctypes.c_void_p(handle)))


def mi355x_gated_attn_sparse_step(ctx, qkv, positions, cache_loc, cache_seqlens, page_table,
                                  block_idx, k_cache, v_cache, k_scale, v_scale, out, workspace,
                                  stream=None):
    """Launch one page-list-driven decode step (block_idx: contiguous int32
    device tensor [Hkv, B, topk], -1 padded); otherwise as mi355x_gated_attn_step."""
    import torch
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    specs = _step_specs(c, c.batch * c.q_len, qkv, positions, cache_loc, cache_seqlens, page_table,
                        k_cache, v_cache, k_scale, v_scale, out, workspace)
    specs.append(("block_idx", block_idx, _dt("int32"), c.num_kv_heads * c.batch * c.sparse_topk,
                  None, True))
    _check_tensors(specs, dev)
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
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    if not 0 <= int(total_q) <= c.batch * c.q_len:
        raise ValueError(f"total_q {total_q} outside 0..batch * q_len = {c.batch * c.q_len}")
    specs = _step_specs(c, int(total_q), qkv, positions, cache_loc, cache_seqlens, page_table,
                        k_cache, v_cache, k_scale, v_scale, out, workspace)
    specs.append(("cu_seqlens_q", cu_seqlens_q, _dt("int32"), c.batch + 1, None, True))
    _check_tensors(specs, dev)
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
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    if int(num_requests) < 1:
        raise ValueError(f"num_requests {num_requests} < 1")
    specs = _step_specs(c, c.batch, qkv, positions, cache_loc, cache_seqlens, page_table, k_cache,
                        v_cache, k_scale, v_scale, out, workspace, page_rows=int(num_requests))
    specs += [("token_req", token_req, _dt("int32"), c.batch, None, True),
              ("block_idx", block_idx, _dt("int32"), c.num_kv_heads * c.batch * c.sparse_topk,
               None, True)]
    _check_tensors(specs, dev)
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
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    T = c.batch * c.q_len
    i32, i64 = _dt("int32"), _dt("int64")
    _check_tensors([("seq_lens", seq_lens, i32, c.batch, None, True),
                    ("page_table", page_table, i32, c.batch * c.max_pages, None, True),
                    ("positions", positions, i64, T, None, True),
                    ("cache_loc", cache_loc, i64, T, None, True),
                    ("cache_seqlens", cache_seqlens, i32, c.batch, None, True)], dev)
    if stream is None:
        stream = torch.cuda.current_stream(seq_lens.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_step_meta(ctx, _ptr(seq_lens), _ptr(page_table), _ptr(positions),
                                             _ptr(cache_loc), _ptr(cache_seqlens),
                                             ctypes.c_void_p(handle)))


def mi355x_gated_attn_page_table(ctx, req_to_token, slot_ids, kv_lens, page_table=None,
                                 kv_indices=None, kv_indptr=None, stream=None):
    """Build the step's physical page table on the device (page "msa.py"
    _build_page_table): int32 req_to_token [max_reqs, req_stride], slot_ids
    [B] and kv_lens [B] in; page_table [B, max_pages] (padded with -1) and/or
    kv_indices (packed) with kv_indptr [B+1] out."""
    import torch
    c, dev = _ctx_entry(ctx)
    if c.batch == 0:
        return
    i32 = _dt("int32")
    if req_to_token is None or req_to_token.dim() != 2:
        raise ValueError("req_to_token must be a 2-D int32 device tensor [max_reqs, req_stride]")
    specs = [("req_to_token", req_to_token, i32, None, None, True),
             ("slot_ids", slot_ids, i32, c.batch, None, True),
             ("kv_lens", kv_lens, i32, c.batch, None, True),
             ("page_table", page_table, i32, c.batch * c.max_pages, None, False),
             ("kv_indices", kv_indices, i32, None, None, False),
             ("kv_indptr", kv_indptr, i32, c.batch + 1, None, kv_indices is not None)]
    _check_tensors(specs, dev)
    if stream is None:
        stream = torch.cuda.current_stream(req_to_token.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_page_table(
        ctx, _ptr(req_to_token), req_to_token.shape[1], req_to_token.shape[0], _ptr(slot_ids),
        _ptr(kv_lens), _ptr(page_table), _ptr(kv_indices), _ptr(kv_indptr),
        ctypes.c_void_p(handle)))


def mi355x_gated_attn_workspace_init(ctx, workspace, stream=None):
    """Zero a new workspace's counters (once, before its first step)."""
    import torch
    _, dev = _ctx_entry(ctx)
    _check_tensors([("workspace", workspace, _dt("uint8", "int8"), None, None, True)], dev)
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(lib().mi355x_gated_attn_workspace_init(ctx, _ptr(workspace), _nbytes(workspace),
                                                  ctypes.c_void_p(handle)))


def mi355x_gated_attn_destroy(ctx):
    _CTX.pop(_ctx_key(ctx), None)
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
