"""Shared helpers of the GPU parity tests: run one step through the C ABI on
cuda:0 and the oracle on the same seeded inputs, and compare to the stated bar
(cache and q bytes exact but for one e4m3 code on at most 0.1% of written
elements; outputs within 2e-2 absolute + 2e-2 relative)."""
from __future__ import annotations

import numpy as np
import torch

import attention_decode_qk_amd as ga
import oracle
import synth

ATOL = 2e-2
RTOL = 2e-2


def oracle_config(x: synth.Inputs) -> oracle.Config:
    w = x.w
    return oracle.Config(batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads,
                         num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                         window=w.window, max_pages=x.max_pages, num_pages=x.num_pages,
                         rope_theta=w.rope_theta, sm_scale=w.sm_scale, kv_scale=w.kv_scale,
                         q_scale=w.q_scale)


def abi_config(x: synth.Inputs) -> ga.Config:
    w = x.w
    return ga.make_config(w.batch, w.q_len, w.page_size, w.window, x.max_pages, x.num_pages,
                          w.rope_theta, w.sm_scale, w.kv_scale, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, w.q_scale, w.sparse_block, w.sparse_topk)


def max_context(x: synth.Inputs) -> int:
    """The bound a serving loop knows: the workload's largest cached length + L."""
    return int(max(x.w.seq_hi, int(x.seq_lens.max(initial=0))) + x.w.q_len)


class Device:
    """The step's inputs as device tensors (byte-exact copies)."""

    def __init__(self, x: synth.Inputs, dev="cuda:0"):
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.qkv = t(x.qkv.view(np.int16))
        self.positions = t(x.positions)
        self.cache_loc = t(x.cache_loc)
        self.cache_seqlens = t(x.cache_seqlens)
        self.page_table = t(x.page_table)
        self.seq_lens = t(x.seq_lens)
        self.k_cache = t(x.k_cache)
        self.v_cache = t(x.v_cache)
        self.k_scale = torch.tensor([x.k_scale], dtype=torch.float32, device=dev)
        self.v_scale = torch.tensor([x.v_scale], dtype=torch.float32, device=dev)
        self.out = torch.zeros((x.w.batch, x.w.q_len, x.w.num_q_heads * x.w.head_dim),
                               dtype=torch.int16, device=dev)
        self.block_idx = t(x.extra["block_idx"]) if "block_idx" in x.extra else None

    def run(self, step: ga.GatedAttnStep, stream=None):
        if self.block_idx is not None:  # page-list-driven decode
            step.sparse(self.qkv, self.positions, self.cache_loc, self.cache_seqlens,
                        self.page_table, self.block_idx, self.k_cache, self.v_cache, self.k_scale,
                        self.v_scale, self.out, stream)
            return
        step(self.qkv, self.positions, self.cache_loc, self.cache_seqlens, self.page_table,
             self.seq_lens, self.k_cache, self.v_cache, self.k_scale, self.v_scale, self.out,
             stream)


class Result:
    def __init__(self, out, k_cache, v_cache, q):
        self.out, self.k_cache, self.v_cache, self.q = out, k_cache, v_cache, q


def run_gpu(x: synth.Inputs, num_splits: int = 0, ctx_bound: int | None = None) -> Result:
    step = ga.GatedAttnStep(abi_config(x), ctx_bound or max_context(x), num_splits)
    d = Device(x)
    d.run(step)
    torch.cuda.synchronize()
    r = Result(d.out.cpu().numpy().view(np.uint16), d.k_cache.cpu().numpy(),
               d.v_cache.cpu().numpy(), step.q_bytes().cpu().numpy())
    r.splits = step.splits
    step.close()
    return r


class Reference:
    """Oracle results: q codes, caches after the stores, and per-row outputs."""

    def __init__(self, x: synth.Inputs):
        self.x = x
        self.cfg = oracle_config(x)
        self.k_cache = x.k_cache.copy()
        self.v_cache = x.v_cache.copy()
        self.q = oracle.prologue(self.cfg, x.qkv, x.positions, x.cache_loc, self.k_cache,
                                 self.v_cache, x.k_scale, x.v_scale)

    def outputs(self, sel_t=None, sel_h=None):
        x = self.x
        if "block_idx" in x.extra:  # page-list-driven decode: all rows, then the selection
            o = oracle.sparse_attention(self.cfg, self.q, self.k_cache, self.v_cache,
                                        x.page_table, x.cache_seqlens, x.extra["block_idx"],
                                        x.w.sparse_block, x.k_scale, x.v_scale)
            o = o.reshape(-1, x.w.head_dim)
            if sel_t is not None:
                o = o[np.asarray(sel_t) * x.w.num_q_heads + np.asarray(sel_h)]
            return oracle.epilogue(self.cfg, np.ascontiguousarray(o), x.qkv, sel_t, sel_h)
        o = oracle.attention(self.cfg, self.q, self.k_cache, self.v_cache, x.page_table,
                             x.cache_seqlens, x.k_scale, x.v_scale, sel_t, sel_h)
        return oracle.epilogue(self.cfg, o, x.qkv, sel_t, sel_h)


def ragged_reference(x: synth.Inputs, r: dict, lens):
    """Oracle result of a ragged batch r = synth.ragged(x, lens): the oracle
    step run request by request (batch 1, q_len lens[b]) on one shared copy of
    the caches.  Each request reads and writes only its own pages, so this is
    the batch's result.  Returns q codes [total_q, Hq, D], the caches, and
    outputs bf16 bits [total_q, Hq*D]."""
    k, v = x.k_cache.copy(), x.v_cache.copy()
    qs, outs = [], []
    cu = r["cu_seqlens_q"]
    for b, n in enumerate(lens):
        if n == 0:
            continue
        cfg = oracle_config(x)
        cfg.batch, cfg.q_len = 1, int(n)
        s = slice(int(cu[b]), int(cu[b + 1]))
        q, out, _ = oracle.step(cfg, np.ascontiguousarray(r["qkv"][s]),
                                np.ascontiguousarray(r["positions"][s]),
                                np.ascontiguousarray(r["cache_loc"][s]),
                                np.ascontiguousarray(r["cache_seqlens"][b:b + 1]),
                                np.ascontiguousarray(x.page_table[b:b + 1]), k, v,
                                x.k_scale, x.v_scale)
        qs.append(q)
        outs.append(out.reshape(int(n), -1))
    H, D = x.w.num_q_heads, x.w.head_dim
    q = np.concatenate(qs) if qs else np.zeros((0, H, D), np.uint8)
    out = np.concatenate(outs) if outs else np.zeros((0, H * D), np.uint16)
    return q, k, v, out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .double().numpy()


def assert_codes_match(got: np.ndarray, ref: np.ndarray, written: int, what: str):
    """Exact, except one adjacent-code step on at most 0.1% of written elements."""
    neq = got != ref
    n = int(neq.sum())
    if n:
        step = np.abs(got.astype(np.int32) - ref.astype(np.int32))[neq]
        assert step.max() == 1, f"{what}: {n} codes differ, max step {step.max()}"
        assert n <= 0.001 * written, f"{what}: {n} of {written} codes differ"


def assert_outputs_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str):
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    err = np.abs(g - r)
    bad = err > ATOL + RTOL * np.abs(r)
    assert not np.isnan(g).any(), f"{what}: NaN in output"
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, "
                           f"max err {err.max():.4g}")


def check_full(x: synth.Inputs, res: Result, ref: Reference, what: str):
    """Whole-output comparison (small cases)."""
    T = x.tokens
    written = T * x.w.num_kv_heads * x.w.head_dim
    assert_codes_match(res.q, ref.q, ref.q.size, what + " q")
    assert_codes_match(res.k_cache, ref.k_cache, written, what + " k_cache")
    assert_codes_match(res.v_cache, ref.v_cache, written, what + " v_cache")
    out_ref = ref.outputs().reshape(res.out.shape)
    assert_outputs_close(res.out, out_ref, what + " out")
