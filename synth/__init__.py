"""Seeded synthetic inputs for the gated-attention decode / verify step.

This module is shared by the tests, the benchmark and the smoke check; it holds
none of the step's arithmetic.  Values are drawn with numpy's PCG64 and cast to
bf16 / float8 e4m3 with torch's CPU casts (library routines), so the oracle and
the HIP library receive identical bytes.

The five named workloads are the decode and verify shapes of the page
"012-attention-local-splits.py" (Config: Hq 16 and Hkv 2 per GPU under TP8,
head_dim 64, page_size 1 as served or 64 in tests, window 2048 with RoPE theta
500000 on sliding layers, sm_scale 1/8, cache scales 1 unless set), with the
batch, context and distribution recipe of each case listed below.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    seq_lo: int            # cached tokens per request, drawn uniformly in [seq_lo, seq_hi]
    seq_hi: int
    window: int            # 0 = full causal attention
    rope_theta: float      # 0 = no RoPE
    page_size: int = 1
    kv_scale: float = 1.0
    qkv_std: float = 1.0
    q_scale: float = 1.0   # q's norm output scale (page "qk_norm"); 1 = page 1's prologue
    sparse_block: int = 0  # > 0: block-sparse decode (page "msa.py") over blocks of this many keys
    sparse_topk: int = 0   # blocks each KV head's list selects
    table: str = "perm"    # "identity": page j of request b is page b*max + j; "perm": shuffled
    num_q_heads: int = 16
    num_kv_heads: int = 2
    head_dim: int = 64
    sm_scale: float = 0.125
    spare_pages: int = 0   # pool pages no request references
    seed: int = 0
    ragged_lo: int = 0     # > 0: a ragged batch, request b keeping ragged_lens(w)[b] new tokens
    prefill_block: int = 0  # > 0: block-sparse prefill (page "msa.py") over blocks of this many keys
    prefill_topk: int = 0   # blocks each query's list selects per KV head

    @property
    def width(self) -> int:
        return (2 * self.num_q_heads + 2 * self.num_kv_heads) * self.head_dim


# The five workloads, each with its fixed seed (1000 + index).
WORKLOADS = {
    # batch 1, one token, 512 cached, full attention, identity page table
    "tiny_decode": Workload("tiny_decode", 1, 1, 512, 512, 0, 0.0, table="identity", seed=1001),
    # batch 32, one token, 4k-16k cached, window 2048, RoPE 5e5, shuffled rows
    "swa_decode": Workload("swa_decode", 32, 1, 4096, 16384, 2048, 500000.0, seed=1002),
    # batch 64, one token, 32768 cached, full attention
    "full_decode_32k": Workload("full_decode_32k", 64, 1, 32768, 32768, 0, 0.0, seed=1003),
    # batch 32, 8-token verify block, 8k-32k cached, window 2048, RoPE 5e5
    "swa_verify": Workload("swa_verify", 32, 8, 8192, 32768, 2048, 500000.0, seed=1004),
    # batch 8, 8-token block, 64k-128k cached, page 64, cache scales 0.5, qkv ~ N(0, 2)
    "paged_scaled_long": Workload("paged_scaled_long", 8, 8, 65536, 131072, 0, 0.0,
                                  page_size=64, kv_scale=0.5, qkv_std=math.sqrt(2.0),
                                  seed=1005),
}
ORDER = ["tiny_decode", "swa_decode", "full_decode_32k", "swa_verify", "paged_scaled_long"]

# Supplementary benchmark rows: the headline's shape with every request at
# 16,384 cached tokens, windowed and full (the "16k ctx" of the headline read
# either way).  Not part of ORDER.
SUPPLEMENTARY = {
    "swa_decode_16k": Workload("swa_decode_16k", 32, 1, 16384, 16384, 2048, 500000.0, seed=1006),
    "full_decode_16k": Workload("full_decode_16k", 32, 1, 16384, 16384, 0, 500000.0, seed=1007),
}
WORKLOADS.update(SUPPLEMENTARY)

# Page-list-driven (top-k block-sparse) decode, page "msa.py": blocks of 128
# keys, one page each (the page's block_size_k == page_size == 128), 16
# selected per KV head (2,048 keys, the headline's window), 8k-32k cached, no
# window, no RoPE.  Synthetic block lists (the real ones come from a trained
# indexer): see make_block_lists.
SPARSE = {
    "sparse_decode": Workload("sparse_decode", 32, 1, 8192, 32768, 0, 0.0, page_size=128,
                              sparse_block=128, sparse_topk=16, seed=1008),
}
WORKLOADS.update(SPARSE)

# Extend / prefill blocks (q_len >> 8) through the same step: a 1,024-token
# chunk per request over an 8k-16k prefix with page 1's window and RoPE, and
# page 2's prefill shape (blocks of 128 keys, one page each, causal from the
# prefix length) as 2,048 new tokens over a 4k-8k prefix, full attention.
EXTEND = {
    "swa_extend": Workload("swa_extend", 4, 1024, 8192, 16384, 2048, 500000.0, seed=1009),
    "full_extend": Workload("full_extend", 2, 2048, 4096, 8192, 0, 0.0, page_size=128, seed=1010),
    # a speculative block just past the verify kernel's 8 tokens over a long
    # full-attention context: 8 units, so the plan splits their keys
    "verify16_32k": Workload("verify16_32k", 4, 16, 32768, 32768, 0, 0.0, seed=1011),
    # page 2's ragged prefill batch: 8 requests keeping 1..1,024 new tokens each
    # (seeded, uniform) over an 8k-16k prefix, page 1's window and RoPE
    "ragged_extend": Workload("ragged_extend", 8, 1024, 8192, 16384, 2048, 500000.0,
                              ragged_lo=1, seed=1012),
    # page 2's block-sparse prefill: 2 requests x 1,024 new tokens over 8k-16k
    # prefixes, every token a query selecting 16 blocks of 128 keys (one page
    # each) per KV head, no window, no RoPE
    "sparse_prefill": Workload("sparse_prefill", 2, 1024, 8192, 16384, 0, 0.0, page_size=128,
                               prefill_block=128, prefill_topk=16, seed=1013),
}
WORKLOADS.update(EXTEND)


@dataclass
class Inputs:
    w: Workload
    qkv: np.ndarray            # uint16 bf16 bits [B, L, width]
    positions: np.ndarray      # int64 [B*L]
    cache_loc: np.ndarray      # int64 [B*L]
    cache_seqlens: np.ndarray  # int32 [B]  = seq_lens + L
    cu_seqlens_q: np.ndarray   # int32 [B+1] = 0, L, 2L, ...
    page_table: np.ndarray     # int32 [B, max_pages], -1 unused
    seq_lens: np.ndarray       # int32 [B]
    k_cache: np.ndarray        # uint8 e4m3 codes [num_pages*P, Hkv, D]
    v_cache: np.ndarray
    k_scale: float
    v_scale: float
    max_pages: int
    num_pages: int
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.w.batch * self.w.q_len


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> float8_e4m3fn codes via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _normal_e4m3(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = to_e4m3_codes(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def make_inputs(w: Workload, seed: int | None = None, seq_lens: np.ndarray | None = None,
                max_pages: int | None = None) -> Inputs:
    """Build one step's inputs.

    Recipe: seq_lens ~ U{seq_lo..seq_hi} (or given); cache_seqlens = seq_lens + L;
    each request owns ceil(cache_seqlens/P) pages taken consecutively from the
    identity or a random permutation of the pool; the page_table row tail is -1;
    the new token i of request b sits at position p = seq_lens[b] + i and flat
    cache row page_table[b, p // P] * P + p % P; the pool holds e4m3(N(0,1));
    qkv = bf16(N(0, qkv_std^2)); the cache scales equal kv_scale.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, L, P = w.batch, w.q_len, w.page_size
    if seq_lens is None:
        seq_lens = rng.integers(w.seq_lo, w.seq_hi, size=B, endpoint=True)
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    assert seq_lens.shape == (B,)
    cache_seqlens = (seq_lens + L).astype(np.int32)
    n_pages = (cache_seqlens.astype(np.int64) + P - 1) // P
    if max_pages is None:
        max_pages = int(-(-(max(w.seq_hi, int(seq_lens.max(initial=0))) + L) // P)) + 1
    assert n_pages.max(initial=0) <= max_pages
    num_pages = int(n_pages.sum()) + w.spare_pages
    if w.table == "identity":
        order = np.arange(num_pages, dtype=np.int64)
    else:
        order = rng.permutation(num_pages).astype(np.int64)
    page_table = np.full((B, max_pages), -1, np.int32)
    off = 0
    for b in range(B):
        page_table[b, : n_pages[b]] = order[off: off + n_pages[b]]
        off += int(n_pages[b])
    positions = (seq_lens[:, None].astype(np.int64) + np.arange(L, dtype=np.int64)[None, :])
    rows = page_table[np.arange(B)[:, None], positions // P].astype(np.int64) * P + positions % P
    rows_total = num_pages * P
    k_cache = _normal_e4m3(rng, (rows_total, w.num_kv_heads, w.head_dim))
    v_cache = _normal_e4m3(rng, (rows_total, w.num_kv_heads, w.head_dim))
    qkv = to_bf16_bits(rng.standard_normal((B, L, w.width), dtype=np.float32) * np.float32(w.qkv_std))
    cu = (np.arange(B + 1, dtype=np.int32) * L).astype(np.int32)
    extra = {}
    if w.sparse_block > 0:
        extra["block_idx"] = make_block_lists(rng, cache_seqlens, w.sparse_block, w.sparse_topk,
                                              w.num_kv_heads)
    return Inputs(w=w, qkv=qkv, positions=positions.reshape(-1).copy(),
                  cache_loc=rows.reshape(-1).copy(), cache_seqlens=cache_seqlens,
                  cu_seqlens_q=cu, page_table=page_table, seq_lens=seq_lens,
                  k_cache=k_cache, v_cache=v_cache, k_scale=float(w.kv_scale),
                  v_scale=float(w.kv_scale), max_pages=int(max_pages), num_pages=num_pages,
                  extra=extra)


def ragged_lens(w: Workload) -> np.ndarray:
    """Segment lengths of a ragged workload: uniform in [ragged_lo, q_len], seeded."""
    rng = np.random.default_rng(w.seed + 1)
    return rng.integers(w.ragged_lo, w.q_len, size=w.batch, endpoint=True).astype(np.int32)


def ragged(x: Inputs, lens: np.ndarray) -> dict:
    """A packed ragged batch cut from uniform inputs x (q_len L): request b keeps
    its first lens[b] new tokens (0 <= lens[b] <= L), so its cached length
    becomes seq_lens[b] + lens[b] while positions, cache rows and projection
    rows stay those of x.  Returns qkv [total_q, width], positions, cache_loc
    [total_q], cache_seqlens [B], cu_seqlens_q [B+1] (0, then running sums of
    lens) and total_q."""
    B, L = x.w.batch, x.w.q_len
    lens = np.asarray(lens, np.int32)
    assert lens.shape == (B,) and lens.min(initial=0) >= 0 and lens.max(initial=0) <= L
    idx = np.concatenate([b * L + np.arange(int(lens[b]), dtype=np.int64) for b in range(B)]
                         + [np.zeros(0, np.int64)])
    width = x.qkv.shape[-1]
    return dict(qkv=np.ascontiguousarray(x.qkv.reshape(B * L, width)[idx]),
                positions=np.ascontiguousarray(x.positions[idx]),
                cache_loc=np.ascontiguousarray(x.cache_loc[idx]),
                cache_seqlens=(x.seq_lens + lens).astype(np.int32),
                cu_seqlens_q=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                total_q=int(lens.sum()))


def make_block_lists(rng: np.random.Generator, cache_seqlens: np.ndarray, block_size: int,
                     topk: int, num_kv_heads: int) -> np.ndarray:
    """int32 [Hkv, B, topk] top-k block lists: per (KV head, request) the
    block holding the query's own position (cache_seqlens - 1) and distinct
    other blocks of the request drawn uniformly, min(topk, blocks) in all, in
    random order, padded with -1."""
    B = len(cache_seqlens)
    out = np.full((num_kv_heads, B, topk), -1, np.int32)
    for g in range(num_kv_heads):
        for b in range(B):
            n = int(-(-int(cache_seqlens[b]) // block_size))
            if n <= 0:
                continue
            others = rng.choice(n - 1, size=min(topk, n) - 1, replace=False) if n > 1 else []
            sel = np.concatenate([[n - 1], np.asarray(others, np.int64)])
            out[g, b, :len(sel)] = rng.permutation(sel)
    return out


def sparse_prefill(x: Inputs, block_size: int, topk: int, seed: int) -> dict:
    """Page-list-driven prefill inputs cut from uniform inputs x (B requests, L
    new tokens each): every new token is a query of its own — token_req its
    request, cache_seqlens its position + 1 — with per-KV-head block lists
    drawn by make_block_lists at that length ([Hkv, B*L, topk]).  Also the
    page table expanded to a row per query (page_table_q) for a plain batch of
    one-token queries."""
    B, L = x.w.batch, x.w.q_len
    T = B * L
    token_req = np.repeat(np.arange(B, dtype=np.int32), L)
    cs = (x.positions + 1).astype(np.int32)
    rng = np.random.default_rng(seed)
    return dict(qkv=np.ascontiguousarray(x.qkv.reshape(T, 1, -1)), positions=x.positions,
                cache_loc=x.cache_loc, token_req=token_req, cache_seqlens=cs,
                page_table_q=np.ascontiguousarray(x.page_table[token_req]),
                block_idx=make_block_lists(rng, cs, block_size, topk, x.w.num_kv_heads))


def small(name: str = "small", batch: int = 3, q_len: int = 1, seq_lo: int = 40, seq_hi: int = 300,
          window: int = 0, rope_theta: float = 0.0, page_size: int = 1, kv_scale: float = 1.0,
          qkv_std: float = 1.0, table: str = "perm", sm_scale: float = 0.125,
          num_q_heads: int = 16, num_kv_heads: int = 2, spare_pages: int = 3,
          seed: int = 7, q_scale: float = 1.0) -> Workload:
    """A workload small enough for the oracle to finish in well under a second."""
    return Workload(name, batch, q_len, seq_lo, seq_hi, window, rope_theta, page_size=page_size,
                    kv_scale=kv_scale, qkv_std=qkv_std, table=table, sm_scale=sm_scale,
                    num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    spare_pages=spare_pages, seed=seed, q_scale=q_scale)


def with_seed(w: Workload, seed: int) -> Workload:
    return replace(w, seed=seed)



# ---- inputs of the per-head QK-norm (page "qk_norm") --------------------------

def to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bit patterns via torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class QkNormWorkload:
    name: str
    rows: int          # tokens
    num_heads: int
    head_dim: int
    row_stride: int    # elements between rows of x (>= num_heads * head_dim)
    dtype: str         # "bf16" or "fp16"
    scale: float       # the output scale
    std: float = 1.0   # x ~ N(0, std^2), cast once
    eps: float = 1e-5
    seed: int = 0


# The page's qk_norm reads a strided view such as the q columns of the fused
# projection row (2304 wide per GPU on page "012-attention-local-splits.py",
# q first); the q scale 5.473 is that page's query factor, folded into q.
QK_NORM_WORKLOADS = {
    "qk_norm_q_prefill": QkNormWorkload("qk_norm_q_prefill", 16384, 16, 64, 2304, "bf16", 5.473,
                                        seed=2001),
    "qk_norm_q_decode": QkNormWorkload("qk_norm_q_decode", 32, 16, 64, 2304, "bf16", 5.473,
                                       seed=2002),
    "qk_norm_fp16_d256": QkNormWorkload("qk_norm_fp16_d256", 8192, 8, 256, 2048, "fp16", 1.0,
                                        seed=2003),
}


def make_qk_norm_input(w: QkNormWorkload, rows: int | None = None) -> np.ndarray:
    """uint16 bit patterns [rows, row_stride] of N(0, std^2) values in w.dtype."""
    rng = np.random.default_rng(w.seed)
    n = w.rows if rows is None else rows
    x = rng.standard_normal((n, w.row_stride), dtype=np.float32) * np.float32(w.std)
    return to_bf16_bits(x) if w.dtype == "bf16" else to_fp16_bits(x)
