"""Pins of the oracle's page-list-driven (top-k block-sparse) decode (page
"msa.py": msa_sparse_decode_main / build_msa_decode_meta: one decode query per
request at its last cached position, keys taken through each KV head's list of
selected blocks, -1 padding).  Checked against designed closed forms, torch's
float64 softmax over an explicit mask, and the dense attention (itself pinned)
when every block is selected."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth


def _cfg(x):
    w = x.w
    return oracle.Config(batch=w.batch, q_len=1, page_size=w.page_size, window=0,
                         max_pages=x.max_pages, num_pages=x.num_pages, rope_theta=0.0,
                         sm_scale=w.sm_scale, kv_scale=w.kv_scale)


def _inputs(batch=3, block=16, topk=5, page_size=4, seq_lo=30, seq_hi=200, seed=3):
    w = synth.small(batch=batch, q_len=1, page_size=page_size, seq_lo=seq_lo, seq_hi=seq_hi,
                    seed=seed)
    w = dataclasses.replace(w, sparse_block=block, sparse_topk=topk)
    return synth.make_inputs(w)


def _rows(x, b, keys):
    P = x.w.page_size
    keys = np.asarray(keys, np.int64)
    return x.page_table[b, keys // P].astype(np.int64) * P + keys % P


def _visible(x, lists, b, g, block):
    cs = int(x.cache_seqlens[b])
    keys = set()
    for j in lists[g, b]:
        if j >= 0:
            keys.update(range(j * block, min((j + 1) * block, cs)))
    return sorted(keys)


def _q(x, rng):
    T = x.w.batch
    return synth.to_e4m3_codes(rng.standard_normal((T, 16, 64)).astype(np.float32))


@pytest.mark.parametrize("block,topk,page_size", [(16, 5, 4), (32, 3, 32), (8, 40, 1)])
def test_uniform_weights_reveal_exactly_the_selected_keys(block, topk, page_size):
    """K = 0 makes every weight equal; V row of key j holds the bits of j (and a
    KV-head marker), so each output is the exact share of visible keys with
    that bit set: the block -> key map, the padding, the clamp below
    cache_seqlens and the per-head lists all show."""
    x = _inputs(block=block, topk=topk, page_size=page_size)
    lists = x.extra["block_idx"].copy()
    lists[1, 0, -1] = -1  # some padding
    B = x.w.batch
    kc = np.zeros_like(x.k_cache)
    vc = np.zeros_like(x.v_cache)
    one = synth.to_e4m3_codes(np.array([1.0], np.float32))[0]
    for b in range(B):
        cs = int(x.cache_seqlens[b])
        rows = _rows(x, b, np.arange(cs))
        for bit in range(12):
            on = ((np.arange(cs) >> bit) & 1).astype(bool)
            vc[rows[on], :, bit] = one
        vc[rows, 1, 40] = one  # KV head 1 marker
    q = _q(x, np.random.default_rng(1))
    o = oracle.sparse_attention(_cfg(x), q, kc, vc, x.page_table, x.cache_seqlens, lists, block)
    for b in range(B):
        for h in range(16):
            g = h // 8
            keys = np.array(_visible(x, lists, b, g, block))
            want = np.zeros(64)
            for bit in range(12):
                want[bit] = np.mean((keys >> bit) & 1)
            want[40] = 1.0 if g == 1 else 0.0
            assert np.allclose(o[b, h], want, atol=1e-12), (b, h)


def test_matches_torch_softmax_over_the_block_mask():
    x = _inputs(batch=4, block=16, topk=6, page_size=8, seq_hi=300, seed=9)
    lists = x.extra["block_idx"].copy()
    lists[0, 2, 3:] = -1
    q = _q(x, np.random.default_rng(2))
    o = oracle.sparse_attention(_cfg(x), q, x.k_cache, x.v_cache, x.page_table, x.cache_seqlens,
                                lists, 16)
    dec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double()
    for b in range(x.w.batch):
        cs = int(x.cache_seqlens[b])
        rows = _rows(x, b, np.arange(cs))
        for g in range(2):
            vis = np.zeros(cs, bool)
            vis[_visible(x, lists, b, g, 16)] = True
            K = dec[torch.from_numpy(x.k_cache[rows, g].astype(np.int64))]
            V = dec[torch.from_numpy(x.v_cache[rows, g].astype(np.int64))]
            Q = dec[torch.from_numpy(q[b, 8 * g:8 * g + 8].astype(np.int64))]
            s = (Q @ K.T) * x.w.sm_scale
            s[:, torch.from_numpy(~vis)] = -torch.inf
            ref = torch.softmax(s, dim=-1) @ V
            assert np.allclose(o[b, 8 * g:8 * g + 8], ref.numpy(), atol=1e-12, rtol=1e-12)


def test_every_block_selected_is_dense_attention():
    x = _inputs(batch=3, block=16, topk=64, page_size=4, seq_hi=250, seed=4)
    B = x.w.batch
    lists = np.full((2, B, 64), -1, np.int32)
    for b in range(B):
        n = -(-int(x.cache_seqlens[b]) // 16)
        for g in range(2):
            lists[g, b, :n] = np.random.default_rng(b + 10 * g).permutation(n)
    q = _q(x, np.random.default_rng(5))
    o = oracle.sparse_attention(_cfg(x), q, x.k_cache, x.v_cache, x.page_table, x.cache_seqlens,
                                lists, 16)
    dense = oracle.attention(_cfg(x), q, x.k_cache, x.v_cache, x.page_table, x.cache_seqlens,
                             x.k_scale, x.v_scale)
    assert np.allclose(o.reshape(dense.shape), dense, atol=1e-12, rtol=1e-12)


def test_repeated_blocks_add_nothing_and_empty_lists_give_zero():
    x = _inputs(batch=2, block=16, topk=4, seed=6)
    lists = x.extra["block_idx"].copy()
    dup = lists.copy()
    dup[:, :, 1] = dup[:, :, 0]
    dup[:, :, 2] = -1
    ref = lists.copy()
    ref[:, :, 1] = -1
    ref[:, :, 2] = -1
    q = _q(x, np.random.default_rng(7))
    args = (_cfg(x), q, x.k_cache, x.v_cache, x.page_table, x.cache_seqlens)
    assert np.array_equal(oracle.sparse_attention(*args, dup, 16), oracle.sparse_attention(*args, ref, 16))
    none = np.full_like(lists, -1)
    assert np.all(oracle.sparse_attention(*args, none, 16) == 0.0)
