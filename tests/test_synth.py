"""The seeded input generator keeps the cross-field invariants the step relies
on (page "012-attention-local-splits.py", Inputs: cache_seqlens = seq_lens + L,
each new token at position seq_lens + i, its cache row given by the page table,
cu_seqlens_q = 0, L, 2L, ..., -1 in the page table's unused tail)."""
import numpy as np
import pytest

import synth


def _check(x):
    w = x.w
    B, L, P = w.batch, w.q_len, w.page_size
    assert np.all(x.seq_lens >= w.seq_lo) and np.all(x.seq_lens <= w.seq_hi)
    np.testing.assert_array_equal(x.cache_seqlens, x.seq_lens + L)
    np.testing.assert_array_equal(x.cu_seqlens_q, np.arange(B + 1) * L)
    pos = x.positions.reshape(B, L)
    np.testing.assert_array_equal(pos, x.seq_lens[:, None] + np.arange(L)[None, :])
    # each new token's cache row is the row the page table gives its position
    rows = x.page_table[np.arange(B)[:, None], pos // P].astype(np.int64) * P + pos % P
    np.testing.assert_array_equal(x.cache_loc.reshape(B, L), rows)
    used = []
    for b in range(B):
        n = -(-int(x.cache_seqlens[b]) // P)
        assert np.all(x.page_table[b, :n] >= 0) and np.all(x.page_table[b, :n] < x.num_pages)
        assert np.all(x.page_table[b, n:] == -1) and n < x.max_pages  # a -1 tail exists
        used.append(x.page_table[b, :n])
    used = np.concatenate(used)
    assert len(np.unique(used)) == len(used)  # no page shared between requests
    assert x.k_cache.shape == (x.num_pages * P, w.num_kv_heads, w.head_dim)
    for c in (x.k_cache, x.v_cache):
        assert not np.any((c & 0x7F) == 0x7F)  # no NaN codes in the pool
    assert x.qkv.shape == (B, L, w.width)
    assert not np.any((x.qkv & 0x7F80) == 0x7F80)  # finite bf16


@pytest.mark.parametrize("kw", [
    dict(batch=3, q_len=1), dict(batch=4, q_len=8, page_size=4), dict(batch=2, q_len=3, page_size=64),
    dict(batch=5, q_len=2, table="identity"),
])
def test_small_workloads_keep_the_invariants(kw):
    _check(synth.make_inputs(synth.small(**kw)))


@pytest.mark.parametrize("name", ["tiny_decode", "swa_decode", "paged_scaled_long"])
def test_named_workloads_keep_the_invariants(name):
    x = synth.make_inputs(synth.WORKLOADS[name])
    _check(x)


def test_generation_is_deterministic():
    w = synth.small(batch=3, q_len=2, page_size=4)
    a, b = synth.make_inputs(w), synth.make_inputs(w)
    for f in ("qkv", "positions", "cache_loc", "page_table", "k_cache", "v_cache"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_identity_table_for_the_tiny_workload():
    x = synth.make_inputs(synth.WORKLOADS["tiny_decode"])
    np.testing.assert_array_equal(x.page_table[0, :513], np.arange(513))
    assert x.cache_loc[0] == 512 and x.positions[0] == 512


def test_ragged_batch_cut_and_its_reference():
    """synth.ragged keeps each request's first lens[b] tokens with their own
    positions, cache rows and projection rows, and cache_seqlens = seq_lens +
    lens; the request-by-request oracle composition used for ragged parity
    equals the oracle's batch step when every segment is at the bound, and a
    request's rows equal a batch of that request alone at its length."""
    from gpu_support import Reference, ragged_reference
    w = synth.small(name="rg", batch=3, q_len=12, window=7, rope_theta=500000.0, page_size=4,
                    seq_lo=20, seq_hi=60)
    x = synth.make_inputs(w, seed=5)
    lens = np.array([12, 5, 0], np.int32)
    r = synth.ragged(x, lens)
    assert r["total_q"] == 17 and list(r["cu_seqlens_q"]) == [0, 12, 17, 17]
    assert list(r["cache_seqlens"]) == list(x.seq_lens + lens)
    np.testing.assert_array_equal(r["positions"][12:], x.positions[12:17])
    np.testing.assert_array_equal(r["qkv"][12:], x.qkv.reshape(36, -1)[12:17])
    full = synth.ragged(x, np.full(3, 12, np.int32))
    q, k, v, out = ragged_reference(x, full, [12, 12, 12])
    ref = Reference(x)
    np.testing.assert_array_equal(q, ref.q)
    np.testing.assert_array_equal(k, ref.k_cache)
    np.testing.assert_array_equal(out, ref.outputs().reshape(36, -1))
    # request 1 alone at length 5
    w1 = synth.small(name="rg1", batch=1, q_len=5, window=7, rope_theta=500000.0, page_size=4,
                     seq_lo=20, seq_hi=60)
    x1 = synth.make_inputs(w1, seed=5, seq_lens=x.seq_lens[1:2])
    x1.qkv = np.ascontiguousarray(x.qkv[1:2, :5])
    x1.page_table = np.ascontiguousarray(x.page_table[1:2])
    x1.positions = np.ascontiguousarray(x.positions[12:17])
    x1.cache_loc = np.ascontiguousarray(x.cache_loc[12:17])
    x1.k_cache, x1.v_cache = x.k_cache, x.v_cache
    x1.max_pages, x1.num_pages = x.max_pages, x.num_pages
    _, _, _, out_r = ragged_reference(x, r, lens)
    np.testing.assert_array_equal(out_r[12:], Reference(x1).outputs().reshape(5, -1))
