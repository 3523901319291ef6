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
