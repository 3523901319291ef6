"""Pins of the oracle's step metadata (positions, cache rows, key counts from
the cached lengths and the page table; page "012-attention-local-splits.py",
`Inputs`; padded slots from page "msa.py", update_msa_decode_cg_meta):
hand-derived cases, and agreement with the seeded generator, which forms the
same fields by its own numpy code when it builds a step's inputs."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _cfg(batch, q_len, page_size, max_pages, num_pages=1 << 20):
    return oracle.Config(batch=batch, q_len=q_len, num_q_heads=16, num_kv_heads=2, head_dim=64,
                         page_size=page_size, window=0, max_pages=max_pages, num_pages=num_pages,
                         rope_theta=0.0, sm_scale=0.125, kv_scale=1.0)


def test_hand_derived_cases(orc):
    cases = json.load(open(os.path.join(HERE, "golden", "meta_cases.json")))["cases"]
    for c in cases:
        B = len(c["seq_lens"])
        cfg = _cfg(B, c["q_len"], c["page_size"], c["max_pages"])
        pos, loc, cs = oracle.step_meta(cfg, np.array(c["seq_lens"], np.int32),
                                        np.array(c["page_table"], np.int32))
        np.testing.assert_array_equal(pos, c["positions"], err_msg=c["why"])
        np.testing.assert_array_equal(loc, c["cache_loc"], err_msg=c["why"])
        np.testing.assert_array_equal(cs, c["cache_seqlens"], err_msg=c["why"])


@pytest.mark.parametrize("kw", [
    dict(batch=4, q_len=1), dict(batch=3, q_len=8, page_size=4), dict(batch=5, q_len=3, page_size=64),
    dict(batch=2, q_len=2, table="identity"),
])
def test_agrees_with_the_generator(orc, kw):
    x = synth.make_inputs(synth.small(**kw))
    w = x.w
    cfg = _cfg(w.batch, w.q_len, w.page_size, x.max_pages, x.num_pages)
    pos, loc, cs = oracle.step_meta(cfg, x.seq_lens, x.page_table)
    np.testing.assert_array_equal(pos, x.positions)
    np.testing.assert_array_equal(loc, x.cache_loc)
    np.testing.assert_array_equal(cs, x.cache_seqlens)


def test_padded_slots_and_the_headline_batch(orc):
    x = synth.make_inputs(synth.WORKLOADS["swa_decode"])
    w = x.w
    seq = x.seq_lens.copy()
    seq[[3, 17]] = 0
    cfg = _cfg(w.batch, w.q_len, w.page_size, x.max_pages, x.num_pages)
    pos, loc, cs = oracle.step_meta(cfg, seq, x.page_table)
    keep = np.ones(w.batch, bool)
    keep[[3, 17]] = False
    np.testing.assert_array_equal(pos[keep], x.positions[keep])
    np.testing.assert_array_equal(loc[keep], x.cache_loc[keep])
    np.testing.assert_array_equal(cs[keep], x.cache_seqlens[keep])
    assert np.all(pos[~keep] == 0) and np.all(loc[~keep] == -1) and np.all(cs[~keep] == 0)
