"""GPU parity: the HIP step through the C ABI against the CPU oracle on the same
seeded inputs.  Bar: q and cache bytes exact (one e4m3 code on at most 0.1% of
written elements allowed); bf16 outputs within 2e-2 absolute + 2e-2 relative.
Small cases and the full-size workloads compare every output row and every
cache and q byte; the full-size ones run in the launch configuration the
benchmark times (automatic plan), with the oracle's (token, head) pairs spread
over the host's cores."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_support import (Reference, assert_codes_match, assert_outputs_close, check_full,
                         run_gpu)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = {
    "decode_full": dict(batch=3, q_len=1, window=0),
    "decode_swa_rope": dict(batch=4, q_len=1, window=64, rope_theta=500000.0),
    "decode_window1": dict(batch=2, q_len=1, window=1),
    "decode_window5_page4": dict(batch=3, q_len=1, window=5, page_size=4),
    "verify2": dict(batch=3, q_len=2, window=0, page_size=16),
    "verify3_swa": dict(batch=2, q_len=3, window=40, rope_theta=500000.0),
    "verify5_page3": dict(batch=2, q_len=5, window=0, page_size=3),
    "verify8_swa": dict(batch=3, q_len=8, window=100, rope_theta=500000.0, page_size=1),
    "verify8_scaled_page64": dict(batch=2, q_len=8, window=0, page_size=64, kv_scale=0.5,
                                  qkv_std=1.4142135),
    "decode_qk_factor": dict(batch=2, q_len=1, window=0, sm_scale=5.473 / 8),
    # the query factor carried by q (page "qk_norm"'s output scale), not sm_scale
    "decode_q_scaled": dict(batch=3, q_len=1, window=0, q_scale=5.473),
    "verify3_swa_q_scaled": dict(batch=2, q_len=3, window=40, rope_theta=500000.0, q_scale=5.473),
    "decode_b1_identity": dict(batch=1, q_len=1, window=0, table="identity"),
    "verify8_window1": dict(batch=2, q_len=8, window=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_case_matches_oracle(name):
    w = synth.small(name=name, seq_lo=20, seq_hi=700, **SMALL[name])
    x = synth.make_inputs(w, seed=100 + len(name))
    _say(f"[gpu] small case {name}: B={w.batch} L={w.q_len} W={w.window} P={w.page_size}")
    res = run_gpu(x)
    check_full(x, res, Reference(x), name)


@pytest.mark.parametrize("q_len", range(1, 9))
@pytest.mark.parametrize("grouping", ["short", "long"])
def test_every_q_len_under_both_token_groupings(q_len, grouping):
    """Every q_len with the plan's two token groupings: a short key bound makes
    ceil(L/2) groups of at most two tokens, a long one ceil(L/4) groups of at
    most four (plan(); with the long bound most splits are empty here)."""
    w = synth.small(name="groups", batch=3, q_len=q_len, window=0 if grouping == "long" else 96,
                    rope_theta=500000.0, seq_lo=30, seq_hi=400, page_size=4)
    x = synth.make_inputs(w, seed=300 + q_len)
    bound = 100000 if grouping == "long" else None
    _say(f"[gpu] groups {grouping}: L={q_len}")
    res = run_gpu(x, ctx_bound=bound)
    check_full(x, res, Reference(x), f"groups {grouping} L={q_len}")


@pytest.mark.parametrize("q_len", [1, 8])
def test_large_batch_single_split(q_len):
    """A batch large enough for the plan to give one split per request (more
    units than compute units): each unit is its own combine (no partials, no
    counter)."""
    w = synth.small(name="wide", batch=300, q_len=q_len, window=64, rope_theta=500000.0,
                    seq_lo=30, seq_hi=200, page_size=4)
    x = synth.make_inputs(w, seed=91)
    _say(f"[gpu] large batch B=300 L={q_len}")
    res = run_gpu(x)
    assert res.splits == 1
    check_full(x, res, Reference(x), f"B=300 L={q_len}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 64])
def test_split_count_invariance(splits):
    """Any split count gives oracle-level results (partials merge exactly in form)."""
    w = synth.small(name="splits", batch=3, q_len=4, window=300, rope_theta=500000.0,
                    seq_lo=500, seq_hi=1500, page_size=2)
    x = synth.make_inputs(w, seed=55)
    _say(f"[gpu] split invariance S={splits}")
    res = run_gpu(x, num_splits=splits)
    assert res.splits == splits
    check_full(x, res, Reference(x), f"splits={splits}")


def test_deterministic_and_repeatable():
    w = synth.small(name="det", batch=4, q_len=2, window=0, seq_lo=100, seq_hi=900)
    x = synth.make_inputs(w, seed=3)
    _say("[gpu] determinism")
    a = run_gpu(x)
    b = run_gpu(x)
    np.testing.assert_array_equal(a.out, b.out)
    np.testing.assert_array_equal(a.k_cache, b.k_cache)


def test_value_codec_exhaustive_through_the_store():
    """All 65,536 bf16 patterns pass through the V store (512 tokens x 128
    values): every stored byte equals the oracle's e4m3 code (finite values
    round to nearest even, |x| >= 448 and infinities saturate, NaN -> NaN code)."""
    w = synth.small(name="codec", batch=512, q_len=1, window=4, seq_lo=3, seq_hi=3)
    x = synth.make_inputs(w, seed=1)
    qkv = x.qkv.reshape(512, -1)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    qkv[:, 18 * 64:20 * 64] = pats
    _say("[gpu] exhaustive V codec")
    res = run_gpu(x)
    ref = Reference(x)
    got = res.v_cache[x.cache_loc].reshape(512, 128)
    exp = ref.v_cache[x.cache_loc].reshape(512, 128)
    nan_ref = (exp & 0x7F) == 0x7F
    np.testing.assert_array_equal(got[~nan_ref], exp[~nan_ref])
    assert np.all((got[nan_ref] & 0x7F) == 0x7F)


def test_padded_slot_stores_nothing_and_outputs_zero():
    """A request slot with cache_seqlens 0 and cache_loc -1 (a padded batch slot)
    writes no cache row and produces a zero output; the others are unaffected."""
    w = synth.small(name="pad", batch=3, q_len=1, window=0, seq_lo=50, seq_hi=200)
    x = synth.make_inputs(w, seed=8)
    x.cache_seqlens[1] = 0
    x.cache_loc[1] = -1
    _say("[gpu] padded slot")
    res = run_gpu(x)
    ref = Reference(x)
    np.testing.assert_array_equal(res.k_cache, ref.k_cache)
    np.testing.assert_array_equal(res.v_cache, ref.v_cache)
    assert np.all(res.out[1] == 0)
    out_ref = ref.outputs().reshape(res.out.shape)
    assert_outputs_close(res.out, out_ref, "pad")


@pytest.mark.parametrize("name", synth.ORDER + list(synth.SUPPLEMENTARY))
def test_full_size_workload(name):
    """Every q and cache byte, and every output row, of one full-size step."""
    w = synth.WORKLOADS[name]
    _say(f"[gpu] full-size {name}: generating inputs")
    x = synth.make_inputs(w)
    _say(f"[gpu] full-size {name}: running step (B={w.batch} L={w.q_len})")
    res = run_gpu(x)
    _say(f"[gpu] full-size {name}: splits={res.splits}; oracle prologue")
    ref = Reference(x)
    written = x.tokens * w.num_kv_heads * w.head_dim
    assert_codes_match(res.q, ref.q, ref.q.size, name + " q")
    assert_codes_match(res.k_cache, ref.k_cache, written, name + " k_cache")
    assert_codes_match(res.v_cache, ref.v_cache, written, name + " v_cache")
    _say(f"[gpu] full-size {name}: oracle attention on all {x.tokens * w.num_q_heads} rows "
         f"({oracle.threads()} threads)")
    out_ref = ref.outputs().reshape(res.out.shape)
    assert_outputs_close(res.out, out_ref, name + " out")


def test_full_size_decode_with_the_query_factor_in_q():
    """The headline decode with page "qk_norm"'s output scale carrying the
    query factor (q_scale 5.473, sm_scale 1/8): every q and cache byte, every
    output row."""
    import dataclasses
    w = dataclasses.replace(synth.WORKLOADS["swa_decode"], name="swa_decode_q_scaled", q_scale=5.473)
    _say("[gpu] full-size swa_decode with q_scale 5.473")
    x = synth.make_inputs(w)
    res = run_gpu(x)
    ref = Reference(x)
    written = x.tokens * w.num_kv_heads * w.head_dim
    assert_codes_match(res.q, ref.q, ref.q.size, "q_scaled q")
    assert_codes_match(res.k_cache, ref.k_cache, written, "q_scaled k_cache")
    assert_codes_match(res.v_cache, ref.v_cache, written, "q_scaled v_cache")
    assert_outputs_close(res.out, ref.outputs().reshape(res.out.shape), "q_scaled out")


def test_graph_replay_matches_eager():
    """Capture the step in a HIP graph and replay it several times with eager
    work and synchronisation in between: every replay equals the eager result
    (the page's warning: a decode kernel that is not graph-safe returns silently
    wrong results that compound across replays)."""
    import attention_decode_qk_amd as ga
    from gpu_support import Device, abi_config, max_context
    w = synth.small(name="graph", batch=4, q_len=3, window=50, rope_theta=500000.0,
                    seq_lo=200, seq_hi=600, page_size=4)
    x = synth.make_inputs(w, seed=21)
    _say("[gpu] graph replay")
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    d = Device(x)
    d.run(step)
    torch.cuda.synchronize()
    eager_out = d.out.clone()
    eager_k, eager_v = d.k_cache.clone(), d.v_cache.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(step, stream=s)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(step, stream=s)
    torch.cuda.synchronize()
    for rep in range(5):
        d.out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, eager_out), f"replay {rep}"
        assert torch.equal(d.k_cache, eager_k) and torch.equal(d.v_cache, eager_v)
        del junk
    step.close()
