"""GPU parity of the step at extend / prefill sizes (q_len > 8: a block of new
tokens per request, causal inside the block from the prefix length on, page 1's
window per query; page 2's prefill calls the same attention with the query
offset = prefix length) against the oracle, through the C ABI.  Bar: q and cache
bytes exact (one e4m3 code on at most 0.1% of written elements allowed); bf16
outputs within 2e-2 absolute + 2e-2 relative."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_support import (Device, Reference, abi_config, assert_codes_match, assert_outputs_close,
                         check_full, max_context, run_gpu)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# 16-token tiles: 9 (one ragged tile), 16 (one whole tile), 17, 33 (a one-token
# tail), 40, 64 and 200 (many tiles, ragged); windows shorter than a tile, than
# the block and longer; pages of 1, 3, 16, 64 rows.
SMALL = {
    "ext9_full": dict(batch=3, q_len=9, window=0),
    "ext16_swa_rope": dict(batch=2, q_len=16, window=24, rope_theta=500000.0),
    "ext17_page16": dict(batch=3, q_len=17, window=0, page_size=16),
    "ext33_scaled_page64": dict(batch=2, q_len=33, window=0, page_size=64, kv_scale=0.5,
                                qkv_std=1.4142135),
    "ext40_window1": dict(batch=2, q_len=40, window=1),
    "ext40_window5_page4": dict(batch=2, q_len=40, window=5, page_size=4),
    "ext64_swa_rope_q_scaled": dict(batch=2, q_len=64, window=100, rope_theta=500000.0,
                                    q_scale=5.473),
    "ext100_window50": dict(batch=2, q_len=100, window=50, rope_theta=500000.0, page_size=16),
    "ext200_page3": dict(batch=2, q_len=200, window=0, page_size=3),
    "ext67_b5_swa": dict(batch=5, q_len=67, window=300, rope_theta=500000.0, page_size=8),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_extend_small_case_matches_oracle(name):
    w = synth.small(name=name, seq_lo=20, seq_hi=700, **SMALL[name])
    x = synth.make_inputs(w, seed=300 + len(name))
    _say(f"[gpu] extend {name}: B={w.batch} L={w.q_len} W={w.window} P={w.page_size}")
    res = run_gpu(x)
    check_full(x, res, Reference(x), f"{name} S={res.splits}")


def test_extend_fresh_prefill_whole_context_in_the_block():
    """Prefixes of 1-3 tokens: the block is (nearly) the whole context, so each
    row's keys are mostly its own block's new keys, read back from the cache."""
    w = synth.small(name="fresh", batch=3, q_len=130, window=0, seq_lo=1, seq_hi=3, page_size=16)
    x = synth.make_inputs(w, seed=9)
    _say("[gpu] extend fresh prefill L=130")
    res = run_gpu(x)
    check_full(x, res, Reference(x), "fresh")


def test_extend_padded_slot_stores_nothing_and_outputs_zero():
    """A slot with cache_seqlens 0 and cache_loc -1 for all its tokens (a padded
    batch slot) writes no cache row and outputs zeros; the others are unaffected."""
    w = synth.small(name="pad", batch=3, q_len=20, window=0, seq_lo=50, seq_hi=200)
    x = synth.make_inputs(w, seed=8)
    L = w.q_len
    x.cache_seqlens[1] = 0
    x.cache_loc[L:2 * L] = -1
    _say("[gpu] extend padded slot")
    res = run_gpu(x)
    ref = Reference(x)
    np.testing.assert_array_equal(res.k_cache, ref.k_cache)
    np.testing.assert_array_equal(res.v_cache, ref.v_cache)
    assert np.all(res.out[1] == 0)
    assert_outputs_close(res.out, ref.outputs().reshape(res.out.shape), "extend pad")


def test_extend_graph_replay_matches_eager():
    """The two launches captured in a HIP graph and replayed several times, with
    eager work and synchronisation between replays: every replay equals eager."""
    import attention_decode_qk_amd as ga
    w = synth.small(name="graph", batch=2, q_len=48, window=40, rope_theta=500000.0,
                    seq_lo=100, seq_hi=400, page_size=4)
    x = synth.make_inputs(w, seed=22)
    _say("[gpu] extend graph replay")
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
        d.run(step, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(step, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        d.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, eager_out), f"replay {rep}"
        assert torch.equal(d.k_cache, eager_k) and torch.equal(d.v_cache, eager_v)
    step.close()


@pytest.mark.parametrize("name", list(synth.EXTEND))
def test_extend_full_size_workload(name):
    """Every q and cache byte and every output row of one full-size extend."""
    w = synth.WORKLOADS[name]
    _say(f"[gpu] full-size {name}: generating inputs")
    x = synth.make_inputs(w)
    _say(f"[gpu] full-size {name}: running step (B={w.batch} L={w.q_len})")
    res = run_gpu(x)
    _say(f"[gpu] full-size {name}: oracle prologue")
    ref = Reference(x)
    written = x.tokens * w.num_kv_heads * w.head_dim
    assert_codes_match(res.q, ref.q, ref.q.size, name + " q")
    assert_codes_match(res.k_cache, ref.k_cache, written, name + " k_cache")
    assert_codes_match(res.v_cache, ref.v_cache, written, name + " v_cache")
    _say(f"[gpu] full-size {name}: oracle attention on all {x.tokens * w.num_q_heads} rows "
         f"({oracle.threads()} threads)")
    out_ref = ref.outputs().reshape(res.out.shape)
    assert_outputs_close(res.out, out_ref, name + " out")


def test_extend_longest_block_served():
    """q_len 65,536 (the longest block the library serves) for one request over a
    1k-3k prefix with page 1's window, RoPE and pages of 16: every q and cache
    byte; every output row of the first and last 1,024 tokens (the window's
    start, the tiles' and splits' ends) and of 1,024 random tokens."""
    w = synth.small(name="longest", batch=1, q_len=65536, window=2048, rope_theta=500000.0,
                    page_size=16, seq_lo=1000, seq_hi=3000)
    _say("[gpu] extend L=65536: generating inputs")
    x = synth.make_inputs(w, seed=5)
    _say("[gpu] extend L=65536: running step")
    res = run_gpu(x)
    _say("[gpu] extend L=65536: oracle prologue")
    ref = Reference(x)
    written = x.tokens * w.num_kv_heads * w.head_dim
    assert_codes_match(res.q, ref.q, ref.q.size, "longest q")
    assert_codes_match(res.k_cache, ref.k_cache, written, "longest k_cache")
    assert_codes_match(res.v_cache, ref.v_cache, written, "longest v_cache")
    T, H = x.tokens, w.num_q_heads
    toks = np.unique(np.concatenate([np.arange(1024), np.arange(T - 1024, T),
                                     np.random.default_rng(3).integers(0, T, 1024)]))
    st = np.repeat(toks, H).astype(np.int64)
    sh = np.tile(np.arange(H), len(toks)).astype(np.int32)
    _say(f"[gpu] extend L=65536: oracle attention on {len(st)} rows ({oracle.threads()} threads)")
    got = res.out.reshape(T, H, w.head_dim)[st, sh]
    assert_outputs_close(got, ref.outputs(st, sh), "longest out")


# Key splits: forced counts (more than a unit's stages leaves some splits empty)
# and the plan's own count for few units over long key ranges.
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("name", ["ext67_b5_swa", "ext33_scaled_page64", "ext200_page3"])
def test_extend_forced_split_counts_match_oracle(name, splits):
    w = synth.small(name=name, seq_lo=20, seq_hi=700, **SMALL[name])
    x = synth.make_inputs(w, seed=300 + len(name))
    _say(f"[gpu] extend {name} S={splits}")
    res = run_gpu(x, num_splits=splits)
    assert res.splits == splits
    check_full(x, res, Reference(x), f"{name} S={splits}")


@pytest.mark.parametrize("kw", [
    dict(batch=1, q_len=16, window=0, seq_lo=3000, seq_hi=5000, page_size=16),
    dict(batch=2, q_len=40, window=500, seq_lo=2000, seq_hi=4000, rope_theta=500000.0),
    dict(batch=3, q_len=9, window=0, seq_lo=1500, seq_hi=2500, page_size=1, kv_scale=0.5,
         qkv_std=1.4142135),
])
def test_extend_few_units_split_by_the_plan(kw):
    """Few units over long key ranges: the plan splits the keys (S > 1) and the
    last split of each unit merges them."""
    w = synth.small(name="few_units", **kw)
    x = synth.make_inputs(w, seed=41)
    res = run_gpu(x)
    _say(f"[gpu] extend few units {kw}: S={res.splits}")
    assert res.splits > 1
    check_full(x, res, Reference(x), f"few units S={res.splits}")


def test_extend_split_graph_replay_matches_eager():
    """Split extend steps captured in a HIP graph and replayed several times
    (each replay re-arms the per-unit counters): every replay equals eager."""
    import attention_decode_qk_amd as ga
    w = synth.small(name="graph_split", batch=1, q_len=20, window=0, seq_lo=2000, seq_hi=2500,
                    page_size=8)
    x = synth.make_inputs(w, seed=23)
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    _say(f"[gpu] extend split graph replay S={step.splits}")
    assert step.splits > 1
    d = Device(x)
    d.run(step)
    torch.cuda.synchronize()
    eager_out = d.out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(step, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(step, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        d.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, eager_out), f"replay {rep}"
    step.close()
    res = run_gpu(x)
    check_full(x, res, Reference(x), "graph split")
