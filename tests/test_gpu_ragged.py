"""GPU parity of ragged extend batches (page "msa.py", msa_sparse_prefill_main:
per-request query segments from cumulative lengths, causal from each
request's prefix, here with dense keys): the packed step through the C ABI
against the oracle step run request by request on one shared cache (each
request reads and writes only its own pages, so the order of the requests is
immaterial and the composition is the batch's result).  Segments of 0, 1, 15,
16, 17 tokens and up to the bound, windows, pages, RoPE, the scaled cache,
key splits, and the bound's own uniform batch.  Bar: q and cache bytes exact
(one e4m3 code on at most 0.1% of written elements), outputs within 2e-2."""
import sys

import numpy as np
import pytest
import torch

import attention_decode_qk_amd as ga
import synth
from gpu_support import (abi_config, assert_codes_match, assert_outputs_close, max_context,
                         ragged_reference)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _run(x, lens, num_splits=0, what="ragged"):
    r = synth.ragged(x, lens)
    step = ga.GatedAttnStep(abi_config(x), max_context(x), num_splits)
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    T = r["total_q"]
    out = torch.zeros((max(T, 1), 1024), dtype=torch.int16, device=DEV)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    qkv = _t(r["qkv"].view(np.int16)) if T else torch.zeros((1, 2304), dtype=torch.int16,
                                                             device=DEV)
    pos = _t(r["positions"]) if T else torch.zeros(1, dtype=torch.int64, device=DEV)
    loc = _t(r["cache_loc"]) if T else torch.zeros(1, dtype=torch.int64, device=DEV)
    step.ragged(qkv, pos, loc, _t(r["cu_seqlens_q"]), T, _t(r["cache_seqlens"]),
                _t(x.page_table), kc, vc, ks, vs, out)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref, out_ref = ragged_reference(x, r, lens)
    q_got = step.q_bytes().cpu().numpy().reshape(-1, 16, 64)[:T]
    written = T * 2 * 64
    assert_codes_match(q_got, q_ref, max(q_ref.size, 1), what + " q")
    assert_codes_match(kc.cpu().numpy(), k_ref, max(written, 1), what + " k_cache")
    assert_codes_match(vc.cpu().numpy(), v_ref, max(written, 1), what + " v_cache")
    if T:
        assert_outputs_close(out.cpu().numpy().view(np.uint16)[:T], out_ref, what + " out")
    splits = step.splits
    step.close()
    return splits


CASES = {
    "mixed_window": (dict(batch=5, q_len=40, window=30, rope_theta=500000.0, page_size=4),
                     [17, 0, 40, 1, 16]),
    "full_pages64_scaled": (dict(batch=4, q_len=70, window=0, page_size=64, kv_scale=0.5,
                                 qkv_std=1.4142135), [70, 9, 33, 15]),
    "short_segments": (dict(batch=6, q_len=24, window=0, rope_theta=500000.0),
                       [1, 2, 3, 24, 8, 0]),
    "wide_window_q_scaled": (dict(batch=3, q_len=100, window=200, page_size=16, q_scale=5.473),
                             [100, 50, 64]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_case_matches_oracle(name):
    kw, lens = CASES[name]
    w = synth.small(name=name, seq_lo=0, seq_hi=600, **kw)
    x = synth.make_inputs(w, seed=1100 + len(name))
    _say(f"[gpu] ragged {name}: B={w.batch} bound L={w.q_len} lens={lens}")
    _run(x, np.array(lens, np.int32), what=name)


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_ragged_key_splits(splits):
    """Few units over long prefixes: the plan's key splits, and forced ones."""
    w = synth.small(name="ragged_split", batch=2, q_len=20, window=0, seq_lo=2000, seq_hi=2500,
                    page_size=8)
    x = synth.make_inputs(w, seed=1200)
    _say(f"[gpu] ragged splits S={splits}")
    got = _run(x, np.array([20, 11], np.int32), num_splits=splits, what=f"ragged S={splits}")
    assert got == splits


def test_ragged_uniform_lengths_equal_the_uniform_step():
    """Every segment at the bound: the ragged call is the uniform step."""
    w = synth.small(name="ragged_full", batch=3, q_len=33, window=64, rope_theta=500000.0,
                    seq_lo=50, seq_hi=300, page_size=4)
    x = synth.make_inputs(w, seed=1300)
    _say("[gpu] ragged at the bound")
    _run(x, np.full(3, 33, np.int32), what="ragged at the bound")


def test_ragged_batch_without_new_tokens_is_a_no_op():
    w = synth.small(name="ragged_none", batch=2, q_len=16, window=0, seq_lo=30, seq_hi=90)
    x = synth.make_inputs(w, seed=1400)
    _say("[gpu] ragged without tokens")
    _run(x, np.zeros(2, np.int32), what="ragged empty")


def test_ragged_graph_replay_matches_eager():
    """The ragged step's two launches captured in a HIP graph and replayed four
    times, with eager work between replays: every replay equals the eager step
    (the step writes the same cache rows with the same codes each time)."""
    w = synth.small(name="ragged_graph", batch=3, q_len=40, window=50, rope_theta=500000.0,
                    seq_lo=100, seq_hi=900, page_size=4)
    x = synth.make_inputs(w, seed=1500)
    lens = np.array([40, 3, 21], np.int32)
    r = synth.ragged(x, lens)
    step = ga.GatedAttnStep(abi_config(x), max_context(x), 2)
    T = r["total_q"]
    args = [_t(r["qkv"].view(np.int16)), _t(r["positions"]), _t(r["cache_loc"]),
            _t(r["cu_seqlens_q"]), T, _t(r["cache_seqlens"]), _t(x.page_table)]
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    eager = torch.zeros((T, 1024), dtype=torch.int16, device=DEV)
    _say("[gpu] ragged graph replay")
    step.ragged(*args, kc, vc, ks, vs, eager)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step.ragged(*args, kc, vc, ks, vs, out, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        del junk
    q_ref, k_ref, v_ref, out_ref = ragged_reference(x, r, lens)
    assert_outputs_close(eager.cpu().numpy().view(np.uint16), out_ref, "ragged graph")
    assert_codes_match(kc.cpu().numpy(), k_ref, T * 128, "ragged graph k_cache")
    step.close()


@pytest.mark.parametrize("batch", [64, 65])
def test_ragged_many_requests(batch):
    """Up to 64 requests deal only the tiles that hold rows over the XCDs (a
    lane per request); 65 keep the padded order.  Many empty and one-token
    segments among longer ones."""
    rng = np.random.default_rng(batch)
    lens = rng.choice([0, 1, 5, 16, 17, 33, 40], size=batch).astype(np.int32)
    w = synth.small(name="ragged_many", batch=batch, q_len=40, window=64, rope_theta=500000.0,
                    seq_lo=20, seq_hi=300, page_size=4)
    x = synth.make_inputs(w, seed=1600 + batch)
    _say(f"[gpu] ragged many requests B={batch} tokens={int(lens.sum())}")
    _run(x, lens, what=f"ragged B={batch}")
