"""GPU parity of the on-device step metadata (positions, cache rows, key counts
from cached lengths and the page table; page "012-attention-local-splits.py",
`Inputs`; padded seq_len == 0 slots from page "msa.py"): bit-exact against the
oracle, and a graph holding metadata + step replayed over a short decode run
(lengths advanced between replays, eager work in between) against the oracle
stepped the same way."""
import sys

import numpy as np
import pytest
import torch

import attention_decode_qk_amd as ga
import oracle
import synth
from gpu_support import (abi_config, assert_codes_match, assert_outputs_close, max_context,
                         oracle_config)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _meta_gpu(step, x, seq_lens):
    B, T = x.w.batch, x.tokens
    pos = torch.full((T,), -7, dtype=torch.int64, device=DEV)
    loc = torch.full((T,), -7, dtype=torch.int64, device=DEV)
    cs = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    step.meta(_t(seq_lens), _t(x.page_table), pos, loc, cs)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), loc.cpu().numpy(), cs.cpu().numpy()


CASES = {
    "decode_p1": dict(batch=5, q_len=1, window=0),
    "verify8_p4": dict(batch=3, q_len=8, window=0, page_size=4),
    "verify3_p64": dict(batch=4, q_len=3, window=0, page_size=64),
    "verify5_p3": dict(batch=3, q_len=5, window=0, page_size=3),
}


@pytest.mark.parametrize("name", list(CASES) + ["swa_decode", "swa_verify", "paged_scaled_long"])
def test_meta_is_bit_exact(name):
    if name in CASES:
        x = synth.make_inputs(synth.small(name=name, **CASES[name]), seed=40 + len(name))
    else:
        x = synth.make_inputs(synth.WORKLOADS[name])
    seq = x.seq_lens.copy()
    if x.w.batch > 2:
        seq[1] = 0  # a padded slot
    _say(f"[gpu] step meta {name}: B={x.w.batch} L={x.w.q_len} P={x.w.page_size}")
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    got = _meta_gpu(step, x, seq)
    ref = oracle.step_meta(oracle_config(x), seq, x.page_table)
    for g, r, what in zip(got, ref, ("positions", "cache_loc", "cache_seqlens")):
        np.testing.assert_array_equal(g, r, err_msg=f"{name} {what}")
    keep = seq > 0
    Lq = x.w.q_len
    np.testing.assert_array_equal(got[2][keep], x.cache_seqlens[keep])
    np.testing.assert_array_equal(got[0].reshape(-1, Lq)[keep], x.positions.reshape(-1, Lq)[keep])
    np.testing.assert_array_equal(got[1].reshape(-1, Lq)[keep], x.cache_loc.reshape(-1, Lq)[keep])
    step.close()


@pytest.mark.parametrize("q_len,window", [(1, 0), (3, 40)])
def test_graph_of_meta_and_step_over_a_decode_run(q_len, window):
    """One graph holds the metadata build and the step.  Between replays the
    host advances every request's cached length by q_len (a decode run) and
    does unrelated eager work; each replay is checked against the oracle, run
    step by step on its own copy of the caches."""
    R = 6
    w = synth.small(name="soak", batch=4, q_len=q_len, window=window, rope_theta=500000.0,
                    seq_lo=150, seq_hi=400, page_size=4)
    # Lengths of the last step; the page table then covers every step's positions.
    x = synth.make_inputs(w, seed=77)
    base = x.seq_lens - (R - 1) * q_len
    _say(f"[gpu] meta+step graph soak L={q_len} W={window}")
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    qkv, pt = _t(x.qkv.view(np.int16)), _t(x.page_table)
    seq = _t(base)
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    pos = torch.zeros(x.tokens, dtype=torch.int64, device=DEV)
    loc = torch.zeros(x.tokens, dtype=torch.int64, device=DEV)
    cs = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    out = torch.zeros((w.batch, q_len, 1024), dtype=torch.int16, device=DEV)

    def run(stream):
        step.meta(seq, pt, pos, loc, cs, stream)
        step(qkv, pos, loc, cs, pt, seq, kc, vc, ks, vs, out, stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(s)
    torch.cuda.synchronize()

    cfg = oracle_config(x)
    k_ref, v_ref = x.k_cache.copy(), x.v_cache.copy()
    for r in range(R):
        lens = (base + r * q_len).astype(np.int32)
        seq.copy_(_t(lens))
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        m_pos, m_loc, m_cs = oracle.step_meta(cfg, lens, x.page_table)
        np.testing.assert_array_equal(pos.cpu().numpy(), m_pos, err_msg=f"replay {r}")
        np.testing.assert_array_equal(loc.cpu().numpy(), m_loc, err_msg=f"replay {r}")
        np.testing.assert_array_equal(cs.cpu().numpy(), m_cs, err_msg=f"replay {r}")
        _, o_ref, _ = oracle.step(cfg, x.qkv, m_pos, m_loc, m_cs, x.page_table, k_ref, v_ref,
                                  x.k_scale, x.v_scale)
        assert_outputs_close(out.cpu().numpy().view(np.uint16), o_ref, f"replay {r}")
        del junk
    written = R * x.tokens * 2 * 64
    assert_codes_match(kc.cpu().numpy(), k_ref, written, "k_cache after the run")
    assert_codes_match(vc.cpu().numpy(), v_ref, written, "v_cache after the run")
    step.close()
