"""The no-allocation step (mi355x_gated_attn_step_noalloc: q, partials and
counters in the library's static per-GPU scratch) against the workspace step
it mirrors, through the C ABI: two calls in a row on one GPU, the second with
a smaller input and another context, each with the same outputs and cache
writes as mi355x_gated_attn_step (the same kernels: byte-identical) and
within the oracle bar."""
import sys

import numpy as np
import pytest
import torch

import attention_decode_qk_amd as ga
import synth
from gpu_support import Device, Reference, abi_config, check_full, max_context

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(x, num_splits):
    """(workspace step result, no-allocation step result) on separate copies of
    the inputs; each a dict of out / k_cache / v_cache as numpy arrays."""
    results = []
    for noalloc in (False, True):
        step = ga.GatedAttnStep(abi_config(x), max_context(x), num_splits)
        d = Device(x)
        if noalloc:
            ga.mi355x_gated_attn_step_noalloc(step.ctx, d.qkv, d.positions, d.cache_loc,
                                              d.cache_seqlens, d.page_table, d.seq_lens,
                                              d.k_cache, d.v_cache, d.k_scale, d.v_scale, d.out)
        else:
            d.run(step)
        torch.cuda.synchronize()
        results.append(dict(out=d.out.cpu().numpy().view(np.uint16), k=d.k_cache.cpu().numpy(),
                            v=d.v_cache.cpu().numpy(), splits=step.splits))
        step.close()
    return results


CASES = [
    # a split verify step (counters and partials in use), then a smaller decode
    ("verify8_swa_split", dict(batch=6, q_len=8, window=300, rope_theta=500000.0, page_size=4,
                               seq_lo=400, seq_hi=1500), 5),
    ("decode_small_split", dict(batch=3, q_len=1, window=0, seq_lo=200, seq_hi=900), 3),
]


def test_noalloc_matches_the_workspace_step_on_two_calls():
    for name, kw, splits in CASES:
        w = synth.small(name=name, **kw)
        x = synth.make_inputs(w, seed=4242 + len(name))
        _say(f"[gpu] no-alloc {name}: B={w.batch} L={w.q_len} S={splits}")
        ref_ws, got = _both(x, splits)
        assert ref_ws["splits"] == got["splits"] == splits
        np.testing.assert_array_equal(got["out"], ref_ws["out"])
        np.testing.assert_array_equal(got["k"], ref_ws["k"])
        np.testing.assert_array_equal(got["v"], ref_ws["v"])
        # and the oracle's bar, on the no-allocation result
        ref = Reference(x)
        res = type("R", (), {})()
        res.out, res.k_cache, res.v_cache = got["out"], got["k"], got["v"]
        res.q = ref.q  # q stays in the static scratch; its bytes are not compared here
        check_full(x, res, ref, f"no-alloc {name}")


def test_noalloc_extend_then_decode():
    """An extend block (q_len > 8: prologue + attention launches, split keys)
    through the static scratch, then a decode: both equal the workspace step."""
    for name, kw, splits in [
        ("extend40_split", dict(batch=2, q_len=40, window=0, page_size=8, seq_lo=1500,
                                seq_hi=2500), 4),
        ("decode_after_extend", dict(batch=2, q_len=1, window=64, rope_theta=500000.0,
                                     seq_lo=100, seq_hi=400), 2),
    ]:
        w = synth.small(name=name, **kw)
        x = synth.make_inputs(w, seed=99 + len(name))
        _say(f"[gpu] no-alloc {name}: B={w.batch} L={w.q_len} S={splits}")
        ref_ws, got = _both(x, splits)
        np.testing.assert_array_equal(got["out"], ref_ws["out"])
        np.testing.assert_array_equal(got["k"], ref_ws["k"])
        np.testing.assert_array_equal(got["v"], ref_ws["v"])
