"""GPU parity of length-balanced splits: without a window (and 2 <= B <= 64,
S > 1) the plan lets the kernel deal a token group's B * S units out to the
requests in proportion to their key counts, so a short request gets one unit
and a long one many.  Cases with very uneven cached lengths (a fresh request
with only its new tokens, one-key requests beside thousands of keys), the
batch limits on both sides (64: balanced, 65: uniform), every q_len grouping,
pages, the scaled cache, and forced split counts from 2 to 64.  Same bar as
the other parity tests: q and cache bytes exact, outputs within 2e-2."""
import sys

import numpy as np
import pytest

import synth
from gpu_support import Reference, check_full, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


UNEVEN = np.array([0, 5, 700, 33, 1500, 2], np.int32)


@pytest.mark.parametrize("q_len", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("splits", [0, 3, 16])
def test_uneven_lengths(q_len, splits):
    w = synth.small(name="balanced", batch=len(UNEVEN), q_len=q_len, window=0,
                    rope_theta=500000.0, page_size=4, seq_lo=0, seq_hi=1500)
    x = synth.make_inputs(w, seed=700 + q_len, seq_lens=UNEVEN)
    _say(f"[gpu] balanced uneven: L={q_len} S={splits or 'plan'}")
    res = run_gpu(x, num_splits=splits)
    check_full(x, res, Reference(x), f"balanced L={q_len} S={splits}")


@pytest.mark.parametrize("batch", [2, 64, 65])
def test_batch_limits(batch):
    """64 requests take the balanced deal (one cached length per lane), 65 the
    uniform one; two requests are the smallest balanced batch."""
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, 2500, size=batch).astype(np.int32)
    lens[0] = 3000
    w = synth.small(name="balanced_b", batch=batch, q_len=1, window=0, page_size=1,
                    seq_lo=1, seq_hi=3000)
    x = synth.make_inputs(w, seed=800 + batch, seq_lens=lens)
    _say(f"[gpu] balanced batch B={batch}")
    res = run_gpu(x, num_splits=4)
    check_full(x, res, Reference(x), f"balanced B={batch}")


def test_scaled_paged_verify():
    """The long-context verify shape in small: q_len 8, pages of 64, scaled
    cache, lengths spread over a factor of 40."""
    lens = np.array([100, 4000, 50, 2200], np.int32)
    w = synth.small(name="balanced_scaled", batch=4, q_len=8, window=0, page_size=64,
                    kv_scale=0.5, qkv_std=1.4142135, seq_lo=50, seq_hi=4000)
    x = synth.make_inputs(w, seed=901, seq_lens=lens)
    ref = Reference(x)
    for s in (2, 16, 64):
        _say(f"[gpu] balanced scaled verify S={s}")
        res = run_gpu(x, num_splits=s)
        check_full(x, res, ref, f"balanced scaled S={s}")


@pytest.mark.parametrize("page_size", [32, 64, 256])
@pytest.mark.parametrize("splits", [0, 5, 24])
def test_whole_block_units_on_page_blocks(page_size, splits):
    """Balanced units of a whole verify block (q_len 8, one group under a long
    key bound) over pages of 32 or more keys, where every 32-key block lies in
    one page and the kernel takes a block's rows from one page entry: uneven
    lengths leave units whose last block runs past their chunk and waves with
    masked filler blocks; the scaled cache on one case."""
    lens = np.array([1, 33, 700, 64, 1500, 95], np.int32)
    w = synth.small(name="page_blocks", batch=len(lens), q_len=8, window=0, page_size=page_size,
                    rope_theta=500000.0, kv_scale=0.5 if page_size == 64 else 1.0,
                    qkv_std=1.4142135 if page_size == 64 else 1.0, seq_lo=1, seq_hi=1500)
    x = synth.make_inputs(w, seed=950 + page_size + splits, seq_lens=lens)
    _say(f"[gpu] page blocks: P={page_size} S={splits or 'plan'}")
    res = run_gpu(x, num_splits=splits, ctx_bound=100000)
    check_full(x, res, Reference(x), f"page blocks P={page_size} S={splits}")
