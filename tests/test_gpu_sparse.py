"""GPU parity of the page-list-driven (top-k block-sparse) decode step (page
"msa.py": msa_sparse_decode_main: one query per request at its last cached
position, keys through each KV head's selected blocks) against the oracle,
through the C ABI: q and cache bytes exact (one e4m3 step on <= 0.1% allowed),
outputs within 2e-2 + 2e-2 |ref|."""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from gpu_support import Reference, assert_codes_match, assert_outputs_close, check_full, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _small(block, topk, seed, **kw):
    base = dict(batch=3, q_len=1, window=0, seq_lo=40, seq_hi=700, page_size=1)
    base.update(kw)
    w = synth.small(name=f"sparse_b{block}_k{topk}", seed=seed, **base)
    return dataclasses.replace(w, sparse_block=block, sparse_topk=topk)


CASES = {
    "b32_k4_p1": (32, 4, dict()),
    "b64_k8_p16": (64, 8, dict(batch=4, page_size=16)),
    "b128_k16_p128": (128, 16, dict(batch=2, seq_lo=2000, seq_hi=6000, page_size=128)),
    "b32_k40_padded": (32, 40, dict(batch=3, seq_lo=40, seq_hi=300)),  # more slots than blocks
    "b32_k6_rope_qscale": (32, 6, dict(rope_theta=500000.0, q_scale=5.473)),
    "b64_k5_scaled_p64": (64, 5, dict(page_size=64, kv_scale=0.5, qkv_std=1.4142135)),
    "b256_k3_p8": (256, 3, dict(batch=5, seq_lo=100, seq_hi=3000, page_size=8)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_small_case_matches_oracle(name):
    block, topk, kw = CASES[name]
    w = _small(block, topk, seed=40 + len(name), **kw)
    x = synth.make_inputs(w)
    _say(f"[gpu] sparse {name}: B={w.batch} block={block} topk={topk} P={w.page_size}")
    res = run_gpu(x)
    check_full(x, res, Reference(x), "sparse " + name)


def test_sparse_lists_without_the_querys_own_block():
    """Lists that leave out the block of the new token's position: its key is not
    attended (the row is still stored), and empty lists give zero rows."""
    w = _small(32, 5, seed=77, batch=4)
    x = synth.make_inputs(w)
    bi = x.extra["block_idx"]
    for g in range(2):
        for b in range(w.batch):
            own = (int(x.cache_seqlens[b]) - 1) // 32
            bi[g, b][bi[g, b] == own] = -1
    bi[1, 2, :] = -1  # an empty list: KV head 1 of request 2 sees nothing
    _say("[gpu] sparse lists without the own block")
    res = run_gpu(x)
    check_full(x, res, Reference(x), "sparse no-own-block")


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_sparse_split_count_invariance(splits):
    w = _small(64, 8, seed=91, batch=3, seq_lo=500, seq_hi=2000)
    x = synth.make_inputs(w)
    _say(f"[gpu] sparse splits={splits}")
    res = run_gpu(x, num_splits=splits)
    check_full(x, res, Reference(x), f"sparse S={splits}")


def test_sparse_decode_full_size():
    """The sparse_decode workload: every q and cache byte, sampled output rows."""
    w = synth.WORKLOADS["sparse_decode"]
    _say("[gpu] full-size sparse_decode: generating inputs")
    x = synth.make_inputs(w)
    res = run_gpu(x)
    _say(f"[gpu] full-size sparse_decode: splits={res.splits}; oracle")
    ref = Reference(x)
    written = x.tokens * w.num_kv_heads * w.head_dim
    assert_codes_match(res.q, ref.q, ref.q.size, "sparse_decode q")
    assert_codes_match(res.k_cache, ref.k_cache, written, "sparse_decode k_cache")
    assert_codes_match(res.v_cache, ref.v_cache, written, "sparse_decode v_cache")
    out_ref = ref.outputs().reshape(res.out.shape)
    assert_outputs_close(res.out, out_ref, "sparse_decode out")
