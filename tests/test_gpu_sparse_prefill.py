"""GPU parity of the page-list-driven (top-k block-sparse) prefill (page
"msa.py", msa_sparse_prefill_main: each new token of a chunk a query with its
own per-KV-head block list, causal from the prefix) against the oracle's
block-sparse step on the same queries as a batch of one-token requests (each
with its request's page-table row and its position + 1 as cached length; the
oracle stores every new row before any attention, as the prefill's first
launch does).  Chunks of 1-40 tokens, blocks of 32-128 keys, lists with and
without the query's own block, pages, RoPE with a q scale, the scaled cache.
Bar: q and cache bytes exact (one e4m3 code on at most 0.1%), outputs within
2e-2 + 2e-2 |ref|."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import attention_decode_qk_amd as ga
import oracle
import synth
from gpu_support import assert_codes_match, assert_outputs_close, oracle_config

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES = {
    "b32_k4_L20": (32, 4, dict(batch=2, q_len=20)),
    "b64_k6_L40_p16_rope": (64, 6, dict(batch=3, q_len=40, page_size=16, rope_theta=500000.0,
                                         q_scale=5.473)),
    "b128_k8_L9_p128": (128, 8, dict(batch=2, q_len=9, page_size=128, seq_lo=1500,
                                     seq_hi=4000)),
    "b32_k3_L1": (32, 3, dict(batch=4, q_len=1)),
    "b64_k5_L16_scaled_p64": (64, 5, dict(batch=2, q_len=16, page_size=64, kv_scale=0.5,
                                          qkv_std=1.4142135)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_prefill_matches_oracle(name):
    block, topk, kw = CASES[name]
    base = dict(window=0, seq_lo=40, seq_hi=900, page_size=1)
    base.update(kw)
    w = synth.small(name=name, **base)
    x = synth.make_inputs(w, seed=1700 + len(name))
    sp = synth.sparse_prefill(x, block, topk, seed=1800 + len(name))
    # drop the own block from one query's lists: its new key is then unseen
    bi = sp["block_idx"].copy()
    bi[:, 0, 0] = -1
    T = x.tokens
    _say(f"[gpu] sparse prefill {name}: T={T} block={block} topk={topk}")
    cfg = ga.make_config(T, 1, w.page_size, 0, x.max_pages, x.num_pages, w.rope_theta,
                         w.sm_scale, w.kv_scale, q_scale=w.q_scale, sparse_block=block,
                         sparse_topk=topk)
    step = ga.GatedAttnStep(cfg, int(sp["cache_seqlens"].max()))
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    out = torch.zeros((T, 1, 1024), dtype=torch.int16, device=DEV)
    step.sparse_prefill(_t(sp["qkv"].view(np.int16)), _t(sp["positions"]), _t(sp["cache_loc"]),
                        _t(sp["token_req"]), w.batch, _t(sp["cache_seqlens"]), _t(x.page_table),
                        _t(bi), kc, vc, ks, vs, out)
    torch.cuda.synchronize()
    ocfg = oracle_config(x)
    ocfg.batch, ocfg.q_len = T, 1
    k_ref, v_ref = x.k_cache.copy(), x.v_cache.copy()
    q_ref, o_ref, _ = oracle.sparse_step(ocfg, sp["qkv"], sp["positions"], sp["cache_loc"],
                                         sp["cache_seqlens"], sp["page_table_q"], bi, block,
                                         k_ref, v_ref, x.k_scale, x.v_scale)
    written = T * 2 * 64
    assert_codes_match(step.q_bytes().cpu().numpy(), q_ref, q_ref.size, name + " q")
    assert_codes_match(kc.cpu().numpy(), k_ref, written, name + " k_cache")
    assert_codes_match(vc.cpu().numpy(), v_ref, written, name + " v_cache")
    assert_outputs_close(out.cpu().numpy().view(np.uint16), o_ref, name + " out")
    step.close()


def test_sparse_prefill_graph_replay_matches_eager():
    """The prefill's two launches captured in a HIP graph and replayed three
    times with eager work between: every replay equals the eager step."""
    block, topk = 64, 4
    w = synth.small(name="sp_graph", batch=2, q_len=24, window=0, seq_lo=100, seq_hi=600,
                    page_size=8, rope_theta=500000.0)
    x = synth.make_inputs(w, seed=1900)
    sp = synth.sparse_prefill(x, block, topk, seed=1901)
    T = x.tokens
    cfg = ga.make_config(T, 1, w.page_size, 0, x.max_pages, x.num_pages, w.rope_theta,
                         w.sm_scale, w.kv_scale, sparse_block=block, sparse_topk=topk)
    step = ga.GatedAttnStep(cfg, int(sp["cache_seqlens"].max()), 2)
    args = [_t(sp["qkv"].view(np.int16)), _t(sp["positions"]), _t(sp["cache_loc"]),
            _t(sp["token_req"]), w.batch, _t(sp["cache_seqlens"]), _t(x.page_table),
            _t(sp["block_idx"])]
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    eager = torch.zeros((T, 1, 1024), dtype=torch.int16, device=DEV)
    _say("[gpu] sparse prefill graph replay")
    step.sparse_prefill(*args, kc, vc, ks, vs, eager)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step.sparse_prefill(*args, kc, vc, ks, vs, out, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        del junk
    step.close()
