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


def _allocator_map(x, rng):
    """The allocator map a step's page table implies (numpy): request b lives
    in map row rows[b], and position p of it in slot page_table[b, p // P] * P +
    p % P; other entries are junk (-7) the builder must not read."""
    P, B = x.w.page_size, x.w.batch
    stride = x.max_pages * P
    rows = rng.permutation(B + 5)[:B].astype(np.int32)
    r2t = np.full((B + 5, stride), -7, np.int32)
    for b in range(B):
        p = np.arange(int(x.cache_seqlens[b]))
        r2t[rows[b], p] = x.page_table[b, p // P] * P + p % P
    return r2t, rows


@pytest.mark.parametrize("name", ["decode_p1", "verify8_p4", "verify3_p64", "verify5_p3",
                                  "swa_decode", "paged_scaled_long", "full_extend"])
def test_page_table_is_bit_exact(name):
    """The device page-table builder (page "msa.py", _build_page_table) against
    the oracle, padded and packed, with a padded slot."""
    if name in CASES:
        x = synth.make_inputs(synth.small(name=name, **CASES[name]), seed=60 + len(name))
    else:
        x = synth.make_inputs(synth.WORKLOADS[name])
    r2t, rows = _allocator_map(x, np.random.default_rng(5))
    kv = x.cache_seqlens.copy()
    if x.w.batch > 2:
        kv[1] = 0
    _say(f"[gpu] page table {name}: B={x.w.batch} P={x.w.page_size} max_pages={x.max_pages}")
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    B = x.w.batch
    table = torch.full((B, x.max_pages), -9, dtype=torch.int32, device=DEV)
    n_total = int(np.where(kv > 0, -(-kv.astype(np.int64) // x.w.page_size), 0).sum())
    packed = torch.full((max(n_total, 1),), -9, dtype=torch.int32, device=DEV)
    indptr = torch.full((B + 1,), -9, dtype=torch.int32, device=DEV)
    ga.mi355x_gated_attn_page_table(step.ctx, _t(r2t), _t(rows), _t(kv), table, packed, indptr)
    torch.cuda.synchronize()
    ref_t, ref_p, ref_i = oracle.page_table(r2t, rows, kv, x.w.page_size, x.max_pages)
    np.testing.assert_array_equal(table.cpu().numpy(), ref_t)
    np.testing.assert_array_equal(packed.cpu().numpy()[:n_total], ref_p)
    np.testing.assert_array_equal(indptr.cpu().numpy(), ref_i)
    keep = kv > 0
    np.testing.assert_array_equal(table.cpu().numpy()[keep], x.page_table[keep])
    step.close()


def test_page_table_meta_and_step_in_one_graph():
    """Page table, metadata and step captured in one graph, replayed three
    times with the map changed between replays (requests moved to other map
    rows and pages): every replay equals the oracle's table, metadata and step."""
    w = synth.small(name="pt_graph", batch=5, q_len=2, window=64, rope_theta=500000.0,
                    page_size=4, seq_lo=100, seq_hi=300)
    x = synth.make_inputs(w, seed=91)
    _say("[gpu] page table + meta + step graph")
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    B, T = w.batch, x.tokens
    rng = np.random.default_rng(11)
    r2t, rows = _allocator_map(x, rng)
    d_r2t, d_rows = _t(r2t), _t(rows)
    kv, seq = _t(x.cache_seqlens), _t(x.seq_lens)
    table = torch.zeros((B, x.max_pages), dtype=torch.int32, device=DEV)
    pos = torch.zeros(T, dtype=torch.int64, device=DEV)
    loc = torch.zeros(T, dtype=torch.int64, device=DEV)
    cs = torch.zeros(B, dtype=torch.int32, device=DEV)
    qkv = _t(x.qkv.view(np.int16))
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    out = torch.zeros((B, w.q_len, 1024), dtype=torch.int16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ga.mi355x_gated_attn_page_table(step.ctx, d_r2t, d_rows, kv, table, stream=s)
            step.meta(seq, table, pos, loc, cs, s)
            step(qkv, pos, loc, cs, table, seq, kc, vc, ks, vs, out, s)
    torch.cuda.synchronize()
    cfg = oracle_config(x)
    for rep in range(3):
        # the same logical cache seen through another map: shuffle the rows
        rows_new = rng.permutation(r2t.shape[0])[:B].astype(np.int32)
        r2t_new = np.full_like(r2t, -7)
        r2t_new[rows_new] = r2t[rows]
        d_r2t.copy_(_t(r2t_new))
        d_rows.copy_(_t(rows_new))
        kc.copy_(_t(x.k_cache))
        vc.copy_(_t(x.v_cache))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_t, _, _ = oracle.page_table(r2t_new, rows_new, x.cache_seqlens, w.page_size,
                                        x.max_pages)
        np.testing.assert_array_equal(table.cpu().numpy(), ref_t, err_msg=f"replay {rep}")
        m_pos, m_loc, m_cs = oracle.step_meta(cfg, x.seq_lens, ref_t)
        np.testing.assert_array_equal(loc.cpu().numpy(), m_loc, err_msg=f"replay {rep}")
        k_ref, v_ref = x.k_cache.copy(), x.v_cache.copy()
        _, o_ref, _ = oracle.step(cfg, x.qkv, m_pos, m_loc, m_cs, ref_t, k_ref, v_ref,
                                  x.k_scale, x.v_scale)
        assert_outputs_close(out.cpu().numpy().view(np.uint16), o_ref, f"replay {rep}")
        assert_codes_match(kc.cpu().numpy(), k_ref, T * 128, f"replay {rep} k_cache")
    step.close()


def test_meta_feeds_an_extend_step_with_an_empty_prefix():
    """Extend (q_len > 8) through the device metadata with a new request
    (seq_lens 0: empty prefix, page "msa.py" prefill) and a padded slot
    (seq_lens -1): the new request's K/V rows are stored and its outputs equal
    the oracle's; the padded slot stores nothing and outputs zeros."""
    w = synth.small(name="meta_extend", batch=3, q_len=20, window=0, page_size=4, seq_lo=30,
                    seq_hi=60)
    x = synth.make_inputs(w, seed=33)
    seq = x.seq_lens.copy()
    seq[0] = 0   # a new request: its 20 tokens at positions 0..19
    seq[2] = -1  # padding
    _say("[gpu] meta -> extend with an empty prefix")
    step = ga.GatedAttnStep(abi_config(x), max_context(x))
    B, T = w.batch, x.tokens
    pos = torch.zeros(T, dtype=torch.int64, device=DEV)
    loc = torch.zeros(T, dtype=torch.int64, device=DEV)
    cs = torch.zeros(B, dtype=torch.int32, device=DEV)
    pt = _t(x.page_table)
    step.meta(_t(seq), pt, pos, loc, cs)
    kc, vc = _t(x.k_cache), _t(x.v_cache)
    ks = torch.tensor([x.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([x.v_scale], dtype=torch.float32, device=DEV)
    out = torch.full((B, w.q_len, 1024), 77, dtype=torch.int16, device=DEV)
    step(_t(x.qkv.view(np.int16)), pos, loc, cs, pt, _t(seq), kc, vc, ks, vs, out)
    torch.cuda.synchronize()
    cfg = oracle_config(x)
    m_pos, m_loc, m_cs = oracle.step_meta(cfg, seq, x.page_table)
    assert list(m_cs) == [w.q_len, int(seq[1]) + w.q_len, 0]
    np.testing.assert_array_equal(loc.cpu().numpy(), m_loc)
    k_ref, v_ref = x.k_cache.copy(), x.v_cache.copy()
    _, o_ref, _ = oracle.step(cfg, x.qkv, m_pos, m_loc, m_cs, x.page_table, k_ref, v_ref,
                              x.k_scale, x.v_scale)
    got = out.cpu().numpy().view(np.uint16)
    assert_outputs_close(got[:2], o_ref[:2], "extend with an empty prefix")
    assert np.all(got[2] == 0)
    written = 2 * w.q_len * 128
    assert_codes_match(kc.cpu().numpy(), k_ref, written, "k_cache")
    assert_codes_match(vc.cpu().numpy(), v_ref, written, "v_cache")
    assert not np.array_equal(k_ref[m_loc[:w.q_len]], x.k_cache[m_loc[:w.q_len]])
    step.close()
