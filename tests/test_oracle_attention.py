"""Pins for the oracle's attention and epilogue (page "012-attention-local-splits.py",
kernel_fn: the FA3 paged causal sliding-window call and rms_norm_gate):
torch's scaled_dot_product_attention and rms_norm as independent library
routines, closed forms from bit-encoded values, and the hand-derived mask cases
in tests/golden/mask_cases.json."""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ONE = 0x38  # e4m3 code of 1.0


def _cfg(orc, x):
    w = x.w
    return orc.Config(batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads,
                      num_kv_heads=w.num_kv_heads, page_size=w.page_size, window=w.window,
                      max_pages=x.max_pages, num_pages=x.num_pages, rope_theta=w.rope_theta,
                      sm_scale=w.sm_scale, kv_scale=w.kv_scale)


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double()


def _rows_of(x, b, keys):
    P = x.w.page_size
    keys = np.asarray(keys, np.int64)
    return x.page_table[b, keys // P].astype(np.int64) * P + keys % P


CASES = [
    dict(batch=3, q_len=1, window=0),
    dict(batch=2, q_len=1, window=5, rope_theta=500000.0),
    dict(batch=2, q_len=3, window=2, page_size=4),
    dict(batch=3, q_len=8, window=0, page_size=4),
    dict(batch=2, q_len=8, window=64, rope_theta=500000.0, page_size=16),
    dict(batch=2, q_len=2, window=0, kv_scale=0.5, page_size=64, qkv_std=1.41),
    dict(batch=2, q_len=1, window=1),
    dict(batch=2, q_len=3, window=0, num_q_heads=4, num_kv_heads=2),
    dict(batch=1, q_len=1, window=0, sm_scale=5.473 / 8),
    # extend / prefill (q_len >> 8): causal inside the block, per-query windows
    dict(batch=2, q_len=40, window=0, page_size=8),
    dict(batch=1, q_len=67, window=24, rope_theta=500000.0, page_size=1),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_attention_matches_torch_sdpa(orc, case):
    """Per (token, head): torch SDPA in float64 over the visible keys gathered
    through the page table; the oracle agrees to 1e-12."""
    w = synth.small(seq_lo=20, seq_hi=150, **case)
    x = synth.make_inputs(w, seed=5)
    cfg = _cfg(orc, x)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    q = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, x.k_scale, x.v_scale)
    o = orc.attention(cfg, q, kc, vc, x.page_table, x.cache_seqlens, x.k_scale, x.v_scale)
    o = o.reshape(x.tokens, w.num_q_heads, 64)
    grp = w.num_q_heads // w.num_kv_heads
    scaled = w.kv_scale != 1.0
    ks = x.k_scale if scaled else 1.0
    vs = x.v_scale if scaled else 1.0
    for t in range(x.tokens):
        b, i = divmod(t, w.q_len)
        p = int(x.cache_seqlens[b]) - w.q_len + i
        lo = max(0, p - w.window + 1) if w.window > 0 else 0
        rows = _rows_of(x, b, np.arange(lo, p + 1))
        for h in range(w.num_q_heads):
            g = h // grp
            qq = _dec(q[t, h])[None, None, None, :]
            K = _dec(kc[rows, g])[None, None]
            V = _dec(vc[rows, g])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, K, V, scale=float(np.float32(w.sm_scale)) * ks)[0, 0, 0].numpy() * vs
            np.testing.assert_allclose(o[t, h], ref, rtol=1e-12, atol=1e-14)


def _bit_encoded_inputs(orc, cache_seqlen, q_len, window, page_size, seed=0, batch=2):
    """All keys zero (so every score is 0 and the weights are uniform); V column c
    of logical key j holds bit c of j (c < 16), column 63 holds 1.0, and the two
    KV heads differ by sign of column 62 (+1 for head 0, -1 for head 1)."""
    w = synth.small(batch=batch, q_len=q_len, window=window, page_size=page_size)
    seq = np.full(batch, cache_seqlen - q_len, np.int32)
    x = synth.make_inputs(w, seed=seed, seq_lens=seq)
    hq, hkv = w.num_q_heads, w.num_kv_heads
    x.k_cache[:] = 0
    x.v_cache[:] = 0
    qkv = x.qkv.reshape(x.tokens, -1)
    qkv[:, hq * 64:(hq + hkv) * 64] = 0  # new keys: x = 0 -> normed 0 -> code 0
    one_bf16, neg_bf16 = 0x3F80, 0xBF80
    for b in range(batch):
        keys = np.arange(cache_seqlen)
        rows = _rows_of(x, b, keys)
        for c in range(16):
            x.v_cache[rows, :, c] = np.where((keys >> c) & 1, ONE, 0)[:, None]
        x.v_cache[rows, :, 63] = ONE
        x.v_cache[rows, 0, 62] = ONE
        x.v_cache[rows, 1, 62] = 0x80 | ONE
        for i in range(q_len):  # the new tokens' values come from the projection
            t = b * q_len + i
            pos = cache_seqlen - q_len + i
            vv = np.zeros((hkv, 64), np.uint16)
            for c in range(16):
                vv[:, c] = one_bf16 if (pos >> c) & 1 else 0
            vv[:, 63] = one_bf16
            vv[0, 62], vv[1, 62] = one_bf16, neg_bf16
            qkv[t, (hq + hkv) * 64:(hq + 2 * hkv) * 64] = vv.reshape(-1)
    return x


def _expected_bits_mean(lo, hi):
    keys = np.arange(lo, hi + 1)
    return np.array([((keys >> c) & 1).mean() for c in range(16)])


def test_mask_golden_cases_closed_form(orc):
    with open(os.path.join(GOLDEN, "mask_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        for P in (1, 4):
            x = _bit_encoded_inputs(orc, case["cache_seqlen"], case["q_len"], case["window"], P)
            cfg = _cfg(orc, x)
            kc, vc = x.k_cache.copy(), x.v_cache.copy()
            q = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, 1.0, 1.0)
            o = orc.attention(cfg, q, kc, vc, x.page_table, x.cache_seqlens, 1.0, 1.0)
            o = o.reshape(x.tokens, 16, 64)
            for t in range(x.tokens):
                lo, hi = case["ranges"][t % case["q_len"]]
                exp = _expected_bits_mean(lo, hi)
                for h in range(16):
                    np.testing.assert_allclose(o[t, h, :16], exp, atol=1e-12, err_msg=str(case))
                    assert abs(o[t, h, 63] - 1.0) < 1e-12
                    # query heads 0-7 read KV head 0, heads 8-15 read KV head 1
                    assert o[t, h, 62] == pytest.approx(1.0 if h < 8 else -1.0, abs=1e-12)


def test_window_one_returns_own_value(orc):
    w = synth.small(batch=3, q_len=3, window=1, rope_theta=500000.0)
    x = synth.make_inputs(w, seed=9)
    cfg = _cfg(orc, x)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    q = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, 1.0, 1.0)
    o = orc.attention(cfg, q, kc, vc, x.page_table, x.cache_seqlens, 1.0, 1.0)
    o = o.reshape(x.tokens, 16, 64)
    for t in range(x.tokens):
        own = _dec(vc[x.cache_loc[t]]).numpy()
        for h in range(16):
            np.testing.assert_array_equal(o[t, h], own[h // 8])


def test_no_visible_key_gives_zero(orc):
    """A padded request slot (cache_seqlens 0) has no keys: o = 0 and out = 0."""
    w = synth.small(batch=2, q_len=1)
    x = synth.make_inputs(w, seed=2)
    cs = x.cache_seqlens.copy()
    cs[1] = 0
    cfg = _cfg(orc, x)
    q = np.zeros((x.tokens, 16, 64), np.uint8)
    o = orc.attention(cfg, q, x.k_cache, x.v_cache, x.page_table, cs, 1.0, 1.0)
    assert np.all(o.reshape(x.tokens, 16, 64)[1] == 0)
    out = orc.epilogue(cfg, o, x.qkv)
    assert np.all(out.reshape(x.tokens, 16, 64)[1] == 0)


def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def test_epilogue_zero_gate_is_half_rmsnorm(orc):
    """gate = 0 => sigmoid = 0.5 exactly, out = bf16(0.5 * rms_norm(bf16(o)))."""
    w = synth.small(batch=2, q_len=2)
    x = synth.make_inputs(w, seed=4)
    cfg = _cfg(orc, x)
    qkv = x.qkv.copy().reshape(x.tokens, -1)
    qkv[:, 20 * 64:] = 0
    rng = np.random.default_rng(1)
    o = rng.standard_normal((x.tokens * 16, 64)) * 0.03
    out = orc.epilogue(cfg, o, qkv)
    ob = torch.from_numpy(o).to(torch.bfloat16).double()
    ref = (0.5 * torch.nn.functional.rms_norm(ob, (64,), eps=1e-5)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    assert (out != ref).mean() <= 0.001
    assert np.all(np.abs(out.astype(np.int32) - ref.astype(np.int32)) <= 1)


def test_epilogue_matches_torch_composition(orc):
    w = synth.small(batch=3, q_len=2, qkv_std=2.0)
    x = synth.make_inputs(w, seed=6)
    cfg = _cfg(orc, x)
    rng = np.random.default_rng(2)
    o = rng.standard_normal((x.tokens * 16, 64)) * 0.05
    out = orc.epilogue(cfg, o, x.qkv)
    gate = _bf16_to_f64(x.qkv.reshape(x.tokens, -1)[:, 20 * 64:]).reshape(-1, 64)
    ob = torch.from_numpy(o).to(torch.bfloat16).double()
    ref = (torch.nn.functional.rms_norm(ob, (64,), eps=1e-5) * torch.sigmoid(gate))
    ref = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (out != ref).mean() <= 0.001
    assert np.all(np.abs(out.astype(np.int32) - ref.astype(np.int32)) <= 1)


def test_step_composes_the_parts(orc):
    """The whole-step entry equals prologue -> attention -> epilogue."""
    w = synth.small(batch=2, q_len=3, window=7, rope_theta=500000.0, page_size=4)
    x = synth.make_inputs(w, seed=8)
    cfg = _cfg(orc, x)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    q, out, o = orc.step(cfg, x.qkv, x.positions, x.cache_loc, x.cache_seqlens, x.page_table,
                         kc, vc, 1.0, 1.0)
    kc2, vc2 = x.k_cache.copy(), x.v_cache.copy()
    q2 = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc2, vc2, 1.0, 1.0)
    o2 = orc.attention(cfg, q2, kc2, vc2, x.page_table, x.cache_seqlens, 1.0, 1.0)
    out2 = orc.epilogue(cfg, o2, x.qkv)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(kc, kc2)
    np.testing.assert_array_equal(out.reshape(-1, 64), out2)


def test_thread_count_does_not_change_the_oracle(orc):
    """The attention loops run their (token, head) pairs (and the sparse step its
    (request, KV head) pairs) on OpenMP threads: one thread and all of them give
    the same bytes, the selected-row form included."""
    w = synth.small(batch=3, q_len=4, window=50, rope_theta=500000.0, page_size=4, seq_lo=60,
                    seq_hi=300)
    x = synth.make_inputs(w, seed=12)
    cfg = _cfg(orc, x)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    q = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, x.k_scale, x.v_scale)
    n0 = orc.threads()
    try:
        outs = []
        for n in (1, max(2, n0)):
            orc.threads(n)
            assert orc.threads() == n or n0 == 1
            o = orc.attention(cfg, q, kc, vc, x.page_table, x.cache_seqlens, x.k_scale, x.v_scale)
            st = np.array([5, 0, 11, 7], np.int64)
            sh = np.array([3, 15, 0, 8], np.int32)
            osel = orc.attention(cfg, q, kc, vc, x.page_table, x.cache_seqlens, x.k_scale,
                                 x.v_scale, st, sh)
            np.testing.assert_array_equal(osel, o[st * 16 + sh])
            outs.append(o)
        np.testing.assert_array_equal(outs[0], outs[1])
    finally:
        orc.threads(n0)
