"""Pins for the oracle's prologue (page "012-attention-local-splits.py",
`_prepare_qkv`): per-head unweighted RMSNorm, interleaved RoPE, q cast and the
K/V cache store.  Checked against torch's own library routines, closed forms
and invariants, never against a retyped copy of the oracle."""
import math

import numpy as np
import pytest
import torch

import synth


def _bf16_bits(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


def _bits_to_f32(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).float().numpy()


def _torch_norm(x_bits):
    """torch's fp32 RMSNorm (library), rounded to bf16."""
    x = torch.from_numpy(_bits_to_f32(x_bits))
    y = torch.nn.functional.rms_norm(x, (x.shape[-1],), eps=1e-5)
    return y.to(torch.bfloat16).float().numpy()


def test_norm_matches_torch_rms_norm(orc):
    rng = np.random.default_rng(11)
    rows = _bf16_bits(rng.standard_normal((400, 64)) * rng.uniform(0.05, 20, (400, 1)))
    diff = 0
    for r in rows:
        y = orc.norm_rope_row(r)
        ref = _torch_norm(r)
        ulps = np.abs(y.view(np.int32) - ref.view(np.int32)) >> 16
        assert ulps.max() <= 1
        diff += int((ulps > 0).sum())
    assert diff <= 0.001 * rows.size


def test_norm_unit_rms_invariant(orc):
    """Before rounding, mean(y^2) = ms / (ms + eps); bf16 rounding moves it by < 2^-7."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        r = _bf16_bits(rng.standard_normal(64) * rng.uniform(0.5, 4))
        x = _bits_to_f32(r).astype(np.float64)
        ms = float((x * x).mean())
        y = orc.norm_rope_row(r).astype(np.float64)
        assert abs(float((y * y).mean()) * (ms + 1e-5) / ms - 1.0) < 2 ** -7


def test_norm_scale_invariance(orc):
    """x and 2^k x (exact in bf16) give the same normed bits once ms is so large
    that fp32(ms + 1e-5) == ms (ms >= 256): then the exact rsqrt scales by 2^-k."""
    rng = np.random.default_rng(13)
    for k in (1, 2, 5, 10):
        r = _bf16_bits(rng.standard_normal(64) * 32.0)
        r2 = _bf16_bits(_bits_to_f32(r) * (2.0 ** k))
        np.testing.assert_array_equal(orc.norm_rope_row(r), orc.norm_rope_row(r2))


def test_rope_position_zero_is_identity(orc):
    rng = np.random.default_rng(14)
    r = _bf16_bits(rng.standard_normal(64))
    np.testing.assert_array_equal(orc.norm_rope_row(r, 0, 500000.0), orc.norm_rope_row(r))


def test_rope_closed_form_rotation(orc):
    """Each pair (2i, 2i+1) is the complex product (e + i o) * exp(i * angle) with
    angle = fp32(fp32(pos) * inv_freq_i), inv_freq from torch's fp32 recipe; the
    first pair has inv_freq 1 so its angle is pos radians."""
    rng = np.random.default_rng(15)
    theta = 500000.0
    invf = (1.0 / (theta ** (torch.arange(0, 64, 2, dtype=torch.float) / 64))).numpy()
    assert invf[0] == 1.0
    for pos in [1, 7, 4095, 16384, 123457, 2 ** 21 - 1]:
        r = _bf16_bits(rng.standard_normal(64))
        y0 = orc.norm_rope_row(r).astype(np.float64)
        y = orc.norm_rope_row(r, pos, theta).astype(np.float64)
        ang = (np.float32(pos) * invf).astype(np.float64)
        z = (y0[0::2] + 1j * y0[1::2]) * np.exp(1j * ang)
        ref = np.empty(64)
        ref[0::2], ref[1::2] = z.real, z.imag
        # half a bf16 ulp (2^-8 relative) of the exact rotation, plus the fp32 roundings of the
        # cos/sin values, the two products and their sum
        mag = np.repeat(np.abs(y0[0::2]) + np.abs(y0[1::2]), 2)
        tol = np.abs(ref) * 2 ** -8 * 1.01 + mag * 2 ** -21
        assert np.all(np.abs(y - ref) <= tol), pos
        # the pair norm is preserved up to bf16 rounding
        n0 = np.hypot(y0[0::2], y0[1::2])
        n1 = np.hypot(y[0::2], y[1::2])
        assert np.all(np.abs(n1 - n0) <= n0 * 2 ** -8 + 1e-6)


def _run_prologue(orc, w, seed=0):
    x = synth.make_inputs(w, seed=seed)
    cfg = orc.Config(batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads,
                     num_kv_heads=w.num_kv_heads, page_size=w.page_size, window=w.window,
                     max_pages=x.max_pages, num_pages=x.num_pages, rope_theta=w.rope_theta,
                     sm_scale=w.sm_scale, kv_scale=w.kv_scale)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    q = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, x.k_scale, x.v_scale)
    return x, cfg, q, kc, vc


@pytest.mark.parametrize("kv_scale", [1.0, 0.5])
def test_value_store_is_the_cast_of_the_raw_projection(orc, kv_scale):
    """V rows are e4m3 of the raw bf16 values (divided by the scale when set): with
    scale 0.5 the division is an exact doubling, so torch's cast of 2v is the pin."""
    w = synth.small(batch=3, q_len=2, kv_scale=kv_scale, qkv_std=1.5, rope_theta=500000.0)
    x, cfg, q, kc, vc = _run_prologue(orc, w)
    hq, hkv = w.num_q_heads, w.num_kv_heads
    v = _bits_to_f32(x.qkv.reshape(x.tokens, -1)[:, (hq + hkv) * 64:(hq + 2 * hkv) * 64])
    v = v / np.float32(kv_scale)
    ref = synth.to_e4m3_codes(v).reshape(x.tokens, hkv, 64)
    np.testing.assert_array_equal(vc[x.cache_loc], ref)


def test_store_touches_only_cache_loc_rows(orc):
    w = synth.small(batch=4, q_len=3, page_size=4, rope_theta=500000.0)
    x, cfg, q, kc, vc = _run_prologue(orc, w)
    mask = np.ones(kc.shape[0], bool)
    mask[x.cache_loc] = False
    np.testing.assert_array_equal(kc[mask], x.k_cache[mask])
    np.testing.assert_array_equal(vc[mask], x.v_cache[mask])


@pytest.mark.parametrize("theta,kv_scale", [(0.0, 1.0), (500000.0, 1.0), (500000.0, 0.5)])
def test_q_and_key_codes_match_torch_composition(orc, theta, kv_scale):
    """q and K codes against a composition of torch library routines: fp32 rms_norm,
    bf16 cast, complex rotation with torch's fp32 angles, division, e4m3 cast.
    Allowed: one code step on at most 0.5% of elements (rsqrt / cos ulps)."""
    w = synth.small(batch=3, q_len=4, rope_theta=theta, kv_scale=kv_scale, qkv_std=1.3)
    x, cfg, q, kc, vc = _run_prologue(orc, w, seed=3)
    hq, hkv = w.num_q_heads, w.num_kv_heads
    qk = torch.from_numpy(_bits_to_f32(x.qkv.reshape(x.tokens, -1)[:, : (hq + hkv) * 64]))
    qk = qk.view(x.tokens, hq + hkv, 64)
    y = torch.nn.functional.rms_norm(qk, (64,), eps=1e-5).to(torch.bfloat16).float()
    if theta:
        invf = 1.0 / (theta ** (torch.arange(0, 64, 2, dtype=torch.float) / 64))
        ang = (torch.from_numpy(x.positions).float()[:, None] * invf[None, :])
        c, s = ang.cos()[:, None, :], ang.sin()[:, None, :]
        e, o = y[..., 0::2], y[..., 1::2]
        y2 = torch.empty_like(y)
        y2[..., 0::2] = (e * c - o * s)
        y2[..., 1::2] = (o * c + e * s)
        y = y2.to(torch.bfloat16).float()
    qref = y[:, :hq].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    key = y[:, hq:]
    if kv_scale != 1.0:
        key = (key / kv_scale).to(torch.bfloat16).float()
    kref = key.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for got, ref in ((q, qref), (kc[x.cache_loc], kref)):
        vg = torch.from_numpy(np.ascontiguousarray(got)).view(torch.float8_e4m3fn).float()
        vr = torch.from_numpy(np.ascontiguousarray(ref)).view(torch.float8_e4m3fn).float()
        neq = got != ref
        assert neq.mean() <= 0.005, neq.mean()
        # mismatches are one code apart
        assert np.all(np.abs(got.astype(int) - ref.astype(int))[neq] == 1)
        assert torch.all(torch.sign(vg) * torch.sign(vr) >= 0)


# ---- q scale before the bf16 rounding (page "qk_norm": the output scale) ----

def _q_codes(orc, w, q_scale, sm_scale=None):
    x = synth.make_inputs(w)
    cfg = orc.Config(batch=w.batch, q_len=w.q_len, page_size=w.page_size, window=w.window,
                     max_pages=x.max_pages, num_pages=x.num_pages, rope_theta=w.rope_theta,
                     sm_scale=w.sm_scale if sm_scale is None else sm_scale, kv_scale=w.kv_scale,
                     q_scale=q_scale)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    q = orc.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, x.k_scale, x.v_scale)
    return x, cfg, q, kc, vc


@pytest.mark.parametrize("q_scale", [5.473, 0.37])
def test_q_scale_without_rope_is_the_pages_qk_norm(orc, q_scale):
    """Without RoPE, q's bf16 values are exactly the page's qk_norm of the q
    columns with that output scale (the independently pinned function), and K
    and V do not depend on the q scale."""
    w = synth.small(batch=3, q_len=2, rope_theta=0.0, qkv_std=1.4)
    x, cfg, q, kc, vc = _q_codes(orc, w, q_scale)
    T = w.batch * w.q_len
    rows = x.qkv.reshape(T, -1)
    normed = orc.qk_norm(rows, 16, 64, orc.QK_BF16, eps=1e-5, scale=q_scale)
    want = synth.to_e4m3_codes(_bits_to_f32(normed)).reshape(T, 16, 64)
    assert np.array_equal(q, want)
    _, _, q1, kc1, vc1 = _q_codes(orc, w, 1.0)
    assert np.array_equal(kc, kc1) and np.array_equal(vc, vc1)
    assert not np.array_equal(q, q1)


def test_q_scale_moved_out_of_the_softmax_scale_keeps_the_output(orc):
    """Scaling q by 2 and halving the softmax scale gives the same attention up to
    e4m3's rounding of the doubled values (exact but in its subnormal band): the
    unrounded attention outputs agree to 1e-3 (observed 1e-4), while a scale
    applied twice moves them by more than 0.1 (observed 1.5)."""
    w = synth.small(batch=2, q_len=3, rope_theta=500000.0, window=64, qkv_std=1.2)
    outs = []
    for qs, sm in ((1.0, w.sm_scale), (2.0, w.sm_scale / 2), (2.0, w.sm_scale)):
        x = synth.make_inputs(w)
        cfg = orc.Config(batch=w.batch, q_len=w.q_len, page_size=w.page_size, window=w.window,
                         max_pages=x.max_pages, num_pages=x.num_pages, rope_theta=w.rope_theta,
                         sm_scale=sm, kv_scale=w.kv_scale, q_scale=qs)
        kc, vc = x.k_cache.copy(), x.v_cache.copy()
        _, _, o = orc.step(cfg, x.qkv, x.positions, x.cache_loc, x.cache_seqlens, x.page_table,
                           kc, vc, x.k_scale, x.v_scale)
        outs.append(o)
    ref, moved, doubled = outs
    assert np.max(np.abs(moved - ref)) <= 1e-3
    assert np.max(np.abs(doubled - ref)) > 0.1
