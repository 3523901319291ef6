"""Pins for the oracle's number formats (bf16 rounding, OCP e4m3, exact rsqrt,
RoPE inverse frequencies) against things other than the oracle itself:
brute-force nearest-code search, torch's CPU casts (library routines), exact
rational arithmetic and hand-derived fixtures."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_torch(orc):
    ref = _torch_e4m3_values()
    for c in range(256):
        got = orc.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
            assert math.copysign(1.0, got) == math.copysign(1.0, ref[c]), c


def test_e4m3_encode_golden_cases(orc):
    with open(os.path.join(GOLDEN, "e4m3_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        assert orc.e4m3_encode(case["x"]) == case["code"], case


def _brute_force_code(x, vals):
    """Nearest finite e4m3 code by exhaustive search; ties go to the code whose
    last mantissa bit is 0; |x| beyond 448 saturates; signed zero kept."""
    best = None
    for c in range(256):
        v = vals[c]
        if math.isnan(v):
            continue
        if (c & 0x80) != (0x80 if math.copysign(1.0, x) < 0 else 0):
            continue  # same sign half only (keeps -0 for tiny negatives)
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c)
    return best[1]


def test_e4m3_encode_exhaustive_over_bf16(orc):
    """Every finite bf16 value: oracle == brute-force nearest code, and == torch's
    cast wherever torch does not overflow to NaN (|x| < 464)."""
    vals = _torch_e4m3_values()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    tcodes = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float8_e4m3fn)
    tcodes = tcodes.view(torch.uint8).numpy()
    n_checked = 0
    for i in range(65536):
        x = xs[i]
        if not math.isfinite(x):
            continue
        got = orc.e4m3_encode(x)
        if abs(x) < 464.0:
            assert got == tcodes[i], (x, got, tcodes[i])
        else:
            assert got == (0xFE if x < 0 else 0x7E), x  # READING: saturation
        if abs(x) <= 448.0 and (i % 7 == 0 or abs(x) < 0.02 or abs(x) > 200):
            assert got == _brute_force_code(x, vals), x
        n_checked += 1
    assert n_checked > 65000


def test_e4m3_nan_keeps_sign(orc):
    assert orc.e4m3_encode(float("nan")) & 0x7F == 0x7F


def test_bf16_round_matches_torch_on_float32(orc):
    rng = np.random.default_rng(3)
    xs = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        np.clip(rng.standard_normal(1000) * 2e38, -3.3e38, 3.3e38).astype(np.float32),
        # exact ties: 8 significant bits plus a half
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -133 * 1.5,
                  3.3895314e38, 3.39e38, 0.0, -0.0], np.float32),
    ])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, r in zip(xs, ref):
        assert orc.bf16_round(float(x)) == int(r), (x, hex(orc.bf16_round(float(x))), hex(int(r)))


def test_bf16_round_of_doubles_is_nearest(orc):
    """Doubles with more than 24 significant bits: compare with the nearest bf16
    found by exact rational comparison of the two neighbours."""
    rng = np.random.default_rng(4)
    for x in rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000)):
        b = orc.bf16_round(float(x))
        v = orc.bf16_to_float(b)
        lo = torch.tensor([v], dtype=torch.float32).view(torch.int32).item()
        nb = [lo - 1, lo + 1]
        fx = Fraction(float(x))
        for n in nb:
            w = torch.tensor([n], dtype=torch.int32).view(torch.float32).item()
            wb = torch.tensor([w], dtype=torch.float32).to(torch.bfloat16).to(torch.float32).item()
            assert abs(Fraction(v) - fx) <= abs(Fraction(wb) - fx)


def _exact_rsqrt_is_correct(a: float, y: float) -> bool:
    """y is the float nearest to 1/sqrt(a): both neighbour midpoints bracket it.
    Checked exactly with rationals: m^2 * a compared with 1."""
    fa = Fraction(a)
    yb = np.float32(y)
    up = np.nextafter(yb, np.float32(np.inf))
    dn = np.nextafter(yb, np.float32(0))
    mu = (Fraction(float(yb)) + Fraction(float(up))) / 2
    md = (Fraction(float(yb)) + Fraction(float(dn))) / 2
    return mu * mu * fa > 1 and md * md * fa < 1


def test_rsqrt_correctly_rounded(orc):
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.uniform(1e-5, 10, 3000), np.exp(rng.uniform(-30, 30, 2000)),
                         [1.0, 4.0, 0.25, 1e-5, 2.0, 3.0]]).astype(np.float32)
    for a in xs:
        assert _exact_rsqrt_is_correct(float(a), orc.rsqrt_cr(float(a))), a


@pytest.mark.parametrize("theta", [500000.0, 10000.0])
def test_inv_freq_matches_torch_fp32_recipe(orc, theta):
    """The page builds inv_freq as 1.0 / (theta ** (arange(0, d, 2, float) / d))
    in torch fp32; torch's CPU routine is the independent check."""
    ref = (1.0 / (theta ** (torch.arange(0, 64, 2, dtype=torch.float) / 64))).numpy()
    got = orc.inv_freq(theta)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert got[0] == 1.0
