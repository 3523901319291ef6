"""Pins of the oracle's page-3 QK-norm (page "qk_norm", vLLM's CuTeDSL fused
QK-norm: the `qk_norm` function and `QKNormDirectKernel.kernel`): each head
group normed without a weight, rstd = rsqrt(sum of squares / head_dim + eps),
fp32 x * rstd (* scale), one rounding to the input's 16-bit type on the store.

Every check compares the oracle with something other than itself: numpy's
binary16 conversion, closed forms, an exact power-of-two invariance, an
independent exact-arithmetic evaluation (fractions and decimal) on tiny inputs,
and torch's float64 rms_norm."""
import decimal
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

BF16, FP16 = oracle.QK_BF16, oracle.QK_FP16


def _bits(values: np.ndarray, dtype: int) -> np.ndarray:
    t = torch.from_numpy(np.asarray(values, np.float32))
    t = t.to(torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _values(bits: np.ndarray, dtype: int) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == BF16 else torch.float16).to(torch.float64).numpy()


def _random_x(rng, M, n, dtype, std=1.0):
    return _bits(rng.standard_normal((M, n)).astype(np.float32) * std, dtype)


# ---- binary16 codec against numpy's float16 --------------------------------

def test_fp16_decode_matches_numpy_exhaustively():
    h = np.arange(65536, dtype=np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_float(int(v)) for v in h])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_fp16_round_matches_numpy():
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(4000) * np.exp2(rng.integers(-30, 18, 4000)))
    # ties, binade edges, the subnormal range and the overflow threshold
    xs += [1 + 2.0**-11, 1 + 3 * 2.0**-11, 2.0**-25, 3 * 2.0**-25, 2.0**-24 * 1.5,
           2.0**-14 * (1 - 2.0**-11), 2.0**-14 - 2.0**-25, 65504.0, 65519.99, 65520.0, 1e9,
           -0.0, 0.0, -(1 + 2.0**-11), 2047.5, 2048.5, 4095.0]
    for x in xs:
        with np.errstate(over="ignore"):
            ref = int(np.array(x, np.float64).astype(np.float16).view(np.uint16))
        assert oracle.fp16_round(x) == ref, x


# ---- closed forms ----------------------------------------------------------

@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("c", [1.0, -2.0, 0.25, 3.0, -0.1, 7.5])
@pytest.mark.parametrize("scale", [1.0, 5.473])
def test_constant_head_without_eps_is_the_scale(dtype, c, scale):
    """x = c over a head and eps = 0: rstd = 1/|c| (rounded once), so each output
    is sign(c) * scale to well within a 16-bit step, i.e. exactly the rounded
    scale."""
    D, H = 64, 3
    x = _bits(np.full((2, H * D), c, np.float32), dtype)
    out = oracle.qk_norm(x, H, D, dtype, eps=0.0, scale=scale)
    want = _bits(np.full(out.shape, np.sign(c) * np.float32(scale), np.float32), dtype)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("k", [-4, 3])
def test_power_of_two_input_scaling_is_exactly_invisible_without_eps(dtype, k):
    rng = np.random.default_rng(11 + k)
    D, H = 128, 2
    # magnitudes in [1/8, 8]: the scaled values stay normal in both formats
    mag = np.exp2(rng.uniform(-3, 3, (5, H * D))) * rng.choice([-1.0, 1.0], (5, H * D))
    x = _bits(mag.astype(np.float32), dtype)
    x2 = _bits(_values(x, dtype).astype(np.float32) * np.float32(2.0**k), dtype)
    assert np.array_equal(_values(x2, dtype), _values(x, dtype) * 2.0**k)  # exact scaling
    a = oracle.qk_norm(x, H, D, dtype, eps=0.0, scale=1.7)
    b = oracle.qk_norm(x2, H, D, dtype, eps=0.0, scale=1.7)
    assert np.array_equal(a, b)


# ---- independent exact evaluation on tiny inputs ----------------------------

def _rsqrt_correctly_rounded(a: np.float32) -> np.float32:
    """fp32 nearest to 1/sqrt(a), from a 60-digit decimal value: the float32
    neighbours of a first guess are compared with it exactly."""
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        t = 1 / decimal.Decimal(float(a)).sqrt()
        f = np.float32(float(t))
        cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
        return min(cands, key=lambda v: abs(decimal.Decimal(float(v)) - t))


def _brute(xbits, H, D, dtype, eps, scale):
    xv = _values(xbits, dtype)
    M = xv.shape[0]
    out = np.zeros((M, H * D), np.float32)
    for r in range(M):
        for h in range(H):
            seg = xv[r, h * D:(h + 1) * D]
            ss = sum((Fraction(float(v)) ** 2 for v in seg), Fraction(0))  # exact
            ss32 = np.float32(float(ss))  # one rounding (ss is exact in float64 here)
            ms = np.float32(ss32 / np.float32(D))
            a = np.float32(ms + np.float32(eps))
            rstd = _rsqrt_correctly_rounded(a)
            y = (seg.astype(np.float32) * rstd).astype(np.float32)
            if scale != 1.0:
                y = (y * np.float32(scale)).astype(np.float32)
            out[r, h * D:(h + 1) * D] = y
    return _bits(out, dtype)


@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("scale", [1.0, 5.473])
@pytest.mark.parametrize("D,H", [(8, 2), (16, 3), (64, 1)])
def test_tiny_inputs_match_an_exact_arithmetic_evaluation(dtype, scale, D, H):
    rng = np.random.default_rng(100 + D + H)
    x = _random_x(rng, 3, H * D, dtype, std=0.7)
    got = oracle.qk_norm(x, H, D, dtype, eps=1e-5, scale=scale)
    assert np.array_equal(got, _brute(x, H, D, dtype, 1e-5, scale))


def test_tiny_eps_dominated_heads_match_the_exact_evaluation():
    """Small inputs, where + eps decides rstd: a dropped or misplaced eps fails."""
    rng = np.random.default_rng(7)
    x = _random_x(rng, 4, 2 * 16, BF16, std=1e-3)
    got = oracle.qk_norm(x, 2, 16, BF16, eps=1e-5, scale=1.0)
    assert np.array_equal(got, _brute(x, 2, 16, BF16, 1e-5, 1.0))


# ---- torch's float64 rms_norm ----------------------------------------------

@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_within_one_step_of_torch_rms_norm(dtype, D):
    rng = np.random.default_rng(D + dtype)
    H, M, scale = 4, 33, 5.473
    x = _random_x(rng, M, H * D, dtype, std=2.0)
    got = _values(oracle.qk_norm(x, H, D, dtype, eps=1e-5, scale=scale), dtype)
    xt = torch.from_numpy(_values(x, dtype)).view(M, H, D)
    ref = (torch.nn.functional.rms_norm(xt, (D,), eps=1e-5) * scale).view(M, H * D).numpy()
    step = np.exp2(np.floor(np.log2(np.abs(ref))) - (7 if dtype == BF16 else 10))
    assert np.all(np.abs(got - ref) <= step * 1.01)


# ---- strided rows -------------------------------------------------------------

def test_columns_past_the_heads_are_never_read():
    rng = np.random.default_rng(5)
    H, D, M = 16, 64, 6
    x = _random_x(rng, M, H * D, BF16)
    wide = np.full((M, 2304), 0x7FC0, np.uint16)  # NaN beyond the normed columns
    wide[:, :H * D] = x
    a = oracle.qk_norm(x, H, D, BF16, scale=5.473)
    b = oracle.qk_norm(wide, H, D, BF16, scale=5.473)
    assert np.array_equal(a, b)


def test_empty_input_gives_empty_output():
    out = oracle.qk_norm(np.zeros((0, 128), np.uint16), 2, 64, BF16)
    assert out.shape == (0, 128)
