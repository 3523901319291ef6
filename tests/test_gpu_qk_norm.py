"""GPU parity of the per-head QK-norm with an output scale (page "qk_norm",
vLLM's CuTeDSL fused QK-norm: the qk_norm function and QKNormDirectKernel's
kernel) against the oracle, through the C ABI.  The definition fixes every
rounding (the sum of squares formed exactly, a correctly rounded rsqrt, fp32
products, one final rounding), so the bar is bit-exact, NaN for NaN."""
import sys

import numpy as np
import pytest
import torch

import attention_decode_qk_amd as ga
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"bf16": (torch.bfloat16, oracle.QK_BF16), "fp16": (torch.float16, oracle.QK_FP16)}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu(xbits: np.ndarray, dtype: str, heads: int, D: int, eps: float, scale: float,
         stream=None) -> np.ndarray:
    tdt, _ = DT[dtype]
    x = torch.from_numpy(np.ascontiguousarray(xbits).view(np.int16)).to(DEV).view(tdt)
    x = x[:, :heads * D]  # strided view: rows keep the full stride
    out = ga.qk_norm(x, D, eps=eps, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def _assert_same(got: np.ndarray, want: np.ndarray, dtype: str):
    assert got.shape == want.shape
    if np.array_equal(got, want):
        return
    tdt, _ = DT[dtype]
    g = torch.from_numpy(got.view(np.int16)).view(tdt).float().numpy()
    w = torch.from_numpy(want.view(np.int16)).view(tdt).float().numpy()
    both_nan = np.isnan(g) & np.isnan(w)
    bad = (got != want) & ~both_nan
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[:4]}"


CASES = [
    # (dtype, head_dim, heads, rows, row_stride, scale, std)
    ("bf16", 64, 16, 1, 2304, 5.473, 1.0),
    ("bf16", 64, 16, 333, 2304, 5.473, 1.0),
    ("bf16", 64, 2, 77, 128, 1.0, 3.0),
    ("bf16", 128, 3, 50, 392, 1.0, 0.01),
    ("bf16", 256, 5, 19, 1280, 0.125, 1.0),
    ("fp16", 64, 16, 333, 1032, 5.473, 1.0),
    ("fp16", 128, 4, 61, 512, 1.0, 2.0),
    ("fp16", 256, 2, 40, 520, 1.0, 1e-3),
    ("fp16", 256, 7, 9, 1792, 2.0, 0.5),
    # more groups than one pass of the capped grid covers (the grid strides),
    # one group per thread and four
    ("bf16", 64, 16, 10000, 2304, 5.473, 1.0),
    ("bf16", 64, 16, 20000, 1024, 1.0, 1.0),
    ("fp16", 256, 8, 9000, 2048, 5.473, 1.0),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=lambda i: "-".join(map(str, CASES[i])))
def test_qk_norm_matches_the_oracle(ci):
    dtype, D, H, M, stride, scale, std = CASES[ci]
    _say(f"[qk_norm] {CASES[ci]}")
    w = synth.QkNormWorkload("t", M, H, D, stride, dtype, scale, std=std, seed=300 + ci)
    x = synth.make_qk_norm_input(w)
    want = oracle.qk_norm(x, H, D, DT[dtype][1], eps=1e-5, scale=scale)
    _assert_same(_gpu(x, dtype, H, D, 1e-5, scale), want, dtype)


@pytest.mark.parametrize("name", list(synth.QK_NORM_WORKLOADS))
def test_qk_norm_workloads_at_full_size(name):
    w = synth.QK_NORM_WORKLOADS[name]
    _say(f"[qk_norm] workload {name}")
    x = synth.make_qk_norm_input(w)
    want = oracle.qk_norm(x, w.num_heads, w.head_dim, DT[w.dtype][1], eps=w.eps, scale=w.scale)
    _assert_same(_gpu(x, w.dtype, w.num_heads, w.head_dim, w.eps, w.scale), want, w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_qk_norm_edge_values(dtype):
    """Zero heads (eps = 0: 0 * inf = NaN on both sides), tiny heads whose mean
    square is subnormal, huge heads, a NaN and an infinity in a head."""
    _say(f"[qk_norm] edges {dtype}")
    D, H = 64, 6
    vals = np.zeros((4, H * D), np.float32)
    rng = np.random.default_rng(9)
    vals[0, 0:D] = 0.0
    vals[0, D:2 * D] = rng.standard_normal(D) * (1e-21 if dtype == "bf16" else 1e-4)
    vals[0, 2 * D:3 * D] = rng.standard_normal(D) * (1e30 if dtype == "bf16" else 6e4)
    vals[0, 3 * D:4 * D] = rng.standard_normal(D)
    vals[0, 3 * D + 5] = np.nan
    vals[0, 4 * D:5 * D] = rng.standard_normal(D)
    vals[0, 4 * D + 9] = np.inf
    vals[1:] = rng.standard_normal((3, H * D))
    bits = synth.to_bf16_bits(vals) if dtype == "bf16" else synth.to_fp16_bits(vals)
    for eps in (0.0, 1e-5):
        want = oracle.qk_norm(bits, H, D, DT[dtype][1], eps=eps, scale=1.5)
        _assert_same(_gpu(bits, dtype, H, D, eps, 1.5), want, dtype)


def test_qk_norm_on_a_side_stream_and_no_rows():
    _say("[qk_norm] side stream")
    w = synth.QkNormWorkload("s", 129, 16, 64, 2304, "bf16", 5.473, seed=5)
    x = synth.make_qk_norm_input(w)
    s = torch.cuda.Stream()
    got = _gpu(x, "bf16", 16, 64, 1e-5, 5.473, stream=s.cuda_stream)
    _assert_same(got, oracle.qk_norm(x, 16, 64, oracle.QK_BF16, scale=5.473), "bf16")
    empty = torch.empty((0, 2304), dtype=torch.bfloat16, device=DEV)[:, :1024]
    assert ga.qk_norm(empty, 64).shape == (0, 1024)
