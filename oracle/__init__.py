"""CPU oracle for the gated-attention decode / verify step (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  It wraps ``oracle.c`` (plain C, built with gcc)
through ctypes and shares nothing with the HIP library.

Every function follows the page "012-attention-local-splits.py" (SGLang's Muse
Spark Open gated attention, H200): the ``_prepare_qkv`` kernel for the
prologue, the ``flash_attn_with_kvcache`` call in ``kernel_fn`` for attention
and ``rms_norm_gate`` for the epilogue.  ``oracle.c`` cites each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]
# The sanitizer build (address + undefined behaviour, host code only): the
# same source into its own library, selected with ORACLE_SANITIZE=1 (the
# process must then preload the ASan runtime, see tests/test_sanitizers.py).
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so (or, sanitize=True, the address and
    undefined-behaviour sanitized liboracle_san.so) with gcc (no GPU toolchain
    involved)."""
    out = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp"
        flags = CFLAGS + (SAN_FLAGS if sanitize else [])
        subprocess.check_call(["gcc", *flags, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("rope_theta", ctypes.c_float),
                ("sm_scale", ctypes.c_float), ("kv_scale", ctypes.c_float),
                ("q_scale", ctypes.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        san = os.environ.get("ORACLE_SANITIZE") == "1"
        path = _SAN_LIB if san else _LIB
        if not os.path.exists(path):
            build(sanitize=san)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_float.restype = ctypes.c_float
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_rsqrt_cr.argtypes = [ctypes.c_float]
        L.orc_rsqrt_cr.restype = ctypes.c_float
        L.orc_inv_freq.argtypes = [ctypes.c_float, ctypes.c_int, P]
        L.orc_inv_freq.restype = None
        L.orc_norm_rope_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_float, P]
        L.orc_norm_rope_row.restype = None
        L.orc_prologue.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, ctypes.c_float,
                                   ctypes.c_float, P]
        L.orc_attention.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, ctypes.c_float,
                                    ctypes.c_float, ctypes.c_int64, P, P, P]
        L.orc_epilogue.argtypes = [ctypes.POINTER(_Cfg), P, P, ctypes.c_int64, P, P, P]
        L.orc_step.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, P, ctypes.c_float,
                               ctypes.c_float, P, P, P]
        for f in ("orc_prologue", "orc_attention", "orc_epilogue", "orc_step"):
            getattr(L, f).restype = ctypes.c_int
        L.orc_fp16_to_double.restype = ctypes.c_double
        L.orc_fp16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_fp16_round.restype = ctypes.c_uint16
        L.orc_fp16_round.argtypes = [ctypes.c_double]
        L.orc_sparse_attention.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_float, ctypes.c_float, P]
        L.orc_sparse_step.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, ctypes.c_int32,
                                      ctypes.c_int32, P, P, ctypes.c_float, ctypes.c_float, P, P, P]
        L.orc_qk_norm.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_float, ctypes.c_float, P]
        L.orc_page_table.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, P, P, P]
        L.orc_page_table.restype = ctypes.c_int
        L.orc_threads.argtypes = [ctypes.c_int]
        L.orc_threads.restype = ctypes.c_int
        _lib = L
    return _lib


@dataclass
class Config:
    """The page's Config: batch, q_len, heads, head_dim, page_size, window,
    rope_theta, the applied softmax scale and the cache-scale value."""
    batch: int
    q_len: int
    num_q_heads: int = 16
    num_kv_heads: int = 2
    head_dim: int = 64
    page_size: int = 1
    window: int = 0
    max_pages: int = 0
    num_pages: int = 0
    rope_theta: float = 0.0
    sm_scale: float = 0.125
    kv_scale: float = 1.0
    q_scale: float = 1.0  # q's norm output scale (page "qk_norm"); 1 = page 1

    def c(self) -> _Cfg:
        return _Cfg(self.batch, self.q_len, self.num_q_heads, self.num_kv_heads, self.head_dim,
                    self.page_size, self.window, self.max_pages, self.num_pages,
                    self.rope_theta, self.sm_scale, self.kv_scale, self.q_scale)


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def threads(n: int = 0) -> int:
    """Set the OpenMP thread count of the oracle's attention loops (n > 0) and
    return the count they will use.  Results do not depend on it: each
    (token, head) pair is computed by one thread in a fixed order."""
    return int(lib().orc_threads(int(n)))


# --- number formats --------------------------------------------------------

def bf16_round(x: float) -> int:
    return int(lib().orc_bf16_round(float(x)))


def bf16_to_float(bits: int) -> float:
    return float(lib().orc_bf16_to_float(int(bits)))


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e4m3_decode(code: int) -> float:
    return float(lib().orc_e4m3_decode(int(code)))


def rsqrt_cr(a: float) -> float:
    return float(lib().orc_rsqrt_cr(float(a)))


def inv_freq(theta: float, head_dim: int = 64) -> np.ndarray:
    out = np.zeros(head_dim // 2, np.float32)
    lib().orc_inv_freq(float(theta), head_dim, _p(out))
    return out


def norm_rope_row(x_bits: np.ndarray, pos: int = 0, theta: float = 0.0) -> np.ndarray:
    """Normed (and, if theta != 0, rotated) bf16-valued row as float32."""
    x = np.ascontiguousarray(x_bits, np.uint16)
    y = np.zeros(x.shape[-1], np.float32)
    lib().orc_norm_rope_row(_p(x), x.shape[-1], int(pos), float(theta), _p(y))
    return y


# --- the step ------------------------------------------------------------------

def prologue(cfg: Config, qkv: np.ndarray, positions: np.ndarray, cache_loc: np.ndarray,
             k_cache: np.ndarray, v_cache: np.ndarray, k_scale: float, v_scale: float):
    """Run the prologue; updates k_cache/v_cache (uint8) in place, returns q e4m3 codes."""
    T = cfg.batch * cfg.q_len
    q = np.zeros((T, cfg.num_q_heads, cfg.head_dim), np.uint8)
    c = cfg.c()
    _check(lib().orc_prologue(ctypes.byref(c), _p(qkv), _p(positions), _p(cache_loc),
                              _p(k_cache), _p(v_cache), float(k_scale), float(v_scale), _p(q)),
           "prologue")
    return q


def attention(cfg: Config, q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
              page_table: np.ndarray, cache_seqlens: np.ndarray, k_scale: float, v_scale: float,
              sel_t: np.ndarray | None = None, sel_h: np.ndarray | None = None) -> np.ndarray:
    """Unrounded (double) attention output for the selected (token, head) pairs,
    or all of them in (token, head) order."""
    T = cfg.batch * cfg.q_len
    n = T * cfg.num_q_heads if sel_t is None else len(sel_t)
    o = np.zeros((n, cfg.head_dim), np.float64)
    st = None if sel_t is None else np.ascontiguousarray(sel_t, np.int64)
    sh = None if sel_h is None else np.ascontiguousarray(sel_h, np.int32)
    c = cfg.c()
    _check(lib().orc_attention(ctypes.byref(c), _p(q), _p(k_cache), _p(v_cache), _p(page_table),
                               _p(cache_seqlens), float(k_scale), float(v_scale), n, _p(st),
                               _p(sh), _p(o)), "attention")
    return o


def epilogue(cfg: Config, o: np.ndarray, qkv: np.ndarray, sel_t: np.ndarray | None = None,
             sel_h: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns of the gated epilogue for the selected pairs."""
    n = o.shape[0]
    out = np.zeros((n, cfg.head_dim), np.uint16)
    st = None if sel_t is None else np.ascontiguousarray(sel_t, np.int64)
    sh = None if sel_h is None else np.ascontiguousarray(sel_h, np.int32)
    o = np.ascontiguousarray(o, np.float64)
    c = cfg.c()
    _check(lib().orc_epilogue(ctypes.byref(c), _p(o), _p(qkv), n, _p(st), _p(sh), _p(out)),
           "epilogue")
    return out


def step_meta(cfg: Config, seq_lens: np.ndarray, page_table: np.ndarray):
    """(positions int64 [T], cache_loc int64 [T], cache_seqlens int32 [B]) of a step."""
    T = cfg.batch * cfg.q_len
    seq = np.ascontiguousarray(seq_lens, np.int32)
    pt = np.ascontiguousarray(page_table, np.int32)
    pos = np.empty(T, np.int64)
    loc = np.empty(T, np.int64)
    cs = np.empty(cfg.batch, np.int32)
    _check(lib().orc_step_meta(ctypes.byref(cfg.c()), _p(seq), _p(pt), _p(pos), _p(loc), _p(cs)),
           "step_meta")
    return pos, loc, cs


def page_table(req_to_token: np.ndarray, slot_ids: np.ndarray, kv_lens: np.ndarray,
               page_size: int, max_pages: int):
    """Page "msa.py" _build_page_table (see orc_page_table): returns (padded page
    table int32 [B, max_pages], packed kv_indices int32, kv_indptr int32 [B+1])."""
    r2t = np.ascontiguousarray(req_to_token, np.int32)
    sid = np.ascontiguousarray(slot_ids, np.int32)
    kvl = np.ascontiguousarray(kv_lens, np.int32)
    B = len(sid)
    n = np.where(kvl > 0, (kvl.astype(np.int64) + page_size - 1) // page_size, 0)
    table = np.empty((B, max_pages), np.int32)
    packed = np.empty(max(int(n.sum()), 1), np.int32)
    indptr = np.empty(B + 1, np.int32)
    _check(lib().orc_page_table(_p(r2t), r2t.shape[1], r2t.shape[0], _p(sid), _p(kvl), B,
                                int(page_size), int(max_pages), _p(table), _p(packed),
                                _p(indptr)), "page_table")
    return table, packed[:int(n.sum())], indptr


def step(cfg: Config, qkv, positions, cache_loc, cache_seqlens, page_table, k_cache, v_cache,
         k_scale: float, v_scale: float):
    """Whole step; caches updated in place.  Returns (q codes, out bf16 bits [B, L, Hq*D],
    unrounded attention output double [T, Hq, D])."""
    T = cfg.batch * cfg.q_len
    q = np.zeros((T, cfg.num_q_heads, cfg.head_dim), np.uint8)
    o = np.zeros((T * cfg.num_q_heads, cfg.head_dim), np.float64)
    out = np.zeros((T * cfg.num_q_heads, cfg.head_dim), np.uint16)
    c = cfg.c()
    _check(lib().orc_step(ctypes.byref(c), _p(qkv), _p(positions), _p(cache_loc),
                          _p(cache_seqlens), _p(page_table), _p(k_cache), _p(v_cache),
                          float(k_scale), float(v_scale), _p(q), _p(o), _p(out)), "step")
    return (q, out.reshape(cfg.batch, cfg.q_len, cfg.num_q_heads * cfg.head_dim),
            o.reshape(T, cfg.num_q_heads, cfg.head_dim))


# Page "qk_norm" (vLLM's CuTeDSL fused QK-norm): the plain definition, see
# orc_qk_norm in oracle.c.
QK_BF16, QK_FP16 = 0, 1


def fp16_round(x: float) -> int:
    """Binary16 bit pattern of x rounded to nearest, ties to even."""
    return int(lib().orc_fp16_round(float(x)))


def fp16_to_float(h: int) -> float:
    return float(lib().orc_fp16_to_double(int(h)))


def qk_norm(x: np.ndarray, num_heads: int, head_dim: int, dtype: int, eps: float = 1e-5,
            scale: float = 1.0) -> np.ndarray:
    """x: uint16 bit patterns [M, row_stride] (bf16 or fp16 per dtype); the
    first num_heads * head_dim columns of each row are normed.  Returns the
    uint16 bit patterns of the [M, num_heads * head_dim] output."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, stride = x.shape
    out = np.zeros((M, num_heads * head_dim), np.uint16)
    _check(lib().orc_qk_norm(_p(x), M, num_heads, head_dim, stride, dtype, ctypes.c_float(eps),
                             ctypes.c_float(scale), _p(out)), "orc_qk_norm")
    return out


# Page "msa.py": page-list-driven (top-k block-sparse) decode, see
# orc_sparse_attention in oracle.c.

def sparse_attention(cfg: Config, q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     page_table: np.ndarray, cache_seqlens: np.ndarray, block_idx: np.ndarray,
                     block_size: int, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Unrounded attention output double [B, Hq, D]; block_idx int32 [Hkv, B, topk]."""
    bi = np.ascontiguousarray(block_idx, np.int32)
    o = np.zeros((cfg.batch, cfg.num_q_heads, cfg.head_dim), np.float64)
    _check(lib().orc_sparse_attention(ctypes.byref(cfg.c()), _p(np.ascontiguousarray(q)),
                                      _p(k_cache), _p(v_cache),
                                      _p(np.ascontiguousarray(page_table, np.int32)),
                                      _p(np.ascontiguousarray(cache_seqlens, np.int32)), _p(bi),
                                      int(block_size), int(bi.shape[-1]), float(k_scale),
                                      float(v_scale), _p(o)), "sparse_attention")
    return o


def sparse_step(cfg: Config, qkv, positions, cache_loc, cache_seqlens, page_table, block_idx,
                block_size: int, k_cache, v_cache, k_scale: float, v_scale: float):
    """Whole sparse decode step; caches updated in place.  Returns (q codes, out
    bf16 bits [B, 1, Hq*D], unrounded attention output double [B, Hq, D])."""
    T = cfg.batch * cfg.q_len
    bi = np.ascontiguousarray(block_idx, np.int32)
    q = np.zeros((T, cfg.num_q_heads, cfg.head_dim), np.uint8)
    o = np.zeros((T * cfg.num_q_heads, cfg.head_dim), np.float64)
    out = np.zeros((T * cfg.num_q_heads, cfg.head_dim), np.uint16)
    _check(lib().orc_sparse_step(ctypes.byref(cfg.c()), _p(qkv), _p(positions), _p(cache_loc),
                                 _p(cache_seqlens), _p(page_table), _p(bi), int(block_size),
                                 int(bi.shape[-1]), _p(k_cache), _p(v_cache), float(k_scale),
                                 float(v_scale), _p(q), _p(o), _p(out)), "sparse_step")
    return (q, out.reshape(cfg.batch, cfg.q_len, cfg.num_q_heads * cfg.head_dim),
            o.reshape(T, cfg.num_q_heads, cfg.head_dim))
