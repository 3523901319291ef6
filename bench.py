"""Benchmark of the gated-attention layer-step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload swa_decode]

A "step" is one layer-step of the whole hot path (norm, RoPE, e4m3 store,
split attention, combine + gated epilogue: one fused kernel) over one batch of
synthetic inputs.  The default
workload is the decode batch the headline metric is quoted on: B=32, L=1,
16 query / 2 KV heads, head_dim 64, page_size 1, window 2048, RoPE theta
5e5, cached lengths uniform in [4096, 16384], shuffled page table.

Cold-cache discipline: the steps round-robin over per-layer pools (own K/V
caches, own page-table permutation and cache rows, own projection rows, same
lengths), enough of them that one round touches at least 1 GiB -- the bytes
the steps read and write, not the pools' size -- four times the 256 MB Infinity
Cache, as a model's layers would.  After one sweep over every pool the
warm-up steps run on pools 0 .. W-1 and the timed steps start at pool W, so a
timed step never reads a pool touched less than a round of pools earlier
(config.timed_min_reuse_bytes reports the smallest such distance).  --shared-table shares pool 0's page table and cache rows
instead, as a serving engine that builds them once per step for every layer
would (measured within noise of the default).  The layer-
steps are captured in HIP graphs outside the timed region (one graph of W
warm-up steps, one of exactly K timed steps) and the timed region is one
replay of the K-step graph, bracketed by synchronisation and HIP events on the
replay stream (a short untimed GPU spin before the start event lets the host
finish submitting the graph, so its submission latency is not counted).  For q_len <= 8 the step is a single kernel, so the time per
step is also the kernel's average duration (the roofline figure); a second,
eager pass with the library's event hook is reported as well (it includes
event overhead).  An extend workload (q_len > 8: swa_extend, full_extend) is
two launches, and its roofline (matrix cores) takes the attention launch's
duration from that event hook, which then brackets that launch alone.

Prints one JSON line (see the design doc for every field).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
SPIN_CYCLES = 5_000_000  # GPU spin ahead of a timed replay (about 2 ms at 2.4 GHz)
METRIC = "µs per layer-step and KV-read HBM GB/s (% of peak), B=32 L=1 16k ctx"
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "f16": 2500.0}  # MI355X dense matrix-core peaks


def _is_extend(workload: str) -> bool:
    """Whether the workload's dominant kernel is the extend attention kernel (a
    block-sparse prefill's is the step kernel, whatever its chunk length)."""
    import synth
    w = synth.WORKLOADS.get(workload)
    return w is not None and w.q_len > 8 and w.prefill_block == 0


def _kernel_prefix(workload: str) -> str:
    if workload.startswith("qk_norm"):
        return "qk_norm"
    return "extend_attn" if _is_extend(workload) else "fused_step"


def counters_file(workload: str) -> str:
    """The committed rocprofv3 counter summary of one workload."""
    return os.path.join(ROOT, "profiles", f"{_kernel_prefix(workload)}_{workload}_counters.md")


def _sources(*kernel_files: str):
    return [os.path.join(ROOT, "attention_decode_qk_amd", "csrc", f)
            for f in (*kernel_files, "kernels.h", "numerics.h")] + \
           [os.path.join(ROOT, "attention_decode_qk_amd", "build.py")]  # compiler flags


KERNEL_SOURCES = _sources("step_kernel.hip", "step_device.h")
EXTEND_SOURCES = _sources("extend_kernel.hip", "step_device.h")
QK_NORM_SOURCES = _sources("qk_norm_kernel.hip")


def workload_sources(workload: str):
    """The sources that build the workload's dominant kernel."""
    if workload.startswith("qk_norm"):
        return QK_NORM_SOURCES
    return EXTEND_SOURCES if _is_extend(workload) else KERNEL_SOURCES


def kernel_source_hash(files=None) -> str:
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def attended_keys(w, cache_seqlens) -> int:
    """Keys a step must read: per request, the union of its queries' visible
    ranges (query i at p = cache_seqlens - L + i sees max(0, p-W+1)..p)."""
    total = 0
    for cs in cache_seqlens.tolist():
        last = cs - 1
        first = max(cs - w.q_len - w.window + 1, 0) if w.window > 0 else 0
        total += max(0, last - first + 1)
    return total


def extend_flops(w, cache_seqlens):
    """Extend / prefill: the attention's algorithmic flops per step, QK^T (fp8
    operands) and PV (f16 operands) separately: 2*D each per (query row,
    visible key), query i of request b at p = cache_seqlens[b] - L + i seeing
    max(0, p-W+1)..p."""
    import numpy as np
    rows = 0
    for cs in cache_seqlens.tolist():
        p = np.arange(cs - w.q_len, cs, dtype=np.int64)
        vis = np.minimum(p + 1, w.window) if w.window > 0 else p + 1
        rows += int(np.maximum(vis, 0).sum())
    f = 2 * w.head_dim * rows * w.num_q_heads
    return f, f


def ragged_accounting(w, x, lens):
    """A ragged batch (request b keeps lens[b] new tokens, cached length
    seq_lens[b] + lens[b]): KV bytes (the union of each request's visible
    keys), the step's algorithmic bytes as for the uniform step, and the
    attention's flops (QK^T, PV)."""
    import numpy as np
    per_token = (w.width * 2 + 2 * w.num_kv_heads * w.head_dim
                 + w.num_q_heads * w.head_dim * 2 + 16)
    keys = pages = rows = 0
    for sl, n in zip(x.seq_lens.tolist(), lens.tolist()):
        if n == 0:
            continue
        cs = sl + n
        first = max(0, cs - n - w.window + 1) if w.window > 0 else 0
        keys += cs - first
        pages += (cs - 1) // w.page_size - first // w.page_size + 1
        p = np.arange(cs - n, cs, dtype=np.int64)
        vis = np.minimum(p + 1, w.window) if w.window > 0 else p + 1
        rows += int(vis.sum())
    kv = keys * w.num_kv_heads * w.head_dim * 2
    f = 2 * w.head_dim * rows * w.num_q_heads
    return kv, kv + 4 * pages + int(lens.sum()) * per_token, f, f


def sparse_prefill_accounting(w, x, sp):
    """Block-sparse prefill: per (KV head, query) the listed blocks' keys below
    the query's cached length, each a half row (one KV head) of K and of V; the
    listed blocks' page-table entries (one page per block) and the lists; per
    token the projection row, K/V row stores, output row, position and cache row."""
    import numpy as np
    bi = sp["block_idx"].astype(np.int64)                  # [Hkv, T, topk]
    cs = sp["cache_seqlens"].astype(np.int64)[None, :, None]
    BS = w.prefill_block
    keys = np.clip(cs - bi * BS, 0, BS) * (bi >= 0)
    kv = int(keys.sum()) * w.head_dim * 2
    pages = int(((keys > 0).sum()) * -(-BS // w.page_size))
    per_token = (w.width * 2 + 2 * w.num_kv_heads * w.head_dim
                 + w.num_q_heads * w.head_dim * 2 + 16)
    lists = 4 * bi.size
    return kv, kv + 4 * pages + lists + x.tokens * per_token


def mfma_peak(f_fp8: float, f_f16: float) -> float:
    """The matrix cores' peak for this mix: both products at their own dtype's
    dense peak, back to back (TFLOP/s)."""
    t = f_fp8 / MFMA_PEAK_TFLOPS["fp8"] + f_f16 / MFMA_PEAK_TFLOPS["f16"]
    return (f_fp8 + f_f16) / t


def sparse_keys(w, x):
    """Page-list-driven decode: per (KV head, request) the keys of its listed
    blocks below the cached length (the union), and the listed blocks' pages."""
    keys = pages = 0
    bi = x.extra["block_idx"]
    for g in range(w.num_kv_heads):
        for b, cs in enumerate(x.cache_seqlens.tolist()):
            seen, pg = set(), set()
            for j in bi[g, b].tolist():
                if j >= 0:
                    ks = range(j * w.sparse_block, min((j + 1) * w.sparse_block, cs))
                    seen.update(ks)
                    pg.update(k // w.page_size for k in ks)
            keys += len(seen)
            pages += len(pg)
    return keys, pages


def algorithmic_bytes(w, x):
    """Per step: KV bytes (the metric's numerator), and the step kernel's
    algorithmic bytes: KV rows and page-table entries of the attended keys, plus
    per token the projection row, its two K/V row stores, its output row and its
    position and cache row.  Page-list-driven decode reads one KV head's half of
    a row per (head, listed key), and its block lists."""
    per_token = (w.width * 2 + 2 * w.num_kv_heads * w.head_dim
                 + w.num_q_heads * w.head_dim * 2 + 16)
    if w.sparse_block > 0:
        keys, pages = sparse_keys(w, x)
        kv = keys * w.head_dim * 2
        lists = 4 * w.num_kv_heads * w.batch * w.sparse_topk
        return kv, kv + 4 * pages + lists + x.tokens * per_token
    keys = attended_keys(w, x.cache_seqlens)
    kv = keys * w.num_kv_heads * w.head_dim * 2
    pages = 0
    for cs in x.cache_seqlens.tolist():
        first = cs - w.q_len - (w.window - 1 if w.window > 0 else cs)
        first = max(first, 0)
        pages += (cs - 1) // w.page_size - first // w.page_size + 1
    return kv, kv + 4 * pages + x.tokens * per_token


def step_accounting(w, x0):
    """(KV bytes, algorithmic bytes) of one step of workload w on its seeded
    inputs x0: the ragged and block-sparse prefill batches count only what
    they keep."""
    import synth
    if w.prefill_block > 0:
        sp0 = synth.sparse_prefill(x0, w.prefill_block, w.prefill_topk, seed=w.seed + 2)
        return sparse_prefill_accounting(w, x0, sp0)
    if w.ragged_lo > 0:
        return ragged_accounting(w, x0, synth.ragged_lens(w))[:2]
    return algorithmic_bytes(w, x0)


def extend_attention_bytes(w, step_bytes: int, tokens: int) -> int:
    """The extend path's attention launch alone: the step's KV and page-table
    bytes, and per token its e4m3 query rows, gate columns and output row (the
    prologue, a launch of its own, reads the projection row and stores q and the
    K/V rows)."""
    step_token = w.width * 2 + 2 * w.num_kv_heads * w.head_dim + w.num_q_heads * w.head_dim * 2 + 16
    attn_token = w.num_q_heads * w.head_dim * (1 + 2 + 2)
    return step_bytes - tokens * (step_token - attn_token)


POOL_MEMORY_LIMIT = 64 << 30  # device bytes the layer pools may take


def layer_pool_count(step_bytes: int, pool_bytes: int, cold_bytes: float) -> int:
    """Layer pools to round-robin over: enough that one round touches at least
    cold_bytes (a step touches step_bytes of its pool, whatever the pool's size),
    within POOL_MEMORY_LIMIT of device memory."""
    n = max(1, -(-int(cold_bytes) // max(1, int(step_bytes))))
    return max(1, min(n, POOL_MEMORY_LIMIT // max(1, int(pool_bytes))))


def load_traffic(workload: str):
    """HBM traffic per launch from the workload's committed counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = counters_file(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^traffic_json:\s*(\{.*\})\s*$", text, re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source_sha256") != kernel_source_hash(workload_sources(workload)):
        return None
    return d.get("traffic_bytes_per_launch")


def reuse_distances(before, timed, step_bytes):
    """For each timed step, the bytes the steps since its pool's previous use
    touched (each step touches step_bytes), given the pools run before the timed
    region; None for a pool never used before."""
    last = {}
    seq = list(before) + list(timed)
    out = []
    for i, li in enumerate(seq):
        if i >= len(before):
            out.append(None if li not in last else (i - last[li] - 1) * step_bytes)
        last[li] = i
    return out


def host_description():
    """The benchmark host's CPU: logical CPUs visible, usable by this process,
    and the model name."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def cpu_baseline(x, budget_s: float):
    """The oracle as it stands on this host (at its current thread count), on
    whole steps of layer pool 0's inputs until the time budget is used (at least
    one step)."""
    import numpy as np
    import oracle
    cfg = oracle.Config(q_scale=x.w.q_scale, batch=x.w.batch, q_len=x.w.q_len,
                        num_q_heads=x.w.num_q_heads,
                        num_kv_heads=x.w.num_kv_heads, head_dim=x.w.head_dim,
                        page_size=x.w.page_size, window=x.w.window, max_pages=x.max_pages,
                        num_pages=x.num_pages, rope_theta=x.w.rope_theta,
                        sm_scale=x.w.sm_scale, kv_scale=x.w.kv_scale)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    n = 0
    t0 = time.perf_counter()
    while True:
        if x.w.sparse_block > 0:
            oracle.sparse_step(cfg, x.qkv, x.positions, x.cache_loc, x.cache_seqlens,
                               x.page_table, x.extra["block_idx"], x.w.sparse_block, kc, vc,
                               x.k_scale, x.v_scale)
        else:
            oracle.step(cfg, x.qkv, x.positions, x.cache_loc, x.cache_seqlens, x.page_table, kc,
                        vc, x.k_scale, x.v_scale)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    del np
    return n, dt


def cpu_baseline_extend(x, budget_s: float):
    """Extend / prefill: a whole step of the oracle takes minutes, so it is timed
    on a sample: the prologue of every token once, then attention + epilogue on
    random (token, head) rows in chunks until the budget is used.  Returns the
    estimated seconds per whole step and the sample's description."""
    import numpy as np
    import oracle
    w = x.w
    cfg = oracle.Config(q_scale=w.q_scale, batch=w.batch, q_len=w.q_len,
                        num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                        head_dim=w.head_dim, page_size=w.page_size, window=w.window,
                        max_pages=x.max_pages, num_pages=x.num_pages, rope_theta=w.rope_theta,
                        sm_scale=w.sm_scale, kv_scale=w.kv_scale)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    t0 = time.perf_counter()
    q = oracle.prologue(cfg, x.qkv, x.positions, x.cache_loc, kc, vc, x.k_scale, x.v_scale)
    t_pro = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    n_rows, t_rows = 0, 0.0
    while t_rows < budget_s:
        st = rng.integers(0, x.tokens, 64).astype(np.int64)
        sh = rng.integers(0, w.num_q_heads, 64).astype(np.int32)
        t1 = time.perf_counter()
        o = oracle.attention(cfg, q, kc, vc, x.page_table, x.cache_seqlens, x.k_scale, x.v_scale,
                             st, sh)
        oracle.epilogue(cfg, o, x.qkv, st, sh)
        t_rows += time.perf_counter() - t1
        n_rows += 64
    total_rows = x.tokens * w.num_q_heads
    est = t_pro + t_rows / n_rows * total_rows
    sample = (f"prologue of all {x.tokens} tokens ({t_pro:.1f} s) + attention and epilogue of "
              f"{n_rows} random (token, head) rows of {total_rows} ({t_rows:.1f} s), scaled to "
              f"the whole step: {est:.0f} s per step; single-threaded")  # (thread count noted by the caller)
    return est, sample


def cpu_baseline_legs(x, kv_bytes, budget_s: float, extend: bool):
    """The oracle as it stands on this host, twice on the same sample: with its
    attention loops on every usable CPU (OpenMP over (token, head) pairs: the
    reported value, cores = the threads used) and on one thread."""
    import oracle
    oracle.build()
    host = host_description()
    legs = {}
    n0 = oracle.threads()
    try:
        for name, n in (("omp", max(1, host["usable_cpus"] or 1)), ("single_thread", 1)):
            used = oracle.threads(n)
            if extend:
                est, sample = cpu_baseline_extend(x, budget_s / 2)
                legs[name] = {"value": round(kv_bytes / est / 1e9, 6), "cores": used,
                              "sample": sample.replace("single-threaded", f"{used} threads")}
            else:
                k, dt = cpu_baseline(x, budget_s / 2)
                legs[name] = {"value": round(k * kv_bytes / dt / 1e9, 4), "cores": used,
                              "sample": f"{k} whole steps of layer pool 0 ({x.w.name}), "
                                        f"{used} threads, {dt:.1f} s"}
    finally:
        oracle.threads(n0)
    top = legs["omp"]
    return {"value": top["value"], "unit": "GB/s", "cores": top["cores"], "kind": "oracle",
            "sample": top["sample"], "single_thread": legs["single_thread"], "host": host}


def qk_norm_bytes(w) -> int:
    """Algorithmic HBM bytes of one call: the normed columns read once, the
    output written once."""
    return 2 * w.rows * w.num_heads * w.head_dim * 2


def run_qk_norm(args, w, dev):
    """The per-head QK-norm (page "qk_norm") on its own: K calls round-robin
    over enough input/output buffer pairs that one round touches the cold
    bytes, graph-captured, one replay timed."""
    import numpy as np
    import torch

    import attention_decode_qk_amd as ga
    import synth
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    x0 = synth.make_qk_norm_input(w)
    call_bytes = qk_norm_bytes(w)
    pool_bytes = x0.nbytes + call_bytes // 2
    n_pools = layer_pool_count(call_bytes, pool_bytes, args.cold_bytes * (1 << 30))
    print(f"[bench] {w.name}: {w.rows} x {w.num_heads} x {w.head_dim} {w.dtype}, stride "
          f"{w.row_stride}; {n_pools} buffer pairs", file=sys.stderr, flush=True)
    base = torch.from_numpy(x0.view(np.int16)).to(dev).view(tdt)
    xs, outs = [], []
    for i in range(n_pools):
        x = base if i == 0 else torch.roll(base, shifts=i, dims=0).contiguous()
        xs.append(x[:, :w.num_heads * w.head_dim])
        outs.append(torch.empty((w.rows, w.num_heads * w.head_dim), dtype=tdt, device=dev))
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())

    def call(i, stream):
        ga.qk_norm(xs[i], w.head_dim, eps=w.eps, scale=w.scale, out=outs[i], stream=stream.cuda_stream)

    with torch.cuda.stream(cap):
        for i in range(n_pools):
            call(i, cap)
    torch.cuda.synchronize()

    def capture(pools):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in pools:
                    call(i, cap)
        return g

    # As for the step: the warm-up on buffer pairs 0 .. W-1, the timed calls from pair W on.
    n_warm = max(1, args.warmup)
    warm_pools = [k % n_pools for k in range(n_warm)]
    cold_pools = [(n_warm + k) % n_pools for k in range(args.steps)]
    g_warm, g_cold, g_hot = capture(warm_pools), capture(cold_pools), capture([0] * args.steps)
    torch.cuda.synchronize()
    reuse = [r for r in reuse_distances(list(range(n_pools)) + warm_pools, cold_pools, call_bytes)
             if r is not None]

    def timed(g):
        g_warm.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN_CYCLES)  # as for the step: the host's submission is not timed
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    t0 = time.perf_counter()
    us = 1000.0 * timed(g_cold) / args.steps
    wall_s = time.perf_counter() - t0
    us_warm = 1000.0 * timed(g_hot) / args.steps
    achieved = call_bytes / (us * 1e-6) / 1e9
    result = {
        "metric": f"µs per call and HBM GB/s (% of peak), per-head QK-norm {w.name}",
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000.0, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "num_heads": w.num_heads,
                   "head_dim": w.head_dim, "row_stride": w.row_stride, "scale": w.scale,
                   "buffer_pairs": n_pools, "touched_bytes_per_round": n_pools * call_bytes,
                   "timed_touched_bytes": args.steps * call_bytes,
                   "timed_min_reuse_bytes": min(reuse) if reuse else None},
        "us_per_call": round(us, 3),
        "warm_single_buffer": {"us_per_call": round(us_warm, 3),
                               "gbs": round(call_bytes / (us_warm * 1e-6) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(w.name), "algorithmic_bytes": call_bytes,
                     "kernel": "qk_norm_kernel", "kernel_source": kernel_source_hash(QK_NORM_SOURCES)},
        "timed_wall_s": round(wall_s, 3),
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        dt_code = oracle.QK_BF16 if w.dtype == "bf16" else oracle.QK_FP16
        rows = max(1, min(w.rows, 4096))
        sample = np.ascontiguousarray(x0[:rows])
        n, t1 = 0, time.perf_counter()
        while True:
            oracle.qk_norm(sample, w.num_heads, w.head_dim, dt_code, eps=w.eps, scale=w.scale)
            n += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t1
        per = 2 * rows * w.num_heads * w.head_dim * 2
        result["cpu_baseline"] = {"value": round(n * per / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"{n} calls on the first {rows} rows, single-threaded "
                                            f"(the QK-norm oracle has no parallel loop), {dt:.1f} s",
                                  "host": host_description()}
    print(json.dumps(result), flush=True)


# ---- profile summaries (profiles/*.md) from rocprofv3's CSV output ----------

PROFILES_DIR = os.path.join(ROOT, "profiles")
KERNEL_NAMES = {"fused_step": "fused_step_kernel", "extend_attn": "extend_attn_kernel",
                "qk_norm": "qk_norm_kernel"}


def _short_kernel(name: str) -> str:
    name = re.sub(r"^void ", "", name).replace("mi355x_ga::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def _find_csv(directory: str, suffix: str) -> str:
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    return files[0]


def summarize_trace(workload: str, trace_dir: str, title: str, command: str) -> str:
    """profiles/<kernel>_<workload>_kernel_trace.md from a rocprofv3
    --kernel-trace --stats run: calls and average / min / max duration of each
    of the library's kernels."""
    import csv
    rows = list(csv.DictReader(open(_find_csv(trace_dir, "kernel_stats.csv"))))
    out = os.path.join(PROFILES_DIR, f"{_kernel_prefix(workload)}_{workload}_kernel_trace.md")
    lines = [f"# Kernel trace: {title}", "", "Command (on the MI355X box, from /tmp):", "", "```",
             command, "```", "",
             f"Kernel sources hash (as `bench.py` computes it): "
             f"`{kernel_source_hash(workload_sources(workload))}`", "",
             "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    for r in rows:
        if "mi355x_ga::" not in r["Name"]:
            continue
        lines.append(f"| {_short_kernel(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def _counter_mean(directory: str, counter: str, kernel: str):
    import csv
    import glob
    vals, full = [], None
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
                full = r["Kernel_Name"]
    if not vals:
        raise SystemExit(f"no {counter} for {kernel} under {directory}")
    return sum(vals) / len(vals), len(vals), full


def summarize_counters(workload: str, dirs, title: str, commands, algorithmic: int) -> str:
    """profiles/<kernel>_<workload>_counters.md from four rocprofv3 --pmc runs
    (FETCH_SIZE and WRITE_SIZE of the workload, then of a 1 GiB device copy):
    HBM bytes per launch, each counter scaled by what it reads for the copy."""
    pref = _kernel_prefix(workload)
    kname = KERNEL_NAMES[pref]
    fetch, nf, full = _counter_mean(dirs[0], "FETCH_SIZE", kname)
    write, _, _ = _counter_mean(dirs[1], "WRITE_SIZE", kname)
    cf, _, _ = _counter_mean(dirs[2], "FETCH_SIZE", "copyBuffer")
    cw, _, _ = _counter_mean(dirs[3], "WRITE_SIZE", "copyBuffer")
    copy = 1 << 30
    fs, ws = copy / (cf * 1024), copy / (cw * 1024)
    fb, wb = round(fetch * 1024 * fs), round(write * 1024 * ws)
    kshort = _short_kernel(full) if pref == "fused_step" else kname
    d = {"kernel": kshort, "kernel_source_sha256": kernel_source_hash(workload_sources(workload)),
         "fetch_kib_per_dispatch": round(fetch, 3), "write_kib_per_dispatch": round(write, 3),
         "copy_fetch_kib": round(cf, 3), "copy_write_kib": round(cw, 3),
         "fetch_scale": round(fs, 5), "write_scale": round(ws, 5), "fetch_bytes": fb,
         "write_bytes": wb, "traffic_bytes_per_launch": fb + wb,
         "algorithmic_bytes_per_launch": algorithmic}
    out = os.path.join(PROFILES_DIR, f"{pref}_{workload}_counters.md")
    lines = [f"# HBM counters: {kshort}, {title}", "",
             "Commands (on the MI355X box, from /tmp), one counter per run:", "", "```", *commands,
             "```", "",
             f"- FETCH_SIZE per dispatch: {fetch:.1f} KiB (mean of {nf} dispatches)",
             f"- WRITE_SIZE per dispatch: {write:.1f} KiB",
             f"- Calibration: a 1 GiB device copy (`bench.py --calibrate-copy`, rocclr copyBuffer) "
             f"reads FETCH_SIZE {cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB per dispatch, so the scale "
             f"factors are {fs:.4f} (fetch) and {ws:.4f} (write).",
             f"- Scaled: {fb / 1e6:.3f} MB read + {wb / 1e6:.3f} MB written = {(fb + wb) / 1e6:.3f} MB "
             f"per launch, against {algorithmic / 1e6:.3f} MB algorithmic (ratio "
             f"{(fb + wb) / algorithmic:.3f}).", "", "traffic_json: " + json.dumps(d)]
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def _old_title(path: str):
    """The workload description on the first line of an existing summary."""
    if os.path.exists(path):
        m = re.match(r"# (?:Kernel trace|HBM counters): (?:.*?, )?(\w+ \(.*\))$",
                     open(path).readline().strip())
        if m:
            return m.group(1)
    return None


SQ_PASSES = (
    "SQ_WAVES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY",
    "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_ACTIVE_INST_ANY SQ_BUSY_CYCLES "
    "SQ_INSTS_LDS SQ_ACTIVE_INST_SCA SQ_INSTS_BRANCH",
    "GRBM_GUI_ACTIVE GRBM_COUNT",
)


def summarize_sq(workloads, root: str) -> str:
    """profiles/fused_step_sq_counters.md: per-wave instruction, wait and
    matrix-core counts of the step kernel from three --pmc passes per workload
    (root/sq_<workload>_<pass>), the kernel's duration from its trace summary."""
    import csv
    import glob
    rows, cmds = [], []
    for w in workloads:
        vals, meta = {}, None
        for i in (1, 2, 3):
            for f in glob.glob(os.path.join(root, f"sq_{w}_{i}", "**", "*counter_collection.csv"),
                               recursive=True):
                for r in csv.DictReader(open(f)):
                    if "fused_step_kernel" in r["Kernel_Name"]:
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                        meta = r
        if meta is None:
            raise SystemExit(f"no SQ counters for {w} under {root}")
        m = {k: sum(v) / len(v) for k, v in vals.items()}
        wv = m["SQ_WAVES"]

        def per(k):
            return m[k] / wv
        trace = open(os.path.join(PROFILES_DIR, f"fused_step_{w}_kernel_trace.md")).read()
        us = float(re.search(r"^\| fused_step_kernel[^|]*\| \d+ \| ([\d.]+) \|", trace, re.M).group(1))
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024  # per SIMD
        frac = busy / (us * 1e-6 * 2.4e9)
        util = 100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] * 1024)
        rows.append(
            f"| {w} | `{_short_kernel(meta['Kernel_Name'])}` | {meta['Workgroup_Size']} | "
            f"{meta['VGPR_Count']}+{meta['Accum_VGPR_Count']} | {int(wv)} | {per('SQ_INSTS_VALU'):.0f} | "
            f"{per('SQ_INSTS_MFMA'):.0f} | {per('SQ_INSTS_VALU_TRANS_F32'):.0f} | "
            f"{per('SQ_INSTS_VMEM_RD'):.0f} | {per('SQ_WAVE_CYCLES'):.0f} | "
            f"{per('SQ_ACTIVE_INST_VALU'):.0f} ({100 * m['SQ_ACTIVE_INST_VALU'] / m['SQ_WAVE_CYCLES']:.0f}%) | "
            f"{per('SQ_WAIT_INST_ANY'):.0f} | {per('SQ_WAIT_ANY'):.0f} "
            f"({100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.0f}%) | {busy:.0f} | "
            f"{100 * frac:.1f}% of {us:.1f} µs | {util:.2f}% |")
        for i, pas in enumerate(SQ_PASSES, 1):
            cmds.append(f"rocprofv3 --pmc {pas} --output-format csv -d $R/gpurun_out/sq_{w}_{i} -o sq -- "
                        f"python3 $R/bench.py --workload {w} --steps 10 --warmup 2 --no-cpu-baseline")
    out = os.path.join(PROFILES_DIR, "fused_step_sq_counters.md")
    lines = [
        "# SQ instruction, wait and matrix-core counters: fused step kernel", "",
        "Commands (on the MI355X box, from /tmp; three passes per workload, within the per-block "
        "counter limits):", "", "```", *cmds, "```", "",
        f"Kernel sources hash (as `bench.py` computes it): `{kernel_source_hash()}`", "",
        "Per wave, mean over the dispatches of the step kernel (wave-cycle counters are in units of 4 "
        "cycles). MFMA busy: `SQ_VALU_MFMA_BUSY_CYCLES` is counted per SIMD; summed over the dispatch "
        "it is divided by the 1,024 SIMDs, then by the kernel-trace average duration at 2.4 GHz "
        "(second-last column). The last column is rocprofv3's own `MfmaUtil` expression (busy cycles / "
        "(GRBM_GUI_ACTIVE x SIMDs)), whose GRBM_GUI_ACTIVE, taken in its own pass, spans the profiler's "
        "serialised dispatch window and so is far longer than the kernel.", "",
        "| workload | kernel | threads | VGPRs+AGPRs | waves | VALU | MFMA | transcendental | vector loads "
        "| wave quad-cycles | VALU-active | waiting on a dependency | waiting (any) | MFMA busy cycles per "
        "SIMD | MFMA busy / kernel time | MfmaUtil |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|", *rows, ""]
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def summarize(args):
    """--summarize trace|counters|sq: write profiles/*.md for the workload(s)
    from rocprofv3's CSV output under --profile-root (trace_<w>,
    pmc_<counter>_<w>, pmc_<counter>_copy, sq_<w>_<pass>), recording the
    commands that made them."""
    import synth
    root = args.profile_root
    R = "$R"
    if args.summarize == "sq":
        print("wrote", summarize_sq(args.workload.split(","), root))
        return
    w = args.workload
    pref = _kernel_prefix(w)
    if args.summarize == "trace":
        out = os.path.join(PROFILES_DIR, f"{pref}_{w}_kernel_trace.md")
        cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {R}/gpurun_out/trace_{w} "
               f"-o {w} -- python3 {R}/bench.py --workload {w} --steps 100 --warmup 10 "
               f"--no-cpu-baseline")
        title = args.title or _old_title(out) or w
        print("wrote", summarize_trace(w, os.path.join(root, f"trace_{w}"), title, cmd))
        return
    out = os.path.join(PROFILES_DIR, f"{pref}_{w}_counters.md")
    cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {R}/gpurun_out/pmc_{c}_{w} -o bench -- "
            f"python3 {R}/bench.py --workload {w} --steps 20 --warmup 2 --no-cpu-baseline"
            for c in ("FETCH_SIZE", "WRITE_SIZE")]
    cmds += [f"rocprofv3 --pmc {c} --output-format csv -d {R}/gpurun_out/pmc_{c}_copy -o copy -- "
             f"python3 {R}/bench.py --calibrate-copy" for c in ("FETCH_SIZE", "WRITE_SIZE")]
    if w in synth.QK_NORM_WORKLOADS:
        alg = qk_norm_bytes(synth.QK_NORM_WORKLOADS[w])
    else:
        wl = synth.WORKLOADS[w]
        x0 = synth.make_inputs(wl)
        alg = step_accounting(wl, x0)[1]
        if pref == "extend_attn":
            tokens = int(synth.ragged_lens(wl).sum()) if wl.ragged_lo > 0 else x0.tokens
            alg = extend_attention_bytes(wl, alg, tokens)
    dirs = [os.path.join(root, d) for d in (f"pmc_FETCH_SIZE_{w}", f"pmc_WRITE_SIZE_{w}",
                                            "pmc_FETCH_SIZE_copy", "pmc_WRITE_SIZE_copy")]
    title = args.title or _old_title(out) or w
    print("wrote", summarize_counters(w, dirs, title, cmds, alg))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="swa_decode")
    ap.add_argument("--cold-bytes", type=float, default=1.0,
                    help="GiB the steps touch in one round over the layer pools (cold cache)")
    ap.add_argument("--shared-table", action="store_true",
                    help="share layer pool 0's page table and cache rows among the pools")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="force a split count (0 = plan)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--summarize", choices=("trace", "counters", "sq"), default=None,
                    help="write profiles/*.md for --workload (comma list for sq) from rocprofv3 "
                         "CSV output under --profile-root; needs no GPU")
    ap.add_argument("--profile-root", default=os.path.join(ROOT, "gpurun_out"),
                    help="--summarize: where the rocprofv3 runs wrote their directories")
    ap.add_argument("--title", default="", help="--summarize: the workload's description")
    ap.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"), help="--summarize: where to write")
    args = ap.parse_args()

    if args.summarize:
        global PROFILES_DIR
        PROFILES_DIR = args.profiles_dir
        summarize(args)
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the step is "
                          "head-sharded with no exchange, so N GPUs run N independent copies; "
                          "--gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import attention_decode_qk_amd as ga
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.workload in synth.QK_NORM_WORKLOADS:
        run_qk_norm(args, synth.QK_NORM_WORKLOADS[args.workload], dev)
        return

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    x0 = synth.make_inputs(w)
    kv_bytes, step_bytes = algorithmic_bytes(w, x0)
    # Page 2's ragged prefill batch: each request keeps its first lens[b] new
    # tokens, packed (ragged_step); the layers' rows are cut the same way.
    # Page 2's block-sparse prefill: every new token a one-token query of the
    # block-sparse step (sparse_prefill_step), its list drawn at its position.
    sprefill = None
    if w.prefill_block > 0:
        sp0 = synth.sparse_prefill(x0, w.prefill_block, w.prefill_topk, seed=w.seed + 2)
        kv_bytes, step_bytes = sparse_prefill_accounting(w, x0, sp0)
        sprefill = dict(token_req=torch.from_numpy(sp0["token_req"]).to(dev),
                        cs=torch.from_numpy(sp0["cache_seqlens"]).to(dev),
                        block_idx=torch.from_numpy(sp0["block_idx"]).to(dev),
                        max_cs=int(sp0["cache_seqlens"].max()))
    ragged = None
    if w.ragged_lo > 0:
        lens = synth.ragged_lens(w)
        r0 = synth.ragged(x0, lens)
        kv_bytes, step_bytes, rf8, rf16 = ragged_accounting(w, x0, lens)
        idx = np.concatenate([b * w.q_len + np.arange(int(n)) for b, n in enumerate(lens)])
        ragged = dict(lens=lens, total=r0["total_q"], idx=torch.from_numpy(idx).to(dev),
                      cu=torch.from_numpy(r0["cu_seqlens_q"]).to(dev),
                      cs=torch.from_numpy(r0["cache_seqlens"]).to(dev),
                      pos=torch.from_numpy(r0["positions"]).to(dev))
    pool_bytes = x0.k_cache.nbytes + x0.v_cache.nbytes + (0 if args.shared_table else x0.page_table.nbytes)
    n_layers = layer_pool_count(step_bytes, pool_bytes, args.cold_bytes * (1 << 30))
    print(f"[bench] {w.name}: B={w.batch} L={w.q_len} W={w.window} P={w.page_size}; "
          f"{n_layers} layer pools of {pool_bytes / 1e6:.1f} MB, {step_bytes / 1e6:.2f} MB "
          f"touched per step", file=sys.stderr, flush=True)

    cfg = ga.make_config(w.batch, w.q_len, w.page_size, w.window, x0.max_pages, x0.num_pages,
                         w.rope_theta, w.sm_scale, w.kv_scale, q_scale=w.q_scale,
                         sparse_block=w.sparse_block, sparse_topk=w.sparse_topk)
    if sprefill is not None:  # a sparse config whose batch counts the queries
        cfg = ga.make_config(x0.tokens, 1, w.page_size, 0, x0.max_pages, x0.num_pages,
                             w.rope_theta, w.sm_scale, w.kv_scale, q_scale=w.q_scale,
                             sparse_block=w.prefill_block, sparse_topk=w.prefill_topk)
    step = ga.GatedAttnStep(cfg, sprefill["max_cs"] if sprefill else int(w.seq_hi + w.q_len),
                            args.splits)

    # Layer pools: pool 0 is the tests' seeded input; the others are drawn on
    # the device with the same recipe (own caches, page-table permutation and
    # projection rows; pool 0's table and cache rows with --shared-table).
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    P = w.page_size
    seq = torch.from_numpy(x0.seq_lens).to(dev)
    cache_seqlens = torch.from_numpy(x0.cache_seqlens).to(dev)
    positions = torch.from_numpy(x0.positions).to(dev)
    n_pages = (x0.cache_seqlens.astype(np.int64) + P - 1) // P
    k_scale = torch.tensor([x0.k_scale], dtype=torch.float32, device=dev)
    v_scale = torch.tensor([x0.v_scale], dtype=torch.float32, device=dev)
    pos_b = torch.from_numpy(x0.positions.reshape(w.batch, w.q_len)).to(dev)
    layers = []
    pt0 = torch.from_numpy(x0.page_table).to(dev)
    for li in range(n_layers):
        pt = pt0
        if li == 0:
            kc = torch.from_numpy(x0.k_cache).to(dev)
            vc = torch.from_numpy(x0.v_cache).to(dev)
            qkv = torch.from_numpy(x0.qkv.view(np.int16)).to(dev)
        else:
            if not args.shared_table:
                perm = torch.randperm(x0.num_pages, generator=gen, device=dev).to(torch.int32)
                pt = torch.full((w.batch, x0.max_pages), -1, dtype=torch.int32, device=dev)
                off = 0
                for b in range(w.batch):
                    pt[b, : n_pages[b]] = perm[off: off + n_pages[b]]
                    off += int(n_pages[b])
            rows = x0.num_pages * P
            kc = torch.randn((rows, w.num_kv_heads, w.head_dim), generator=gen, device=dev) \
                .to(torch.float8_e4m3fn).view(torch.uint8)
            vc = torch.randn((rows, w.num_kv_heads, w.head_dim), generator=gen, device=dev) \
                .to(torch.float8_e4m3fn).view(torch.uint8)
            qkv = (torch.randn((w.batch, w.q_len, w.width), generator=gen, device=dev)
                   * w.qkv_std).to(torch.bfloat16).view(torch.int16)
        cl = (pt.gather(1, pos_b // P).to(torch.int64) * P + pos_b % P).reshape(-1).contiguous()
        out = torch.empty((w.batch, w.q_len, w.num_q_heads * w.head_dim), dtype=torch.int16,
                          device=dev)
        if sprefill is not None:  # one-token queries
            out = torch.empty((x0.tokens, 1, w.num_q_heads * w.head_dim), dtype=torch.int16,
                              device=dev)
        if ragged is not None:  # the packed rows of the kept tokens
            qkv = qkv.view(w.batch * w.q_len, w.width)[ragged["idx"]].contiguous()
            cl = cl[ragged["idx"]].contiguous()
            out = torch.empty((ragged["total"], w.num_q_heads * w.head_dim), dtype=torch.int16,
                              device=dev)
        layers.append(dict(qkv=qkv, cache_loc=cl, page_table=pt, k_cache=kc, v_cache=vc, out=out))
    torch.cuda.synchronize()

    # Page-list-driven decode: pool 0's block lists serve every layer (each
    # layer's own page table and caches still make its rows its own).
    block_idx = (torch.from_numpy(x0.extra["block_idx"]).to(dev) if w.sparse_block > 0 else None)

    def run(li, stream=None):
        L_ = layers[li]
        if sprefill is not None:
            step.sparse_prefill(L_["qkv"].view(x0.tokens, 1, w.width), positions, L_["cache_loc"],
                                sprefill["token_req"], w.batch, sprefill["cs"], L_["page_table"],
                                sprefill["block_idx"], L_["k_cache"], L_["v_cache"], k_scale,
                                v_scale, L_["out"], stream)
            return
        if ragged is not None:
            step.ragged(L_["qkv"], ragged["pos"], L_["cache_loc"], ragged["cu"], ragged["total"],
                        ragged["cs"], L_["page_table"], L_["k_cache"], L_["v_cache"], k_scale,
                        v_scale, L_["out"], stream)
            return
        if block_idx is not None:
            step.sparse(L_["qkv"], positions, L_["cache_loc"], cache_seqlens, L_["page_table"],
                        block_idx, L_["k_cache"], L_["v_cache"], k_scale, v_scale, L_["out"], stream)
            return
        step(L_["qkv"], positions, L_["cache_loc"], cache_seqlens, L_["page_table"], seq,
             L_["k_cache"], L_["v_cache"], k_scale, v_scale, L_["out"], stream)

    # HIP graphs captured outside the timed region: one holding the W warm-up
    # layer-steps and one holding exactly the K timed layer-steps, the layers
    # taken round-robin (cold) or all layer 0 (warm).  A single graph launch
    # runs its kernels back to back, so the host's launch cost is not timed.
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())

    def capture(pools):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for li in pools:
                    run(li, cap)
        return g

    # Order of execution: one sweep over every pool, the warm-up graph on pools
    # 0 .. W-1, then the timed graph starting at pool W, so that no timed step
    # reads a pool touched since the sweep (until the rotation wraps round, a
    # whole round of pools later).
    n_warm = max(1, args.warmup)
    warm_pools = [k % n_layers for k in range(n_warm)]
    cold_pools = [(n_warm + k) % n_layers for k in range(args.steps)]
    sweep = list(range(n_layers))
    with torch.cuda.stream(cap):
        for li in sweep:
            run(li, cap)
    torch.cuda.synchronize()
    g_warm = capture(warm_pools)
    g_cold = capture(cold_pools)
    g_hot = capture([0] * args.steps)
    torch.cuda.synchronize()
    reuse = reuse_distances(sweep + warm_pools, cold_pools, step_bytes)

    def timed(g):
        g_warm.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # A short spin on the GPU (untimed, ahead of the start event) keeps the
        # device busy while the host submits the graph, so the interval holds
        # the K steps' device time rather than the host's submission latency.
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    t_wall0 = time.perf_counter()
    ms_total = timed(g_cold)
    wall_s = time.perf_counter() - t_wall0
    ms_warm = timed(g_hot)
    us_step = 1000.0 * ms_total / args.steps
    us_warm = 1000.0 * ms_warm / args.steps

    # Kernel duration: eager steps with the event hook, host enqueueing ahead of
    # a spinning GPU so the kernels run back to back.
    n_k = min(args.steps, 200)
    torch.cuda.synchronize()
    ga.mi355x_gated_attn_timing(step.ctx, True)
    torch.cuda._sleep(int(5e7))
    for k in range(n_k):
        run(k % n_layers)
    kernel_ms, n_timed = ga.mi355x_gated_attn_timing_read(step.ctx)
    ga.mi355x_gated_attn_timing(step.ctx, False)
    torch.cuda.synchronize()
    kernel_us = 1000.0 * kernel_ms / max(1, n_timed)

    # The on-device step metadata (built once per step for all layers): K
    # launches in one graph, round-robin over the layer pools' page tables.
    # The block-sparse prefill's queries carry their own rows and positions
    # (token_req), so it has no such metadata.
    meta_us = None
    if sprefill is None:
        m_pos = torch.empty(x0.tokens, dtype=torch.int64, device=dev)
        m_loc = torch.empty(x0.tokens, dtype=torch.int64, device=dev)
        m_cs = torch.empty(w.batch, dtype=torch.int32, device=dev)
        g_meta = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            step.meta(seq, layers[0]["page_table"], m_pos, m_loc, m_cs, cap)
            torch.cuda.synchronize()
            with torch.cuda.graph(g_meta, stream=cap):
                for k in range(args.steps):
                    step.meta(seq, layers[k % n_layers]["page_table"], m_pos, m_loc, m_cs, cap)
        torch.cuda.synchronize()
        meta_us = 1000.0 * timed(g_meta) / args.steps

    # A decode or verify step is one kernel, or two where the plan merges the
    # splits in a second launch (combine_kernel, the long-context verify): the
    # roofline takes the graph-timed time of the whole step either way, so a
    # second launch never flatters it (rocprofv3's kernel trace lists both).
    # An extend step is two launches: its roofline takes the attention kernel's
    # event-timed duration (the hook brackets that launch alone).
    extend = w.q_len > 8 and sprefill is None
    achieved = step_bytes / (us_step * 1e-6) / 1e9
    traffic = load_traffic(w.name)
    if extend:
        f8, f16 = (rf8, rf16) if ragged is not None else extend_flops(w, x0.cache_seqlens)
        peak = mfma_peak(f8, f16)
        achieved_tf = (f8 + f16) / (kernel_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved_tf, 2), "peak": round(peak, 1),
                    "unit": "TFLOP/s", "frac": round(achieved_tf / peak, 4), "traffic": traffic,
                    "algorithmic_flops": {"qk_fp8": f8, "pv_f16": f16},
                    "peak_rule": "QK^T at the fp8 dense peak (5.0 PFLOP/s) and PV at the f16 "
                                 "one (2.5), back to back",
                    "algorithmic_bytes": extend_attention_bytes(
                        w, step_bytes, int(ragged["total"]) if ragged is not None else x0.tokens),
                    "kernel": "extend_attn_kernel", "kernel_us": round(kernel_us, 3),
                    "kernel_source": kernel_source_hash(EXTEND_SOURCES)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "algorithmic_bytes": step_bytes,
                    "kernel": "fused_step_kernel", "kernel_source": kernel_source_hash()}
    timed_reuse = [r for r in reuse if r is not None]
    result = {
        "metric": METRIC,
        "value": round(kv_bytes / (us_step * 1e-6) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size, "window": w.window,
                   "rope_theta": w.rope_theta, "sm_scale": w.sm_scale, "kv_scale": w.kv_scale,
                   "seq_lens": [w.seq_lo, w.seq_hi], "splits": step.splits,
                   "layer_pools": n_layers, "touched_bytes_per_round": n_layers * step_bytes,
                   "timed_touched_bytes": args.steps * step_bytes,
                   "timed_min_reuse_bytes": min(timed_reuse) if timed_reuse else None,
                   "pool_bytes_allocated": n_layers * pool_bytes,
                   "page_table": "shared by the layers" if args.shared_table else "per layer"},
        "us_per_layer_step": round(us_step, 3),
        "kv_bytes_per_step": kv_bytes,
        "kv_gbs_pct_of_peak": round(100.0 * kv_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "kernel_us": round(us_step, 3),
        "eager_event_kernel_us": round(kernel_us, 3),
        "step_meta_us": None if meta_us is None else round(meta_us, 3),
        "warm_single_pool": {"us_per_layer_step": round(us_warm, 3),
                             "kv_gbs": round(kv_bytes / (us_warm * 1e-6) / 1e9, 1)},
        "roofline": roofline,
        "timed_wall_s": round(wall_s, 3),
    }
    if extend:
        result["kernel_us"] = round(kernel_us, 3)  # the attention launch; the step has two
        n_tok = ragged["total"] if ragged is not None else x0.tokens
        result["tokens_per_s"] = round(n_tok / (us_step * 1e-6), 1)
        if ragged is not None:
            result["config"]["segments"] = [int(n) for n in ragged["lens"]]
    if sprefill is not None:
        result["tokens_per_s"] = round(x0.tokens / (us_step * 1e-6), 1)
        result["config"]["prefill_block"] = w.prefill_block
        result["config"]["prefill_topk"] = w.prefill_topk
    if not args.no_cpu_baseline and (ragged is not None or sprefill is not None):
        pass  # the sampled oracle baselines are written for uniform batches
    elif not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_legs(x0, kv_bytes, args.cpu_seconds, extend)
    print(json.dumps(result), flush=True)
    step.close()


if __name__ == "__main__":
    main()
