"""Host-side byte accounting of bench.py: the keys a step must read are the
union of its queries' visible ranges (page "012-attention-local-splits.py",
kernel_fn's flash_attn_with_kvcache call: causal, with window_size (W-1, 0)
on sliding layers and no window on full layers), checked against a brute-force
union over the queries."""
import numpy as np
import pytest

import bench
import synth


def _brute_keys(w, cache_seqlens):
    total = 0
    for cs in cache_seqlens.tolist():
        seen = set()
        for i in range(w.q_len):
            p = cs - w.q_len + i
            lo = max(0, p - w.window + 1) if w.window > 0 else 0
            seen.update(range(lo, p + 1))
        total += len(seen)
    return total


@pytest.mark.parametrize("kw", [
    dict(batch=3, q_len=1, window=0), dict(batch=3, q_len=1, window=16),
    dict(batch=4, q_len=8, window=0, page_size=4), dict(batch=2, q_len=8, window=32, page_size=16),
])
def test_attended_keys_is_the_union_of_the_visible_ranges(kw):
    w = synth.small(**kw)
    x = synth.make_inputs(w)
    assert bench.attended_keys(w, x.cache_seqlens) == _brute_keys(w, x.cache_seqlens)


def test_full_attention_reads_every_cached_key():
    w = synth.small(batch=5, q_len=2, window=0)
    x = synth.make_inputs(w)
    assert bench.attended_keys(w, x.cache_seqlens) == int(np.sum(x.cache_seqlens))


def test_algorithmic_bytes_count_kv_rows_pages_and_token_rows():
    w = synth.small(batch=2, q_len=1, window=0, page_size=4)
    x = synth.make_inputs(w)
    kv, total = bench.algorithmic_bytes(w, x)
    assert kv == int(np.sum(x.cache_seqlens)) * w.num_kv_heads * w.head_dim * 2
    pages = int(np.sum((x.cache_seqlens + w.page_size - 1) // w.page_size))
    per_token = w.width * 2 + 2 * w.num_kv_heads * w.head_dim + w.num_q_heads * w.head_dim * 2 + 16
    assert total == kv + 4 * pages + x.tokens * per_token


def test_layer_pools_cover_the_cold_bytes_by_what_a_step_touches():
    # A windowed step touches ~17 MB of a ~90 MB pool: the round must cover 1 GiB
    # of touched bytes, not of allocated pools (the Infinity Cache is 256 MB).
    n = bench.layer_pool_count(17_261_056, 89_500_000, 1 << 30)
    assert n == 63 and n * 17_261_056 >= 1 << 30
    assert bench.layer_pool_count(600_000_000, 600_000_000, 1 << 30) == 2
    assert bench.layer_pool_count(1 << 31, 1 << 31, 1 << 30) == 1
    # Device memory bounds the count.
    assert bench.layer_pool_count(1000, 1 << 30, 1 << 30) == bench.POOL_MEMORY_LIMIT // (1 << 30)


def test_traffic_comes_only_from_the_workloads_own_counters():
    assert bench.load_traffic("no_such_workload") is None
    import os
    if os.path.exists(bench.counters_file("swa_decode")):
        t = bench.load_traffic("swa_decode")
        assert t is None or t > 0


def test_sparse_bytes_count_each_heads_listed_keys_once():
    import dataclasses
    w = dataclasses.replace(synth.small(batch=3, q_len=1, page_size=8, seq_lo=100, seq_hi=400),
                            sparse_block=32, sparse_topk=4)
    x = synth.make_inputs(w)
    kv, total = bench.algorithmic_bytes(w, x)
    brute = 0
    for g in range(2):
        for b, cs in enumerate(x.cache_seqlens.tolist()):
            keys = set()
            for j in x.extra["block_idx"][g, b].tolist():
                if j >= 0:
                    keys.update(k for k in range(j * 32, (j + 1) * 32) if k < cs)
            brute += len(keys)
    assert kv == brute * 64 * 2
    assert total > kv


@pytest.mark.parametrize("kw", [dict(batch=3, q_len=20, window=0), dict(batch=2, q_len=40, window=7),
                                dict(batch=2, q_len=33, window=100, seq_lo=2, seq_hi=9)])
def test_extend_flops_count_every_visible_row_key_pair(kw):
    """2*D flops per (query row, visible key) for each product, by brute force
    over the rows."""
    w = synth.small(**kw)
    x = synth.make_inputs(w)
    pairs = 0
    for cs in x.cache_seqlens.tolist():
        for i in range(w.q_len):
            p = cs - w.q_len + i
            lo = max(0, p - w.window + 1) if w.window > 0 else 0
            pairs += len(range(lo, p + 1))
    f8, f16 = bench.extend_flops(w, x.cache_seqlens)
    assert f8 == f16 == 2 * w.head_dim * w.num_q_heads * pairs


def test_mfma_peak_of_the_mix():
    assert bench.mfma_peak(1.0, 0.0) == pytest.approx(5000.0)
    assert bench.mfma_peak(0.0, 1.0) == pytest.approx(2500.0)
    assert bench.mfma_peak(1.0, 1.0) == pytest.approx(2.0 / (1 / 5000.0 + 1 / 2500.0))


def test_extend_workloads_use_their_own_counter_files():
    assert bench.counters_file("swa_extend").endswith("extend_attn_swa_extend_counters.md")
    assert bench.counters_file("swa_decode").endswith("fused_step_swa_decode_counters.md")


def test_ragged_accounting_reduces_to_the_uniform_one():
    """With every segment at the bound, the ragged batch's KV bytes, step bytes
    and flops are the uniform step's; shorter segments count only their own
    tokens, keys and rows."""
    import numpy as np
    w = synth.small(name="acct", batch=3, q_len=40, window=30, rope_theta=500000.0, page_size=4,
                    seq_lo=50, seq_hi=200)
    x = synth.make_inputs(w, seed=3)
    kv, step_b, f8, f16 = bench.ragged_accounting(w, x, np.full(3, 40, np.int32))
    assert (kv, step_b) == bench.algorithmic_bytes(w, x)
    assert (f8, f16) == bench.extend_flops(w, x.cache_seqlens)
    kv1, step1, g8, _ = bench.ragged_accounting(w, x, np.array([40, 0, 0], np.int32))
    s = int(x.seq_lens[0])
    assert kv1 == (s + 40 - max(0, s - 30 + 1)) * 2 * 64 * 2
    assert g8 == 2 * 64 * 16 * sum(min(p + 1, 30) for p in range(s, s + 40))


def test_sparse_prefill_accounting_counts_the_listed_keys():
    """Block-sparse prefill: KV bytes are, per (KV head, query), the keys of its
    listed blocks below its cached length, a 64-byte half row of K and of V
    each (brute force over the lists)."""
    import dataclasses
    w = dataclasses.replace(synth.small(name="spacct", batch=2, q_len=6, window=0, page_size=32,
                                        seq_lo=40, seq_hi=200),
                            prefill_block=32, prefill_topk=3)
    x = synth.make_inputs(w, seed=4)
    sp = synth.sparse_prefill(x, 32, 3, seed=9)
    kv, step_b = bench.sparse_prefill_accounting(w, x, sp)
    keys = 0
    for g in range(2):
        for t in range(x.tokens):
            cs = int(sp["cache_seqlens"][t])
            for j in sp["block_idx"][g, t].tolist():
                if j >= 0:
                    keys += len([k for k in range(32 * j, 32 * j + 32) if k < cs])
    assert kv == keys * 64 * 2
    assert step_b > kv


def test_timed_steps_never_reread_a_recently_touched_pool():
    """After the sweep over every pool and the warm-up on pools 0 .. W-1, the
    timed steps start at pool W: each timed step's pool was last touched a whole
    round of pools earlier (n - 1 steps), for the driver's 20 timed steps after
    5 warm-up ones as for the default 400 after 40."""
    import bench
    step = 17_261_056
    n = bench.layer_pool_count(step, 89_500_000, float(1 << 30))
    assert n * step >= 1 << 30
    for warm, steps in ((5, 20), (40, 400), (1, 1)):
        warm_pools = [k % n for k in range(warm)]
        cold = [(warm + k) % n for k in range(steps)]
        r = bench.reuse_distances(list(range(n)) + warm_pools, cold, step)
        assert all(x is not None for x in r)
        assert min(r) == (n - 1) * step, (warm, steps, min(r))
    # the old order (timed from pool 0 right after a warm-up on pools 0..4) re-read them
    r = bench.reuse_distances(list(range(n)) + [0, 1, 2, 3, 4], list(range(20)), step)
    assert min(r) == 4 * step


def _write_csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_writes_trace_and_counter_summaries(tmp_path):
    """--summarize turns rocprofv3 CSV output into the profiles' summaries:
    the kernel table and a traffic line that bench.py reads back, scaled by the
    copy calibration (a copy that counts twice its bytes halves the reading)."""
    import json
    import re
    import subprocess
    import sys
    root, out = tmp_path / "runs", tmp_path / "profiles"
    out.mkdir()
    kname = "void mi355x_ga::(anonymous namespace)::fused_step_kernel<1, 1, 0>(mi355x_ga::StepParams)"
    _write_csv(root / "trace_swa_decode" / "box" / "swa_decode_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[kname, 110, 1100000, 10000, 99.0, 9500, 12000], ["copyBuffer", 3, 1, 1, 1.0, 1, 1]])
    counters = {"FETCH_SIZE": 1000.0, "WRITE_SIZE": 10.0}
    for c, v in counters.items():
        _write_csv(root / f"pmc_{c}_swa_decode" / "box" / "bench_counter_collection.csv",
                   ["Counter_Name", "Kernel_Name", "Counter_Value"], [[c, kname, v], [c, kname, v]])
        copy_kib = (2 if c == "FETCH_SIZE" else 1) * (1 << 20)
        _write_csv(root / f"pmc_{c}_copy" / "box" / "copy_counter_collection.csv",
                   ["Counter_Name", "Kernel_Name", "Counter_Value"], [[c, "copyBuffer", copy_kib]])
    for mode in ("trace", "counters"):
        subprocess.run([sys.executable, bench.__file__, "--summarize", mode, "--workload", "swa_decode",
                        "--profile-root", str(root), "--profiles-dir", str(out), "--title", "t"],
                       check=True, capture_output=True)
    trace = (out / "fused_step_swa_decode_kernel_trace.md").read_text()
    assert "| fused_step_kernel<1, 1, 0> | 110 | 10.000 | 9.500 | 12.000 |" in trace
    assert "copyBuffer" not in trace
    text = (out / "fused_step_swa_decode_counters.md").read_text()
    d = json.loads(re.search(r"^traffic_json:\s*(\{.*\})\s*$", text, re.M).group(1))
    assert d["fetch_bytes"] == 1000 * 1024 // 2 and d["write_bytes"] == 10 * 1024
    wl = synth.WORKLOADS["swa_decode"]
    assert d["algorithmic_bytes_per_launch"] == bench.step_accounting(wl, synth.make_inputs(wl))[1]
    assert d["kernel_source_sha256"] == bench.kernel_source_hash()
