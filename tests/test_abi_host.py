"""Host-side tests of the C-ABI library (no GPU needed): it loads, exports every
symbol the header declares, and validates configurations, plans and step
arguments with the documented status codes before touching a device."""
import ctypes
import os
import re

import pytest

import attention_decode_qk_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ga.LIB_PATH):
        from attention_decode_qk_amd import build
        build.build(force=False)
    return ga.lib()


def _declared_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(mi355x_(?:gated_attn|qk_norm)\w*)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol(L):
    declared = _declared_symbols()
    assert len(declared) >= 8
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert declared == set(ga.EXPORTED)


def cfg(**kw):
    base = dict(batch=32, q_len=1, page_size=1, window=2048, max_pages=16386, num_pages=400000,
                rope_theta=500000.0)
    base.update(kw)
    return ga.make_config(**base)


def test_supports_accepts_the_served_shapes(L):
    for q_len in list(range(1, 9)) + [9, 16, 67, 4096, 65536]:
        assert ga.mi355x_gated_attn_supports(cfg(q_len=q_len)) == ga.MI355X_GA_OK
    assert ga.mi355x_gated_attn_supports(cfg(batch=0)) == ga.MI355X_GA_OK
    assert ga.mi355x_gated_attn_supports(cfg(page_size=64, window=0, rope_theta=0.0,
                                             kv_scale=0.5)) == ga.MI355X_GA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=128), ga.MI355X_GA_UNSUPPORTED),
    (dict(num_q_heads=15), ga.MI355X_GA_UNSUPPORTED),
    (dict(num_q_heads=8, num_kv_heads=1), ga.MI355X_GA_UNSUPPORTED),
    (dict(q_len=65537), ga.MI355X_GA_UNSUPPORTED),
    (dict(batch=65536, q_len=65536), ga.MI355X_GA_UNSUPPORTED),
    (dict(q_len=0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(batch=-1), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(page_size=0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(window=-1), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(max_pages=0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(num_pages=0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(rope_theta=-1.0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(rope_theta=float("inf")), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(sm_scale=0.0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(sm_scale=float("nan")), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(kv_scale=-0.5), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(q_scale=0.0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(q_scale=float("inf")), ga.MI355X_GA_INVALID_ARGUMENT),
])
def test_supports_rejects(L, kw, status):
    assert ga.mi355x_gated_attn_supports(cfg(**kw)) == status
    assert ga.mi355x_gated_attn_last_error() != ""
    with pytest.raises(ga.GatedAttnError) as e:
        ga.mi355x_gated_attn_prepare(cfg(**kw))
    assert e.value.status == status


def test_prepare_plan_workspace_layout(L):
    c = cfg(batch=32, q_len=8)
    ctx = ga.mi355x_gated_attn_prepare(c)
    try:
        ws, s = ga.mi355x_gated_attn_plan(ctx, 32776, 4)
        assert s == 4
        T = 32 * 8
        q = T * 16 * 64
        po = -(-q // 256) * 256
        pml = -(-(po + s * T * 16 * 64 * 2) // 256) * 256  # partial o / l: f16
        cnt = -(-(pml + s * T * 16 * 2 * 4) // 256) * 256
        assert ws == -(-(cnt + 32 * 2 * 4) // 256) * 256  # window 2048, q_len 8: two token groups of four
        ws0, s0 = ga.mi355x_gated_attn_plan(ctx, 32776, 0)
        assert 1 <= s0 <= 256
        with pytest.raises(ga.GatedAttnError):
            ga.mi355x_gated_attn_plan(ctx, 100, 257)
        with pytest.raises(ga.GatedAttnError):
            ga.mi355x_gated_attn_plan(ctx, -1, 0)
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_auto_split_count_fills_the_chip(L):
    """Automatic plans: about one work unit per compute unit, at least one
    32-key block per wave, never more than 256 splits."""
    cases = [(1, 1, 0, 513), (32, 1, 2048, 16385), (64, 1, 0, 32769), (32, 8, 2048, 32776),
             (8, 8, 0, 131080)]
    for B, Lq, W, ctxlen in cases:
        ctx = ga.mi355x_gated_attn_prepare(cfg(batch=B, q_len=Lq, window=W))
        try:
            _, s = ga.mi355x_gated_attn_plan(ctx, ctxlen, 0)
            keys = min(ctxlen, W + Lq - 1) if W else ctxlen
            assert s <= max(1, -(-keys // 128))
            assert s <= 256
            per_req = (-(-Lq // 2) if Lq <= 4 else -(-Lq // 4)) if keys <= 4096 else 1
            groups = B * per_req  # work units per split
            assert groups * s <= 256 + groups
        finally:
            ga.mi355x_gated_attn_destroy(ctx)


def _raw_step(L, ctx, **over):
    """Call the C step with fake (never dereferenced on the host) pointers."""
    P = ctypes.c_void_p
    args = dict(qkv=P(0x1000), positions=P(0x2000), cache_loc=P(0x3000), cache_seqlens=P(0x4000),
                page_table=P(0x5000), seq_lens=P(0x6000), k_cache=P(0x10000), v_cache=P(0x20000),
                k_scale=P(0x7000), v_scale=P(0x8000), out=P(0x9000), workspace=P(0x100000),
                ws_bytes=1 << 30, stream=None)
    args.update(over)
    return L.mi355x_gated_attn_step(ctx, args["qkv"], args["positions"], args["cache_loc"],
                                    args["cache_seqlens"], args["page_table"], args["seq_lens"],
                                    args["k_cache"], args["v_cache"], args["k_scale"],
                                    args["v_scale"], args["out"], args["workspace"],
                                    args["ws_bytes"], args["stream"])


def test_step_argument_errors_are_reported_before_any_launch(L):
    ctx = ga.mi355x_gated_attn_prepare(cfg(kv_scale=0.5))
    try:
        assert _raw_step(L, ctx) == ga.MI355X_GA_INVALID_ARGUMENT  # not planned yet
        ws, _ = ga.mi355x_gated_attn_plan(ctx, 16385, 0)
        for name in ("qkv", "cache_loc", "cache_seqlens", "page_table", "k_cache", "v_cache",
                     "out", "workspace", "positions", "k_scale", "v_scale"):
            assert _raw_step(L, ctx, **{name: None}) == ga.MI355X_GA_INVALID_ARGUMENT, name
        assert _raw_step(L, ctx, ws_bytes=ws - 1) == ga.MI355X_GA_WORKSPACE_TOO_SMALL
        assert _raw_step(L, ctx, workspace=ctypes.c_void_p(0x100010)) == \
            ga.MI355X_GA_INVALID_ARGUMENT
        assert "aligned" in ga.mi355x_gated_attn_last_error()
        assert L.mi355x_gated_attn_step(None, *([None] * 12), 0, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_unscaled_rope_free_step_needs_no_scales_or_positions(L):
    ctx = ga.mi355x_gated_attn_prepare(cfg(rope_theta=0.0, window=0))
    try:
        ws, _ = ga.mi355x_gated_attn_plan(ctx, 1000, 0)
        rc = _raw_step(L, ctx, positions=None, k_scale=None, v_scale=None, ws_bytes=ws)
        # past argument validation: only the device check remains (no GPU here)
        assert rc in (ga.MI355X_GA_OK, ga.MI355X_GA_INVALID_ARGUMENT, ga.MI355X_GA_HIP_ERROR)
        if rc == ga.MI355X_GA_INVALID_ARGUMENT:
            assert "device" in ga.mi355x_gated_attn_last_error()
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_workspace_init_validates_before_launch(L):
    ctx = ga.mi355x_gated_attn_prepare(cfg())
    try:
        P = ctypes.c_void_p
        assert L.mi355x_gated_attn_workspace_init(ctx, P(0x100000), 1 << 30, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT  # before plan
        ws, _ = ga.mi355x_gated_attn_plan(ctx, 16385, 0)
        assert L.mi355x_gated_attn_workspace_init(ctx, None, ws, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
        assert L.mi355x_gated_attn_workspace_init(ctx, P(0x100000), ws - 1, None) == \
            ga.MI355X_GA_WORKSPACE_TOO_SMALL
        assert L.mi355x_gated_attn_workspace_init(None, P(0x100000), ws, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


@pytest.mark.parametrize("q_len", [1, 8, 100])
def test_empty_batch_is_a_no_op(L, q_len):
    ctx = ga.mi355x_gated_attn_prepare(cfg(batch=0, q_len=q_len))
    try:
        ga.mi355x_gated_attn_plan(ctx, 100, 0)
        assert L.mi355x_gated_attn_step(ctx, *([None] * 12), 0, None) == ga.MI355X_GA_OK
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_destroy_accepts_null(L):
    ga.mi355x_gated_attn_destroy(None)


def test_timing_hook_without_steps(L):
    ctx = ga.mi355x_gated_attn_prepare(cfg())
    try:
        ga.mi355x_gated_attn_timing(ctx, True)
        ms, n = ga.mi355x_gated_attn_timing_read(ctx)
        assert n == 0 and ms == 0.0
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_plan_rejects_a_launch_beyond_the_grid_limit(L):
    """B * token groups * splits workgroups must fit one launch (2^31 - 1);
    q_len 8 makes one group over a long key range and two over a short one,
    q_len 3 one and two."""
    ctx = ga.mi355x_gated_attn_prepare(cfg(batch=1 << 28, q_len=8, window=0))
    try:
        ga.mi355x_gated_attn_plan(ctx, 100000, 7)  # 2^28 * 1 * 7 < 2^31
        ga.mi355x_gated_attn_plan(ctx, 1000, 3)  # 2^28 * 2 * 3 < 2^31
        for max_context, splits in ((100000, 8), (1000, 4)):  # 2^28 * 8 = 2^28 * 2 * 4 = 2^31
            with pytest.raises(ga.GatedAttnError) as e:
                ga.mi355x_gated_attn_plan(ctx, max_context, splits)
            assert e.value.status == ga.MI355X_GA_UNSUPPORTED
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    ctx = ga.mi355x_gated_attn_prepare(cfg(batch=1 << 28, q_len=3, window=0))
    try:
        ga.mi355x_gated_attn_plan(ctx, 100000, 7)  # one group of three: 2^28 * 7 < 2^31
        with pytest.raises(ga.GatedAttnError) as e:
            ga.mi355x_gated_attn_plan(ctx, 1000, 4)  # two groups (pairs): 2^28 * 2 * 4 = 2^31
        assert e.value.status == ga.MI355X_GA_UNSUPPORTED
        ga.mi355x_gated_attn_plan(ctx, 1000, 3)
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_short_key_ranges_use_groups_of_two_tokens(L):
    """Up to q_len 4 a short key range takes pairs of tokens, longer blocks
    groups of four; a long range one group; the counters region holds one
    int32 per (request, token group)."""
    for Lq, max_context, groups in ((8, 100000, 1), (8, 4096, 2), (3, 1000, 2), (3, 100000, 1),
                                    (1, 1000, 1), (4, 4000, 2), (4, 5000, 1), (5, 4000, 2), (5, 5000, 1)):
        c = cfg(batch=7, q_len=Lq, window=0)
        ctx = ga.mi355x_gated_attn_prepare(c)
        try:
            ws, s = ga.mi355x_gated_attn_plan(ctx, max_context, 2)
            T = 7 * Lq
            po = -(-(T * 16 * 64) // 256) * 256
            pml = -(-(po + s * T * 16 * 64 * 2) // 256) * 256  # partial o / l: f16
            cnt = -(-(pml + s * T * 16 * 2 * 4) // 256) * 256
            assert ws == -(-(cnt + 7 * groups * 4) // 256) * 256, (Lq, max_context)
        finally:
            ga.mi355x_gated_attn_destroy(ctx)


def test_step_meta_validates_before_launch(L):
    """Metadata builder: NULL pointers are rejected on the host, B == 0 is a no-op."""
    P = ctypes.c_void_p
    ctx = ga.mi355x_gated_attn_prepare(cfg(batch=4, q_len=2))
    try:
        args = [P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000)]
        for k in range(5):
            bad = list(args)
            bad[k] = None
            assert L.mi355x_gated_attn_step_meta(ctx, *bad, None) == ga.MI355X_GA_INVALID_ARGUMENT
        assert L.mi355x_gated_attn_step_meta(None, *args, None) == ga.MI355X_GA_INVALID_ARGUMENT
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    ctx = ga.mi355x_gated_attn_prepare(cfg(batch=0))
    try:
        assert L.mi355x_gated_attn_step_meta(ctx, None, None, None, None, None, None) == ga.MI355X_GA_OK
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


# ---- per-head QK-norm (page "qk_norm") ---------------------------------------

def test_qk_norm_serves_the_pages_head_dims(L):
    """The page's launch-shape table covers a head with 8, 16 or 32 threads of
    eight 16-bit values (no tail path): head_dim 64, 128, 256 for bf16/fp16."""
    served = {(d, h) for d in (0, 1, 2, -1) for h in range(1, 600)
              if ga.mi355x_qk_norm_supports(d, h)}
    assert served == {(d, h) for d in (0, 1) for h in (64, 128, 256)}


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 1), (dict(dtype=2), 1),
    (dict(M=-1), 2), (dict(num_heads=0), 2),
    (dict(x_row_stride=1000), 2),                 # shorter than 16 * 64
    (dict(x_row_stride=1028), 2),                 # not a multiple of 8
    (dict(x=None), 2), (dict(out=None), 2),       # NULL with M > 0
    (dict(x=0x1008), 2), (dict(out=0x2004), 2),   # not 16-byte aligned
])
def test_qk_norm_rejects_bad_arguments_before_any_launch(L, kw, status):
    args = dict(x=0x1000, out=0x2000, M=4, num_heads=16, head_dim=64, x_row_stride=2304, dtype=0,
                eps=1e-5, scale=1.0, stream=None)
    args.update(kw)
    rc = L.mi355x_qk_norm(args["x"], args["out"], args["M"], args["num_heads"], args["head_dim"],
                          args["x_row_stride"], args["dtype"], ctypes.c_float(args["eps"]),
                          ctypes.c_float(args["scale"]), args["stream"])
    assert rc == status
    assert ga.mi355x_gated_attn_last_error() != ""


def test_qk_norm_of_no_rows_is_a_no_op(L):
    assert L.mi355x_qk_norm(None, None, 0, 16, 64, 1024, 0, ctypes.c_float(1e-5),
                            ctypes.c_float(5.473), None) == 0


def test_qk_norm_binding_checks_shapes_like_the_page():
    import torch
    x = torch.zeros((4, 100), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ga.qk_norm(x, 64)  # 100 is not a multiple of 64
    with pytest.raises(ValueError):
        ga.qk_norm(torch.zeros((4, 64, 2), dtype=torch.bfloat16), 64)
    with pytest.raises(ga.GatedAttnError):
        ga.qk_norm(torch.zeros((4, 128), dtype=torch.float32), 64)
    assert ga.qk_norm(torch.zeros((0, 128), dtype=torch.bfloat16), 64).shape == (0, 128)
    assert ga.supports_qk_norm(torch.float16, 256) and not ga.supports_qk_norm(torch.float32, 64)


# ---- page-list-driven (top-k block-sparse) decode (page "msa.py") -------------

@pytest.mark.parametrize("kw,status", [
    (dict(sparse_block=128, sparse_topk=16, window=0), ga.MI355X_GA_OK),
    (dict(sparse_block=32, sparse_topk=256, window=0), ga.MI355X_GA_OK),
    (dict(sparse_block=128, sparse_topk=16), ga.MI355X_GA_UNSUPPORTED),            # a window
    (dict(sparse_block=128, sparse_topk=16, window=0, q_len=2), ga.MI355X_GA_UNSUPPORTED),
    (dict(sparse_block=48, sparse_topk=16, window=0), ga.MI355X_GA_UNSUPPORTED),    # not x32
    (dict(sparse_block=128, sparse_topk=257, window=0), ga.MI355X_GA_UNSUPPORTED),
    (dict(sparse_block=128, sparse_topk=0, window=0), ga.MI355X_GA_INVALID_ARGUMENT),
    (dict(sparse_block=-32, sparse_topk=4, window=0), ga.MI355X_GA_INVALID_ARGUMENT),
])
def test_sparse_configs(L, kw, status):
    assert ga.mi355x_gated_attn_supports(cfg(**kw)) == status


def test_sparse_plan_sizes_splits_for_the_listed_keys(L):
    """topk * block keys per KV head, one KV head per wave: B = 32 with 16
    blocks of 128 gives 2,048 keys, eight splits (one unit per CU)."""
    ctx = ga.mi355x_gated_attn_prepare(cfg(sparse_block=128, sparse_topk=16, window=0))
    try:
        _, s = ga.mi355x_gated_attn_plan(ctx, 1 << 20, 0)
        assert s == 8
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_dense_and_sparse_steps_refuse_each_others_configs(L):
    P = ctypes.c_void_p
    sparse = ga.mi355x_gated_attn_prepare(cfg(sparse_block=128, sparse_topk=16, window=0))
    dense = ga.mi355x_gated_attn_prepare(cfg())
    try:
        ga.mi355x_gated_attn_plan(sparse, 1 << 20, 0)
        ga.mi355x_gated_attn_plan(dense, 16385, 0)
        assert _raw_step(L, sparse) == ga.MI355X_GA_INVALID_ARGUMENT  # dense step, sparse config
        args = [P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), P(0x6000), P(0x10000),
                P(0x20000), P(0x7000), P(0x8000), P(0x9000), P(0x100000)]
        assert L.mi355x_gated_attn_sparse_step(dense, *args, 1 << 30, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
        no_list = list(args)
        no_list[5] = None
        assert L.mi355x_gated_attn_sparse_step(sparse, *no_list, 1 << 30, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
    finally:
        ga.mi355x_gated_attn_destroy(sparse)
        ga.mi355x_gated_attn_destroy(dense)


@pytest.mark.parametrize("batch,q_len", [(5, 9), (5, 100), (5, 4096), (1, 64)])
def test_extend_plan_splits_only_when_the_units_do_not_fill_the_chip(L, batch, q_len):
    """q_len > 8 (extend / prefill): one unit per (request, 16-token tile, KV
    head); S = min(ceil(256 / units), stages / 4, 32) key splits over the
    64-key stages of the key bound; the workspace holds q, then (S > 1) f16
    partial rows and fp32 (m, l) per split and unit row, then one counter per unit."""
    tiles = -(-q_len // 16)
    units = batch * 2 * tiles
    for max_context, window in ((200000, 0), (5000, 0), (300, 0), (200000, 2048)):
        ctx = ga.mi355x_gated_attn_prepare(cfg(batch=batch, q_len=q_len, window=window), 0)
        try:
            nbytes, splits = ga.mi355x_gated_attn_plan(ctx, max_context, 0)
            keys = min(max_context, window + q_len - 1) if window else max_context
            want = max(1, min(-(-256 // units), -(-keys // 64) // 4, 32))
            assert splits == want, (batch, q_len, max_context, window)
            al = lambda x: -(-x // 256) * 256
            q = al(batch * q_len * 16 * 64)
            rows = units * 128
            po = al(q + (splits * rows * 64 * 2 if splits > 1 else 0))
            pml = al(po + (splits * rows * 2 * 4 if splits > 1 else 0))
            assert nbytes == al(pml + 4 * units)
            forced, s3 = ga.mi355x_gated_attn_plan(ctx, max_context, 3)
            assert s3 == 3 and forced == al(al(al(q + 3 * rows * 128) + 3 * rows * 8) + 4 * units)
        finally:
            ga.mi355x_gated_attn_destroy(ctx)


def test_extend_refuses_page_list_driven_configs(L):
    assert ga.mi355x_gated_attn_supports(
        cfg(q_len=16, window=0, sparse_block=32, sparse_topk=4)) == ga.MI355X_GA_UNSUPPORTED


def test_ragged_step_validates_before_any_launch(L):
    """The ragged extend entry point: a dense extend config only (q_len > 8
    bounding every segment), a cu_seqlens_q array, and total_q within
    0..B*q_len, all checked on the host with no launch; an empty batch is a
    no-op."""
    P = ctypes.c_void_p
    ext = ga.mi355x_gated_attn_prepare(cfg(batch=4, q_len=64, window=0))
    dec = ga.mi355x_gated_attn_prepare(cfg(batch=4, q_len=8, window=0))
    empty = ga.mi355x_gated_attn_prepare(cfg(batch=0, q_len=64, window=0))
    try:
        ws, _ = ga.mi355x_gated_attn_plan(ext, 5000, 0)
        ga.mi355x_gated_attn_plan(dec, 5000, 0)

        def call(ctx, cu=P(0x4000), total=100):
            return L.mi355x_gated_attn_ragged_step(
                ctx, P(0x1000), P(0x2000), P(0x3000), cu, total, P(0x5000), P(0x6000),
                P(0x10000), P(0x20000), P(0x7000), P(0x8000), P(0x9000), P(0x100000), ws, None)
        assert call(dec) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "q_len" in ga.mi355x_gated_attn_last_error()
        assert call(ext, cu=None) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "cu_seqlens_q" in ga.mi355x_gated_attn_last_error()
        assert call(ext, total=-1) == ga.MI355X_GA_INVALID_ARGUMENT
        assert call(ext, total=4 * 64 + 1) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "total_q" in ga.mi355x_gated_attn_last_error()
        assert call(empty) == ga.MI355X_GA_OK
        assert L.mi355x_gated_attn_ragged_step(None, *([None] * 4), 0, *([None] * 8), 0, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
    finally:
        for c in (ext, dec, empty):
            ga.mi355x_gated_attn_destroy(c)


def test_sparse_prefill_step_validates_before_any_launch(L):
    """Page-list-driven prefill: a sparse config only, token_req and block_idx
    present, at least one page-table row; an empty batch is a no-op."""
    P = ctypes.c_void_p
    sparse = ga.mi355x_gated_attn_prepare(cfg(batch=40, sparse_block=64, sparse_topk=4, window=0))
    dense = ga.mi355x_gated_attn_prepare(cfg(batch=40, window=0))
    empty = ga.mi355x_gated_attn_prepare(cfg(batch=0, sparse_block=64, sparse_topk=4, window=0))
    try:
        ws, _ = ga.mi355x_gated_attn_plan(sparse, 1 << 16, 0)
        ga.mi355x_gated_attn_plan(dense, 1 << 16, 0)

        def call(ctx, tr=P(0x4000), nreq=2, bi=P(0x6000)):
            return L.mi355x_gated_attn_sparse_prefill_step(
                ctx, P(0x1000), P(0x2000), P(0x3000), tr, nreq, P(0x5000), P(0x5800), bi,
                P(0x10000), P(0x20000), P(0x7000), P(0x8000), P(0x9000), P(0x100000), ws, None)
        assert call(dense) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "dense" in ga.mi355x_gated_attn_last_error()
        assert call(sparse, tr=None) == ga.MI355X_GA_INVALID_ARGUMENT
        assert call(sparse, bi=None) == ga.MI355X_GA_INVALID_ARGUMENT
        assert call(sparse, nreq=0) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "num_requests" in ga.mi355x_gated_attn_last_error()
        assert call(empty) == ga.MI355X_GA_OK
    finally:
        for c in (sparse, dense, empty):
            ga.mi355x_gated_attn_destroy(c)


def _good_step_tensors(c):
    """CPU tensors of the right dtypes and sizes for config c (the binding checks
    dtype and size before device and layout)."""
    import torch
    T = c.batch * c.q_len
    width = (2 * c.num_q_heads + 2 * c.num_kv_heads) * c.head_dim
    cache = c.num_pages * c.page_size * c.num_kv_heads * c.head_dim
    return dict(
        qkv=torch.zeros(T * width, dtype=torch.int16),
        positions=torch.zeros(T, dtype=torch.int64),
        cache_loc=torch.zeros(T, dtype=torch.int64),
        cache_seqlens=torch.zeros(c.batch, dtype=torch.int32),
        page_table=torch.zeros(c.batch * c.max_pages, dtype=torch.int32),
        seq_lens=torch.zeros(c.batch, dtype=torch.int32),
        k_cache=torch.zeros(cache, dtype=torch.uint8),
        v_cache=torch.zeros(cache, dtype=torch.uint8),
        k_scale=torch.ones(1, dtype=torch.float32),
        v_scale=torch.ones(1, dtype=torch.float32),
        out=torch.zeros(T * c.num_q_heads * c.head_dim, dtype=torch.bfloat16),
        workspace=torch.zeros(256, dtype=torch.uint8))


@pytest.mark.parametrize("name,bad,msg", [
    ("qkv", lambda t: t.float(), "dtype"),
    ("qkv", lambda t: t[:-8], "elements"),
    ("positions", lambda t: t.int(), "dtype"),
    ("positions", lambda t: t[:-1], "elements"),
    ("cache_loc", lambda t: t.int(), "dtype"),
    ("cache_loc", lambda t: t.repeat(2), "elements"),
    ("cache_seqlens", lambda t: t.long(), "dtype"),
    ("cache_seqlens", lambda t: t[:-1], "elements"),
    ("page_table", lambda t: t.long(), "dtype"),
    ("page_table", lambda t: t[:-1], "elements"),
    ("seq_lens", lambda t: t.long(), "dtype"),
    ("k_cache", lambda t: t.half(), "dtype"),
    ("k_cache", lambda t: t[:-1], "at least"),
    ("v_cache", lambda t: t[:-64], "at least"),
    ("k_scale", lambda t: t.double(), "dtype"),
    ("k_scale", lambda t: t.repeat(2), "elements"),
    ("k_scale", lambda t: None, "required"),
    ("v_scale", lambda t: t.half(), "dtype"),
    ("v_scale", lambda t: None, "required"),
    ("out", lambda t: t.float(), "dtype"),
    ("out", lambda t: t[:-1], "elements"),
    ("workspace", lambda t: t.float(), "dtype"),
])
def test_binding_checks_every_tensor_against_the_config(L, name, bad, msg):
    """The step wrapper checks each tensor's dtype and size against the
    context's config (and its device and layout) before any pointer reaches the
    C ABI: a mis-sized or mistyped tensor raises ValueError naming it."""
    c = cfg(batch=3, q_len=2, max_pages=40, num_pages=100, page_size=4, kv_scale=0.5)
    ctx = ga.mi355x_gated_attn_prepare(c)
    try:
        t = _good_step_tensors(c)
        t[name] = bad(t[name])
        with pytest.raises(ValueError, match=msg) as e:
            ga.mi355x_gated_attn_step(ctx, t["qkv"], t["positions"], t["cache_loc"],
                                      t["cache_seqlens"], t["page_table"], t["seq_lens"],
                                      t["k_cache"], t["v_cache"], t["k_scale"], t["v_scale"],
                                      t["out"], t["workspace"])
        assert name in str(e.value)
        # right dtypes and sizes on the host: the device check is what remains
        good = _good_step_tensors(c)
        with pytest.raises(ValueError, match="device tensor"):
            ga.mi355x_gated_attn_step(ctx, *[good[k] for k in (
                "qkv", "positions", "cache_loc", "cache_seqlens", "page_table", "seq_lens",
                "k_cache", "v_cache", "k_scale", "v_scale", "out", "workspace")])
    finally:
        ga.mi355x_gated_attn_destroy(ctx)


def test_binding_checks_the_variants_own_tensors(L):
    """block_idx (sparse), cu_seqlens_q and total_q (ragged), token_req and the
    page-table rows (sparse prefill) and the metadata tensors are checked too;
    positions may be absent without RoPE and the scales without a scaled cache."""
    import torch
    # sparse decode: block_idx [Hkv, B, topk]
    c = cfg(batch=3, q_len=1, window=0, max_pages=40, num_pages=100, page_size=4,
            sparse_block=32, sparse_topk=5)
    ctx = ga.mi355x_gated_attn_prepare(c)
    try:
        t = _good_step_tensors(c)
        args = [t[k] for k in ("qkv", "positions", "cache_loc", "cache_seqlens", "page_table")]
        rest = [t[k] for k in ("k_cache", "v_cache", "k_scale", "v_scale", "out", "workspace")]
        with pytest.raises(ValueError, match="block_idx: 29 elements"):
            ga.mi355x_gated_attn_sparse_step(ctx, *args, torch.zeros(29, dtype=torch.int32), *rest)
        with pytest.raises(ValueError, match="block_idx: dtype"):
            ga.mi355x_gated_attn_sparse_step(ctx, *args, torch.zeros(30, dtype=torch.int64), *rest)
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    # ragged: cu_seqlens_q [B+1], total_q bounds, packed rows of total_q tokens
    c = cfg(batch=2, q_len=16, window=0, max_pages=40, num_pages=100, page_size=4,
            rope_theta=0.0)
    ctx = ga.mi355x_gated_attn_prepare(c)
    try:
        t = _good_step_tensors(c)
        n = 20
        W = 2304
        qkv = torch.zeros(n * W, dtype=torch.int16)
        loc = torch.zeros(n, dtype=torch.int64)
        out = torch.zeros(n * 1024, dtype=torch.int16)
        common = (t["cache_seqlens"], t["page_table"], t["k_cache"], t["v_cache"], None, None,
                  out, t["workspace"])
        with pytest.raises(ValueError, match="total_q 33"):
            ga.mi355x_gated_attn_ragged_step(ctx, qkv, None, loc, torch.zeros(3, dtype=torch.int32),
                                             33, *common)
        with pytest.raises(ValueError, match="qkv: "):
            ga.mi355x_gated_attn_ragged_step(ctx, qkv, None, loc, torch.zeros(3, dtype=torch.int32),
                                             19, *common)
        with pytest.raises(ValueError, match="cu_seqlens_q: 2 elements"):
            ga.mi355x_gated_attn_ragged_step(ctx, qkv, None, loc, torch.zeros(2, dtype=torch.int32),
                                             n, *common)
        with pytest.raises(ValueError, match="device tensor"):  # positions may be absent
            ga.mi355x_gated_attn_ragged_step(ctx, qkv, None, loc, torch.zeros(3, dtype=torch.int32),
                                             n, *common)
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    # sparse prefill: page_table has num_requests rows, token_req one per query
    c = cfg(batch=6, q_len=1, window=0, max_pages=40, num_pages=100, page_size=4,
            sparse_block=32, sparse_topk=2)
    ctx = ga.mi355x_gated_attn_prepare(c)
    try:
        t = _good_step_tensors(c)
        pt2 = torch.zeros(2 * 40, dtype=torch.int32)
        rest = (t["k_cache"], t["v_cache"], t["k_scale"], t["v_scale"], t["out"], t["workspace"])
        bi = torch.zeros(2 * 6 * 2, dtype=torch.int32)
        with pytest.raises(ValueError, match="page_table: 240 elements"):
            ga.mi355x_gated_attn_sparse_prefill_step(ctx, t["qkv"], t["positions"], t["cache_loc"],
                                                     torch.zeros(6, dtype=torch.int32), 2,
                                                     t["cache_seqlens"], t["page_table"], bi, *rest)
        with pytest.raises(ValueError, match="token_req: 5 elements"):
            ga.mi355x_gated_attn_sparse_prefill_step(ctx, t["qkv"], t["positions"], t["cache_loc"],
                                                     torch.zeros(5, dtype=torch.int32), 2,
                                                     t["cache_seqlens"], pt2, bi, *rest)
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    # step metadata
    c = cfg(batch=3, q_len=2, max_pages=40, num_pages=100)
    ctx = ga.mi355x_gated_attn_prepare(c)
    try:
        i32 = lambda n: torch.zeros(n, dtype=torch.int32)
        i64 = lambda n: torch.zeros(n, dtype=torch.int64)
        with pytest.raises(ValueError, match="positions: 5 elements"):
            ga.mi355x_gated_attn_step_meta(ctx, i32(3), i32(120), i64(5), i64(6), i32(3))
        with pytest.raises(ValueError, match="cache_seqlens: dtype"):
            ga.mi355x_gated_attn_step_meta(ctx, i32(3), i32(120), i64(6), i64(6), i64(3))
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    with pytest.raises(ValueError, match="unknown or destroyed"):
        ga.mi355x_gated_attn_step_meta(ctx, i32(3), i32(120), i64(6), i64(6), i32(3))


def test_noalloc_step_rejects_plans_beyond_its_static_scratch(L):
    """The no-allocation step refuses, before touching a device, a plan whose
    q and partials exceed the static scratch (an extend block of 65,536
    tokens needs 64 MiB of q alone), and an unplanned or NULL context."""
    big = cfg(batch=1, q_len=65536, window=2048)
    ctx = ga.mi355x_gated_attn_prepare(big)
    try:
        assert L.mi355x_gated_attn_step_noalloc(ctx, *([None] * 12)) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "plan" in ga.mi355x_gated_attn_last_error()
        ga.mi355x_gated_attn_plan(ctx, 70000, 0)
        assert L.mi355x_gated_attn_step_noalloc(ctx, *([None] * 12)) == \
            ga.MI355X_GA_WORKSPACE_TOO_SMALL
        assert "static scratch" in ga.mi355x_gated_attn_last_error()
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    assert L.mi355x_gated_attn_step_noalloc(None, *([None] * 12)) == ga.MI355X_GA_INVALID_ARGUMENT
    small = ga.mi355x_gated_attn_prepare(cfg(batch=0))
    try:
        ga.mi355x_gated_attn_plan(small, 100, 0)
        assert L.mi355x_gated_attn_step_noalloc(small, *([None] * 12)) == ga.MI355X_GA_OK
    finally:
        ga.mi355x_gated_attn_destroy(small)


def test_page_table_validates_before_any_launch(L):
    ctx = ga.mi355x_gated_attn_prepare(cfg(batch=3, max_pages=10))
    P = ctypes.c_void_p
    try:
        f = L.mi355x_gated_attn_page_table
        good = [P(0x1000), 16, 4, P(0x2000), P(0x3000), P(0x4000), None, None]
        assert f(ctx, *good[:5], None, None, None, None) == ga.MI355X_GA_INVALID_ARGUMENT
        assert "neither" in ga.mi355x_gated_attn_last_error()
        assert f(ctx, None, 16, 4, P(0x2000), P(0x3000), P(0x4000), None, None, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
        assert f(ctx, P(0x1000), 0, 4, P(0x2000), P(0x3000), P(0x4000), None, None, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
        assert f(ctx, P(0x1000), 16, 4, P(0x2000), P(0x3000), None, P(0x5000), None, None) == \
            ga.MI355X_GA_INVALID_ARGUMENT
        assert "kv_indptr" in ga.mi355x_gated_attn_last_error()
        assert f(None, *good, None) == ga.MI355X_GA_INVALID_ARGUMENT
    finally:
        ga.mi355x_gated_attn_destroy(ctx)
    empty = ga.mi355x_gated_attn_prepare(cfg(batch=0))
    try:
        assert L.mi355x_gated_attn_page_table(empty, None, 1, 1, *([None] * 6)) == ga.MI355X_GA_OK
    finally:
        ga.mi355x_gated_attn_destroy(empty)
