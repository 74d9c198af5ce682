"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars: bf16 storage with fp32 accumulation -> max |err| <= 2e-2 and relative L2
error <= 5e-3; the float32 path -> relative L2 error <= 1e-5.  Small cases are
compared element by element over the whole output; the full-size workloads
are run whole on the GPU and compared on sampled (batch, head) slices, each of
which the oracle computes independently (heads never interact).
"""

import numpy as np
import pytest

from oracle import squad_oracle as so
from sub_quadratic_factorized_amd import binding as bd
from sub_quadratic_factorized_amd import workloads as wl

from gpu_common import assert_close, assert_close_bf16_output, host_to_device, log, to_f64, workload_device_inputs

pytestmark = pytest.mark.gpu

OPS = {
    "fwd": (bd.squad_attn_fwd, so.squad_attention),
    "local": (bd.squad_attn_local, so.local_pass),
    "global": (bd.squad_attn_global, so.global_pass),
    "reversed": (bd.squad_attn_fwd_reversed, so.squad_attention_reversed),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def run_small(geo, dtype, op="fwd", seed=0, qk_scale=1.0, B=1, heads=2, d=64, key_ramp=0.0,
              magnitude_scaled=False):
    T, Hs, Ws, wt, wh, ww = geo
    n = T * Hs * Ws
    log(f"case op={op} dtype={dtype} B={B} heads={heads} d={d} grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww} "
        f"qk_scale={qk_scale}")
    q, k, v = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed)
    if qk_scale != 1.0:
        # larger logits; values stay N(0, 1) so the absolute error bar keeps its meaning
        q, k = (wl.bf16_bits_to_f32(wl.bf16_round_bits(x * np.float32(qk_scale))) if dtype == "bf16"
                else x * np.float32(qk_scale) for x in (q, k))
    if key_ramp:
        # keys grow along the grid's x axis, which runs inside every window and
        # across windows, so later key blocks of a problem hold larger logits
        # and the running maximum must be refreshed
        x = np.arange(n, dtype=np.float32) % Ws
        ramp = (1.0 + key_ramp * x / Ws)[None, :, None, None]
        k = k * ramp
        if dtype == "bf16":
            k = wl.bf16_bits_to_f32(wl.bf16_round_bits(k))
    qd, kd, vd = host_to_device((q, k, v), dtype)
    gpu_fn, ref_fn = OPS[op]
    out = gpu_fn(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    ref = ref_fn(q, k, v, (B, heads, T, Hs, Ws, wt, wh, ww, d))
    return assert_close(to_f64(out), ref, dtype, op, magnitude_scaled=magnitude_scaled)


# ---------------------------------------------------------------------------
# The tiny fp32 workload (both readings of its value recipe)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_prescaled"])
@pytest.mark.parametrize("op", list(OPS))
def test_tiny_workload_f32(name, op):
    w = wl.WORKLOADS[name]
    log(f"case workload={name} op={op}")
    q, k, v = wl.full_inputs_f32(w)
    qd, kd, vd = host_to_device((q, k, v), "f32")
    gpu_fn, ref_fn = OPS[op]
    out = gpu_fn(qd, kd, vd, (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww))
    assert_close(to_f64(out), ref_fn(q, k, v, w.geometry()), "f32", f"{name}/{op}")


@pytest.mark.parametrize("op", list(OPS))
def test_tiny_geometry_bf16(op):
    run_small((3, 4, 4, 3, 2, 2), "bf16", op)


# ---------------------------------------------------------------------------
# Full-size workloads, sampled heads
# ---------------------------------------------------------------------------

# every head of the two native blocks; six heads of the 4x blocks, the first
# and last head of each batch element among them
SAMPLES = {
    "wan5b_704p": [(0, h) for h in range(24)],
    "wan1p3b_480p": [(0, h) for h in range(12)],
    "wan5b_4x": [(0, 0), (0, 5), (0, 11), (0, 16), (0, 19), (0, 23)],
    "wan14b_4x_cfg": [(0, 0), (0, 17), (0, 39), (1, 0), (1, 22), (1, 39)],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_workload_bf16_sampled_heads(name):
    import torch
    w = wl.WORKLOADS[name]
    log(f"case workload={name} op=fwd (generating inputs)")
    qd, kd, vd = workload_device_inputs(w)
    out = bd.squad_attn_fwd(qd, kd, vd, (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww))
    torch.cuda.synchronize()
    table = so.window_slot_table(w.T, w.Hs, w.Ws, w.wt, w.wh, w.ww)
    for b, h in SAMPLES[name]:
        q, k, v = wl.head_slices_f64(w, b, h)
        assert_close_bf16_output(to_f64(out[b, :, h, :]), so.squad_head(q, k, v, table), f"{name} b={b} h={h}")
    del qd, kd, vd, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("op", ["local", "global", "reversed"])
def test_headline_workload_each_pass(op):
    import torch
    w = wl.WORKLOADS["wan5b_704p"]
    log(f"case workload=wan5b_704p op={op}")
    qd, kd, vd = workload_device_inputs(w)
    out = OPS[op][0](qd, kd, vd, (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww))
    torch.cuda.synchronize()
    table = so.window_slot_table(w.T, w.Hs, w.Ws, w.wt, w.wh, w.ww)
    head_fn = {"local": so.local_pass_head, "global": so.global_pass_head, "reversed": so.squad_reversed_head}[op]
    for b, h in [(0, 5), (0, 13), (0, 17)]:
        q, k, v = wl.head_slices_f64(w, b, h)
        assert_close_bf16_output(to_f64(out[b, :, h, :]), head_fn(q, k, v, table), f"{op} h={h}")


# ---------------------------------------------------------------------------
# Edge cases: ragged lengths on every launch configuration, extremes, layouts
# ---------------------------------------------------------------------------

# (T, Hs, Ws, wt, wh, ww): m = wt*wh*ww, N_w = n/m
RAGGED = [
    (1, 6, 10, 1, 3, 5),      # m=15  N_w=4
    (3, 10, 12, 3, 2, 2),     # m=12  N_w=30
    (2, 9, 34, 1, 1, 17),     # m=17  N_w=36
    (1, 11, 99, 1, 1, 33),    # m=33  N_w=33
    (4, 5, 60, 2, 5, 10),     # m=100 N_w=12
    (2, 14, 100, 2, 1, 100),  # m=200 N_w=14
    (1, 7, 600, 1, 1, 200),   # m=200 N_w=21 (13 tiles)
    (2, 5, 300, 1, 1, 300),   # m=300 N_w=10 (19 tiles)
    (1, 4, 800, 1, 1, 400),   # m=400 N_w=8  (25 tiles)
    (1, 3, 330, 1, 3, 1),     # m=3   N_w=330
]


@pytest.mark.parametrize("geo", RAGGED, ids=[f"m{g[3]*g[4]*g[5]}_nw{g[0]*g[1]*g[2]//(g[3]*g[4]*g[5])}" for g in RAGGED])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_lengths(geo, dtype):
    run_small(geo, dtype, "fwd", heads=2, d=128 if dtype == "bf16" else 64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_head_dims(dtype, d):
    run_small((3, 4, 8, 3, 2, 2), dtype, "fwd", heads=3, d=d, B=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_window_is_full_attention(dtype):
    # N_w = 1, m = 512 (the longest local problem)
    run_small((8, 8, 8, 8, 8, 8), dtype, "fwd", heads=1, d=64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_token_windows(dtype):
    # m = 1, N_w = 512 (the longest global problem)
    run_small((8, 8, 8, 1, 1, 1), dtype, "fwd", heads=1, d=64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_both_lengths_at_maximum_region(dtype):
    # m = 512 with N_w = 64, then m = 64 with N_w = 512
    run_small((8, 64, 64, 8, 8, 8), dtype, "fwd", heads=1, d=64)
    run_small((8, 64, 64, 1, 8, 8), dtype, "fwd", heads=1, d=64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sharp_attention(dtype):
    # logit std ~ 9 (Q, K scaled by 3): near one-hot rows copy single values,
    # so outputs reach max|V|; the absolute bar is applied relative to |O|
    run_small((3, 10, 12, 3, 2, 2), dtype, "fwd", qk_scale=3.0, d=128, magnitude_scaled=True)
    run_small((2, 14, 100, 2, 1, 100), dtype, "fwd", qk_scale=3.0, d=128, magnitude_scaled=True)
    run_small((1, 4, 800, 1, 1, 400), dtype, "fwd", qk_scale=3.0, d=64, magnitude_scaled=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_running_maximum_refresh(dtype):
    # logits rise along each problem's rows: every few key blocks the block
    # maximum exceeds the running one by more than the refresh headroom
    run_small((1, 4, 800, 1, 1, 400), dtype, "fwd", qk_scale=1.5, key_ramp=3.0, d=64, magnitude_scaled=True)
    run_small((2, 14, 100, 2, 1, 100), dtype, "local", qk_scale=1.5, key_ramp=3.0, d=128, magnitude_scaled=True)
    run_small((1, 3, 330, 1, 3, 1), dtype, "global", qk_scale=1.5, key_ramp=3.0, d=128, magnitude_scaled=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_in_place_equals_out_of_place(dtype):
    import torch
    geo = (3, 10, 12, 3, 2, 2)
    T, Hs, Ws, wt, wh, ww = geo
    q, k, v = wl.random_geometry_inputs(1, 4, T * Hs * Ws, 128, dtype, seed=7)
    qd, kd, vd = host_to_device((q, k, v), dtype)
    for fn in (bd.squad_attn_local, bd.squad_attn_global, bd.squad_attn_fwd, bd.squad_attn_fwd_reversed):
        ref = fn(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
        buf = vd.clone()
        fn(qd, kd, buf, (T, Hs, Ws), (wt, wh, ww), out=buf)
        torch.cuda.synchronize()
        assert torch.equal(buf, ref), fn.__name__


def test_deterministic():
    import torch
    w = wl.WORKLOADS["wan5b_704p"]
    qd, kd, vd = workload_device_inputs(w)
    a = bd.squad_attn_fwd(qd, kd, vd, (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww))
    b = bd.squad_attn_fwd(qd, kd, vd, (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_side_stream_matches_default_stream():
    # the calls enqueue on the stream they are given (torch's current one by default): on a side
    # stream, after waiting for the inputs, forward and backward give the default stream's bits
    import torch
    w = wl.WORKLOADS["wan5b_704p"]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    qd, kd, vd = workload_device_inputs(w)
    dod = wl.device_inputs(w, seed=1)[0]
    ref = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    ref_g = bd.squad_attn_bwd(qd, kd, vd, ref, dod, grid, window)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = bd.squad_attn_fwd(qd, kd, vd, grid, window)
        grads = bd.squad_attn_bwd(qd, kd, vd, out, dod, grid, window)
    out2 = torch.empty_like(qd)
    bd.squad_attn_fwd(qd, kd, vd, grid, window, out=out2, stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(out, ref) and torch.equal(out2, ref)
    assert all(torch.equal(a, b) for a, b in zip(grads, ref_g))


def test_empty_batch_is_noop():
    import torch
    q = torch.empty((0, 48, 2, 64), device="cuda", dtype=torch.bfloat16)
    out = bd.squad_attn_fwd(q, q.clone(), q.clone(), (3, 4, 4), (3, 2, 2))
    assert out.shape == q.shape


def test_rejections_raise():
    import torch
    q = torch.zeros((1, 48, 2, 64), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(bd.SquadError) as e:
        bd.squad_attn_fwd(q, q.clone(), q.clone(), (3, 4, 4), (3, 3, 2))
    assert e.value.status == bd.SQUAD_ERR_SHAPE
    with pytest.raises(bd.SquadError) as e:
        bd.squad_attn_fwd(q, q, q.clone(), (3, 4, 4), (3, 2, 2), out=q)
    assert e.value.status == bd.SQUAD_ERR_ALIAS


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("op", ["fwd", "reversed"])
def test_many_heads_small_dim(dtype, op):
    # 32 heads at d=64: 64 windows x 64 slots per head, row stride 2048
    run_small((4, 32, 32, 4, 4, 4), dtype, op, heads=32, d=64)


# ---------------------------------------------------------------------------
# Long problems: whole on the 2- and 3-tile instances up to 24 tiles, split
# into query parts beyond (problem count a multiple of 8, not in place), else
# whole with their two query parts in turn and the value rows kept in LDS
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("geo,heads", [
    ((21, 8, 8, 21, 4, 4), 8),     # m = 336: 21 tiles on the 3-tile instance, 32 local problems
    ((5, 10, 16, 5, 5, 8), 2),     # m = 200: 13 tiles on the 2-tile instance, ragged last block
    ((5, 16, 10, 5, 8, 10), 4),    # m = 400: 2 parts of 13 + 12 tiles
    ((8, 8, 16, 8, 8, 8), 4),      # m = 512: 2 parts of 16 + 16 tiles
])
@pytest.mark.parametrize("op", ["fwd", "local"])
def test_split_long_problems(geo, heads, op):
    run_small(geo, "bf16", op, heads=heads, d=128, seed=17)


def test_split_long_problems_head_dim_64():
    run_small((21, 8, 8, 21, 4, 4), "bf16", "local", heads=8, d=64, seed=18)   # whole, 3 tiles per wave
    run_small((5, 16, 10, 5, 8, 10), "bf16", "local", heads=4, d=64, seed=18)  # 2 parts


@pytest.mark.parametrize("geo,heads,op,d", [
    ((5, 16, 10, 5, 8, 10), 3, "local", 128),   # m = 400, 6 problems: resident values, buffer loader
    ((5, 16, 10, 5, 8, 10), 3, "fwd", 128),
    ((5, 16, 10, 5, 8, 10), 3, "local", 64),
    ((2, 20, 75, 1, 2, 3), 1, "global", 128),   # N_w = 500 (32 tiles), 6 problems, out of place
    ((2, 20, 75, 1, 2, 3), 1, "global", 64),
])
def test_long_problems_not_split_out_of_place(geo, heads, op, d):
    run_small(geo, "bf16", op, heads=heads, d=d, seed=21)


def test_split_many_slots_global():
    # global pass over N_w = 200 windows at each of 8 slots x 2 heads (16 problems,
    # 13 tiles: whole on the 2-tile instance)
    run_small((2, 20, 80, 1, 2, 4), "bf16", "global", heads=2, d=64, seed=19)


@pytest.mark.parametrize("fn", ["local", "global", "fwd", "reversed"])
def test_in_place_long_problems_against_oracle(fn):
    # lengths that split into query parts when not in place (m = 336 local,
    # N_w = 400 global, problem counts multiples of 8): in place a pass is
    # never split across workgroups; a problem of 25-32 query tiles runs its
    # two query parts one after the other with the value rows kept in LDS
    # (N_w = 400 and 500 global, m = 400 local, 6 problems for N_w = 500), at
    # d = 64 and 128
    import torch
    for geo, heads, d in (((21, 8, 8, 21, 4, 4), 8, 64), ((2, 20, 80, 1, 2, 4), 2, 64),
                          ((2, 20, 80, 1, 2, 4), 2, 128), ((2, 20, 75, 1, 2, 3), 1, 128),
                          ((1, 20, 40, 1, 20, 20), 2, 128), ((1, 20, 40, 1, 20, 20), 2, 64)):
        T, Hs, Ws, wt, wh, ww = geo
        log(f"case in-place {fn} grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww} heads={heads}")
        q, k, v = wl.random_geometry_inputs(1, heads, T * Hs * Ws, d, "bf16", seed=23)
        qd, kd, vd = host_to_device((q, k, v), "bf16")
        gpu_fn, ref_fn = OPS[fn]
        buf = vd.clone()
        gpu_fn(qd, kd, buf, (T, Hs, Ws), (wt, wh, ww), out=buf)
        torch.cuda.synchronize()
        assert_close(to_f64(buf), ref_fn(q, k, v, (1, heads, T, Hs, Ws, wt, wh, ww, d)), "bf16", f"in place {fn}")


@pytest.mark.parametrize("op", ["fwd", "local", "reversed"])
def test_tensors_beyond_4gib_per_batch_element(op):
    # 48 tokens x 360,000 heads x d = 128 in bf16 spans 4.4 GB per tensor: the
    # local pass then takes its 64-bit loader (the 32-bit one needs a batch
    # element to span less than 4 GiB) and every pass addresses rows beyond
    # 2^32 bytes; sampled heads, first and last included, against the oracle
    import torch
    T, Hs, Ws, wt, wh, ww = 3, 4, 4, 3, 2, 2
    heads, d = 360_000, 128
    n = T * Hs * Ws
    log(f"case {op} beyond 4 GiB: grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww} heads={heads} d={d}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    q, k, v = (torch.randn(1, n, heads, d, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(3))
    gpu_fn, ref_fn = OPS[op]
    out = gpu_fn(q, k, v, (T, Hs, Ws), (wt, wh, ww))
    torch.cuda.synchronize()
    for h in (0, 1, 180_001, heads - 1):
        qs, ks, vs = (to_f64(x[:, :, h:h + 1, :].contiguous()) for x in (q, k, v))
        ref = ref_fn(qs, ks, vs, (1, 1, T, Hs, Ws, wt, wh, ww, d))
        assert_close(to_f64(out[:, :, h:h + 1, :].contiguous()), ref, "bf16", f"{op} beyond 4 GiB, head {h}")
    del q, k, v, out
    torch.cuda.empty_cache()


def test_graph_capture_replays_match_eager():
    # the forward enqueues kernels only (no memset, no allocation), so it can
    # be captured; every replay, with eager work and synchronisation between
    # replays, must reproduce the eager result exactly
    import torch
    T, Hs, Ws, wt, wh, ww = 3, 10, 12, 3, 2, 2
    q, k, v = wl.random_geometry_inputs(1, 4, T * Hs * Ws, 128, "bf16", seed=29)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    eager = bd.squad_attn_fwd(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    out = torch.empty_like(qd)
    bd.squad_attn_fwd(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww), out=out)  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bd.squad_attn_fwd(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww), out=out)
    for i in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        bd.squad_attn_local(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))  # eager work between replays
        torch.cuda.synchronize()
