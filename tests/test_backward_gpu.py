"""GPU parity of the backward (squad_attn_bwd through the C ABI) against the
oracle's gradients on the same seeded inputs and upstream gradient.  `out` is
the GPU forward's own output, as a caller would pass it."""

import numpy as np
import pytest

from oracle import squad_oracle as so
from sub_quadratic_factorized_amd import binding as bd
from sub_quadratic_factorized_amd import workloads as wl

from gpu_common import errors, host_to_device, log, to_f64, _record

pytestmark = pytest.mark.gpu

# Bars on each gradient's relative L2 error.  float32: as the forward.  bf16:
# one bf16 rounding (round to nearest even) perturbs a value by about 1.1e-3
# relative RMS; the gradients pass through about six (Y and dY stored, P or
# dS entering each MFMA, the forward's O inside D, the global pass's dq and dk
# contributions stored, the stored gradient), which add to ~2.7e-3 in
# quadrature, and the difference dP - D inside dS = P (dP - D) amplifies that
# somewhat (~3.5e-3 to 5e-3 expected).  The forward's bar is 5e-3 for half as
# many roundings; the gradients get twice that.
F32_GRAD_REL_L2 = 1e-5
BF16_GRAD_REL_L2 = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def check_grads(got, ref, dtype, what):
    bar = BF16_GRAD_REL_L2 if dtype == "bf16" else F32_GRAD_REL_L2
    worst = 0.0
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        max_abs, rel = errors(g, r)
        log(f"  {what} {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} max|ref|={np.max(np.abs(r)):.3f}")
        _record({"case": f"{what} {name}", "dtype": dtype, "max_abs": max_abs, "rel_l2": rel,
                 "max_ref": float(np.max(np.abs(r)))})
        worst = max(worst, rel)
    assert worst <= bar, (what, worst)


def run_bwd(geo, dtype, B=1, heads=2, d=64, seed=0):
    import torch
    T, Hs, Ws, wt, wh, ww = geo
    n = T * Hs * Ws
    log(f"case bwd dtype={dtype} B={B} heads={heads} d={d} grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww}")
    q, k, v = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed)
    do = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed + 1000)[0]
    qd, kd, vd, dod = host_to_device((q, k, v, do), dtype)
    out = bd.squad_attn_fwd(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    dq, dk, dv = bd.squad_attn_bwd(qd, kd, vd, out, dod, (T, Hs, Ws), (wt, wh, ww))
    torch.cuda.synchronize()
    ref = so.squad_backward(q, k, v, do, (B, heads, T, Hs, Ws, wt, wh, ww, d))
    check_grads([to_f64(t) for t in (dq, dk, dv)], ref, dtype, f"bwd {geo}")


# one block, ragged blocks, several blocks, more query tiles than waves, long
# windows (m = 336 as the 4x workloads), many windows; local windows of 7, 10
# and 12 key tiles (m = 100, 150 ragged, 192 whole: the one-sweep local
# backward on 8 and 12 waves, the latter with every K block of LDS in use);
# local windows of 15 key tiles (m = 240: the two-sweep kernel with the saved
# log-sum-exp on 8 waves); global passes of 110 (7 key tiles, ragged, as the
# headline's) and 128 windows (8 whole tiles) over single-token and two-token
# windows
GEOS = [
    (3, 4, 4, 3, 2, 2),
    (2, 6, 8, 1, 3, 4),
    (4, 8, 12, 2, 4, 4),
    (3, 10, 12, 3, 5, 4),
    (21, 8, 8, 21, 4, 4),
    (2, 24, 20, 1, 1, 2),
    (5, 8, 10, 5, 4, 5),
    (3, 10, 20, 3, 5, 10),
    (3, 8, 16, 3, 8, 8),
    (3, 8, 20, 3, 8, 10),
    (1, 10, 22, 1, 1, 2),
    (1, 8, 16, 1, 1, 1),
]


@pytest.mark.parametrize("geo", GEOS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_small(geo, dtype):
    run_bwd(geo, dtype)


@pytest.mark.parametrize("geo", [(3, 4, 4, 3, 4, 4), (3, 4, 4, 1, 1, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_degenerate_windows(geo, dtype):
    # one window spanning the grid (the global pass over a single row: P = 1, its dS = 0) and
    # single-token windows (the local pass is the identity): problems of length 1 in one pass
    run_bwd(geo, dtype, heads=2, d=64, seed=51)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_head_dim_128_batch(dtype):
    run_bwd((3, 8, 10, 3, 2, 5), dtype, B=2, heads=3, d=128, seed=4)


@pytest.mark.parametrize("geo", [(3, 10, 20, 3, 5, 10), (3, 8, 16, 3, 8, 8)])
def test_backward_one_sweep_12_waves_batch_head_dim_128(geo):
    # local windows of 10 (ragged) and 12 key tiles at d = 128 on the second
    # batch element too: the one-sweep local backward on 12 waves, whose rows
    # are 32-bit offsets from each (b, h) slice
    run_bwd(geo, "bf16", B=2, heads=3, d=128, seed=61)


def test_backward_headline_sampled_heads():
    import torch
    w = wl.WORKLOADS["wan5b_704p"]
    log("case bwd workload=wan5b_704p (generating inputs)")
    qd, kd, vd = wl.device_inputs(w, seed=0)
    dod = wl.device_inputs(w, seed=1)[0]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    out = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    dq, dk, dv = bd.squad_attn_bwd(qd, kd, vd, out, dod, grid, window)
    torch.cuda.synchronize()
    table = so.window_slot_table(*grid, *window)
    for h in (0, 17):
        q, k, v = wl.head_slices_f64(w, 0, h)
        do = to_f64(dod[0, :, h, :])
        ref = so.squad_backward_head(q, k, v, do, table)
        check_grads([to_f64(t[0, :, h, :]) for t in (dq, dk, dv)], ref, "bf16", f"wan5b_704p h={h}")


@pytest.mark.parametrize("geo", [(3, 4, 4, 3, 2, 2), (3, 8, 16, 3, 8, 8)])
def test_backward_beyond_one_sweep_row_offsets(geo):
    # a batch element of n * heads * d >= 2^30 elements: the local pass's backward
    # leaves the one-sweep kernel (32-bit row offsets) for the two-sweep kernel
    # with the saved log-sum-exp, on 8 waves (m = 12, one key tile) and on 12
    # (m = 192, 12 key tiles); sampled heads, first and last included
    import torch
    T, Hs, Ws, wt, wh, ww = geo
    n, d = T * Hs * Ws, 128
    heads = -(-(1 << 30) // (n * d))
    assert n * heads * d >= 1 << 30
    grid, window = (T, Hs, Ws), (wt, wh, ww)
    log(f"case bwd beyond the one-sweep gate: grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww} heads={heads} d={d}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(43)
    q, k, v, do = (torch.randn(1, n, heads, d, device="cuda", dtype=torch.bfloat16, generator=gen)
                   for _ in range(4))
    out = bd.squad_attn_fwd(q, k, v, grid, window)
    dq, dk, dv = bd.squad_attn_bwd(q, k, v, out, do, grid, window)
    torch.cuda.synchronize()
    table = so.window_slot_table(*grid, *window)
    for h in (0, heads // 2 + 1, heads - 1):
        qs, ks, vs, ds = (to_f64(x[0, :, h, :]) for x in (q, k, v, do))
        ref = so.squad_backward_head(qs, ks, vs, ds, table)
        check_grads([to_f64(t[0, :, h, :]) for t in (dq, dk, dv)], ref, "bf16", f"beyond gate {geo} h={h}")
    del q, k, v, do, out, dq, dk, dv
    torch.cuda.empty_cache()


def test_backward_deterministic():
    import torch
    geo = (2, 6, 8, 1, 3, 4)
    q, k, v = wl.random_geometry_inputs(1, 2, 96, 64, "bf16", seed=9)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    out = bd.squad_attn_fwd(qd, kd, vd, geo[:3], geo[3:])
    a = bd.squad_attn_bwd(qd, kd, vd, out, vd, geo[:3], geo[3:])
    b = bd.squad_attn_bwd(qd, kd, vd, out, vd, geo[:3], geo[3:])
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_cfg_pair_second_batch_element():
    # the 14B CFG pair (B = 2, 40 heads, m = 336): a head of the second batch element
    import torch
    w = wl.WORKLOADS["wan14b_4x_cfg"]
    log("case bwd workload=wan14b_4x_cfg (generating inputs)")
    qd, kd, vd = wl.device_inputs(w, seed=0)
    dod = wl.device_inputs(w, seed=1)[0]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    out = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    dq, dk, dv = bd.squad_attn_bwd(qd, kd, vd, out, dod, grid, window)
    torch.cuda.synchronize()
    table = so.window_slot_table(*grid, *window)
    q, k, v = wl.head_slices_f64(w, 1, 39)
    ref = so.squad_backward_head(q, k, v, to_f64(dod[1, :, 39, :]), table)
    check_grads([to_f64(t[1, :, 39, :]) for t in (dq, dk, dv)], ref, "bf16", "wan14b_4x_cfg b=1 h=39")
    del qd, kd, vd, dod, out, dq, dk, dv
    torch.cuda.empty_cache()


def test_backward_long_windows_sampled_heads():
    # the 4x 5B block: m = 336 (three groups of query / key tiles per window), N_w = 220
    import torch
    w = wl.WORKLOADS["wan5b_4x"]
    log("case bwd workload=wan5b_4x (generating inputs)")
    qd, kd, vd = wl.device_inputs(w, seed=0)
    dod = wl.device_inputs(w, seed=1)[0]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    out = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    dq, dk, dv = bd.squad_attn_bwd(qd, kd, vd, out, dod, grid, window)
    torch.cuda.synchronize()
    table = so.window_slot_table(*grid, *window)
    for h in (5,):
        q, k, v = wl.head_slices_f64(w, 0, h)
        do = to_f64(dod[0, :, h, :])
        ref = so.squad_backward_head(q, k, v, do, table)
        check_grads([to_f64(t[0, :, h, :]) for t in (dq, dk, dv)], ref, "bf16", f"wan5b_4x h={h}")
    del qd, kd, vd, dod, out, dq, dk, dv
    torch.cuda.empty_cache()


# ---- saved activations: squad_attn_fwd_save + squad_attn_bwd_saved ----------
# The pair runs the same kernels as squad_attn_fwd and squad_attn_bwd minus the
# backward's recomputation of the local pass, so its results must be those of
# the recomputing pair bit for bit (which the oracle checks above); the saved
# Y must be the local pass alone, and the saved log-sum-exp that of each row's
# window scores (log2 units of q.k * log2(e) / sqrt(d)).

def run_saved(geo, dtype, B=1, heads=2, d=64, seed=0):
    import torch
    T, Hs, Ws, wt, wh, ww = geo
    grid, window = (T, Hs, Ws), (wt, wh, ww)
    n = T * Hs * Ws
    log(f"case saved dtype={dtype} B={B} heads={heads} d={d} grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww}")
    q, k, v = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed)
    do = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed + 1000)[0]
    qd, kd, vd, dod = host_to_device((q, k, v, do), dtype)
    out_ref = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    y_ref = bd.squad_attn_local(qd, kd, vd, grid, window)
    out, y, lse = bd.squad_attn_fwd_save(qd, kd, vd, grid, window)
    ref = bd.squad_attn_bwd(qd, kd, vd, out_ref, dod, grid, window)
    got = bd.squad_attn_bwd_saved(qd, kd, vd, out, dod, y, lse, grid, window)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(y, y_ref)
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    if dtype == "bf16":
        # every row's log-sum-exp from its window's scores, float64 on the bf16 inputs; the
        # kernel sums the probabilities as rounded to bf16 for its P V product (unit roundoff
        # 2^-8 each), so its log2 of the sum is exact to 2^-8 * log2(e) ~ 5.6e-3
        qf, kf = to_f64(qd), to_f64(kd)
        table = so.window_slot_table(*grid, *window)
        lse_h = to_f64(lse)
        c = np.log2(np.e) / np.sqrt(d)
        for b in range(B):
            for h in range(heads):
                for rows in table:
                    s = qf[b, rows, h, :] @ kf[b, rows, h, :].T * c
                    mx = s.max(axis=1, keepdims=True)
                    want = mx[:, 0] + np.log2(np.exp2(s - mx).sum(axis=1))
                    np.testing.assert_allclose(lse_h[b, rows, h], want, rtol=0, atol=6e-3)
    return q, k, v, do, got


@pytest.mark.parametrize("geo", [GEOS[0], GEOS[3], GEOS[4], GEOS[9]])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_saved_activations_match_recompute(geo, dtype):
    T, Hs, Ws, wt, wh, ww = geo
    q, k, v, do, got = run_saved(geo, dtype)
    ref = so.squad_backward(q, k, v, do, (1, 2, T, Hs, Ws, wt, wh, ww, 64))
    check_grads([to_f64(t) for t in got], ref, dtype, f"saved {geo}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_saved_activations_batch_head_dim_128(dtype):
    geo = (3, 8, 10, 3, 2, 5)
    T, Hs, Ws, wt, wh, ww = geo
    q, k, v, do, got = run_saved(geo, dtype, B=2, heads=3, d=128, seed=7)
    ref = so.squad_backward(q, k, v, do, (2, 3, T, Hs, Ws, wt, wh, ww, 128))
    check_grads([to_f64(t) for t in got], ref, dtype, f"saved B=2 {geo}")


def test_saved_activations_headline():
    import torch
    w = wl.WORKLOADS["wan5b_704p"]
    log("case saved workload=wan5b_704p (generating inputs)")
    qd, kd, vd = wl.device_inputs(w, seed=0)
    dod = wl.device_inputs(w, seed=1)[0]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    out_ref = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    out, y, lse = bd.squad_attn_fwd_save(qd, kd, vd, grid, window)
    assert torch.equal(out, out_ref)
    del out_ref
    ref = bd.squad_attn_bwd(qd, kd, vd, out, dod, grid, window)
    got = bd.squad_attn_bwd_saved(qd, kd, vd, out, dod, y, lse, grid, window)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    del ref
    table = so.window_slot_table(*grid, *window)
    q, k, v = wl.head_slices_f64(w, 0, 11)
    ref11 = so.squad_backward_head(q, k, v, to_f64(dod[0, :, 11, :]), table)
    check_grads([to_f64(t[0, :, 11, :]) for t in got], ref11, "bf16", "saved wan5b_704p h=11")
    del qd, kd, vd, dod, out, y, lse, got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_wrapper_matches_entry_points(dtype):
    # squad_attention through torch autograd: the saved-activation pair, so the same bits as
    # squad_attn_fwd and squad_attn_bwd
    import torch
    geo = (4, 8, 12, 2, 4, 4)
    T, Hs, Ws, wt, wh, ww = geo
    grid, window = (T, Hs, Ws), (wt, wh, ww)
    q, k, v = wl.random_geometry_inputs(1, 2, T * Hs * Ws, 64, dtype, seed=41)
    do = wl.random_geometry_inputs(1, 2, T * Hs * Ws, 64, dtype, seed=42)[0]
    qd, kd, vd, dod = host_to_device((q, k, v, do), dtype)
    leaves = [t.clone().requires_grad_(True) for t in (qd, kd, vd)]
    out = bd.squad_attention(*leaves, grid, window)
    out.backward(dod)
    ref = bd.squad_attn_fwd(qd, kd, vd, grid, window)
    ref_g = bd.squad_attn_bwd(qd, kd, vd, ref, dod, grid, window)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref)
    assert all(torch.equal(t.grad, g) for t, g in zip(leaves, ref_g))


@pytest.mark.parametrize("saved", [False, True])
def test_graph_capture_backward_replays_match_eager(saved):
    # the backward enqueues kernels only (its workspace is the caller's), so it can be captured;
    # every replay, with eager work and synchronisation between replays, reproduces the eager result
    import torch
    T, Hs, Ws, wt, wh, ww = 3, 10, 12, 3, 2, 2
    grid, window = (T, Hs, Ws), (wt, wh, ww)
    B, heads, d = 1, 4, 128
    q, k, v = wl.random_geometry_inputs(B, heads, T * Hs * Ws, d, "bf16", seed=61)
    do = wl.random_geometry_inputs(B, heads, T * Hs * Ws, d, "bf16", seed=62)[0]
    qd, kd, vd, dod = host_to_device((q, k, v, do), "bf16")
    out, y, lse = bd.squad_attn_fwd_save(qd, kd, vd, grid, window)
    need = (bd.squad_attn_bwd_saved_workspace_bytes if saved else bd.squad_attn_bwd_workspace_bytes)(
        B, heads, T, Hs, Ws, wt, wh, ww, d, bd.SQUAD_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(qd) for _ in range(3)]

    def run():
        if saved:
            bd.squad_attn_bwd_saved(qd, kd, vd, out, dod, y, lse, grid, window, *grads, workspace=ws)
        else:
            bd.squad_attn_bwd(qd, kd, vd, out, dod, grid, window, *grads, workspace=ws)

    run()  # eager, and the warm-up outside capture
    torch.cuda.synchronize()
    eager = [g.clone() for g in grads]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for i in range(4):
        for g in grads:
            g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(g, e) for g, e in zip(grads, eager)), f"replay {i}"
        bd.squad_attn_fwd(qd, kd, vd, grid, window)  # eager work between replays
        torch.cuda.synchronize()
