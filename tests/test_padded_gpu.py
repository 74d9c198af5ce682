"""GPU parity of the padded entry point (grids a window does not tile) against
the oracle's reflect-padded SQuad on the same seeded inputs, plus its side
conditions: a tiling window reduces to squad_attn_fwd exactly, stale workspace
contents do not matter, and in-place use over v is refused."""

import numpy as np
import pytest

from oracle import squad_oracle as so
from sub_quadratic_factorized_amd import binding as bd
from sub_quadratic_factorized_amd import workloads as wl

from gpu_common import assert_close, host_to_device, log, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def run_padded(geo, dtype, B=1, heads=2, d=64, seed=0, stale_workspace=False):
    import torch
    T, Hs, Ws, wt, wh, ww = geo
    n = T * Hs * Ws
    _, Hp, Wp = so.padded_grid(T, Hs, Ws, wt, wh, ww)
    log(f"case padded dtype={dtype} B={B} heads={heads} d={d} grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww} "
        f"padded={T}x{Hp}x{Wp}")
    q, k, v = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed)
    qd, kd, vd = host_to_device((q, k, v), dtype)
    dt = bd.SQUAD_BF16 if dtype == "bf16" else bd.SQUAD_F32
    need = bd.squad_attn_padded_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dt)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    if stale_workspace:
        ws.fill_(0xFF)  # NaN patterns in either dtype
    out = torch.full_like(qd, float("nan"))
    bd.squad_attn_fwd_padded(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww), out=out, workspace=ws)
    ref = so.squad_attention_padded(q, k, v, (B, heads, T, Hs, Ws, wt, wh, ww, d))
    return assert_close(to_f64(out), ref, dtype, f"padded {geo}")


# (grid, window): both margins, right only, bottom only, one frame, long
# windows (several query tiles per wave), many windows (Q read straight from
# memory), the solver's window for a small 5B-aspect grid
PADDED = [
    (2, 5, 7, 2, 3, 2),
    (3, 10, 13, 3, 4, 5),
    (21, 11, 20, 21, 1, 3),
    (4, 9, 9, 2, 4, 4),
    (1, 30, 52, 1, 7, 11),
    (3, 12, 17, 3, 12, 5),
]


@pytest.mark.parametrize("geo", PADDED)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_small(geo, dtype):
    run_padded(geo, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_long_windows(dtype):
    # m = 315 (20 query tiles) on a 21x30x55 padded grid, N_w = 110
    run_padded((21, 30, 52, 21, 3, 5), dtype, heads=1, d=128)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_many_windows(dtype):
    # N_w = 476 windows of 9 tokens (30 query tiles in the global pass)
    run_padded((2, 40, 50, 1, 3, 3), dtype, heads=1, d=64)


def test_padded_headline_grid_other_window():
    # the 5B grid with a 21x2x3 window: 40 columns padded to 42, 154 windows of 126
    run_padded((21, 22, 40, 21, 2, 3), "bf16", heads=3, d=128)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_batch_and_heads(dtype):
    run_padded((2, 6, 10, 1, 4, 3), dtype, B=2, heads=5, d=128, seed=3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stale_workspace_is_overwritten(dtype):
    run_padded((3, 10, 13, 3, 4, 5), dtype, stale_workspace=True, seed=7)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiling_window_is_squad_attn_fwd(dtype):
    import torch
    T, Hs, Ws, wt, wh, ww = 3, 8, 12, 3, 2, 4
    q, k, v = wl.random_geometry_inputs(2, 3, T * Hs * Ws, 64, dtype, seed=5)
    qd, kd, vd = host_to_device((q, k, v), dtype)
    a = bd.squad_attn_fwd(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    b = bd.squad_attn_fwd_padded(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_padded_in_place_over_v_is_refused():
    q, k, v = wl.random_geometry_inputs(1, 2, 2 * 5 * 7, 64, "bf16", seed=1)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    with pytest.raises(bd.SquadError) as e:
        bd.squad_attn_fwd_padded(qd, kd, vd, (2, 5, 7), (2, 3, 2), out=vd)
    assert e.value.status == bd.SQUAD_ERR_ALIAS


def test_padded_small_workspace_is_refused():
    import torch
    q, k, v = wl.random_geometry_inputs(1, 2, 2 * 5 * 7, 64, "bf16", seed=1)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(bd.SquadError) as e:
        bd.squad_attn_fwd_padded(qd, kd, vd, (2, 5, 7), (2, 3, 2), workspace=ws)
    assert e.value.status == bd.SQUAD_ERR_WORKSPACE


def test_solved_windows_run():
    # the window rule's choice on small grids of the three backbones' aspect ratios
    for grid in [(21, 6, 11), (21, 8, 14), (5, 9, 16)]:
        win = bd.squad_window_solve(grid)
        run_padded(grid + win, "bf16", heads=2, d=128, seed=sum(grid))


@pytest.mark.parametrize("stale", [False, True])
def test_padded_long_global_pass_reads_y_from_workspace(stale):
    # 420 windows at each of 4 slots (27 query tiles; B*heads*m = 8): the local pass writes Y into
    # the workspace and the global pass reads it there, split into two query parts
    run_padded((1, 21, 79, 1, 1, 4), "bf16", heads=2, d=64, seed=21, stale_workspace=stale)
    run_padded((1, 21, 79, 1, 1, 4), "bf16", heads=2, d=128, seed=22)


def test_padded_split_long_windows():
    # m = 315 with 4 heads: 440 local problems of 20 tiles, whole on the 3-tile instance
    run_padded((21, 30, 52, 21, 3, 5), "bf16", heads=4, d=128, seed=11)
    # m = 400 with 8 heads: 24 local problems of 25 tiles (grid padded to 5x24x10), two query parts
    run_padded((5, 17, 10, 5, 8, 10), "bf16", heads=8, d=128, seed=12)


def test_padded_long_global_pass_full_grid_sampled_heads():
    # the window-rule sweep's largest grid (1.3B aspect, 21x67x116, window 21x4x5, padded to
    # 21x68x120): 408 windows of 420 tokens; the global pass reads Y from the workspace and runs in
    # two query parts, the local pass too (not in place); two heads against the oracle
    import torch
    T, Hs, Ws, wt, wh, ww = 21, 67, 116, 21, 4, 5
    heads, d = 4, 128
    n = T * Hs * Ws
    log(f"case padded full grid {T}x{Hs}x{Ws} window {wt}x{wh}x{ww} heads={heads}")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    qd, kd, vd = (torch.randn(1, n, heads, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    out = bd.squad_attn_fwd_padded(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    torch.cuda.synchronize()
    for h in (0, 3):
        q, k, v = (to_f64(t[0, :, h, :]) for t in (qd, kd, vd))
        ref = so.squad_head_padded(q, k, v, (T, Hs, Ws), (wt, wh, ww))
        assert_close(to_f64(out[0, :, h, :]), ref, "bf16", f"padded {T}x{Hs}x{Ws} h={h}")
    del qd, kd, vd, out
    torch.cuda.empty_cache()
