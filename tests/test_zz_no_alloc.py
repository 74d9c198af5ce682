"""The padded forward without allocation (squad_attn_fwd_padded_noalloc,
through the C ABI) against the workspace entry point squad_attn_fwd_padded on
the same inputs: two calls in a row, the second on a smaller input, each equal
bit for bit to the workspace entry point's output and within the parity bar of
the oracle."""

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


def run_pair(B, heads, d, grid, window, dtype, seed, heads_checked):
    import torch
    T, Hs, Ws = grid
    n = T * Hs * Ws
    log(f"case noalloc dtype={dtype} B={B} heads={heads} d={d} grid={T}x{Hs}x{Ws} window={window}")
    q, k, v = wl.random_geometry_inputs(B, heads, n, d, dtype, seed=seed)
    qd, kd, vd = host_to_device((q, k, v), dtype)
    need = bd.squad_attn_padded_workspace_bytes(B, heads, *grid, *window, d, bd._dtype_code(qd))
    assert 0 < need <= bd.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref_out = torch.empty_like(qd)
    bd.squad_attn_fwd_padded(qd, kd, vd, grid, window, out=ref_out, workspace=ws)
    out = torch.full_like(qd, float("nan"))
    bd.squad_attn_fwd_padded_noalloc(qd, kd, vd, grid, window, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    geo = (1, 1, T, Hs, Ws, *window, d)
    for b, h in heads_checked:
        ref = so.squad_attention_padded(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], geo)
        assert_close(to_f64(out[b:b + 1, :, h:h + 1]), ref, dtype, f"noalloc b={b} h={h}")


def test_noalloc_two_calls_second_smaller():
    # 21x23x42 with a 21x2x3 window (one padded row per frame: 882 padded
    # positions per batch element), then 2x5x7 with 2x3x2 (13 per frame pair)
    run_pair(2, 8, 128, (21, 23, 42), (21, 2, 3), "bf16", 71, [(0, 0), (1, 7)])
    run_pair(1, 2, 64, (2, 5, 7), (2, 3, 2), "bf16", 72, [(0, 0), (0, 1)])


def test_noalloc_float32_and_tiling_window():
    import torch
    run_pair(1, 3, 64, (3, 7, 9), (3, 2, 4), "f32", 73, [(0, 0), (0, 2)])
    # a window that tiles the grid: the plain forward, no scratch used
    q, k, v = wl.random_geometry_inputs(1, 2, 3 * 4 * 4, 64, "bf16", seed=74)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    ref = bd.squad_attn_fwd(qd, kd, vd, (3, 4, 4), (3, 2, 2))
    out = bd.squad_attn_fwd_padded_noalloc(qd, kd, vd, (3, 4, 4), (3, 2, 2))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_long_global_pass_in_place():
    # 2x20x79 padded to 2x20x80 with 1x2x4 windows: a 400-window global pass,
    # which the workspace entry point splits into query parts (Y in its
    # workspace) and the no-allocation one runs in place, each problem's value
    # rows kept in LDS across its two query parts; both within the bar of the
    # oracle and of each other
    import torch
    for d in (64, 128):
        B, heads, grid, window = 1, 2, (2, 20, 79), (1, 2, 4)
        T, Hs, Ws = grid
        n = T * Hs * Ws
        log(f"case noalloc long global pass d={d}")
        q, k, v = wl.random_geometry_inputs(B, heads, n, d, "bf16", seed=75 + d)
        qd, kd, vd = host_to_device((q, k, v), "bf16")
        ref_out = bd.squad_attn_fwd_padded(qd, kd, vd, grid, window)
        out = bd.squad_attn_fwd_padded_noalloc(qd, kd, vd, grid, window, out=torch.full_like(qd, float("nan")))
        torch.cuda.synchronize()
        ref = so.squad_attention_padded(q, k, v, (B, heads, T, Hs, Ws, *window, d))
        assert_close(to_f64(out), ref, "bf16", f"noalloc long global d={d}")
        assert_close(to_f64(out), to_f64(ref_out), "bf16", f"noalloc vs workspace entry d={d}")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # 924 padded positions x 142 heads x 128 x 2 bytes > 32 MiB: refused before any launch
    import torch
    q = torch.zeros(1, 21 * 22 * 40, 142, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bd.SquadError) as e:
        bd.squad_attn_fwd_padded_noalloc(q, q, q, (21, 22, 40), (21, 2, 3), out=torch.empty_like(q))
    assert e.value.status == bd.SQUAD_ERR_SCRATCH
