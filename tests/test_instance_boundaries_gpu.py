"""GPU parity at the lengths where the bf16 pass changes its launch: 12 / 13
query tiles (1 -> 2 tiles per wave), 16 / 17 (2 -> 3), 24 / 25 (3 tiles ->
query parts or resident values), 26 and 32 (the longest problems), each
length as the local pass (windows of that many tokens) and as the global
pass (that many windows), out of place and in place, with a problem count
that is a multiple of 8 (long problems split into query parts when not in
place) and one that is not (resident values).  Every output element is
compared with the fp64 oracle at the bf16 bar."""

import pytest

from oracle import squad_oracle as so
from sub_quadratic_factorized_amd import binding as bd
from sub_quadratic_factorized_amd import workloads as wl

from gpu_common import assert_close, host_to_device, log, to_f64

pytestmark = pytest.mark.gpu

LENGTHS = [192, 193, 256, 257, 384, 385, 416, 512]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def _geometry(pass_, L):
    # local: 2 windows of 1 x 1 x L; global: L windows of 1 x 1 x 2 (2 slots)
    return (1, 2, L, 1, 1, L) if pass_ == "local" else (1, 1, 2 * L, 1, 1, 2)


@pytest.mark.parametrize("L", LENGTHS)
@pytest.mark.parametrize("pass_", ["local", "global"])
@pytest.mark.parametrize("heads", [4, 3], ids=["8_problems", "6_problems"])
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_launch_boundaries(L, pass_, heads, in_place):
    import torch
    T, Hs, Ws, wt, wh, ww = geo = _geometry(pass_, L)
    d = 64
    n = T * Hs * Ws
    log(f"case {pass_} L={L} heads={heads} in_place={in_place} grid={T}x{Hs}x{Ws} window={wt}x{wh}x{ww} d={d}")
    q, k, v = wl.random_geometry_inputs(1, heads, n, d, "bf16", seed=31 + L)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    gpu_fn = bd.squad_attn_local if pass_ == "local" else bd.squad_attn_global
    ref_fn = so.local_pass if pass_ == "local" else so.global_pass
    if in_place:
        out = vd.clone()
        gpu_fn(qd, kd, out, (T, Hs, Ws), (wt, wh, ww), out=out)
    else:
        out = gpu_fn(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    torch.cuda.synchronize()
    ref = ref_fn(q, k, v, (1, heads, T, Hs, Ws, wt, wh, ww, d))
    assert_close(to_f64(out), ref, "bf16", f"{pass_} L={L}")


@pytest.mark.parametrize("L", [257, 385, 512])
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_launch_boundaries_head_dim_128(L, in_place):
    import torch
    T, Hs, Ws, wt, wh, ww = _geometry("global", L)
    heads, d = 3, 128
    n = T * Hs * Ws
    log(f"case global L={L} heads={heads} in_place={in_place} d={d}")
    q, k, v = wl.random_geometry_inputs(1, heads, n, d, "bf16", seed=41 + L)
    qd, kd, vd = host_to_device((q, k, v), "bf16")
    if in_place:
        out = vd.clone()
        bd.squad_attn_global(qd, kd, out, (T, Hs, Ws), (wt, wh, ww), out=out)
    else:
        out = bd.squad_attn_global(qd, kd, vd, (T, Hs, Ws), (wt, wh, ww))
    torch.cuda.synchronize()
    ref = so.global_pass(q, k, v, (1, heads, T, Hs, Ws, wt, wh, ww, d))
    assert_close(to_f64(out), ref, "bf16", f"global L={L} d=128")
