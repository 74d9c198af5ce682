"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects every invalid argument on the host before any HIP
call (so fake pointers are safe here)."""

import os
import re

import pytest

from sub_quadratic_factorized_amd import binding as bd
from oracle import squad_oracle as so

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "squad_attn.h")

# a valid geometry: the 5B native shape
GEO = dict(B=1, heads=24, T=21, Hs=22, Ws=40, wt=21, wh=2, ww=4, d=128)
BYTES = 1 * 18480 * 24 * 128 * 2
A = 1 << 40  # fake, well separated, 16-byte aligned addresses
Q, K, V, O = A, A + 4 * BYTES, A + 8 * BYTES, A + 12 * BYTES


def call(name="squad_attn_fwd", q=Q, k=K, v=V, out=O, dtype=bd.SQUAD_BF16, **over):
    g = dict(GEO)
    g.update(over)
    return bd.call_raw(name, q, k, v, out, g["B"], g["heads"], g["T"], g["Hs"], g["Ws"],
                       g["wt"], g["wh"], g["ww"], g["d"], dtype)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(squad_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = bd.lib()
    names = declared_functions()
    assert set(bd.ALL_SYMBOLS) == set(names)
    for n in names:
        assert getattr(lib, n) is not None
    assert lib.squad_attn_abi_version() == 4


def test_exports_via_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", bd.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (squad_\w+)", out))
    assert set(declared_functions()) <= exported


@pytest.mark.parametrize("name", bd.COMPUTE_ENTRY_POINTS)
def test_shape_errors(name):
    S = bd.SQUAD_ERR_SHAPE
    assert call(name, B=-1) == S
    assert call(name, heads=-2) == S
    for key in ("T", "Hs", "Ws", "wt", "wh", "ww", "d"):
        assert call(name, **{key: 0}) == S, key
        assert call(name, **{key: -3}) == S, key
    assert call(name, wh=3) == S                    # 22 % 3 != 0
    assert call(name, ww=3) == S                    # 40 % 3 != 0
    assert call(name, wt=4) == S                    # 21 % 4 != 0
    assert call(name, T=1 << 16, Hs=1 << 16, Ws=1, wt=1, wh=1, ww=1) == S  # n >= 2^31
    # element count overflow (B*n*heads*d >= 2^62)
    assert call(name, B=1 << 30, heads=1 << 30, T=1 << 10, Hs=1, Ws=1, wt=1, wh=1, ww=1) == S
    # problem count beyond a 31-bit grid
    assert call(name, B=1 << 20, heads=1 << 10, T=512, Hs=1, Ws=1, wt=1, wh=1, ww=1, d=64) == S
    # token stride heads * d beyond 31 bits
    assert call(name, B=1, heads=1 << 24, T=1, Hs=1, Ws=1, wt=1, wh=1, ww=1, d=128) == S


@pytest.mark.parametrize("name", bd.COMPUTE_ENTRY_POINTS)
def test_unsupported(name):
    U = bd.SQUAD_ERR_UNSUPPORTED
    assert call(name, dtype=7) == U
    assert call(name, dtype=-1) == U
    assert call(name, d=96) == U
    assert call(name, d=256) == U
    assert call(name, d=32) == U
    # window of 1024 tokens > max length
    assert call(name, T=4, Hs=16, Ws=16, wt=4, wh=16, ww=16) == U
    # 1024 windows of one token: N_w > max length
    assert call(name, T=4, Hs=16, Ws=16, wt=1, wh=1, ww=1) == U
    # shape errors win over unsupported (documented order)
    assert call(name, d=96, wh=3) == bd.SQUAD_ERR_SHAPE


@pytest.mark.parametrize("name", bd.COMPUTE_ENTRY_POINTS)
def test_null_align_alias(name):
    assert call(name, q=0) == bd.SQUAD_ERR_NULL
    assert call(name, k=0) == bd.SQUAD_ERR_NULL
    assert call(name, v=0) == bd.SQUAD_ERR_NULL
    assert call(name, out=0) == bd.SQUAD_ERR_NULL
    assert call(name, q=0, dtype=9) == bd.SQUAD_ERR_UNSUPPORTED  # order: unsupported before null
    for key in ("q", "k", "v", "out"):
        for off in (2, 8):
            assert call(name, **{key: {"q": Q, "k": K, "v": V, "out": O}[key] + off}) == bd.SQUAD_ERR_ALIGN
    assert call(name, q=0, out=O + 8) == bd.SQUAD_ERR_NULL       # order: null before align
    assert call(name, out=Q) == bd.SQUAD_ERR_ALIAS
    assert call(name, out=K + 16) == bd.SQUAD_ERR_ALIAS
    assert call(name, out=Q - BYTES + 16) == bd.SQUAD_ERR_ALIAS  # tail of out overlaps head of q
    assert call(name, out=V + 16) == bd.SQUAD_ERR_ALIAS          # partial overlap with v
    assert call(name, out=V - 16) == bd.SQUAD_ERR_ALIAS
    assert call(name, out=K - BYTES, dtype=bd.SQUAD_F32) == bd.SQUAD_ERR_ALIAS  # f32 buffers are twice as long


def check(q=Q, k=K, v=V, out=O, dtype=bd.SQUAD_BF16, **over):
    g = dict(GEO)
    g.update(over)
    return bd.squad_attn_check(q, k, v, out, g["B"], g["heads"], g["T"], g["Hs"], g["Ws"],
                               g["wt"], g["wh"], g["ww"], g["d"], dtype)


def test_check_accepts_what_would_launch():
    assert check() == bd.SQUAD_OK
    assert check(out=V) == bd.SQUAD_OK                 # in place over v
    assert check(out=Q + BYTES) == bd.SQUAD_OK         # adjacent buffers do not overlap
    assert check(out=Q - BYTES) == bd.SQUAD_OK
    assert check(dtype=bd.SQUAD_F32, out=Q + 2 * BYTES) == bd.SQUAD_OK
    assert check(dtype=bd.SQUAD_F32, out=Q + BYTES) == bd.SQUAD_ERR_ALIAS
    assert check(d=64) == bd.SQUAD_OK
    assert check(T=8, Hs=8, Ws=8, wt=8, wh=8, ww=8) == bd.SQUAD_OK      # one window of 512
    assert check(T=8, Hs=8, Ws=8, wt=1, wh=1, ww=1) == bd.SQUAD_OK      # 512 windows of one token
    assert check(T=8, Hs=8, Ws=16, wt=8, wh=8, ww=16) == bd.SQUAD_ERR_UNSUPPORTED
    assert check(B=0, q=0) == bd.SQUAD_OK


@pytest.mark.parametrize("name", bd.COMPUTE_ENTRY_POINTS)
def test_check_matches_entry_points_on_rejections(name):
    cases = [dict(B=-1), dict(wh=3), dict(d=96), dict(dtype=4), dict(q=0), dict(out=O + 4), dict(out=K + 32),
             dict(B=0, q=0)]
    for c in cases:
        assert call(name, **c) == check(**c), c


@pytest.mark.parametrize("name", bd.COMPUTE_ENTRY_POINTS)
def test_empty_problem_is_a_noop(name):
    assert call(name, B=0, q=0, k=0, v=0, out=0) == bd.SQUAD_OK
    assert call(name, heads=0, q=0, k=0, v=0, out=0) == bd.SQUAD_OK
    assert call(name, B=0, wh=3) == bd.SQUAD_ERR_SHAPE


def test_max_len():
    for d in (64, 128):
        for dt in (bd.SQUAD_BF16, bd.SQUAD_F32):
            assert bd.squad_attn_max_len(d, dt) == 512
    assert bd.squad_attn_max_len(96, bd.SQUAD_BF16) == 0
    assert bd.squad_attn_max_len(128, 5) == 0


def test_flops_and_bytes_helpers():
    from sub_quadratic_factorized_amd import workloads as wl
    for w in wl.WORKLOADS.values():
        f = bd.squad_attn_flops(*w.geometry())
        assert f == so.squad_flops(*w.geometry())
        es = 2 if w.dtype == "bf16" else 4
        dt = bd.SQUAD_BF16 if w.dtype == "bf16" else bd.SQUAD_F32
        assert bd.squad_attn_bytes(*w.geometry(), dt) == 8 * w.B * w.n * w.heads * w.d * es
    assert bd.squad_attn_flops(1, 24, 21, 22, 40, 21, 2, 4, 128) == 63_128_862_720
    assert bd.squad_attn_flops(1, 24, 21, 22, 40, 21, 3, 4, 128) == -1
    assert bd.squad_attn_bytes(1, 24, 21, 22, 40, 21, 2, 4, 128, 9) == -1
    assert bd.squad_attn_flops(0, 24, 21, 22, 40, 21, 2, 4, 128) == 0


def test_status_strings():
    for s in range(9):  # every status the header defines
        assert isinstance(bd.status_str(s), str) and bd.status_str(s)
    assert bd.status_str(123) == "unknown status"
    assert bd.lib().squad_attn_last_hip_error() == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        bd.lib()


# ---------------------------------------------------------------------------
# Padded grids (window need not tile the grid)
# ---------------------------------------------------------------------------

# 5B grid with a 21x2x3 window: Ws = 40 padded to 42 (one mirrored column pair)
PGEO = dict(B=1, heads=24, T=21, Hs=22, Ws=40, wt=21, wh=2, ww=3, d=128)
PAD_BYTES = 1 * 21 * 22 * 2 * 24 * 128 * 2    # 21 frames x 22 rows x 2 padded columns
WS = A + 16 * BYTES


def pcall(fn="check", q=Q, k=K, v=V, out=O, ws=WS, ws_bytes=PAD_BYTES, dtype=bd.SQUAD_BF16, **over):
    g = dict(PGEO)
    g.update(over)
    args = (q, k, v, out, ws, ws_bytes, g["B"], g["heads"], g["T"], g["Hs"], g["Ws"], g["wt"], g["wh"], g["ww"],
            g["d"], dtype)
    if fn == "check":
        return bd.squad_attn_check_padded(*args)
    return bd.lib().squad_attn_fwd_padded(*args, None)


def test_padded_workspace_size():
    assert bd.squad_attn_padded_workspace_bytes(*PGEO.values(), bd.SQUAD_BF16) == PAD_BYTES
    assert bd.squad_attn_padded_workspace_bytes(*PGEO.values(), bd.SQUAD_F32) == 2 * PAD_BYTES
    assert bd.squad_attn_padded_workspace_bytes(*GEO.values(), bd.SQUAD_BF16) == 0      # tiles: nothing padded
    assert bd.squad_attn_padded_workspace_bytes(*GEO.values(), 5) == -1
    g = dict(PGEO, wt=4)
    assert bd.squad_attn_padded_workspace_bytes(*g.values(), bd.SQUAD_BF16) == -1      # T % wt != 0
    # both margins: 2x5x7 grid, 2x3x2 window -> 2x6x8 padded, 48 - 35 = 13 padded positions per frame pair
    assert bd.squad_attn_padded_workspace_bytes(1, 2, 2, 5, 7, 2, 3, 2, 64, bd.SQUAD_F32) == 2 * 13 * 2 * 64 * 4


@pytest.mark.parametrize("fn", ["check", "fwd"])
def test_padded_rejections(fn):
    # every case is rejected on the host, so the compute entry point is safe to
    # call with fake pointers; the check function must agree with it
    S, U, N, W, AL, AS = (bd.SQUAD_ERR_SHAPE, bd.SQUAD_ERR_UNSUPPORTED, bd.SQUAD_ERR_NULL, bd.SQUAD_ERR_WORKSPACE,
                          bd.SQUAD_ERR_ALIGN, bd.SQUAD_ERR_ALIAS)
    assert pcall(fn, wt=4) == S                      # time axis never padded
    assert pcall(fn, wh=23) == S                     # window taller than the grid: mirror would overrun
    assert pcall(fn, ww=41) == S
    assert pcall(fn, B=-1) == S
    assert pcall(fn, T=8, Hs=8, Ws=8, wt=8, wh=8, ww=9) == S    # ww > Ws
    assert pcall(fn, d=96) == U
    assert pcall(fn, dtype=3) == U
    assert pcall(fn, T=8, Hs=15, Ws=15, wt=8, wh=8, ww=9) == U  # m = 576 > 512
    assert pcall(fn, T=1, Hs=1000, Ws=1100, wt=1, wh=100, ww=99, d=64) == U   # Wp = 1188 > 1023
    assert pcall(fn, q=0) == N
    assert pcall(fn, ws=0) == W
    assert pcall(fn, ws_bytes=PAD_BYTES - 16) == W
    assert pcall(fn, q=0, ws=0) == N                  # null before workspace
    assert pcall(fn, ws=WS + 8) == AL
    assert pcall(fn, out=O + 8) == AL
    assert pcall(fn, ws=0, out=O + 8) == W            # workspace before align
    assert pcall(fn, out=V) == AS                     # padded: no in-place over v
    assert pcall(fn, out=K + 32) == AS
    assert pcall(fn, ws=O + 32) == AS                 # workspace overlapping out
    assert pcall(fn, ws=Q - PAD_BYTES + 16) == AS     # workspace tail over q


def test_padded_check_accepts_what_would_launch():
    assert pcall() == bd.SQUAD_OK
    assert pcall(ws=Q - PAD_BYTES) == bd.SQUAD_OK                     # adjacent to q
    assert pcall(T=8, Hs=15, Ws=15, wt=8, wh=8, ww=8) == bd.SQUAD_OK  # m = 512 on a 16x16 padded grid
    # a window that tiles: workspace unused (NULL is fine) and out == v allowed
    assert pcall(ww=4, ws=0, ws_bytes=0) == bd.SQUAD_OK
    assert pcall(ww=4, ws=0, ws_bytes=0, out=V) == bd.SQUAD_OK
    assert pcall(B=0, q=0, ws=0) == bd.SQUAD_OK
    assert pcall("fwd", B=0, q=0, k=0, v=0, out=0, ws=0) == bd.SQUAD_OK   # empty: nothing enqueued


def ncall(q=Q, k=K, v=V, out=O, dtype=bd.SQUAD_BF16, **over):
    g = dict(PGEO)
    g.update(over)
    return bd.lib().squad_attn_fwd_padded_noalloc(q, k, v, out, g["B"], g["heads"], g["T"], g["Hs"], g["Ws"],
                                                  g["wt"], g["wh"], g["ww"], g["d"], dtype, None)


def test_noalloc_rejections_before_any_hip_call():
    # the padded entry point's checks without a workspace, and the fixed
    # scratch's limit: 924 padded positions x heads x 128 x 2 bytes fits
    # 32 MiB up to 141 heads
    assert bd.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert 924 * 141 * 128 * 2 <= bd.NOALLOC_SCRATCH_BYTES < 924 * 142 * 128 * 2
    assert ncall(heads=142) == bd.SQUAD_ERR_SCRATCH
    assert ncall(heads=71, dtype=bd.SQUAD_F32) == bd.SQUAD_ERR_SCRATCH
    assert ncall(heads=142, q=0) == bd.SQUAD_ERR_NULL           # null before scratch
    assert ncall(wt=4) == bd.SQUAD_ERR_SHAPE
    assert ncall(ww=41) == bd.SQUAD_ERR_SHAPE
    assert ncall(d=96) == bd.SQUAD_ERR_UNSUPPORTED
    assert ncall(q=0) == bd.SQUAD_ERR_NULL
    assert ncall(out=O + 8) == bd.SQUAD_ERR_ALIGN
    assert ncall(out=V) == bd.SQUAD_ERR_ALIAS                   # padded: no in-place over v
    assert ncall(out=K + 32) == bd.SQUAD_ERR_ALIAS
    assert ncall(B=0, q=0, k=0, v=0, out=0) == bd.SQUAD_OK      # empty: nothing enqueued
    assert "scratch" in bd.status_str(bd.SQUAD_ERR_SCRATCH)


def test_padded_flops_and_bytes_helpers():
    for geo in [(1, 24, 21, 22, 40, 21, 2, 3, 128), (2, 3, 2, 5, 7, 2, 3, 2, 64), (1, 24, 21, 22, 40, 21, 2, 4, 128)]:
        assert bd.squad_attn_flops_padded(*geo) == so.squad_flops_padded(*geo)
        B, heads, T, Hs, Ws, wt, wh, ww, d = geo
        _, Hp, Wp = so.padded_grid(T, Hs, Ws, wt, wh, ww)
        n, n_p = T * Hs * Ws, T * Hp * Wp
        assert bd.squad_attn_bytes_padded(*geo, bd.SQUAD_BF16) == (7 * n_p + n) * B * heads * d * 2
    assert bd.squad_attn_flops_padded(1, 24, 21, 22, 40, 21, 2, 4, 128) == bd.squad_attn_flops(
        1, 24, 21, 22, 40, 21, 2, 4, 128)
    assert bd.squad_attn_flops_padded(1, 1, 21, 22, 40, 4, 2, 3, 128) == -1


def test_window_solver_matches_oracle_rule():
    for T in (1, 2, 21):
        for Hs in range(1, 64, 5):
            for Ws in range(1, 120, 9):
                assert bd.squad_window_solve((T, Hs, Ws)) == so.solve_window(T, Hs, Ws), (T, Hs, Ws)
    assert bd.squad_window_solve((21, 22, 40)) == (21, 2, 4)
    assert bd.squad_window_solve((21, 30, 52)) == (21, 2, 4)
    with pytest.raises(bd.SquadError):
        bd.squad_window_solve((0, 4, 4))
    with pytest.raises(bd.SquadError):
        bd.squad_window_solve((1 << 11, 1 << 10, 1 << 10))


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

DO, DQ, DK, DV = A + 16 * BYTES, A + 20 * BYTES, A + 24 * BYTES, A + 28 * BYTES
BWS = A + 32 * BYTES
# Y, dY and the global pass's dq, dk contributions in bf16, then float32 row log-sum-exp and D
# (256-byte rounded: exact here)
BWS_BYTES = 4 * BYTES + 2 * 18480 * 24 * 4


def bcall(fn="check", q=Q, k=K, v=V, out=O, dout=DO, dq=DQ, dk=DK, dv=DV, ws=BWS, ws_bytes=BWS_BYTES,
          dtype=bd.SQUAD_BF16, **over):
    g = dict(GEO)
    g.update(over)
    args = (q, k, v, out, dout, dq, dk, dv, ws, ws_bytes, g["B"], g["heads"], g["T"], g["Hs"], g["Ws"], g["wt"],
            g["wh"], g["ww"], g["d"], dtype)
    if fn == "check":
        return bd.squad_attn_check_bwd(*args)
    return bd.lib().squad_attn_bwd(*args, None)


def test_bwd_workspace_and_helpers():
    assert bd.squad_attn_bwd_workspace_bytes(*GEO.values(), bd.SQUAD_BF16) == BWS_BYTES
    assert bd.squad_attn_bwd_workspace_bytes(*GEO.values(), bd.SQUAD_F32) == 4 * 2 * BYTES  # no log-sum-exp region
    assert bd.squad_attn_bwd_workspace_bytes(*dict(GEO, wh=3).values(), bd.SQUAD_BF16) == -1
    assert bd.squad_attn_bwd_workspace_bytes(*dict(GEO, B=0).values(), bd.SQUAD_BF16) == 0
    assert bd.squad_attn_bwd_flops(*GEO.values()) == 2.5 * 63_128_862_720
    assert bd.squad_attn_bwd_flops(*GEO.values()) == so.squad_backward_flops(*GEO.values())
    e = 18480 * 24 * 128
    assert bd.squad_attn_bwd_bytes(*GEO.values(), bd.SQUAD_BF16) == e * 2 * 21
    assert bd.squad_attn_bwd_bytes(*GEO.values(), bd.SQUAD_F32) == e * 4 * 22


@pytest.mark.parametrize("fn", ["check", "bwd"])
def test_bwd_rejections(fn):
    assert bcall(fn, wh=3) == bd.SQUAD_ERR_SHAPE
    assert bcall(fn, d=96) == bd.SQUAD_ERR_UNSUPPORTED
    for key in ("q", "k", "v", "out", "dout", "dq", "dk", "dv"):
        assert bcall(fn, **{key: 0}) == bd.SQUAD_ERR_NULL, key
    assert bcall(fn, ws=0) == bd.SQUAD_ERR_WORKSPACE
    assert bcall(fn, ws_bytes=BWS_BYTES - 1) == bd.SQUAD_ERR_WORKSPACE
    assert bcall(fn, dq=0, ws=0) == bd.SQUAD_ERR_NULL
    for key in ("q", "dout", "dv", "ws"):
        assert bcall(fn, **{key: {"q": Q, "dout": DO, "dv": DV, "ws": BWS}[key] + 8}) == bd.SQUAD_ERR_ALIGN, key
    assert bcall(fn, dq=Q) == bd.SQUAD_ERR_ALIAS
    assert bcall(fn, dk=DO + 16) == bd.SQUAD_ERR_ALIAS
    assert bcall(fn, dv=O) == bd.SQUAD_ERR_ALIAS
    assert bcall(fn, dk=DQ) == bd.SQUAD_ERR_ALIAS
    assert bcall(fn, dv=DK + 32) == bd.SQUAD_ERR_ALIAS
    assert bcall(fn, ws=V + 16) == bd.SQUAD_ERR_ALIAS
    assert bcall(fn, dq=BWS + BWS_BYTES - 16) == bd.SQUAD_ERR_ALIAS


def test_bwd_check_accepts_what_would_launch():
    assert bcall() == bd.SQUAD_OK
    assert bcall(out=Q, dout=K) == bd.SQUAD_OK           # inputs may overlap one another
    assert bcall(dtype=bd.SQUAD_F32, q=A, k=A + 2 * BYTES, v=A + 4 * BYTES, out=A + 6 * BYTES,
                 dout=A + 8 * BYTES, dq=A + 10 * BYTES, dk=A + 12 * BYTES, dv=A + 14 * BYTES,
                 ws=A + 16 * BYTES, ws_bytes=8 * BYTES) == bd.SQUAD_OK
    assert bcall("bwd", B=0, q=0, k=0, v=0, out=0, dout=0, dq=0, dk=0, dv=0, ws=0) == bd.SQUAD_OK


# ---------------------------------------------------------------------------
# saved activations: squad_attn_fwd_save / squad_attn_bwd_saved (rejections only: a valid call would launch)

Y, LSE = A + 40 * BYTES, A + 44 * BYTES
SWS = A + 48 * BYTES
LSE_BYTES = 18480 * 24 * 4
SWS_BYTES = 3 * BYTES + LSE_BYTES  # dY and the dq, dk contributions in bf16, float32 row D


def fcall(q=Q, k=K, v=V, out=O, y=Y, lse=LSE, dtype=bd.SQUAD_BF16, **over):
    g = dict(GEO)
    g.update(over)
    return bd.lib().squad_attn_fwd_save(q, k, v, out, y, lse, g["B"], g["heads"], g["T"], g["Hs"], g["Ws"],
                                        g["wt"], g["wh"], g["ww"], g["d"], dtype, None)


def scall(q=Q, k=K, v=V, out=O, dout=DO, y=Y, lse=LSE, dq=DQ, dk=DK, dv=DV, ws=SWS, ws_bytes=SWS_BYTES,
          dtype=bd.SQUAD_BF16, **over):
    g = dict(GEO)
    g.update(over)
    return bd.lib().squad_attn_bwd_saved(q, k, v, out, dout, y, lse, dq, dk, dv, ws, ws_bytes, g["B"], g["heads"],
                                         g["T"], g["Hs"], g["Ws"], g["wt"], g["wh"], g["ww"], g["d"], dtype, None)


def test_saved_workspace_size():
    assert bd.squad_attn_bwd_saved_workspace_bytes(*GEO.values(), bd.SQUAD_BF16) == SWS_BYTES
    assert bd.squad_attn_bwd_saved_workspace_bytes(*GEO.values(), bd.SQUAD_F32) == 3 * 2 * BYTES
    assert bd.squad_attn_bwd_saved_workspace_bytes(*dict(GEO, wh=3).values(), bd.SQUAD_BF16) == -1
    assert bd.squad_attn_bwd_saved_workspace_bytes(*dict(GEO, B=0).values(), bd.SQUAD_BF16) == 0
    assert bd.squad_attn_bwd_saved_workspace_bytes(*GEO.values(), 7) == -1
    # the saved variant needs the recomputing one's workspace less Y and the log-sum-exp
    assert BWS_BYTES - SWS_BYTES == BYTES + LSE_BYTES


def test_fwd_save_rejections():
    assert fcall(wh=3) == bd.SQUAD_ERR_SHAPE
    assert fcall(d=96) == bd.SQUAD_ERR_UNSUPPORTED
    assert fcall(q=0) == bd.SQUAD_ERR_NULL
    assert fcall(y=0) == bd.SQUAD_ERR_NULL
    assert fcall(lse=0) == bd.SQUAD_ERR_NULL                      # bf16 needs the log-sum-exp
    assert fcall(y=Y + 8) == bd.SQUAD_ERR_ALIGN
    assert fcall(lse=LSE + 4) == bd.SQUAD_ERR_ALIGN
    assert fcall(y=O) == bd.SQUAD_ERR_ALIAS                       # y is not the output
    assert fcall(y=V + 16) == bd.SQUAD_ERR_ALIAS
    assert fcall(y=Q - BYTES + 16) == bd.SQUAD_ERR_ALIAS          # tail over q
    assert fcall(lse=K + 64) == bd.SQUAD_ERR_ALIAS
    assert fcall(lse=Y + BYTES - 16) == bd.SQUAD_ERR_ALIAS        # over y's tail
    assert fcall(out=Q) == bd.SQUAD_ERR_ALIAS                     # the forward's own rule first


def test_bwd_saved_rejections():
    assert scall(wh=3) == bd.SQUAD_ERR_SHAPE
    for key in ("q", "dout", "dv", "y", "lse"):
        assert scall(**{key: 0}) == bd.SQUAD_ERR_NULL, key
    assert scall(y=Y + 8) == bd.SQUAD_ERR_ALIGN
    assert scall(lse=LSE + 4) == bd.SQUAD_ERR_ALIGN
    assert scall(y=DQ) == bd.SQUAD_ERR_ALIAS                      # y over a gradient
    assert scall(lse=DV + 64) == bd.SQUAD_ERR_ALIAS
    assert scall(lse=Y + 16) == bd.SQUAD_ERR_ALIAS
    assert scall(ws=0) == bd.SQUAD_ERR_WORKSPACE
    assert scall(ws_bytes=SWS_BYTES - 1) == bd.SQUAD_ERR_WORKSPACE
    assert scall(y=SWS + 256) == bd.SQUAD_ERR_ALIAS               # y inside the workspace
    assert scall(lse=SWS + SWS_BYTES - 16) == bd.SQUAD_ERR_ALIAS
    assert scall(dq=Q) == bd.SQUAD_ERR_ALIAS                      # the backward's own rules still hold
    # float32 ignores lse (here odd): the call gets as far as the workspace, too small for float32
    assert scall(dtype=bd.SQUAD_F32, lse=3) == bd.SQUAD_ERR_WORKSPACE


def test_padded_workspace_holds_y_for_long_global_passes():
    # grid 1x21x79 padded to 1x21x80, window 1x1x4: 420 windows (27 query tiles) in the global pass,
    # 21 padded tokens; with B*heads*m a multiple of 8 the bf16 workspace also holds Y of the 1659
    # real tokens, after the side buffer rounded up to 256 bytes
    side = 1 * 21 * 2 * 64 * 2
    assert bd.squad_attn_padded_workspace_bytes(1, 2, 1, 21, 79, 1, 1, 4, 64, bd.SQUAD_BF16) == \
        (side + 255) // 256 * 256 + 1659 * 2 * 64 * 2
    assert bd.squad_attn_padded_workspace_bytes(1, 2, 1, 21, 79, 1, 1, 4, 64, bd.SQUAD_F32) == 2 * side
    # B*heads*m = 4: the global pass could not split, so the side buffer alone
    assert bd.squad_attn_padded_workspace_bytes(1, 1, 1, 21, 79, 1, 1, 4, 64, bd.SQUAD_BF16) == side // 2
    # 384 windows (24 tiles) or fewer: the side buffer alone
    assert bd.squad_attn_padded_workspace_bytes(1, 2, 1, 21, 71, 1, 1, 4, 64, bd.SQUAD_BF16) == 1 * 21 * 2 * 64 * 2
