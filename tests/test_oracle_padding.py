"""Pins for the oracle's window rule and reflect padding (CPU only).

The rule is pinned by what the pages state about it (it recovers the trained
21x2x4 window at both native grids; the closed-form cost of the window it picks
matches the printed attention FLOPs); the padding by library reflect padding
(torch), hand-worked tiny grids, a pure-Python brute force over the padded
token set, and the uniform-attention closed form.  Planted mistakes in copies
of the padded oracle must each fail one of these.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import squad_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def golden():
    with open(os.path.join(GOLDEN, "window_rule.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Window rule
# ---------------------------------------------------------------------------

def test_rule_recovers_trained_window_at_native_grids():
    g = golden()["recovers_trained_window"]
    for name, grid in g["grids"].items():
        assert so.solve_window(*grid) == tuple(g["window"]), name


def test_printed_native_flops_match_closed_form_of_solved_window():
    g = golden()
    tol = g["closed_form_rel_tolerance"]
    for p in g["native_points"]:
        T, Hs, Ws = p["grid"]
        win = so.solve_window(T, Hs, Ws)
        f = so.squad_flops_padded(1, p["heads"], T, Hs, Ws, *win, p["d"]) / 1e12
        assert abs(f - p["squad_tflops"]) / p["squad_tflops"] <= tol, (p["backbone"], f)
        full = so.full_attention_flops(1, p["heads"], T * Hs * Ws, p["d"]) / 1e12
        assert abs(full - p["full_tflops"]) / p["full_tflops"] <= 0.004


@pytest.mark.parametrize("grid", [(21, 22, 40), (21, 30, 52), (21, 45, 80), (21, 11, 20), (21, 7, 13),
                                  (13, 60, 104), (1, 5, 7), (1, 1, 9), (3, 64, 64), (21, 90, 160)])
def test_rule_constraints(grid):
    T, Hs, Ws = grid
    wt, wh, ww = so.solve_window(T, Hs, Ws)
    assert wt == T                                     # whole temporal extent
    assert 1 <= wh <= Hs and 1 <= ww <= Ws
    _, Hp, Wp = so.padded_grid(T, Hs, Ws, wt, wh, ww)
    assert Hp % wh == 0 and Wp % ww == 0 and Hp - Hs < wh and Wp - Ws < ww
    # a neighbour of the continuous optimum: each extent within one of it
    area = math.sqrt(T * Hs * Ws) / T
    assert abs(wh - math.sqrt(area * Hs / Ws)) < 1 or wh in (1, Hs)
    assert abs(ww - math.sqrt(area * Ws / Hs)) < 1 or ww in (1, Ws)
    # never worse than rounding both extents to nearest
    def cost(wh_, ww_):
        m = T * wh_ * ww_
        n_p = T * (-(-Hs // wh_) * wh_) * (-(-Ws // ww_) * ww_)
        return n_p * m + n_p * n_p / m
    rh = min(max(round(math.sqrt(area * Hs / Ws)), 1), Hs)
    rw = min(max(round(math.sqrt(area * Ws / Hs)), 1), Ws)
    assert cost(wh, ww) <= cost(rh, rw) * (1 + 1e-12)


def test_rule_closed_form_never_below_the_optimum():
    # AM-GM: n m + n^2/m >= 2 n^1.5, and padding only adds tokens
    for Hs in range(1, 40, 3):
        for Ws in range(1, 60, 5):
            T = 21
            win = so.solve_window(T, Hs, Ws)
            n = T * Hs * Ws
            f = so.squad_flops_padded(1, 1, T, Hs, Ws, *win, 1)
            assert f >= 8 * n ** 1.5 * (1 - 1e-12)


# ---------------------------------------------------------------------------
# Reflect padding
# ---------------------------------------------------------------------------

def test_reflect_pad_by_hand():
    # one row a b c extended to 5: a b c b a; one column likewise; a 2x2 grid to 3x3
    row = np.array([[1.0], [2.0], [3.0]])
    assert so.reflect_pad_tokens(row, 1, 1, 3, 1, 5)[:, 0].tolist() == [1, 2, 3, 2, 1]
    assert so.reflect_pad_tokens(row, 1, 3, 1, 5, 1)[:, 0].tolist() == [1, 2, 3, 2, 1]
    sq = np.array([[1.0], [2.0], [3.0], [4.0]])      # [[1, 2], [3, 4]]
    assert so.reflect_pad_tokens(sq, 1, 2, 2, 3, 3)[:, 0].tolist() == [1, 2, 1, 3, 4, 3, 1, 2, 1]


@pytest.mark.parametrize("shape", [(2, 5, 7, 3, 9, 12), (3, 4, 4, 3, 6, 6), (1, 9, 2, 3, 9, 3)])
def test_reflect_pad_matches_library(shape):
    T, Hs, Ws, d, Hp, Wp = shape
    x = rand((T * Hs * Ws, d), 7)
    got = so.reflect_pad_tokens(x, T, Hs, Ws, Hp, Wp)
    g = torch.from_numpy(x.reshape(T, Hs, Ws, d)).permute(0, 3, 1, 2)           # [T, d, Hs, Ws]
    ref = torch.nn.functional.pad(g, (0, Wp - Ws, 0, Hp - Hs), mode="reflect")
    ref = ref.permute(0, 2, 3, 1).reshape(T * Hp * Wp, d).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(so.crop_tokens(got, T, Hp, Wp, Hs, Ws), x)


# ---------------------------------------------------------------------------
# Padded SQuad, parametrised by the implementation so mutants can be fed in
# ---------------------------------------------------------------------------

def brute_force_padded(q, k, v, T, Hs, Ws, wt, wh, ww):
    """Pure Python: the padded token set as coordinates with their mirrored
    sources, the two softmax passes by loops over token pairs, real tokens out."""
    Hp, Wp = -(-Hs // wh) * wh, -(-Ws // ww) * ww
    mirror = lambda i, size: i if i < size else 2 * size - 2 - i
    pts = [(t, y, x) for t in range(T) for y in range(Hp) for x in range(Wp)]
    src = [(t * Hs + mirror(y, Hs)) * Ws + mirror(x, Ws) for (t, y, x) in pts]
    d = len(q[0])
    win = lambda p: (p[0] // wt, p[1] // wh, p[2] // ww)
    slot = lambda p: (p[0] % wt, p[1] % wh, p[2] % ww)

    def attend(group_of, vals):
        out = []
        for a in range(len(pts)):
            keys = [b for b in range(len(pts)) if group_of(pts[b]) == group_of(pts[a])]
            s = {b: sum(q[src[a]][e] * k[src[b]][e] for e in range(d)) / math.sqrt(d) for b in keys}
            mx = max(s.values())
            ex = {b: math.exp(s[b] - mx) for b in keys}
            tot = sum(ex.values())
            out.append([sum(ex[b] * vals[b][e] for b in keys) / tot for e in range(len(vals[0]))])
        return out

    y = attend(win, [v[s] for s in src])
    o = attend(slot, y)
    keep = [i for i, (t, yy, xx) in enumerate(pts) if yy < Hs and xx < Ws]
    return np.array([o[i] for i in keep])


PADDED_GEOS = [(2, 3, 5, 2, 2, 2), (1, 5, 7, 1, 3, 2), (2, 4, 3, 1, 3, 2)]


def check_padded_brute_force(impl, geo=PADDED_GEOS[0], d=4, seed=21):
    T, Hs, Ws, wt, wh, ww = geo
    n = T * Hs * Ws
    q, k, v = rand((n, d), seed), rand((n, d), seed + 1), rand((n, d), seed + 2)
    ref = brute_force_padded(q.tolist(), k.tolist(), v.tolist(), *geo)
    return np.max(np.abs(impl(q, k, v, (T, Hs, Ws), (wt, wh, ww)) - ref)) < 1e-12


def check_padded_uniform(impl, geo=(2, 5, 7, 2, 3, 4), d=3, seed=31):
    # Q = 0: both passes average uniformly, so every real token receives the
    # mean of V over the padded grid, where a real token counts once per mirror
    # image of it (counted here with library reflect padding of an index grid)
    T, Hs, Ws, wt, wh, ww = geo
    Hp, Wp = -(-Hs // wh) * wh, -(-Ws // ww) * ww
    n = T * Hs * Ws
    idx = torch.arange(Hs * Ws, dtype=torch.float64).reshape(1, 1, Hs, Ws)
    img = torch.nn.functional.pad(idx, (0, Wp - Ws, 0, Hp - Hs), mode="reflect").reshape(-1).long()
    mult = torch.bincount(img, minlength=Hs * Ws).double().numpy()
    k, v = rand((n, d), seed), rand((n, d), seed + 1)
    vg = v.reshape(T, Hs * Ws, d)
    expect = (mult[None, :, None] * vg).sum(axis=(0, 1)) / (T * Hp * Wp)
    got = impl(np.zeros((n, d)), k, v, (T, Hs, Ws), (wt, wh, ww))
    return np.max(np.abs(got - expect)) < 1e-12


def check_padded_tiling_reduces(impl, seed=41):
    # a window that tiles the grid: no padding, identical to the plain operator
    T, Hs, Ws, wt, wh, ww, d = 3, 4, 6, 3, 2, 3, 5
    n = T * Hs * Ws
    q, k, v = rand((n, d), seed), rand((n, d), seed + 1), rand((n, d), seed + 2)
    ref = so.squad_head(q, k, v, so.window_slot_table(T, Hs, Ws, wt, wh, ww))
    return np.array_equal(impl(q, k, v, (T, Hs, Ws), (wt, wh, ww)), ref)


PADDED_CHECKS = [check_padded_brute_force, check_padded_uniform, check_padded_tiling_reduces,
                 lambda impl: check_padded_brute_force(impl, geo=PADDED_GEOS[1], d=3, seed=51),
                 lambda impl: check_padded_brute_force(impl, geo=PADDED_GEOS[2], d=3, seed=61)]


def test_padded_brute_force_pins():
    for geo in PADDED_GEOS:
        assert check_padded_brute_force(so.squad_head_padded, geo=geo)


def test_padded_uniform_attention_closed_form():
    assert check_padded_uniform(so.squad_head_padded)


def test_padded_reduces_to_plain_when_window_tiles():
    assert check_padded_tiling_reduces(so.squad_head_padded)


def test_padded_whole_tensor_wrapper():
    B, heads, T, Hs, Ws, d = 2, 3, 2, 5, 7, 4
    win = (2, 3, 2)
    n = T * Hs * Ws
    q, k, v = rand((B, n, heads, d), 1), rand((B, n, heads, d), 2), rand((B, n, heads, d), 3)
    out = so.squad_attention_padded(q, k, v, (B, heads, T, Hs, Ws, *win, d))
    for b in range(B):
        for h in range(heads):
            ref = so.squad_head_padded(q[b, :, h], k[b, :, h], v[b, :, h], (T, Hs, Ws), win)
            assert np.array_equal(out[b, :, h], ref)


# planted mistakes in copies of the padded oracle

def _pad_with(mode, front=False):
    def impl(q, k, v, grid, window):
        T, Hs, Ws = grid
        _, Hp, Wp = so.padded_grid(T, Hs, Ws, *window)
        tab = so.window_slot_table(T, Hp, Wp, *window)

        def pad(a):
            g = a.reshape(T, Hs, Ws, -1)
            w = [(0, 0), (Hp - Hs, 0) if front else (0, Hp - Hs), (Wp - Ws, 0) if front else (0, Wp - Ws), (0, 0)]
            return np.pad(g, w, mode=mode).reshape(T * Hp * Wp, -1)

        o = so.squad_head(pad(q), pad(k), pad(v), tab).reshape(T, Hp, Wp, -1)
        o = o[:, Hp - Hs:, Ws - Ws + (Wp - Ws):] if front else o[:, :Hs, :Ws]
        return o.reshape(T * Hs * Ws, -1)
    return impl


def _mut_edge_repeated(q, k, v, grid, window):
    return _pad_with("symmetric")(q, k, v, grid, window)


def _mut_padded_at_front(q, k, v, grid, window):
    return _pad_with("reflect", front=True)(q, k, v, grid, window)


def _mut_zero_padding(q, k, v, grid, window):
    return _pad_with("constant")(q, k, v, grid, window)


def _mut_pad_values_only(q, k, v, grid, window):
    # queries and keys of padded tokens taken from the wrong source (edge copies)
    T, Hs, Ws = grid
    _, Hp, Wp = so.padded_grid(T, Hs, Ws, *window)
    tab = so.window_slot_table(T, Hp, Wp, *window)
    edge = lambda a: np.pad(a.reshape(T, Hs, Ws, -1), [(0, 0), (0, Hp - Hs), (0, Wp - Ws), (0, 0)],
                            mode="edge").reshape(T * Hp * Wp, -1)
    refl = lambda a: so.reflect_pad_tokens(a, T, Hs, Ws, Hp, Wp)
    return so.crop_tokens(so.squad_head(edge(q), edge(k), refl(v), tab), T, Hp, Wp, Hs, Ws)


def _mut_padded_tokens_masked(q, k, v, grid, window):
    # padded tokens dropped as keys (a mask instead of padding): only real keys
    T, Hs, Ws = grid
    _, Hp, Wp = so.padded_grid(T, Hs, Ws, *window)
    tab = so.window_slot_table(T, Hp, Wp, *window)
    real = so.crop_tokens(np.arange(T * Hp * Wp), T, Hp, Wp, Hs, Ws)
    is_real = np.zeros(T * Hp * Wp, bool)
    is_real[real] = True
    pad = lambda a: so.reflect_pad_tokens(a, T, Hs, Ws, Hp, Wp)
    qp, kp, vp = pad(q), pad(k), pad(v)

    def masked(qq, kk, vv, rows_tab):
        out = np.zeros_like(vv)
        for rows in rows_tab:
            keys = rows[is_real[rows]]
            s = qq[rows] @ kk[keys].T / math.sqrt(qq.shape[1])
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[rows] = (p / p.sum(axis=1, keepdims=True)) @ vv[keys]
        return out
    y = masked(qp, kp, vp, tab)
    o = masked(qp, kp, y, tab.T)
    return so.crop_tokens(o, T, Hp, Wp, Hs, Ws)


@pytest.mark.parametrize("mutant", [_mut_edge_repeated, _mut_padded_at_front, _mut_zero_padding,
                                    _mut_pad_values_only, _mut_padded_tokens_masked])
def test_padding_pins_catch_planted_mistakes(mutant):
    assert all(chk(so.squad_head_padded) for chk in PADDED_CHECKS)
    assert not all(chk(mutant) for chk in PADDED_CHECKS), mutant.__name__
