"""Pins for the oracle's gradients (CPU only).

The gradients are pinned by automatic differentiation in torch (float64)
through a forward built from torch's own scaled-dot-product attention with
boolean masks (an implementation that shares nothing with the oracle's
re-indexed formulas), central finite differences, and closed forms the chain
rule must satisfy: dV = W^T dO for the effective weight W, keys' gradients
summing to zero over every attention, and a single window reducing to library
attention's gradient.  Planted mistakes in copies of the backward must each
fail one of these.
"""

import math

import numpy as np
import pytest
import torch

from oracle import squad_oracle as so

GEOS = [(3, 4, 4, 3, 2, 2), (2, 3, 4, 1, 3, 2), (2, 4, 6, 2, 2, 3)]


def rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


def inputs(geo, d, seed):
    n = geo[0] * geo[1] * geo[2]
    return [rand((n, d), seed + i) for i in range(4)]


def torch_grads(q, k, v, do, geo):
    """Autograd of Attn_G(Q, K, Attn_L(Q, K, V)) with torch SDPA and masks."""
    same_window, same_slot = so.dense_masks(*geo)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    sdpa = torch.nn.functional.scaled_dot_product_attention
    mw, ms = torch.from_numpy(same_window), torch.from_numpy(same_slot)
    y = sdpa(tq[None], tk[None], tv[None], attn_mask=mw)[0]
    o = sdpa(tq[None], tk[None], y[None], attn_mask=ms)[0]
    o.backward(torch.from_numpy(np.asarray(do, dtype=np.float64)))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# checks parametrised by the per-head backward so mutants can be fed in

def check_autograd(impl, geo=GEOS[0], d=8, seed=1):
    q, k, v, do = inputs(geo, d, seed)
    got = impl(q, k, v, do, so.window_slot_table(*geo))
    ref = torch_grads(q, k, v, do, geo)
    return all(np.max(np.abs(g - r)) < 1e-12 for g, r in zip(got, ref))


def check_finite_differences(impl, geo=GEOS[1], d=4, seed=11):
    q, k, v, do = inputs(geo, d, seed)
    table = so.window_slot_table(*geo)
    grads = impl(q, k, v, do, table)
    loss = lambda q_, k_, v_: float(np.sum(so.squad_head(q_, k_, v_, table) * do))
    h = 1e-6
    g = np.random.Generator(np.random.PCG64(seed))
    for which in range(3):
        for _ in range(6):
            i, e = int(g.integers(len(q))), int(g.integers(d))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][i, e] += h
            up = loss(*args)
            args[which][i, e] -= 2 * h
            down = loss(*args)
            if abs((up - down) / (2 * h) - grads[which][i, e]) > 1e-7:
                return False
    return True


def check_dv_is_effective_weight_transpose(impl, geo=GEOS[2], d=5, seed=21):
    q, k, v, do = inputs(geo, d, seed)
    _, _, W = so.effective_weights(q, k, *geo)
    return np.max(np.abs(impl(q, k, v, do, so.window_slot_table(*geo))[2] - W.T @ do)) < 1e-12


def check_key_gradients_sum_to_zero(impl, geo=GEOS[0], d=6, seed=31):
    # every attention's dS rows sum to zero, so its keys' gradients do; summed
    # over all windows and all slots the keys' total is zero per head
    q, k, v, do = inputs(geo, d, seed)
    dk = impl(q, k, v, do, so.window_slot_table(*geo))[1]
    return np.max(np.abs(dk.sum(axis=0))) < 1e-12


def check_single_window(impl, seed=41):
    # one window = the grid: the global pass is the identity, the gradient is
    # library attention's (torch autograd through unmasked SDPA)
    T, Hs, Ws, d = 2, 3, 4, 8
    q, k, v, do = inputs((T, Hs, Ws), d, seed)
    got = impl(q, k, v, do, so.window_slot_table(T, Hs, Ws, T, Hs, Ws))
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0].backward(
        torch.from_numpy(do))
    return all(np.max(np.abs(g - r.grad.numpy())) < 1e-12 for g, r in zip(got, (tq, tk, tv)))


ALL = [check_autograd, check_finite_differences, check_dv_is_effective_weight_transpose,
       check_key_gradients_sum_to_zero, check_single_window,
       lambda impl: check_autograd(impl, geo=GEOS[1], d=3, seed=51),
       lambda impl: check_autograd(impl, geo=GEOS[2], d=5, seed=61)]


@pytest.mark.parametrize("chk", ALL)
def test_backward_pin(chk):
    assert chk(so.squad_backward_head)


def test_whole_tensor_backward():
    B, heads, T, Hs, Ws, wt, wh, ww, d = 2, 3, 2, 4, 6, 2, 2, 3, 4
    n = T * Hs * Ws
    q, k, v, do = (rand((B, n, heads, d), s) for s in range(4))
    got = so.squad_backward(q, k, v, do, (B, heads, T, Hs, Ws, wt, wh, ww, d))
    table = so.window_slot_table(T, Hs, Ws, wt, wh, ww)
    for b in range(B):
        for h in range(heads):
            ref = so.squad_backward_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], table)
            for g, r in zip(got, ref):
                assert np.array_equal(g[b, :, h], r)


def test_value_gradient_totals():
    # each pass's weights are row-stochastic, so summed over tokens dV equals dO
    q, k, v, do = inputs(GEOS[0], 7, 71)
    dv = so.squad_backward_head(q, k, v, do, so.window_slot_table(*GEOS[0]))[2]
    assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) < 1e-12


class _CountingNumpy:
    """Stands in for numpy inside the oracle module: every np.matmul the oracle
    executes adds 2 FLOPs per multiply-add of the product it actually formed
    (each output element sums a.shape[-1] products), whatever its batch shape."""

    def __init__(self):
        self.flops = 0

    def __getattr__(self, name):
        return getattr(np, name)

    def matmul(self, a, b):
        a, b = np.asarray(a), np.asarray(b)
        out = np.matmul(a, b)
        self.flops += 2 * out.size * a.shape[-1]
        return out


COUNT_GEOS = [(2, 3, 3, 4, 4, 3, 2, 2, 8), (1, 2, 2, 6, 8, 1, 3, 4, 5), (1, 1, 4, 2, 6, 2, 1, 3, 3)]


def counted_flops(monkeypatch, geo, seed=5):
    """(forward, backward) FLOPs counted from the products the oracle runs: the
    forward, and the backward less the local pass it recomputes (the forward
    does not keep Y, and the backward's count leaves that recompute out)."""
    B, heads, T, Hs, Ws = geo[:5]
    d = geo[-1]
    q, k, v, do = (rand((B, T * Hs * Ws, heads, d), seed + i) for i in range(4))
    counter = _CountingNumpy()
    monkeypatch.setattr(so, "np", counter)
    so.squad_attention(q, k, v, geo)
    fwd = counter.flops
    counter.flops = 0
    so.squad_backward(q, k, v, do, geo)
    bwd_total = counter.flops
    counter.flops = 0
    so.local_pass(q, k, v, geo)
    recompute = counter.flops
    monkeypatch.undo()
    return fwd, bwd_total - recompute


def check_flop_counts(monkeypatch, fwd_fn, bwd_fn):
    for geo in COUNT_GEOS:
        fwd, bwd = counted_flops(monkeypatch, geo)
        if fwd != fwd_fn(*geo) or bwd != bwd_fn(*geo):
            return False
    return True


def test_flop_counts_match_the_products_executed(monkeypatch):
    # the closed forms against the matmuls the oracle's two passes and their
    # gradients actually run (five L x L x d products per attention in the
    # backward, two in the forward), on three small geometries
    assert check_flop_counts(monkeypatch, so.squad_flops, so.squad_backward_flops)
    # and at the headline shape, the ratio the count implies
    assert so.squad_backward_flops(1, 24, 21, 22, 40, 21, 2, 4, 128) == 5 * 63_128_862_720 // 2


@pytest.mark.parametrize("factor", [2, 3, 4])
def test_flop_count_pin_catches_planted_miscounts(monkeypatch, factor):
    # a backward counted as 2F, 3F or 4F instead of 2.5F (F the forward's
    # count: e.g. the score recompute forgotten, the recompute of Y included,
    # or one product too many) must fail the pin
    mutant = lambda *geo: factor * so.squad_flops(*geo)
    assert not check_flop_counts(monkeypatch, so.squad_flops, mutant)


# planted mistakes in copies of the backward

def _bwd_with(attn_bwd, chain="y"):
    def impl(q, k, v, do, table):
        y = so.local_pass_head(q, k, v, table)
        vals = {"y": y, "v": v}[chain]

        def run(qq, kk, vv, dd, rows):
            dq, dk, dvv = attn_bwd(qq[rows], kk[rows], vv[rows], dd[rows])
            out = [np.empty(np.shape(qq)) for _ in range(3)]
            out[0][rows], out[1][rows], out[2][rows] = dq, dk, dvv
            return out
        dq_g, dk_g, dy = run(q, k, vals, do, np.ascontiguousarray(table.T))
        dq_l, dk_l, dv = run(q, k, v, dy, table)
        return dq_l + dq_g, dk_l + dk_g, dv
    return impl


def _attn_bwd_mut(kind):
    def f(q, k, v, do):
        d = q.shape[-1]
        s = q @ np.swapaxes(k, -1, -2) / math.sqrt(d)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        p = p / p.sum(axis=-1, keepdims=True)
        dv = np.swapaxes(p, -1, -2) @ do
        dp = do @ np.swapaxes(v, -1, -2)
        ds = p * dp if kind == "no_jacobian_correction" else p * (dp - (p * dp).sum(axis=-1, keepdims=True))
        sc = 1.0 if kind == "no_scale" else 1 / math.sqrt(d)
        dq = ds @ k * sc
        dk = np.swapaxes(ds, -1, -2) @ q * sc
        if kind == "swapped_qk":
            dq, dk = dk, dq
        if kind == "transposed_p":
            dv = p @ do
        return dq, dk, dv
    return f


def _mut_global_values_are_v(q, k, v, do, table):
    return _bwd_with(so.softmax_attention_backward, chain="v")(q, k, v, do, table)


def _mut_no_global_chain(q, k, v, do, table):
    # local backward fed dO directly instead of the global pass's value gradient
    y = so.local_pass_head(q, k, v, table)
    dq_g, dk_g, _ = so._pass_backward(q, k, y, do, np.ascontiguousarray(table.T))
    dq_l, dk_l, dv = so._pass_backward(q, k, v, do, table)
    return dq_l + dq_g, dk_l + dk_g, dv


def _mut_local_only_qk(q, k, v, do, table):
    y = so.local_pass_head(q, k, v, table)
    _, _, dy = so._pass_backward(q, k, y, do, np.ascontiguousarray(table.T))
    return so._pass_backward(q, k, v, dy, table)


MUTANTS = [_bwd_with(_attn_bwd_mut(k)) for k in ("no_jacobian_correction", "no_scale", "swapped_qk", "transposed_p")]
MUTANTS += [_mut_global_values_are_v, _mut_no_global_chain, _mut_local_only_qk]


@pytest.mark.parametrize("mutant", MUTANTS)
def test_backward_pins_catch_planted_mistakes(mutant):
    assert not all(chk(mutant) for chk in ALL)
