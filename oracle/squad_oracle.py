"""fp64 CPU oracle for SQuad-Attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  The HIP library never calls it, and it shares no code
with the HIP path (it does not import the package; inputs arrive as arrays).

What is computed (SQuad: Sub-Quadratic Attention Distillation for Efficient
Video Generation):

* The operator composes two plain softmax attentions run one after the other,
  with only re-indexing in between, every position along the axis a pass does
  not attend over acting as one more head (agihunt.info summary, method paragraph; paperpeel full
  text, sec. 3.2 and appendix E "Cost of the two passes").
* Local pass: tokens mix within fixed windows of about sqrt(n) tokens, cut from
  the latent grid and spanning the whole temporal extent (agihunt.info summary;
  paperpeel full text, sec. 1, last paragraph).
* Global pass: tokens at the same position inside each window mix across all
  windows (paperpeel full text, sec. 1; appendix "Reachability").  The local
  output feeds the value stream of the global pass (gist.science explainer,
  "Operador de Atencao SQuad").  Since nothing but re-indexing sits between the
  passes and no parameters are added, the global pass takes the same Q and K
  re-indexed.
* Each attention is the plain softmax(Q K^T / sqrt(d)) V (paperpeel full text,
  sec. 1), non-causal, every query attending to its own key too.

Readings where the pages are silent (listed again in the design notes):
  token order inside the grid is (t, y, x) row-major; windows are aligned,
  non-overlapping tiles anchored at the origin; the slot of a token is its
  in-window offset (t % wt, y % wh, x % ww); the scale is 1/sqrt(d) in both
  passes.

Every function is pinned by tests/test_oracle.py against closed forms, library
attention, brute force over token pairs and the FLOP counts the pages print.
"""

from __future__ import annotations

import math
import numpy as np


# ---------------------------------------------------------------------------
# Re-indexing: window c and slot j of every token
# ---------------------------------------------------------------------------

def window_slot_table(T, Hs, Ws, wt, wh, ww):
    """Token index of (window c, slot j) as an int64 array of shape [N_w, m].

    Windows are the aligned (wt, wh, ww) tiles of the (T, Hs, Ws) grid, numbered
    in (t, y, x) row-major order of their tile coordinates; the slot is the
    token's offset inside its window, numbered the same way.  Token (t, y, x)
    has index (t * Hs + y) * Ws + x.
    """
    if T % wt or Hs % wh or Ws % ww:
        raise ValueError("window must tile the grid")
    Ct, Cy, Cx = T // wt, Hs // wh, Ws // ww
    table = np.empty((Ct * Cy * Cx, wt * wh * ww), dtype=np.int64)
    for ct in range(Ct):
        for cy in range(Cy):
            for cx in range(Cx):
                c = (ct * Cy + cy) * Cx + cx
                for jt in range(wt):
                    for jy in range(wh):
                        for jx in range(ww):
                            j = (jt * wh + jy) * ww + jx
                            t, y, x = ct * wt + jt, cy * wh + jy, cx * ww + jx
                            table[c, j] = (t * Hs + y) * Ws + x
    return table


# ---------------------------------------------------------------------------
# One plain softmax attention
# ---------------------------------------------------------------------------

def softmax_attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v over the last two axes, in float64.

    q, k: [..., L, d]; v: [..., L, dv].  The row maximum is subtracted before
    exponentiating, which leaves the softmax unchanged.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.matmul(p, v)


# ---------------------------------------------------------------------------
# The two passes on one (batch, head) slice: arrays [n, d]
# ---------------------------------------------------------------------------

def local_pass_head(q, k, v, table):
    """Attn_L: every window attends within itself.  q, k, v: [n, d] -> [n, d]."""
    out = np.empty(np.shape(v), dtype=np.float64)
    # gather [N_w, m, d]: the slots of a window form the sequence and each
    # window is an independent attention (a batch entry)
    out[table] = softmax_attention(q[table], k[table], v[table])
    return out


def global_pass_head(q, k, v, table):
    """Attn_G: tokens sharing a slot attend across all windows.  [n, d] -> [n, d]."""
    cols = table.T  # [m, N_w]: the attended axis (windows) becomes the sequence
    out = np.empty(np.shape(v), dtype=np.float64)
    out[cols] = softmax_attention(q[cols], k[cols], v[cols])
    return out


def squad_head(q, k, v, table):
    """Local pass, then global pass with the same q, k and the local output as values."""
    y = local_pass_head(q, k, v, table)
    return global_pass_head(q, k, y, table)


def squad_reversed_head(q, k, v, table):
    """The other order (global first, then local), as in the ordering ablation."""
    y = global_pass_head(q, k, v, table)
    return local_pass_head(q, k, y, table)


# ---------------------------------------------------------------------------
# Whole tensors in [B, n, heads, d] layout
# ---------------------------------------------------------------------------

def _per_head(fn, q, k, v, geom):
    B, heads, T, Hs, Ws, wt, wh, ww, d = geom
    table = window_slot_table(T, Hs, Ws, wt, wh, ww)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            out[b, :, h, :] = fn(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], table)
    return out


def squad_attention(q, k, v, geom):
    """O = Attn_G(Q, K, Attn_L(Q, K, V)) for [B, n, heads, d] inputs; geom =
    (B, heads, T, Hs, Ws, wt, wh, ww, d)."""
    return _per_head(squad_head, q, k, v, geom)


def local_pass(q, k, v, geom):
    return _per_head(local_pass_head, q, k, v, geom)


def global_pass(q, k, v, geom):
    return _per_head(global_pass_head, q, k, v, geom)


def squad_attention_reversed(q, k, v, geom):
    return _per_head(squad_reversed_head, q, k, v, geom)


# ---------------------------------------------------------------------------
# Dense n x n form (tiny n only): masks and the effective weight matrix
# ---------------------------------------------------------------------------

def token_coords(T, Hs, Ws):
    """(t, y, x) of every token index, [n, 3]."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hs), np.arange(Ws), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)


def dense_masks(T, Hs, Ws, wt, wh, ww):
    """Boolean [n, n] masks: same window (local pass) and same slot (global pass).

    Built from grid coordinates alone (no window/slot table), as an independent
    formulation of the two index sets.
    """
    c = token_coords(T, Hs, Ws)
    w = np.array([wt, wh, ww])
    win = c // w
    slot = c % w
    same_window = np.all(win[:, None, :] == win[None, :, :], axis=-1)
    same_slot = np.all(slot[:, None, :] == slot[None, :, :], axis=-1)
    return same_window, same_slot


def masked_softmax_weights(q, k, mask):
    """Row-stochastic [n, n] matrix softmax over the allowed keys of q k^T / sqrt(d)."""
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) / math.sqrt(q.shape[-1])
    s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.where(mask, np.exp(s), 0.0)
    return p / p.sum(axis=1, keepdims=True)


def effective_weights(q, k, T, Hs, Ws, wt, wh, ww):
    """(A_L, A_G, W) for one head: the local weights (beta), the global weights
    (alpha) and the effective weight W = A_G A_L, whose entry for target (c, j)
    and source (c', j') is alpha^j_{c->c'} beta^{c'}_{j->j'} (paperpeel full
    text, appendix "Unrolling the composition" / "Reachability")."""
    same_window, same_slot = dense_masks(T, Hs, Ws, wt, wh, ww)
    a_local = masked_softmax_weights(q, k, same_window)
    a_global = masked_softmax_weights(q, k, same_slot)
    return a_local, a_global, a_global @ a_local


# ---------------------------------------------------------------------------
# FLOP count of the two passes
# ---------------------------------------------------------------------------

def squad_flops(B, heads, T, Hs, Ws, wt, wh, ww, d):
    """FLOPs of the operator counting 2 per multiply-add in the two matmuls of
    each softmax attention (scores and weighted sum), nothing else.

    The local pass runs B*heads*N_w attentions of length m, the global pass
    B*heads*m attentions of length N_w; one attention of length L costs
    2 * (L*L*d) * 2 FLOPs.
    """
    n = T * Hs * Ws
    m = wt * wh * ww
    n_w = n // m
    local = B * heads * n_w * (2 * 2 * m * m * d)
    glob = B * heads * m * (2 * 2 * n_w * n_w * d)
    return local + glob


def full_attention_flops(B, heads, n, d):
    """FLOPs of one full softmax attention over n tokens, same counting rule."""
    return B * heads * 2 * 2 * n * n * d


# ---------------------------------------------------------------------------
# Window rule and reflect padding (grids a window does not tile)
# ---------------------------------------------------------------------------
#
# SQuad paper appendix, "What is measured" and "Conformance to the theoretical
# curves is quantitative": the window is chosen afresh for every latent grid so
# that its volume m follows sqrt(n); it always spans the whole temporal extent
# (wt = T) and its spatial extents keep the grid's aspect ratio; m must be a
# whole number of tokens, and where the window does not divide the grid the grid
# is extended with mirror images.  The pages print no formula beyond this.
# Reading taken: the continuous optimum has wt = T, wh * ww = sqrt(n) / T and
# wh : ww = Hs : Ws; each spatial extent is rounded down or up (kept within
# 1..extent), and of those (at most four) windows the one with the least
# closed-form cost 4hd(n_p m + n_p^2 / m) on its padded grid (n_p tokens) wins;
# ties go to the aspect ratio closer to the grid's, then to the smaller window.
# This recovers the trained 21 x 2 x 4 window at both native grids (21 x 22 x 40
# and 21 x 30 x 52), as the pages state.

def padded_extent(size, w):
    """Smallest multiple of w that is >= size."""
    return -(-size // w) * w


def solve_window(T, Hs, Ws):
    """(wt, wh, ww) for the grid (T, Hs, Ws) under the rule above."""
    from fractions import Fraction
    n = T * Hs * Ws
    area = math.sqrt(n) / T
    wh_c = math.sqrt(area * Hs / Ws)
    ww_c = math.sqrt(area * Ws / Hs)
    cands = set()
    for wh in (math.floor(wh_c), math.ceil(wh_c)):
        for ww in (math.floor(ww_c), math.ceil(ww_c)):
            cands.add((min(max(wh, 1), Hs), min(max(ww, 1), Ws)))

    def key(c):
        wh, ww = c
        m = T * wh * ww
        n_p = T * padded_extent(Hs, wh) * padded_extent(Ws, ww)
        cost = Fraction(n_p * m * m + n_p * n_p, m)       # n_p m + n_p^2 / m, exactly
        a, b = wh * Ws, ww * Hs                            # wh/ww against Hs/Ws
        aspect = Fraction(max(a, b), min(a, b))
        return (cost, aspect, m, wh)

    wh, ww = min(cands, key=key)
    return T, wh, ww


def reflect_pad_tokens(x, T, Hs, Ws, Hp, Wp):
    """[n, ...] in (t, y, x) order -> [T*Hp*Wp, ...]: the grid extended at the
    bottom and right to (T, Hp, Wp) by mirroring (reading: padding at the far
    end only; the time axis is never padded since wt = T)."""
    if Hp - Hs > Hs - 1 or Wp - Ws > Ws - 1:
        raise ValueError("reflect padding must be shorter than the axis")
    g = np.asarray(x).reshape((T, Hs, Ws) + np.shape(x)[1:])
    widths = [(0, 0), (0, Hp - Hs), (0, Wp - Ws)] + [(0, 0)] * (g.ndim - 3)
    return np.pad(g, widths, mode="reflect").reshape((T * Hp * Wp,) + np.shape(x)[1:])


def crop_tokens(x, T, Hp, Wp, Hs, Ws):
    """Inverse of the padding's layout change: the (T, Hs, Ws) tokens of a
    (T, Hp, Wp) token array, in (t, y, x) order."""
    g = np.asarray(x).reshape((T, Hp, Wp) + np.shape(x)[1:])
    return g[:, :Hs, :Ws].reshape((T * Hs * Ws,) + np.shape(x)[1:])


def padded_grid(T, Hs, Ws, wt, wh, ww):
    if T % wt:
        raise ValueError("the window must span whole frames (T % wt == 0)")
    return T, padded_extent(Hs, wh), padded_extent(Ws, ww)


def squad_head_padded(q, k, v, grid, window):
    """SQuad on a grid the window need not tile: reflect-pad Q, K and V, run
    both passes on the padded grid (padded tokens are ordinary keys, values and
    queries there), keep the outputs of the real tokens.  [n, d] -> [n, d]."""
    T, Hs, Ws = grid
    _, Hp, Wp = padded_grid(T, Hs, Ws, *window)
    table = window_slot_table(T, Hp, Wp, *window)
    qp, kp, vp = (reflect_pad_tokens(a, T, Hs, Ws, Hp, Wp) for a in (q, k, v))
    return crop_tokens(squad_head(qp, kp, vp, table), T, Hp, Wp, Hs, Ws)


def squad_attention_padded(q, k, v, geom):
    """squad_attention for any window with wt | T; geom = (B, heads, T, Hs, Ws,
    wt, wh, ww, d)."""
    B, heads, T, Hs, Ws, wt, wh, ww, d = geom
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            out[b, :, h, :] = squad_head_padded(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :],
                                                (T, Hs, Ws), (wt, wh, ww))
    return out


def squad_flops_padded(B, heads, T, Hs, Ws, wt, wh, ww, d):
    """FLOPs of the operator on the padded grid (the work actually done)."""
    _, Hp, Wp = padded_grid(T, Hs, Ws, wt, wh, ww)
    return squad_flops(B, heads, T, Hp, Wp, wt, wh, ww, d)



# ---------------------------------------------------------------------------
# Gradients (the backward pass)
# ---------------------------------------------------------------------------
#
# The pages train through the operator (flow-matching fine-tuning and DMD2
# distillation, SQuad paper sec. 3.3 and sec. 4), so it must be differentiated;
# they print no backward.  What follows is the chain rule applied to the two
# softmax attentions as defined above, nothing else: for one attention
# O = P V with P = softmax(S) and S = Q K^T / sqrt(d), and an upstream
# gradient dO,
#     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
#     dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
# (rowsum(P * dP) = rowsum(dO * O) is the softmax Jacobian's correction).
# SQuad: O = Attn_G(Q, K, Y) with Y = Attn_L(Q, K, V); the global pass's value
# gradient is the local pass's upstream gradient, and Q and K collect
# contributions from both passes.

def softmax_attention_backward(q, k, v, do):
    """(dq, dk, dv) of softmax(q k^T / sqrt(d)) v over the last two axes, float64."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    d = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) / math.sqrt(d)
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) / math.sqrt(d)
    return dq, dk, dv


def _pass_backward(q, k, vals, dout, rows):
    """Backward of one pass whose problems are the rows of the index table
    `rows` ([problems, L] token indices): gradients in token order."""
    dq, dk, dvals = softmax_attention_backward(q[rows], k[rows], vals[rows], dout[rows])
    gq, gk, gv = (np.empty(np.shape(q), dtype=np.float64) for _ in range(3))
    gq[rows], gk[rows], gv[rows] = dq, dk, dvals
    return gq, gk, gv


def squad_backward_head(q, k, v, do, table):
    """(dQ, dK, dV) of O = Attn_G(Q, K, Attn_L(Q, K, V)) for one head, given
    dO; [n, d] each.  The local output Y is recomputed."""
    y = local_pass_head(q, k, v, table)
    dq_g, dk_g, dy = _pass_backward(q, k, y, do, np.ascontiguousarray(table.T))
    dq_l, dk_l, dv = _pass_backward(q, k, v, dy, table)
    return dq_l + dq_g, dk_l + dk_g, dv


def squad_backward(q, k, v, do, geom):
    """Whole-tensor gradients for [B, n, heads, d] inputs; geom as squad_attention."""
    B, heads, T, Hs, Ws, wt, wh, ww, d = geom
    table = window_slot_table(T, Hs, Ws, wt, wh, ww)
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    out = [np.empty(q.shape, dtype=np.float64) for _ in range(3)]
    for b in range(B):
        for h in range(heads):
            g = squad_backward_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], table)
            for o, gi in zip(out, g):
                o[b, :, h] = gi
    return tuple(out)


def squad_backward_flops(B, heads, T, Hs, Ws, wt, wh, ww, d):
    """FLOPs of the gradients counted like the forward's (2 per multiply-add
    of each matmul): per attention of length L the scores S and the four
    products dP, dV, dQ, dK, five L x L x d products against the forward's
    two, so 2.5 times squad_flops (recomputing the local output, which the
    forward does not keep, is not counted here)."""
    return 5 * squad_flops(B, heads, T, Hs, Ws, wt, wh, ww, d) // 2
