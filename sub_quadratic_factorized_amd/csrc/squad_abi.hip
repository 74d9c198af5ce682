// Host side of the SQuad-Attention C ABI (declared in include/squad_attn.h):
// argument validation (pure host code, before any HIP call), the pass
// geometry, and the launch sequence of each entry point.
#include "squad_attn.h"
#include "squad_internal.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

namespace squad {

namespace {

thread_local int g_last_hip_error = 0;

enum class Kind { kFwd, kLocal, kGlobal, kReversed };

struct Problem {
    int B, heads, T, Hs, Ws, wt, wh, ww, d, dtype;
    int64_t n, m, nw;
    int64_t elems;  // B*n*heads*d
    size_t bytes;   // elems * sizeof(dtype)
    // padded grids: extents the window tiles, tokens per batch element of the
    // padded grid, and of the side buffer (padded positions only); N_w above
    // then counts the windows of the padded grid
    int Hp = 0, Wp = 0;
    int64_t np = 0, npad = 0;
    // the padded entry point's workspace: the side buffer (B*npad*heads*d in
    // the dtype) and, at ybuf_off when that is not 0, Y of the real tokens
    size_t ws_bytes = 0, ybuf_off = 0;
};

int esize(int dtype) { return dtype == SQUAD_BF16 ? 2 : 4; }

// Shape checks only: SQUAD_OK, SQUAD_ERR_SHAPE (with pr filled on success).
// *empty is set when B == 0 or heads == 0.
squad_status_t check_shape(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d, Problem* pr,
                           bool* empty) {
    *empty = false;
    if (B < 0 || heads < 0) return SQUAD_ERR_SHAPE;
    if (T < 1 || Hs < 1 || Ws < 1 || wt < 1 || wh < 1 || ww < 1 || d < 1) return SQUAD_ERR_SHAPE;
    if (T % wt != 0 || Hs % wh != 0 || Ws % ww != 0) return SQUAD_ERR_SHAPE;
    const int64_t n = (int64_t)T * Hs * Ws;  // < 2^93 is impossible: each factor < 2^31
    if (n >= ((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    const int64_t m = (int64_t)wt * wh * ww;
    const int64_t nw = n / m;
    pr->B = B;
    pr->heads = heads;
    pr->T = T;
    pr->Hs = Hs;
    pr->Ws = Ws;
    pr->wt = wt;
    pr->wh = wh;
    pr->ww = ww;
    pr->d = d;
    pr->n = n;
    pr->m = m;
    pr->nw = nw;
    if (B == 0 || heads == 0) {
        *empty = true;
        pr->elems = 0;
        return SQUAD_OK;
    }
    // element count B*n*heads*d must stay below 2^62, and the token stride
    // heads*d (an int in the kernels) below 2^31
    const long double el = (long double)B * (long double)n * (long double)heads * (long double)d;
    if (el >= (long double)((int64_t)1 << 62)) return SQUAD_ERR_SHAPE;
    if ((int64_t)heads * d >= ((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    pr->elems = (int64_t)B * n * heads * d;
    // every pass launches at most B*heads*max(m, N_w) problems
    const long double probs = (long double)B * heads * (long double)(m > nw ? m : nw);
    if (probs >= (long double)((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    return SQUAD_OK;
}

// Shape checks of the padded entry points: the window must span whole frames
// (T % wt == 0) and be no larger than the grid spatially (mirror padding is
// shorter than the axis it extends); the grid is extended at the bottom and
// right to multiples of wh and ww.  Same outcomes as check_shape otherwise.
squad_status_t check_shape_padded(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d,
                                  Problem* pr, bool* empty) {
    *empty = false;
    if (B < 0 || heads < 0) return SQUAD_ERR_SHAPE;
    if (T < 1 || Hs < 1 || Ws < 1 || wt < 1 || wh < 1 || ww < 1 || d < 1) return SQUAD_ERR_SHAPE;
    if (T % wt != 0 || wh > Hs || ww > Ws) return SQUAD_ERR_SHAPE;
    const int64_t Hp = ((int64_t)Hs + wh - 1) / wh * wh, Wp = ((int64_t)Ws + ww - 1) / ww * ww;
    const int64_t np = (int64_t)T * Hp * Wp;
    if (np >= ((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    const int64_t n = (int64_t)T * Hs * Ws;
    const int64_t m = (int64_t)wt * wh * ww;
    pr->B = B;
    pr->heads = heads;
    pr->T = T;
    pr->Hs = Hs;
    pr->Ws = Ws;
    pr->wt = wt;
    pr->wh = wh;
    pr->ww = ww;
    pr->d = d;
    pr->n = n;
    pr->m = m;
    pr->nw = np / m;
    pr->Hp = (int)Hp;
    pr->Wp = (int)Wp;
    pr->np = np;
    pr->npad = np - n;
    if (B == 0 || heads == 0) {
        *empty = true;
        pr->elems = 0;
        return SQUAD_OK;
    }
    const long double el = (long double)B * (long double)np * (long double)heads * (long double)d;
    if (el >= (long double)((int64_t)1 << 62)) return SQUAD_ERR_SHAPE;
    if ((int64_t)heads * d >= ((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    pr->elems = (int64_t)B * n * heads * d;
    const long double probs = (long double)B * heads * (long double)(m > pr->nw ? m : pr->nw);
    if (probs >= (long double)((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    return SQUAD_OK;
}

bool overlaps(const void* a, const void* b, size_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bytes && y < x + bytes;
}

squad_status_t validate(const void* q, const void* k, const void* v, const void* out, int B, int heads, int T,
                        int Hs, int Ws, int wt, int wh, int ww, int d, int dtype, Problem* pr, bool* empty) {
    squad_status_t s = check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, pr, empty);
    if (s != SQUAD_OK) return s;
    if (*empty) return SQUAD_OK;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return SQUAD_ERR_UNSUPPORTED;
    const int maxlen = squad_attn_max_len(d, dtype);
    if (maxlen == 0) return SQUAD_ERR_UNSUPPORTED;
    if (pr->m > maxlen || pr->nw > maxlen) return SQUAD_ERR_UNSUPPORTED;
    pr->dtype = dtype;
    if (!q || !k || !v || !out) return SQUAD_ERR_NULL;
    if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v) | ((uintptr_t)out)) & 15u) return SQUAD_ERR_ALIGN;
    pr->bytes = (size_t)pr->elems * (size_t)esize(dtype);
    if (overlaps(out, q, pr->bytes) || overlaps(out, k, pr->bytes)) return SQUAD_ERR_ALIAS;
    if (out != v && overlaps(out, v, pr->bytes)) return SQUAD_ERR_ALIAS;
    return SQUAD_OK;
}

PassGeom make_geom(const Problem& pr, bool global);

// The padded entry point's workspace (pr shaped by check_shape_padded, dtype
// set): the side buffer, and, when the grid is padded and the bf16 global pass
// would split its problems were it not in place, Y of every real token after
// it, so that the local pass writes Y there and the global pass reads its
// values from there and writes `out` (not in place).
// With allow_y false (the fixed scratch of the no-allocation entry point) the
// workspace is the side buffer alone and the global pass runs in place.
void padded_workspace(Problem* pr, bool allow_y = true) {
    const size_t es = (size_t)esize(pr->dtype);
    const size_t side = (size_t)pr->B * (size_t)pr->npad * (size_t)pr->heads * (size_t)pr->d * es;
    pr->ybuf_off = 0;
    pr->ws_bytes = side;
    if (allow_y && pr->npad > 0 && pr->dtype == SQUAD_BF16 && pass_bf16_splits(make_geom(*pr, true))) {
        pr->ybuf_off = (side + 255) & ~(size_t)255;
        pr->ws_bytes = pr->ybuf_off + (size_t)pr->B * (size_t)pr->n * (size_t)pr->heads * (size_t)pr->d * es;
    }
}

// Arguments of the padded entry points: the checks of validate() in the same
// order, plus the side buffer (SQUAD_ERR_WORKSPACE after the NULL checks).
// When the window tiles the grid nothing is padded, the workspace is ignored
// and out == v stays allowed; otherwise out must not overlap v at all (the
// mirror images of a window's padded rows are other windows' rows of v).
// fixed_scratch: the workspace is the library's own scratch of ws_size bytes
// (ws unused): a side buffer larger than it is SQUAD_ERR_SCRATCH, and the
// workspace's pointer checks do not apply.
squad_status_t validate_padded(const void* q, const void* k, const void* v, const void* out, const void* ws,
                               size_t ws_size, int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww,
                               int d, int dtype, Problem* pr, bool* empty, bool fixed_scratch = false) {
    squad_status_t s = check_shape_padded(B, heads, T, Hs, Ws, wt, wh, ww, d, pr, empty);
    if (s != SQUAD_OK) return s;
    if (*empty) return SQUAD_OK;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return SQUAD_ERR_UNSUPPORTED;
    const int maxlen = squad_attn_max_len(d, dtype);
    if (maxlen == 0) return SQUAD_ERR_UNSUPPORTED;
    if (pr->m > maxlen || pr->nw > maxlen) return SQUAD_ERR_UNSUPPORTED;
    const bool padded = pr->npad > 0;
    if (padded && (T > kMaxPaddedT || pr->Hp > kMaxPaddedHW || pr->Wp > kMaxPaddedHW)) return SQUAD_ERR_UNSUPPORTED;
    pr->dtype = dtype;
    if (!q || !k || !v || !out) return SQUAD_ERR_NULL;
    padded_workspace(pr, !fixed_scratch);
    if (fixed_scratch) {
        if (padded && ws_size < pr->ws_bytes) return SQUAD_ERR_SCRATCH;
    } else if (padded && (!ws || ws_size < pr->ws_bytes)) {
        return SQUAD_ERR_WORKSPACE;
    }
    const bool caller_ws = padded && !fixed_scratch;
    uintptr_t bits = ((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v) | ((uintptr_t)out);
    if (caller_ws) bits |= (uintptr_t)ws;
    if (bits & 15u) return SQUAD_ERR_ALIGN;
    pr->bytes = (size_t)pr->elems * (size_t)esize(dtype);
    if (overlaps(out, q, pr->bytes) || overlaps(out, k, pr->bytes)) return SQUAD_ERR_ALIAS;
    if ((padded || out != v) && overlaps(out, v, pr->bytes)) return SQUAD_ERR_ALIAS;
    if (caller_ws) {
        const uintptr_t w = (uintptr_t)ws, e = w + pr->ws_bytes;
        for (const void* t : {q, k, v, out}) {
            const uintptr_t a = (uintptr_t)t;
            if (a < e && w < a + pr->bytes) return SQUAD_ERR_ALIAS;
        }
    }
    return SQUAD_OK;
}

PassGeom make_geom(const Problem& pr, bool global) {
    const bool padded = pr.npad > 0;
    const int Hp = padded ? pr.Hp : pr.Hs, Wp = padded ? pr.Wp : pr.Ws;
    PassGeom g;
    g.n = pr.n;
    g.heads = pr.heads;
    g.L = (int)(global ? pr.nw : pr.m);
    g.P = (int)(global ? pr.m : pr.nw);
    g.nprob = (int)((int64_t)pr.B * pr.heads * g.P);
    g.Hs = pr.Hs;
    g.Ws = pr.Ws;
    g.wt = pr.wt;
    g.wh = pr.wh;
    g.ww = pr.ww;
    g.Cy = Hp / pr.wh;
    g.Cx = Wp / pr.ww;
    g.parts = 1;
    g.part_tiles = (g.L + 15) / 16;
    g.nitems = g.nprob;
    g.div_parts = make_fastdiv(1);
    g.pad = padded ? 1 : 0;
    g.Hp = Hp;
    g.Wp = Wp;
    g.pad_per_frame = pr.Hs * (Wp - pr.Ws) + (Hp - pr.Hs) * Wp;
    g.npad = padded ? pr.npad : 0;
    g.global = global ? 1 : 0;
    g.div_heads = make_fastdiv((uint32_t)g.heads);
    g.div_P = make_fastdiv((uint32_t)g.P);
    g.div_wins_t = make_fastdiv((uint32_t)(g.Cy * g.Cx));
    g.div_Cx = make_fastdiv((uint32_t)g.Cx);
    g.div_slots_t = make_fastdiv((uint32_t)(pr.wh * pr.ww));
    g.div_ww = make_fastdiv((uint32_t)pr.ww);
    return g;
}

hipError_t run_pass(const Problem& pr, bool global, const void* q, const void* k, const void* vals, void* out,
                    void* ypad, hipStream_t st) {
    const PassGeom g = make_geom(pr, global);
    if (pr.dtype == SQUAD_BF16) return launch_pass_bf16(g, pr.d, q, k, vals, out, ypad, nullptr, st);
    return launch_pass_f32(g, pr.d, q, k, vals, out, ypad, st);
}

// Both passes over all heads, in order, on the caller's stream; the second
// pass reads the first pass's output from `out` (and, on a padded grid, from
// the side buffer ypad) and updates `out` in place.
hipError_t run_two_passes(const Problem& pr, bool local_first, const void* q, const void* k, const void* v,
                          void* out, void* ypad, hipStream_t st) {
    hipError_t e = run_pass(pr, !local_first, q, k, v, out, ypad, st);
    if (e == hipSuccess) e = run_pass(pr, local_first, q, k, out, out, ypad, st);
    return e;
}

// Workspace of the backward: Y (the recomputed local output; not with saved
// activations), dY and the global pass's contributions to dQ and dK, all in
// the dtype, then (bf16 only) the local pass's rows' log-sum-exp (not with
// saved activations) and D, float32 [B, n, heads] each; every region starts on
// a 256-byte boundary.
struct BwdLayout {
    size_t y, dy, gq, gk, lse, dl, total;
};

BwdLayout bwd_layout(const Problem& pr, bool saved) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t e = (size_t)pr.elems, t = up(e * esize(pr.dtype));
    const bool bf16 = pr.dtype == SQUAD_BF16;
    const size_t rows = bf16 ? up(e / pr.d * 4) : 0;
    BwdLayout l;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t p = at;
        at += bytes;
        return p;
    };
    l.y = saved ? 0 : take(t);
    l.dy = take(t);
    l.gq = take(t);
    l.gk = take(t);
    l.lse = saved ? 0 : take(rows);
    l.dl = take(rows);
    l.total = at;
    return l;
}

// The activations squad_attn_fwd_save keeps: y as q ([B, n, heads, d] in the
// dtype) and, in bf16, lse ([B, n, heads] float32).  Both non-NULL (lse in bf16
// only), 16-byte aligned, and overlapping none of `tensors` (a forward's
// output, or a backward's gradients) nor each other.
squad_status_t check_saved(const Problem& pr, const void* y, const void* lse, const void* const* tensors,
                           int ntensors) {
    const bool bf16 = pr.dtype == SQUAD_BF16;
    if (!y || (bf16 && !lse)) return SQUAD_ERR_NULL;
    if (((uintptr_t)y | (bf16 ? (uintptr_t)lse : 0)) & 15u) return SQUAD_ERR_ALIGN;
    const size_t lse_bytes = (size_t)pr.elems / (size_t)pr.d * 4;
    for (int i = 0; i < ntensors; ++i) {
        if (overlaps(y, tensors[i], pr.bytes)) return SQUAD_ERR_ALIAS;
        if (bf16) {
            const uintptr_t a = (uintptr_t)lse, b = (uintptr_t)tensors[i];
            if (a < b + pr.bytes && b < a + lse_bytes) return SQUAD_ERR_ALIAS;
        }
    }
    if (bf16) {
        const uintptr_t a = (uintptr_t)lse, b = (uintptr_t)y;
        if (a < b + pr.bytes && b < a + lse_bytes) return SQUAD_ERR_ALIAS;
    }
    return SQUAD_OK;
}

// Arguments of squad_attn_fwd_save: the forward's checks, then y and lse,
// which must not overlap q, k, v or out.
squad_status_t validate_save(const void* q, const void* k, const void* v, const void* out, const void* y,
                             const void* lse, int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d,
                             int dtype, Problem* pr, bool* empty) {
    const squad_status_t s = validate(q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, pr, empty);
    if (s != SQUAD_OK || *empty) return s;
    const void* others[4] = {q, k, v, out};
    return check_saved(*pr, y, lse, others, 4);
}

// Arguments of squad_attn_bwd: the forward's checks on (q, k, v, out), then
// dout and the three gradients, then (saved activations) y and lse, then the
// workspace; gradients must not overlap any input, one another or the
// workspace, and the saved activations must not overlap the gradients or the
// workspace.
squad_status_t validate_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                            const void* dq, const void* dk, const void* dv, const void* ws, size_t ws_size, int B,
                            int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype, Problem* pr,
                            bool* empty, bool saved = false, const void* y = nullptr, const void* lse = nullptr) {
    squad_status_t s = check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, pr, empty);
    if (s != SQUAD_OK) return s;
    if (*empty) return SQUAD_OK;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return SQUAD_ERR_UNSUPPORTED;
    const int maxlen = squad_attn_max_len(d, dtype);
    if (maxlen == 0) return SQUAD_ERR_UNSUPPORTED;
    if (pr->m > maxlen || pr->nw > maxlen) return SQUAD_ERR_UNSUPPORTED;
    pr->dtype = dtype;
    if (!q || !k || !v || !out || !dout || !dq || !dk || !dv) return SQUAD_ERR_NULL;
    pr->bytes = (size_t)pr->elems * (size_t)esize(dtype);
    if (saved) {
        const void* grads[3] = {dq, dk, dv};
        const squad_status_t s2 = check_saved(*pr, y, lse, grads, 3);
        if (s2 != SQUAD_OK) return s2;
    }
    const BwdLayout lay = bwd_layout(*pr, saved);
    if (!ws || ws_size < lay.total) return SQUAD_ERR_WORKSPACE;
    const uintptr_t bits = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout |
                           (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)ws;
    if (bits & 15u) return SQUAD_ERR_ALIGN;
    const void* grads[3] = {dq, dk, dv};
    const void* ins[5] = {q, k, v, out, dout};
    const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + lay.total;
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(grads[i], ins[j], pr->bytes)) return SQUAD_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(grads[i], grads[j], pr->bytes)) return SQUAD_ERR_ALIAS;
    }
    for (const void* t : {q, k, v, out, dout, dq, dk, dv}) {
        const uintptr_t a = (uintptr_t)t;
        if (a < w1 && w0 < a + pr->bytes) return SQUAD_ERR_ALIAS;
    }
    if (saved) {
        const uintptr_t a = (uintptr_t)y;
        if (a < w1 && w0 < a + pr->bytes) return SQUAD_ERR_ALIAS;
        const uintptr_t b = (uintptr_t)lse;
        if (dtype == SQUAD_BF16 && b < w1 && w0 < b + (size_t)pr->elems / (size_t)d * 4) return SQUAD_ERR_ALIAS;
    }
    return SQUAD_OK;
}

// The local pass into y (in bf16 also its rows' log-sum-exp into lse).
hipError_t run_local_saving(const Problem& pr, const void* q, const void* k, const void* v, void* y, float* lse,
                            hipStream_t st) {
    const PassGeom g = make_geom(pr, false);
    if (pr.dtype == SQUAD_BF16) return launch_pass_bf16(g, pr.d, q, k, v, y, nullptr, lse, st);
    return launch_pass_f32(g, pr.d, q, k, v, y, nullptr, st);
}

// The backward's three kernels, or two when the caller passes the local
// output Y (and in bf16 its rows' log-sum-exp) that squad_attn_fwd_save kept.
hipError_t run_backward(const Problem& pr, const void* q, const void* k, const void* v, const void* out,
                        const void* dout, void* dq, void* dk, void* dv, void* ws, hipStream_t st,
                        const void* y_saved = nullptr, const float* lse_saved = nullptr) {
    const bool saved = y_saved != nullptr;
    const BwdLayout lay = bwd_layout(pr, saved);
    char* w = static_cast<char*>(ws);
    void* dy = w + lay.dy;
    void *gq = w + lay.gq, *gk = w + lay.gk;
    const bool bf16 = pr.dtype == SQUAD_BF16;
    float* dl = bf16 ? reinterpret_cast<float*>(w + lay.dl) : nullptr;
    const void* y = y_saved;
    const float* lse = lse_saved;
    hipError_t e = hipSuccess;
    if (!saved) {
        // the forward kept only O: recompute the local output Y (and, in
        // bf16, its rows' log-sum-exp, which the local pass's backward reuses)
        float* lse_w = bf16 ? reinterpret_cast<float*>(w + lay.lse) : nullptr;
        e = run_local_saving(pr, q, k, v, w + lay.y, lse_w, st);
        if (e != hipSuccess) return e;
        y = w + lay.y;
        lse = lse_w;
    }
    // global pass (values Y, output O): its dQ, dK contributions, dY and, in
    // bf16, the local pass's D = rowsum(dY * Y)
    const PassGeom gg = make_geom(pr, true);
    BwdArgs ag{q, k, y, out, dout, nullptr, nullptr, gq, gk, dy, nullptr, nullptr, dl};
    e = bf16 ? launch_bwd_pass_bf16(gg, pr.d, ag, st) : launch_bwd_pass_f32(gg, pr.d, ag, st);
    if (e != hipSuccess) return e;
    // local pass (values V, output Y, upstream dY): adds the global pass's share
    const PassGeom gl = make_geom(pr, false);
    BwdArgs al{q, k, v, y, dy, gq, gk, dq, dk, dv, lse, dl, nullptr};
    return bf16 ? launch_bwd_pass_bf16(gl, pr.d, al, st) : launch_bwd_pass_f32(gl, pr.d, al, st);
}

squad_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return SQUAD_OK;
    g_last_hip_error = (int)e;
    return SQUAD_ERR_HIP;
}

// The window rule: wt = T, the continuous optimum wh*ww = sqrt(n)/T with
// wh : ww = Hs : Ws, each spatial extent rounded down or up (within
// 1..extent), and of those windows the least 4hd(n_p m + n_p^2/m) on the
// padded grid (n_p tokens); ties to the aspect ratio closer to the grid's, then
// to the smaller m, then the smaller wh.  Costs compare exactly as fractions.
void solve_window(int T, int Hs, int Ws, int* out_wh, int* out_ww) {
    typedef unsigned __int128 u128;
    const double n = (double)T * (double)Hs * (double)Ws;
    const double area = sqrt(n) / T;
    const double whc = sqrt(area * Hs / Ws), wwc = sqrt(area * Ws / Hs);
    const int whs[2] = {(int)floor(whc), (int)ceil(whc)}, wws[2] = {(int)floor(wwc), (int)ceil(wwc)};
    bool have = false;
    u128 best_num = 0, best_den = 1, best_amax = 0, best_amin = 1;
    int64_t best_m = 0;
    int best_wh = 1, best_ww = 1;
    for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b) {
            const int wh = whs[a] < 1 ? 1 : (whs[a] > Hs ? Hs : whs[a]);
            const int ww = wws[b] < 1 ? 1 : (wws[b] > Ws ? Ws : wws[b]);
            const u128 m = (u128)T * wh * ww;
            const u128 np = (u128)T * (u128)((Hs + wh - 1) / wh * wh) * (u128)((Ws + ww - 1) / ww * ww);
            const u128 num = np * m * m + np * np, den = m;  // n_p m + n_p^2 / m
            const u128 x = (u128)wh * Ws, y = (u128)ww * Hs;
            const u128 amax = x > y ? x : y, amin = x > y ? y : x;
            bool better = !have;
            if (have) {
                const u128 l = num * best_den, r = best_num * den;
                if (l != r) {
                    better = l < r;
                } else {
                    const u128 al = amax * best_amin, ar = best_amax * amin;
                    if (al != ar) better = al < ar;
                    else if ((int64_t)m != best_m) better = (int64_t)m < best_m;
                    else better = wh < best_wh;
                }
            }
            if (better) {
                have = true;
                best_num = num;
                best_den = den;
                best_amax = amax;
                best_amin = amin;
                best_m = (int64_t)m;
                best_wh = wh;
                best_ww = ww;
            }
        }
    *out_wh = best_wh;
    *out_ww = best_ww;
}

squad_status_t run(Kind kind, const void* q, const void* k, const void* v, void* out, int B, int heads, int T, int Hs,
                   int Ws, int wt, int wh, int ww, int d, int dtype, hipStream_t st) {
    Problem pr;
    bool empty = false;
    const squad_status_t s = validate(q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, &pr, &empty);
    if (s != SQUAD_OK || empty) return s;
    hipError_t e = hipSuccess;
    switch (kind) {
        case Kind::kFwd:
            e = run_two_passes(pr, true, q, k, v, out, nullptr, st);
            break;
        case Kind::kReversed:
            e = run_two_passes(pr, false, q, k, v, out, nullptr, st);
            break;
        case Kind::kLocal:
            e = run_pass(pr, false, q, k, v, out, nullptr, st);
            break;
        case Kind::kGlobal:
            e = run_pass(pr, true, q, k, v, out, nullptr, st);
            break;
    }
    return hip_status(e);
}

// ---- fixed scratch of squad_attn_fwd_padded_noalloc ------------------------
// Device memory of the library's own, so that the entry point allocates
// nothing: each device the library runs on holds one copy until the process
// ends.  On the host the name `scratch` is only a stand-in for the symbol, not
// a device address; the address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[SQUAD_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// This device's scratch address (looked up on the first call on a device), or
// null with *err set.
void* scratch_on_current_device(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        if (ptr == nullptr) {
            *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    if (dev < 64) cached[dev] = cus;
    return cus;
}

}  // namespace squad

extern "C" {

squad_status_t squad_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int heads, int T,
                              int Hs, int Ws, int wt, int wh, int ww, int d, int dtype, hipStream_t stream) {
    return squad::run(squad::Kind::kFwd, q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, stream);
}

squad_status_t squad_attn_local(const void* q, const void* k, const void* v, void* out, int B, int heads, int T,
                                int Hs, int Ws, int wt, int wh, int ww, int d, int dtype, hipStream_t stream) {
    return squad::run(squad::Kind::kLocal, q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, stream);
}

squad_status_t squad_attn_global(const void* q, const void* k, const void* v, void* out, int B, int heads, int T,
                                 int Hs, int Ws, int wt, int wh, int ww, int d, int dtype, hipStream_t stream) {
    return squad::run(squad::Kind::kGlobal, q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, stream);
}

squad_status_t squad_attn_fwd_reversed(const void* q, const void* k, const void* v, void* out, int B, int heads,
                                       int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype,
                                       hipStream_t stream) {
    return squad::run(squad::Kind::kReversed, q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, stream);
}

squad_status_t squad_attn_fwd_padded(const void* q, const void* k, const void* v, void* out, void* workspace,
                                     size_t workspace_bytes, int B, int heads, int T, int Hs, int Ws, int wt, int wh,
                                     int ww, int d, int dtype, hipStream_t stream) {
    squad::Problem pr;
    bool empty = false;
    const squad_status_t s = squad::validate_padded(q, k, v, out, workspace, workspace_bytes, B, heads, T, Hs, Ws,
                                                    wt, wh, ww, d, dtype, &pr, &empty);
    if (s != SQUAD_OK || empty) return s;
    if (pr.ybuf_off > 0) {
        void* ybuf = static_cast<char*>(workspace) + pr.ybuf_off;
        hipError_t e = squad::run_pass(pr, false, q, k, v, ybuf, workspace, stream);
        if (e == hipSuccess) e = squad::run_pass(pr, true, q, k, ybuf, out, workspace, stream);
        return squad::hip_status(e);
    }
    return squad::hip_status(
        squad::run_two_passes(pr, true, q, k, v, out, pr.npad > 0 ? workspace : nullptr, stream));
}

squad_status_t squad_attn_fwd_padded_noalloc(const void* q, const void* k, const void* v, void* out, int B, int heads,
                                             int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype,
                                             hipStream_t stream) {
    squad::Problem pr;
    bool empty = false;
    const squad_status_t s = squad::validate_padded(q, k, v, out, nullptr, SQUAD_NOALLOC_SCRATCH_BYTES, B, heads, T,
                                                    Hs, Ws, wt, wh, ww, d, dtype, &pr, &empty, true);
    if (s != SQUAD_OK || empty) return s;
    void* side = nullptr;
    if (pr.npad > 0) {
        hipError_t e = hipSuccess;
        side = squad::scratch_on_current_device(&e);
        if (side == nullptr) return squad::hip_status(e);
    }
    // the side buffer is written whole by the local pass before the global
    // pass reads it, so nothing of an earlier call's contents is used
    return squad::hip_status(squad::run_two_passes(pr, true, q, k, v, out, side, stream));
}

squad_status_t squad_attn_check_padded(const void* q, const void* k, const void* v, const void* out,
                                       const void* workspace, size_t workspace_bytes, int B, int heads, int T, int Hs,
                                       int Ws, int wt, int wh, int ww, int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    return squad::validate_padded(q, k, v, out, workspace, workspace_bytes, B, heads, T, Hs, Ws, wt, wh, ww, d,
                                  dtype, &pr, &empty);
}

long long squad_attn_padded_workspace_bytes(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d,
                                            int dtype) {
    squad::Problem pr;
    bool empty = false;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return -1;
    if (squad::check_shape_padded(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1;
    if (empty) return 0;
    const long double bytes = (long double)B * (pr.npad + pr.n) * heads * d * squad::esize(dtype) + 256;
    if (bytes >= 9.0e18L) return -1;
    pr.dtype = dtype;
    squad::padded_workspace(&pr);
    return (long long)pr.ws_bytes;
}

double squad_attn_flops_padded(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d) {
    squad::Problem pr;
    bool empty = false;
    if (squad::check_shape_padded(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1.0;
    if (empty) return 0.0;
    return 4.0 * (double)B * heads * (double)d * (double)pr.np * (double)(pr.m + pr.nw);
}

double squad_attn_bytes_padded(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return -1.0;
    if (squad::check_shape_padded(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1.0;
    if (empty) return 0.0;
    const double row = (double)B * heads * d * squad::esize(dtype);
    return row * (7.0 * (double)pr.np + (double)pr.n);
}

squad_status_t squad_window_solve(int T, int Hs, int Ws, int* wt, int* wh, int* ww) {
    if (T < 1 || Hs < 1 || Ws < 1) return SQUAD_ERR_SHAPE;
    if ((int64_t)T * Hs * Ws >= ((int64_t)1 << 31)) return SQUAD_ERR_SHAPE;
    if (!wt || !wh || !ww) return SQUAD_ERR_NULL;
    squad::solve_window(T, Hs, Ws, wh, ww);
    *wt = T;
    return SQUAD_OK;
}

squad_status_t squad_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int heads,
                              int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype, hipStream_t stream) {
    squad::Problem pr;
    bool empty = false;
    const squad_status_t s = squad::validate_bwd(q, k, v, out, dout, dq, dk, dv, workspace, workspace_bytes, B,
                                                 heads, T, Hs, Ws, wt, wh, ww, d, dtype, &pr, &empty);
    if (s != SQUAD_OK || empty) return s;
    return squad::hip_status(squad::run_backward(pr, q, k, v, out, dout, dq, dk, dv, workspace, stream));
}

squad_status_t squad_attn_check_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                    const void* dq, const void* dk, const void* dv, const void* workspace,
                                    size_t workspace_bytes, int B, int heads, int T, int Hs, int Ws, int wt, int wh,
                                    int ww, int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    return squad::validate_bwd(q, k, v, out, dout, dq, dk, dv, workspace, workspace_bytes, B, heads, T, Hs, Ws, wt,
                               wh, ww, d, dtype, &pr, &empty);
}

long long squad_attn_bwd_workspace_bytes(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d,
                                         int dtype) {
    squad::Problem pr;
    bool empty = false;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return -1;
    if (squad::check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1;
    if (empty) return 0;
    pr.dtype = dtype;
    return (long long)squad::bwd_layout(pr, false).total;
}

long long squad_attn_bwd_saved_workspace_bytes(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww,
                                               int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return -1;
    if (squad::check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1;
    if (empty) return 0;
    pr.dtype = dtype;
    return (long long)squad::bwd_layout(pr, true).total;
}

squad_status_t squad_attn_fwd_save(const void* q, const void* k, const void* v, void* out, void* y, float* lse,
                                   int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype,
                                   hipStream_t stream) {
    squad::Problem pr;
    bool empty = false;
    const squad_status_t s =
        squad::validate_save(q, k, v, out, y, lse, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, &pr, &empty);
    if (s != SQUAD_OK || empty) return s;
    hipError_t e = squad::run_local_saving(pr, q, k, v, y, dtype == SQUAD_BF16 ? lse : nullptr, stream);
    if (e == hipSuccess) e = squad::run_pass(pr, true, q, k, y, out, nullptr, stream);
    return squad::hip_status(e);
}

squad_status_t squad_attn_bwd_saved(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                    const void* y, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                                    size_t workspace_bytes, int B, int heads, int T, int Hs, int Ws, int wt, int wh,
                                    int ww, int d, int dtype, hipStream_t stream) {
    squad::Problem pr;
    bool empty = false;
    const squad_status_t s = squad::validate_bwd(q, k, v, out, dout, dq, dk, dv, workspace, workspace_bytes, B,
                                                 heads, T, Hs, Ws, wt, wh, ww, d, dtype, &pr, &empty, true, y, lse);
    if (s != SQUAD_OK || empty) return s;
    return squad::hip_status(squad::run_backward(pr, q, k, v, out, dout, dq, dk, dv, workspace, stream, y,
                                                 dtype == SQUAD_BF16 ? lse : nullptr));
}

double squad_attn_bwd_flops(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d) {
    const double f = squad_attn_flops(B, heads, T, Hs, Ws, wt, wh, ww, d);
    return f < 0 ? f : 2.5 * f;
}

double squad_attn_bwd_bytes(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return -1.0;
    if (squad::check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1.0;
    if (empty) return 0.0;
    const double e = (double)pr.elems, es = squad::esize(dtype);
    // recompute Y: 3 reads + 1 write; global pass: q, k, Y, O, dO read, dY and
    // the dQ, dK contributions written; local pass: q, k, v, dY and the
    // contributions read (and Y, for D, in float32 only), dq, dk, dv written
    // (per-row float32 log-sum-exp and D not counted)
    return e * es * (4.0 + 8.0 + (dtype == SQUAD_BF16 ? 9.0 : 10.0));
}

squad_status_t squad_attn_check(const void* q, const void* k, const void* v, const void* out, int B, int heads,
                                int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    return squad::validate(q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, &pr, &empty);
}

int squad_attn_max_len(int d, int dtype) {
    if (d != 64 && d != 128) return 0;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return 0;
    return squad::kMaxLen;
}

double squad_attn_flops(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d) {
    squad::Problem pr;
    bool empty = false;
    if (squad::check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1.0;
    if (empty) return 0.0;
    return 4.0 * (double)B * heads * (double)d * (double)pr.n * (double)(pr.m + pr.nw);
}

double squad_attn_bytes(int B, int heads, int T, int Hs, int Ws, int wt, int wh, int ww, int d, int dtype) {
    squad::Problem pr;
    bool empty = false;
    if (dtype != SQUAD_BF16 && dtype != SQUAD_F32) return -1.0;
    if (squad::check_shape(B, heads, T, Hs, Ws, wt, wh, ww, d, &pr, &empty) != SQUAD_OK) return -1.0;
    if (empty) return 0.0;
    return 8.0 * (double)pr.elems * (double)squad::esize(dtype);
}

const char* squad_status_str(int status) {
    switch (status) {
        case SQUAD_OK: return "ok";
        case SQUAD_ERR_NULL: return "null pointer argument";
        case SQUAD_ERR_SHAPE:
            return "invalid shape (non-positive extent, window not tiling the grid, or size overflow)";
        case SQUAD_ERR_UNSUPPORTED: return "unsupported dtype, head dim, or sequence length";
        case SQUAD_ERR_ALIAS: return "a written buffer overlaps another buffer of the call (only out == v is allowed)";
        case SQUAD_ERR_ALIGN: return "pointer not 16-byte aligned";
        case SQUAD_ERR_HIP: return "HIP runtime or launch error";
        case SQUAD_ERR_WORKSPACE: return "workspace missing or smaller than squad_attn_padded_workspace_bytes";
        case SQUAD_ERR_SCRATCH:
            return "the padded positions' local outputs need more than the no-allocation entry point's fixed "
                   "scratch (SQUAD_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int squad_attn_last_hip_error(void) { return squad::g_last_hip_error; }

int squad_attn_abi_version(void) { return 4; }

}  // extern "C"
