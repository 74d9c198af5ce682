// Internal declarations shared by the SQuad-Attention HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace squad {

// Longest attended sequence (m for the local pass, N_w for the global pass)
// any kernel instance accepts.
constexpr int kMaxLen = 512;

// Exact unsigned division of 0 <= n < 2^31 by a fixed 1 <= d < 2^31 with one
// multiply and shift (Granlund & Montgomery, "Division by invariant integers
// using multiplication", 1994, thm. 4.2 with N = 31): with 2^(l-1) < d <= 2^l,
// m = floor(2^(31+l) / d) + 1 < 2^32 + 1 and q = floor(n * m / 2^(31+l)).
struct FastDiv {
    uint64_t m;
    uint32_t shift;  // 31 + l
    uint32_t d;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    FastDiv f;
    f.d = d;
    f.shift = 31 + l;
    f.m = ((1ull << (31 + l)) / d) + 1;
    return f;
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.shift);
}

// One pass seen as a batch of independent softmax attentions ("problems").
//
// The local pass has B*heads*N_w problems: (b, h, window c), each over the
// m tokens of c.  The global pass has B*heads*m problems: (b, h, slot j), each
// over the N_w tokens that sit at slot j of every window.  Token (c, j) has
// index win_origin(c) + slot_offset(j) because the token index is linear in the
// grid coordinates; a problem therefore maps its row r to
//   local : win_origin(problem) + slot_offset(r)
//   global: slot_offset(problem) + win_origin(r).
struct PassGeom {
    int64_t n;      // tokens per batch element, T*Hs*Ws
    int heads;
    int L;          // rows per problem (m local, N_w global)
    int P;          // problems per (b, h) (N_w local, m global)
    int nprob;      // B*heads*P
    int Hs, Ws;     // grid extents (T is implied); the real grid when pad = 1
    int wt, wh, ww; // window extents
    int Cy, Cx;     // windows along y and x (of the padded grid when pad = 1)
    int global;     // 0: local pass, 1: global pass
    // divisors of the problem decode and of the row maps
    FastDiv div_heads, div_P;         // problem -> (b, pi, h)
    FastDiv div_wins_t, div_Cx;       // window c -> (ct, cy, cx): Cy*Cx, Cx
    FastDiv div_slots_t, div_ww;      // slot j -> (jt, jy, jx): wh*ww, ww
    // Padded grids (pad = 1).  The window tiles the grid (T, Hp, Wp) that
    // extends (T, Hs, Ws) at the bottom and right by mirror images; windows,
    // slots, Cy and Cx then refer to the padded grid, and a row is named by its
    // packed padded coordinates (see pack_coords) instead of a token offset.
    // The local outputs of padded tokens live in a side buffer of npad tokens
    // per batch element ([B, npad, heads, d]).
    // Long problems may be split by query rows into `parts` work items of
    // part_tiles 16-row query tiles (the last may have fewer); each item
    // streams all the problem's keys and values.  Items of one problem are 8
    // apart (nitems = nprob * parts; splitting needs nprob % 8 == 0 and a pass
    // that is not in place).  Only the bf16 forward splits; everything else
    // has parts = 1.
    int parts, part_tiles, nitems;
    FastDiv div_parts;
    int pad;
    int Hp, Wp;
    int pad_per_frame;  // Hs*(Wp - Ws) + (Hp - Hs)*Wp padded tokens per frame
    int64_t npad;       // T * pad_per_frame
};

// Packed (t, y, x) of the padded grid: 11 bits of t, 10 of y and of x.  The
// fields of a window origin and of an in-window offset add without carries,
// so a row's coordinates are one integer addition away from its problem's.
constexpr int kMaxPaddedT = 2047;
constexpr int kMaxPaddedHW = 1023;

__host__ __device__ inline int pack_coords(int t, int y, int x) { return (t << 20) | (y << 10) | x; }

// Packed origin of window c of the padded grid.
__host__ __device__ inline int win_coords(const PassGeom& g, int c) {
    const int ct = (int)fdiv((uint32_t)c, g.div_wins_t);
    const int r = c - ct * (int)g.div_wins_t.d;
    const int cy = (int)fdiv((uint32_t)r, g.div_Cx);
    const int cx = r - cy * g.Cx;
    return pack_coords(ct * g.wt, cy * g.wh, cx * g.ww);
}

// Packed in-window offset of slot j.
__host__ __device__ inline int slot_coords(const PassGeom& g, int j) {
    const int jt = (int)fdiv((uint32_t)j, g.div_slots_t);
    const int r = j - jt * (int)g.div_slots_t.d;
    const int jy = (int)fdiv((uint32_t)r, g.div_ww);
    return pack_coords(jt, jy, r - jy * g.ww);
}

// Position i of an axis of length size extended past its end by mirroring
// about the last element (the edge itself is not repeated).
__host__ __device__ inline int mirror(int i, int size) { return i < size ? i : 2 * (size - 1) - i; }

// Token of the real grid whose values a padded position carries.
__host__ __device__ inline int mirrored_token(const PassGeom& g, int p) {
    const int t = p >> 20, y = (p >> 10) & 1023, x = p & 1023;
    return (t * g.Hs + mirror(y, g.Hs)) * g.Ws + mirror(x, g.Ws);
}

__host__ __device__ inline bool is_real(const PassGeom& g, int p) {
    return ((p >> 10) & 1023) < g.Hs && (p & 1023) < g.Ws;
}

// Index of a padded (not real) position in the side buffer: frame-major;
// within a frame first the right margin of the real rows, then the bottom rows.
__host__ __device__ inline int pad_index(const PassGeom& g, int p) {
    const int t = p >> 20, y = (p >> 10) & 1023, x = p & 1023;
    const int within = y < g.Hs ? y * (g.Wp - g.Ws) + (x - g.Ws) : g.Hs * (g.Wp - g.Ws) + (y - g.Hs) * g.Wp + x;
    return t * g.pad_per_frame + within;
}

// Token index of slot 0 of window c (windows numbered row-major over their
// tile coordinates (ct, cy, cx)).
__host__ __device__ inline int win_origin(const PassGeom& g, int c) {
    const int ct = (int)fdiv((uint32_t)c, g.div_wins_t);
    const int r = c - ct * (int)g.div_wins_t.d;
    const int cy = (int)fdiv((uint32_t)r, g.div_Cx);
    const int cx = r - cy * g.Cx;
    return ((ct * g.wt) * g.Hs + cy * g.wh) * g.Ws + cx * g.ww;
}

// Offset, in tokens, of in-window slot j (slots numbered row-major over the
// in-window offset (jt, jy, jx)).
__host__ __device__ inline int slot_offset(const PassGeom& g, int j) {
    const int jt = (int)fdiv((uint32_t)j, g.div_slots_t);
    const int r = j - jt * (int)g.div_slots_t.d;
    const int jy = (int)fdiv((uint32_t)r, g.div_ww);
    const int jx = r - jy * g.ww;
    return (jt * g.Hs + jy) * g.Ws + jx;
}

// (b, pi, h) of problem p: heads vary fastest, then the problem index within
// the (b, h) slice, then the batch element.
struct ProblemIndex {
    int b, pi, h;
};

__host__ __device__ inline ProblemIndex decode_problem(const PassGeom& g, int p) {
    const int t = (int)fdiv((uint32_t)p, g.div_heads);
    const int b = (int)fdiv((uint32_t)t, g.div_P);
    return ProblemIndex{b, t - b * g.P, p - t * g.heads};
}

// Kernel launchers.  Each validates nothing (the ABI layer did) and returns the
// launch status.  `vals` may equal `out` (in-place update, race-free because
// every workgroup reads all rows of its problems before writing them, and the
// problems of a pass partition the rows).
// `ypad` is the side buffer of padded grids (unused when g.pad == 0): the
// local pass writes the outputs of padded rows there, the global pass reads
// its values for padded rows from it and stores real rows only.
// `lse_out` (bf16, unpadded grids; may be null): receives each row's
// log-sum-exp in log2 units of the scores scaled by log2(e)/sqrt(d),
// [B, n, heads] float32.
hipError_t launch_pass_bf16(const PassGeom& g, int d, const void* q, const void* k,
                            const void* vals, void* out, void* ypad, float* lse_out, hipStream_t stream);
hipError_t launch_pass_f32(const PassGeom& g, int d, const void* q, const void* k,
                           const void* vals, void* out, void* ypad, hipStream_t stream);

// Whether launch_pass_bf16 splits the problems of g into query parts when the
// pass is not in place (vals != out); in place it never does.
bool pass_bf16_splits(const PassGeom& g);

// Operands of one pass's backward (unpadded grids).  q, k, vals: the pass's
// inputs; out: its output O; dout: the upstream gradient dO.  The kernels
// write dQ and dK (plus addq / addk when those are not null: the other pass's
// contributions, in the kernels' dtype) and dV of the values.  The bf16
// kernels read and write bf16 tensors, with float32 sums inside; the float32
// kernels are float32 throughout.  bf16 only, each may be null (the float32
// kernels take neither): lse, the rows' log-sum-exp as launch_pass_bf16
// writes it; dd_in, the rows' D = rowsum(dO * O) (then `out` is not read);
// vdot, receives rowsum(dV * V) of every values row (dV as stored), which is
// D for the backward of the pass that produced the values.  The per-row
// arrays are [B, n, heads] float32.
struct BwdArgs {
    const void *q, *k, *vals, *out, *dout;
    const void *addq, *addk;
    void *dq, *dk, *dvals;
    const float* lse;
    const float* dd_in;
    float* vdot;
};

hipError_t launch_bwd_pass_bf16(const PassGeom& g, int d, const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_pass_f32(const PassGeom& g, int d, const BwdArgs& a, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace squad
