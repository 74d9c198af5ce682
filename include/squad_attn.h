/*
 * squad_attn.h -- C ABI of the SQuad-Attention forward pass on AMD Instinct
 * MI355X (gfx950).
 *
 * The operator (SQuad: Sub-Quadratic Attention Distillation for Efficient
 * Video Generation) replaces one full softmax self-attention over the n latent
 * tokens of a video DiT block by two plain softmax attentions composed
 * (agihunt.info summary, method paragraph; paperpeel full text, sec. 3.2):
 *
 *   local pass   Y[c,j] = sum_{j'} softmax_{j'}(<Q[c,j], K[c,j']> / sqrt(d)) V[c,j']
 *                over the m = wt*wh*ww tokens of window c (every window spans
 *                the full temporal extent in the pages' configuration);
 *   global pass  O[c,j] = sum_{c'} softmax_{c'}(<Q[c,j], K[c',j]> / sqrt(d)) Y[c',j]
 *                over the N_w = n/m windows, at the fixed in-window slot j
 *                (paperpeel full text, appendix "Reachability"),
 *
 * where [c,j] is the token at slot j of window c, the global pass reuses the
 * block's Q and K (only re-indexing sits between the passes and the method adds
 * no parameters) and the local output is its value stream (gist.science
 * explainer, "Operador de Atencao SQuad").  Both softmaxes are non-causal and
 * include the query's own key.
 *
 * Layout.  q, k, v and out are contiguous device buffers [B, n, heads, d] of
 * one dtype, n = T*Hs*Ws tokens in (t, y, x) row-major order: element
 * (b, i, h, e) sits at ((b*n + i)*heads + h)*d + e.  Windows are the aligned
 * (wt, wh, ww) tiles of the (T, Hs, Ws) grid, numbered in row-major order of
 * their tile coordinates; the slot of a token is its in-window offset
 * (t%wt, y%wh, x%ww), numbered row-major.
 *
 * Ownership.  The caller allocates and owns every buffer.  The library keeps no
 * per-call state and allocates nothing; out doubles as the intermediate Y of
 * squad_attn_fwd, so no workspace is needed (the padded entry point takes one
 * for the padded positions; its no-allocation variant uses a fixed device
 * buffer of the library's own instead).  Prior contents of out are
 * ignored; they are undefined after a failed launch.
 *
 * Semantics.  Every compute entry point is asynchronous on `stream` (0 = the
 * null stream): it validates its arguments on the host, before any HIP call,
 * enqueues its kernels and returns.  Device faults surface at the caller's
 * next synchronisation.  out may be the very same buffer as v (the update is
 * then in place); any other overlap of out with q, k or v is rejected.
 * B == 0 or heads == 0 is an empty problem: SQUAD_OK, nothing is enqueued and
 * the pointers are not inspected.
 *
 * Errors (checked in this order; the first failing check is returned):
 *   SQUAD_ERR_SHAPE       a negative B or heads; any other dimension < 1;
 *                         T % wt, Hs % wh or Ws % ww != 0; the element count
 *                         B*n*heads*d overflowing 62 bits, or heads*d 31 bits;
 *                         B*heads*max(m, N_w) not fitting a 31-bit launch grid.
 *   SQUAD_ERR_UNSUPPORTED unknown dtype; d not in {64, 128}; m or N_w above
 *                         squad_attn_max_len(d, dtype).
 *   SQUAD_ERR_NULL        q, k, v or out is NULL.
 *   SQUAD_ERR_ALIGN       a pointer not 16-byte aligned.
 *   SQUAD_ERR_ALIAS       out overlaps q or k, or overlaps v without being v.
 *   SQUAD_ERR_HIP         a HIP runtime call or kernel launch failed
 *                         (squad_attn_last_hip_error() gives the hipError_t).
 */
#ifndef SQUAD_ATTN_H
#define SQUAD_ATTN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQUAD_BF16 = 0, /* bfloat16 storage, bf16 MFMA with fp32 accumulation */
    SQUAD_F32 = 1   /* float32 storage and arithmetic (debug / reference path) */
} squad_dtype_t;

typedef enum {
    SQUAD_OK = 0,
    SQUAD_ERR_NULL = 1,
    SQUAD_ERR_SHAPE = 2,
    SQUAD_ERR_UNSUPPORTED = 3,
    SQUAD_ERR_ALIAS = 4,
    SQUAD_ERR_ALIGN = 5,
    SQUAD_ERR_HIP = 6,
    SQUAD_ERR_WORKSPACE = 7,
    SQUAD_ERR_SCRATCH = 8
} squad_status_t;

/* Size of the fixed device scratch of squad_attn_fwd_padded_noalloc. */
#define SQUAD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* out = Attn_G(q, k, Attn_L(q, k, v)): the SQuad-Attention forward pass.
 * Enqueues the local pass (writing Y into out) and then the global pass
 * (reading Y from out and writing O over it, each workgroup reading its whole
 * read set before it writes the same rows). */
squad_status_t squad_attn_fwd(const void* q, const void* k, const void* v, void* out,
                              int B, int heads, int T, int Hs, int Ws,
                              int wt, int wh, int ww, int d,
                              int dtype, hipStream_t stream);

/* out = Attn_L(q, k, v): the local (in-window) pass alone. */
squad_status_t squad_attn_local(const void* q, const void* k, const void* v, void* out,
                                int B, int heads, int T, int Hs, int Ws,
                                int wt, int wh, int ww, int d,
                                int dtype, hipStream_t stream);

/* out = Attn_G(q, k, v): the global (cross-window, same-slot) pass alone. */
squad_status_t squad_attn_global(const void* q, const void* k, const void* v, void* out,
                                 int B, int heads, int T, int Hs, int Ws,
                                 int wt, int wh, int ww, int d,
                                 int dtype, hipStream_t stream);

/* out = Attn_L(q, k, Attn_G(q, k, v)): the reverse order the pages ablate
 * (paperpeel full text, sec. 4.4 and appendix "On the ordering"). */
squad_status_t squad_attn_fwd_reversed(const void* q, const void* k, const void* v, void* out,
                                       int B, int heads, int T, int Hs, int Ws,
                                       int wt, int wh, int ww, int d,
                                       int dtype, hipStream_t stream);

/* Grids a window does not tile (paperpeel full text, appendix paragraph
 * "Conformance to the theoretical curves is quantitative": such windows are
 * handled by extending the grid with mirror images).
 *
 * out = the real tokens of SQuad on the padded grid: the (T, Hs, Ws) grid is
 * extended at the bottom and right to (T, Hp, Wp), Hp = ceil(Hs/wh)*wh and
 * Wp = ceil(Ws/ww)*ww, each added position carrying the q, k and v of its
 * mirror image about the last row or column (the edge is not repeated; padded
 * position y >= Hs mirrors row 2*(Hs-1) - y, likewise x); both passes run over
 * the padded grid, padded tokens being ordinary queries, keys and values, and
 * only the outputs of the real tokens are written.  The time axis is never
 * padded: T % wt must be 0.  Nothing is copied: the kernels address mirror
 * images directly.
 *
 * q, k, v, out: [B, n, heads, d] as for squad_attn_fwd (n = T*Hs*Ws, the real
 * grid).  workspace: device buffer of at least
 * squad_attn_padded_workspace_bytes(...) bytes, 16-byte aligned, holding the
 * local outputs of the padded positions between the two passes and, in bf16
 * when the global pass has more than 384 windows and B*heads*m is a multiple
 * of 8, the local outputs of the real tokens too (the global pass then reads
 * its values there instead of from `out`, which lets it split its long
 * problems into query parts) (contents on entry ignored, undefined
 * afterwards; must not overlap q, k, v or out; one workspace must not be used
 * by two calls that may run at the same time).
 * When the window tiles the grid the call is squad_attn_fwd: the workspace is
 * not used (it may be NULL) and out may be v.  Otherwise out must not overlap
 * v either (mirror images read other windows' rows of v).
 *
 * Errors as squad_attn_fwd, except: SQUAD_ERR_SHAPE for T % wt != 0, wh > Hs
 * or ww > Ws (instead of any non-tiling window), with the sizes taken on the
 * padded grid; SQUAD_ERR_UNSUPPORTED also for a padded grid with T > 2047 or
 * Hp or Wp > 1023; SQUAD_ERR_WORKSPACE (after the NULL checks) for a NULL or
 * too small workspace when padding is needed. */
squad_status_t squad_attn_fwd_padded(const void* q, const void* k, const void* v, void* out,
                                     void* workspace, size_t workspace_bytes,
                                     int B, int heads, int T, int Hs, int Ws,
                                     int wt, int wh, int ww, int d,
                                     int dtype, hipStream_t stream);

/* squad_attn_fwd_padded for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and the same `out` bit for bit when squad_attn_fwd_padded's
 * workspace would hold only the padded positions, with no workspace argument.
 * The padded positions' local outputs go to a fixed scratch buffer of the
 * library's own, SQUAD_NOALLOC_SCRATCH_BYTES (32 MiB) of device memory that
 * each device the library runs on holds until the process ends; its address
 * is looked up once per device, on the first call on it.  The call makes no
 * allocation (no hipMalloc, no hipFree, no allocating library routine).  The
 * global pass always runs in place on `out` (no region for Y).
 *
 * Every call on one device shares that device's scratch and it keeps the last
 * call's contents: calls that may overlap in time on one device (different
 * streams, or different host threads, without ordering between them) race on
 * it and must not be issued.  Nothing needs to start at zero: the local pass
 * writes the whole side buffer before the global pass reads it.
 *
 * Arguments and errors as squad_attn_fwd_padded without the workspace, except
 * SQUAD_ERR_SCRATCH (after the NULL checks, before any HIP call) when
 * B * (padded positions per batch element) * heads * d * sizeof(dtype)
 * exceeds SQUAD_NOALLOC_SCRATCH_BYTES.  When the window tiles the grid the
 * call is squad_attn_fwd and uses no scratch. */
squad_status_t squad_attn_fwd_padded_noalloc(const void* q, const void* k, const void* v, void* out,
                                             int B, int heads, int T, int Hs, int Ws,
                                             int wt, int wh, int ww, int d,
                                             int dtype, hipStream_t stream);

/* Validation only for squad_attn_fwd_padded (pure host function). */
squad_status_t squad_attn_check_padded(const void* q, const void* k, const void* v, const void* out,
                                       const void* workspace, size_t workspace_bytes,
                                       int B, int heads, int T, int Hs, int Ws,
                                       int wt, int wh, int ww, int d, int dtype);

/* Bytes of workspace squad_attn_fwd_padded needs: B * (padded positions per
 * batch element) * heads * d * sizeof(dtype), plus, in the case above, that
 * rounded up to 256 bytes and B * n * heads * d * sizeof(dtype) after it; 0
 * when the window tiles the grid or the problem is empty; -1 on a shape or
 * dtype the padded entry point rejects.  Pure host function. */
long long squad_attn_padded_workspace_bytes(int B, int heads, int T, int Hs, int Ws,
                                            int wt, int wh, int ww, int d, int dtype);

/* FLOPs of one squad_attn_fwd_padded call, counted as squad_attn_flops on the
 * padded grid (the work done): 4*B*heads*d*n_p*(m + N_w), n_p = T*Hp*Wp,
 * N_w = n_p/m.  -1 on a rejected shape.  Pure host function. */
double squad_attn_flops_padded(int B, int heads, int T, int Hs, int Ws,
                               int wt, int wh, int ww, int d);

/* Algorithmic HBM bytes of one squad_attn_fwd_padded call: each pass reads
 * three rows per padded-grid token-head, the local pass writes one per padded
 * token-head and the global pass one per real token-head:
 * (7*n_p + n)*B*heads*d*sizeof(dtype).  -1 on a rejected shape or dtype. */
double squad_attn_bytes_padded(int B, int heads, int T, int Hs, int Ws,
                               int wt, int wh, int ww, int d, int dtype);

/* The window of the pages' FLOP-conformance sweep for a (T, Hs, Ws) grid
 * (paperpeel full text, appendix paragraph "What is measured": the window
 * spans the whole temporal extent, its spatial extents keep the grid's aspect
 * ratio and its volume follows sqrt(n); integer extents, padding where it does
 * not divide the grid).  Rule: wt = T; the continuous optimum
 * wh*ww = sqrt(n)/T with wh:ww = Hs:Ws; wh and ww each rounded down or up
 * (kept within 1..Hs and 1..Ws); of those windows the least closed-form cost
 * 4hd(n_p*m + n_p^2/m) on the padded grid, ties to the aspect ratio nearer the
 * grid's, then to the smaller window.  Gives 21x2x4 at 21x22x40 and at
 * 21x30x52, as the pages state.  SQUAD_ERR_SHAPE for an extent < 1 or
 * T*Hs*Ws >= 2^31; SQUAD_ERR_NULL for a NULL output pointer.  Pure host
 * function. */
squad_status_t squad_window_solve(int T, int Hs, int Ws, int* wt, int* wh, int* ww);

/* Gradients of squad_attn_fwd (the chain rule of its two softmax attentions;
 * the pages train through the operator, SQuad paper sec. 3.3 and sec. 4, but
 * print no backward):
 *   global pass O = Attn_G(q, k, Y):  dY, and dq, dk contributions;
 *   local pass  Y = Attn_L(q, k, v):  dv, and dq, dk contributions with dY as
 *                                     the upstream gradient;
 * where for one attention with P = softmax(q k^T / sqrt(d)), D = rowsum(dO*O),
 * dS = P * (dO v^T - D): dq = dS k / sqrt(d), dk = dS^T q / sqrt(d),
 * dv = P^T dO.
 *
 * q, k, v: the forward's inputs; out: its output O; dout: dL/dO; dq, dk, dv:
 * receive dL/dq, dL/dk, dL/dv.  All [B, n, heads, d] of one dtype, as for
 * squad_attn_fwd (windows must tile the grid).  workspace: device buffer of at
 * least squad_attn_bwd_workspace_bytes(...) bytes, 16-byte aligned: the
 * recomputed local output Y, dY and the global pass's dq, dk contributions,
 * all in the dtype, and, in bf16, float32 per row of Y: its log-sum-exp
 * (which the local pass's backward reuses instead of recomputing it) and
 * D = rowsum(dY * Y) (which the global pass's backward computes from what it
 * holds, so the local pass's backward does not read Y) (contents on entry
 * ignored; one workspace must not serve calls that may run at the same
 * time).  Three kernels are enqueued on `stream`: the local pass (recomputing
 * Y), the global pass's backward, the local pass's backward.  In bf16, P and
 * dS enter the MFMAs rounded to bf16 and the global pass's dq, dk
 * contributions are stored in bf16; sums are float32.
 *
 * Errors as squad_attn_fwd for the shape, dtype and sizes; SQUAD_ERR_NULL for
 * any NULL tensor; SQUAD_ERR_WORKSPACE for a NULL or too small workspace;
 * SQUAD_ERR_ALIGN for any pointer not 16-byte aligned; SQUAD_ERR_ALIAS if a
 * gradient overlaps an input, another gradient or the workspace, or the
 * workspace overlaps an input (inputs may overlap one another). */
squad_status_t squad_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                              int B, int heads, int T, int Hs, int Ws,
                              int wt, int wh, int ww, int d,
                              int dtype, hipStream_t stream);

/* squad_attn_fwd for training: the same two kernels and the same `out` (bit
 * for bit), and the local pass's output Y, which squad_attn_fwd keeps only
 * inside `out`, written to `y` instead (the global pass then reads its values
 * from `y`), plus, in bf16, the log-sum-exp of Y's rows to `lse` ([B, n,
 * heads] float32, in log2 units of the scores scaled by log2(e)/sqrt(d)), so
 * that squad_attn_bwd_saved need not recompute them.  Same HBM traffic as
 * squad_attn_fwd (the extra lse is 1/(2d) of a tensor).  y: [B, n, heads, d]
 * in the dtype.  Errors as squad_attn_fwd; then SQUAD_ERR_NULL for a NULL y
 * (or lse in bf16; lse is ignored in float32), SQUAD_ERR_ALIGN for y or lse
 * not 16-byte aligned, SQUAD_ERR_ALIAS if y or lse overlaps q, k, v, out or
 * each other.  Two kernels on `stream`. */
squad_status_t squad_attn_fwd_save(const void* q, const void* k, const void* v, void* out, void* y, float* lse,
                                   int B, int heads, int T, int Hs, int Ws,
                                   int wt, int wh, int ww, int d,
                                   int dtype, hipStream_t stream);

/* squad_attn_bwd from the activations squad_attn_fwd_save kept (y, and lse in
 * bf16; both unchanged since) instead of recomputing them: the same two
 * backward kernels and the same gradients bit for bit, without the local
 * pass's recomputation.  workspace: at least
 * squad_attn_bwd_saved_workspace_bytes(...) bytes (dY and the global pass's
 * dq, dk contributions, and in bf16 the local pass's D).  Errors as
 * squad_attn_bwd; SQUAD_ERR_NULL, SQUAD_ERR_ALIGN for y and lse as for the
 * tensors; SQUAD_ERR_ALIAS also if y or lse overlaps a gradient or the
 * workspace. */
squad_status_t squad_attn_bwd_saved(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                    const void* y, const float* lse, void* dq, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes,
                                    int B, int heads, int T, int Hs, int Ws,
                                    int wt, int wh, int ww, int d,
                                    int dtype, hipStream_t stream);

/* Bytes of workspace squad_attn_bwd_saved needs (0 for an empty problem, -1
 * on a shape or dtype it rejects).  Pure host function. */
long long squad_attn_bwd_saved_workspace_bytes(int B, int heads, int T, int Hs, int Ws,
                                               int wt, int wh, int ww, int d, int dtype);

/* Validation only for squad_attn_bwd (pure host function). */
squad_status_t squad_attn_check_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                    const void* dq, const void* dk, const void* dv,
                                    const void* workspace, size_t workspace_bytes,
                                    int B, int heads, int T, int Hs, int Ws,
                                    int wt, int wh, int ww, int d, int dtype);

/* Bytes of workspace squad_attn_bwd needs (0 for an empty problem, -1 on a
 * shape or dtype it rejects).  Pure host function. */
long long squad_attn_bwd_workspace_bytes(int B, int heads, int T, int Hs, int Ws,
                                         int wt, int wh, int ww, int d, int dtype);

/* FLOPs of the gradients counted like squad_attn_flops: per attention the
 * scores and the products dP, dV, dQ, dK, i.e. 2.5 * squad_attn_flops
 * (recomputing Y is not counted).  -1 on a rejected shape.  Pure host
 * function. */
double squad_attn_bwd_flops(int B, int heads, int T, int Hs, int Ws,
                            int wt, int wh, int ww, int d);

/* HBM bytes of one squad_attn_bwd call as its three kernels move them:
 * E*sizeof(dtype)*21 in bf16 and E*sizeof(dtype)*22 in float32, with
 * E = B*n*heads*d (recompute of Y: 3 reads, 1 write; global backward: q, k,
 * Y, O, dO read, dY and the dq, dk contributions written; local backward: q,
 * k, v, dY and the contributions read, and Y in float32 only, dq, dk, dv
 * written; the per-row float32 arrays are not counted).  -1 on a rejected
 * shape or dtype.  Pure host function. */
double squad_attn_bwd_bytes(int B, int heads, int T, int Hs, int Ws,
                            int wt, int wh, int ww, int d, int dtype);

/* Validation only: the status any compute entry point would return for these
 * arguments before launching (SQUAD_OK when it would launch).  Pure host
 * function: makes no HIP call and never dereferences the pointers. */
squad_status_t squad_attn_check(const void* q, const void* k, const void* v, const void* out,
                                int B, int heads, int T, int Hs, int Ws,
                                int wt, int wh, int ww, int d, int dtype);

/* Largest m or N_w the kernels accept for head dim d and dtype (0 if the pair
 * is unsupported).  Pure host function. */
int squad_attn_max_len(int d, int dtype);

/* FLOPs of one squad_attn_fwd call counting 2 per multiply-add of the two
 * matmuls of each pass: 4*B*heads*d*n*(m + N_w) (paperpeel full text, appendix
 * FLOP conformance paragraph: cost 4hd(nm + n^2/m)).  Returns -1 on a shape the
 * compute entry points would reject with SQUAD_ERR_SHAPE.  Pure host function. */
double squad_attn_flops(int B, int heads, int T, int Hs, int Ws,
                        int wt, int wh, int ww, int d);

/* Algorithmic HBM bytes of one squad_attn_fwd call as two unfused passes,
 * each reading three [B, n, heads, d] tensors and writing one:
 * 8*B*n*heads*d*sizeof(dtype).  -1 on a rejected shape or dtype. */
double squad_attn_bytes(int B, int heads, int T, int Hs, int Ws,
                        int wt, int wh, int ww, int d, int dtype);

/* Static description of a status code (never NULL). */
const char* squad_status_str(int status);

/* hipError_t of the last SQUAD_ERR_HIP returned on the calling thread
 * (0 if none). */
int squad_attn_last_hip_error(void);

/* Version of this ABI (bumped on any change; 2 adds the padded entry points,
 * the backward and SQUAD_ERR_WORKSPACE; 3 the saved-activation forward and
 * backward, and the padded workspace's region for Y; 4 the padded forward
 * without allocation and SQUAD_ERR_SCRATCH). */
int squad_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SQUAD_ATTN_H */
