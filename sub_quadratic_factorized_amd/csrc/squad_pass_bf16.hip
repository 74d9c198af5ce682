// bf16 MFMA kernel for one SQuad-Attention pass on gfx950 (CDNA4).
//
// A pass is a batch of independent softmax attentions ("problems", see
// PassGeom): softmax(Q K^T / sqrt(d)) V over the L rows of a window (local
// pass) or of one slot across all windows (global pass).  The re-indexing
// between the passes is only the row-address map applied on load and store; no
// view is ever materialised in HBM.
//
// Workgroup organisation
//   * Persistent: a workgroup walks work items blockIdx.x, +gridDim.x, ...: a
//     whole problem, or for problems of more than 24 query tiles in a pass
//     that is not in place one of the 2 parts of its query rows.  An item is
//     owned by one workgroup, which reads all of its rows before it writes
//     any (this is what makes the in-place global pass safe).  Problems of
//     more than 24 tiles that are not split take their query rows in two
//     parts one after the other, the first part keeping every value row in
//     LDS for the second, so no value row is read from memory after the first
//     part's outputs are written.
//   * The work of an item (of each query part of it, above) is NB =
//     ceil(L/32) steps.  Step b brings in 32 rows of K and of V (block b of
//     this problem) and 32 rows of Q (block b of the NEXT item's query rows).
//     Every thread stages one 16-byte chunk of each in registers, PD steps
//     ahead of use: ~PD * 3 * 32 * D * 2 bytes per workgroup are in flight
//     while the MFMAs run.  Loads are unconditional
//     (rows past the end clamped to the last row; steps past the last item
//     read one fixed chunk, or, through buffer descriptors, nothing), so each
//     stays in flight until its data is stored.
//   * K and V blocks go to double-buffered LDS slots (one barrier per step);
//     Q blocks go to an LDS Q stage from which each wave copies its 16-row
//     query tiles into registers at the first step of the problem.
//   * Scores are computed transposed, S^T = K Q^T (16x16x32 bf16 MFMA): each
//     lane then holds 4+4 keys of one query row, which is the B-operand layout
//     of O^T = V^T P^T, so probabilities never leave registers.  V stays
//     row-major in LDS and is fetched with the transposing LDS read.  The row
//     sum of P is one more MFMA against a tile of ones.
//   * Softmax is online across key blocks in the exp2 domain with a lazily
//     refreshed running maximum (refreshed only when a block's maximum exceeds
//     it by more than 2^8), so the accumulator rescale is rare and P <= 256;
//     the cross-lane reduction of the block maximum runs only then.
//     On request (the training forward's local pass, and the backward's
//     recompute of it) each row's log-sum-exp is stored as well.
#include "squad_internal.h"
#include "squad_layout.h"
#include "squad_mfma.h"

#include <mutex>

namespace squad {
namespace {

constexpr int BR = kBlockRows;
constexpr float kRescaleHeadroom = 8.0f;  // log2 units

template <int D>
using Geo = BlockGeo<D>;

// D: head dim; QT: 16-row query tiles per wave; MAXW: waves per workgroup
// (upper bound, >= NCH/64 so every thread stages exactly one chunk per tensor);
// PD: steps in flight (even); WPE: waves per SIMD the register budget is sized
// for; LMAX: longest problem of this instance (sizes the LDS Q stage); QSTAGE:
// stream Q through the LDS stage (else each wave loads its Q tiles straight
// into registers at a problem's first step, for problems too long to stage).
// A work item is a problem or, for long problems (PassGeom::parts > 1), one
// part of its query rows; the item streams all of the problem's keys and
// values either way.
// GP: the global pass (rows of a problem are windows at one slot) rather than
// the local pass (rows are the slots of one window).  PAD: a padded grid (rows
// named by packed padded coordinates; q, k and the local pass's values read
// through mirror images; padded rows of Y in the side buffer yp).  SPLIT:
// items are parts of problems (PassGeom::parts > 1); otherwise items are
// whole problems and the part logic compiles away.  FAST (unpadded grids whose
// batch elements span less than 4 GiB per tensor): loads and stores go
// through buffer descriptors based at a problem's base row, so a chunk's
// address is a single 32-bit offset, and loads of dead steps return zeros
// without a memory access.  VRES (resident values; whole problems of up to
// 2 * QT * 16 * waves rows, Q straight from memory): an item is a problem
// whose query rows are taken in parts of QT * 16 * waves rows one after the
// other, each part a pass over all key blocks; the first part stores every
// value block in its own LDS slot and the later parts read them there, their
// value loads dead.  All value rows are in LDS before the first part's
// outputs are written, so the in-place global pass stays safe, and each
// value row is read from memory once.
template <int D, int QT, int PD, int LMAX, bool QSTAGE, bool GP, bool PAD, bool SPLIT, bool FAST, bool VRES>
__device__ __forceinline__ void pass_body(const PassGeom& g, const uint16_t* __restrict__ qp,
                                          const uint16_t* __restrict__ kp, const uint16_t* vp, uint16_t* op,
                                          uint16_t* yp, float* lse_out, float scale_log2) {
    using G = Geo<D>;
    constexpr int OPH = QT >= 3 ? 2 : 1;  // parts the K and V operands of a step are read in
    static_assert(PD % 2 == 0, "the LDS buffer of a step must be known at compile time");
    constexpr int QROWS = QSTAGE ? (LMAX + BR - 1) / BR * BR : 1;
    __shared__ __attribute__((aligned(16))) uint16_t kbuf[2][BR * G::KSTR];
    static_assert(!VRES || (!QSTAGE && !SPLIT), "resident values: whole problems, Q straight from memory");
    constexpr int VBUFS = VRES ? (LMAX + BR - 1) / BR : 2;
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[VBUFS][BR * G::VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t qstage[QROWS * G::KSTR];
    __shared__ uint32_t tab[kMaxLen];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int L = g.L;
    const int NB = (L + BR - 1) / BR;  // key / value blocks of a problem
    // rows of the Q stage filled per item (all of a problem's, or of a part's)
    constexpr int QCAP = QSTAGE ? (LMAX + BR - 1) / BR * BR : 0;
    const int nmine = (g.nitems - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    // VRES: query parts of prow rows, one after another
    const int prow = VRES ? QT * 16 * (int)(blockDim.x >> 6) : L;
    const int vparts = VRES ? (L + prow - 1) / prow : 1;
    const int total = nmine * NB * vparts;  // steps
    const int row_stride = g.heads * D;
    const bool ragged = NB * BR != L;
    // this thread's chunk of every block: row ld_row of the block, 16-byte column ld_col
    const bool stager = tid < G::NCH;
    const int ch = stager ? tid : G::NCH - 1;
    const int ld_row = ch / G::KC;
    const int ld_col = (ch % G::KC) * 8;

    // row r of any problem of this pass sits at a fixed token offset from the
    // problem's base token (padded grids: at fixed packed coordinates; FAST:
    // the offset in bytes, and the table filled up to whole blocks with the
    // last row, so the loader needs no clamp)
    static_assert(!(FAST && PAD), "FAST is for unpadded grids");
    for (int r = tid; r < (FAST ? NB * BR : L); r += blockDim.x) {
        const int rr = FAST ? min(r, L - 1) : r;
        const int tv = PAD ? (GP ? win_coords(g, rr) : slot_coords(g, rr))
                           : (GP ? win_origin(g, rr) : slot_offset(g, rr));
        tab[r] = FAST ? (uint32_t)tv * (uint32_t)(row_stride * 2) : (uint32_t)tv;
    }
    __syncthreads();

    // A work item: unpadded, the offset of its problem's base token row (row
    // r adds tab[r] * row_stride elements, FAST tab[r] bytes); padded, the
    // (b, h) offsets into the tensors
    // and into the side buffer, and the packed base coordinates; and its query
    // rows q0 .. q0 + qn - 1 of the problem.
    struct Prob {
        int64_t off, yoff;
        int base, q0, qn;
    };
    auto problem = [&](int it) -> Prob {
        int p = (int)blockIdx.x + it * (int)gridDim.x, part = 0;
        if (SPLIT) {  // item 8 (c * parts + part) + x -> problem 8 c + x
            const int y = p >> 3;
            const int c = (int)fdiv((uint32_t)y, g.div_parts);
            part = y - c * g.parts;
            p = c * 8 + (p & 7);
        }
        const int q0 = SPLIT ? part * g.part_tiles * 16 : 0;
        const int qn = SPLIT ? min(L - q0, g.part_tiles * 16) : L;
        const ProblemIndex pr = decode_problem(g, p);
        if (PAD)
            return Prob{(int64_t)pr.b * g.n * row_stride + (int64_t)pr.h * D,
                        (int64_t)pr.b * g.npad * row_stride + (int64_t)pr.h * D,
                        GP ? slot_coords(g, pr.pi) : win_coords(g, pr.pi), q0, qn};
        const int base = GP ? slot_offset(g, pr.pi) : win_origin(g, pr.pi);
        return Prob{((int64_t)pr.b * g.n + base) * row_stride + (int64_t)pr.h * D, 0, 0, q0, qn};
    };
    // offset, in q, k and the local pass's values, of the row with table entry tv
    auto src_off = [&](const Prob& pr, uint32_t tv) -> int64_t {
        if (PAD) return pr.off + (int64_t)mirrored_token(g, pr.base + (int)tv) * row_stride;
        if (FAST) return pr.off + (int64_t)(tv >> 1);
        return pr.off + (int64_t)tv * row_stride;
    };
    // FAST: a buffer descriptor based at a problem's base row covering the
    // rest of the tensor (none when the problem is dead)
    const int64_t tensor_elems = (int64_t)(g.nprob / g.P) * g.n * D;
    auto rsrc = [&](const void* base, const Prob& pr, bool live) {
        const int64_t left = (tensor_elems - pr.off) * 2;
        const uint32_t nrec = !live ? 0u : left >= (int64_t)0xffffffffu ? 0xffffffffu : (uint32_t)left;
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(static_cast<const uint16_t*>(base)) + (live ? pr.off : 0), 0, (int)nrec,
            0x00020000);
    };

    // ---- loader -------------------------------------------------------------
    // Step (it, b) stages K and V rows of block b of item it and Q rows of
    // block b of item it+1's query rows.  Past-the-end rows are clamped to
    // the last row (their scores are masked, their probabilities zero, their
    // outputs never stored); Q blocks past an item's query rows read a dead
    // address.
    u32x4 sk[PD], sv[PD], sq[PD];
    int ld_it = 0, ld_b = 0, ld_part = 0;
    // loads of steps past the last problem, and of Q past the last problem,
    // all read the first 16 bytes of the tensor (one cached line, never used;
    // FAST: a descriptor without records, which returns zeros)
    bool ld_dead = nmine <= 0;
    bool q_dead = nmine <= 1;
    Prob ld_p = nmine > 0 ? problem(0) : Prob{0, 0, 0, 0, 1};
    Prob ld_q = nmine > 1 ? problem(1) : Prob{0, 0, 0, 0, 1};

    // FAST: descriptors of the loader's problems, and this thread's row
    // offsets for the next call (read one call ahead)
    const uint32_t col_bytes = (uint32_t)ld_col * 2u;
    __amdgpu_buffer_rsrc_t rk, rv, rq, rdead;
    uint32_t nk_off = 0, nq_off = 0;
    if constexpr (FAST) {
        rk = rsrc(kp, ld_p, !ld_dead);
        rv = rsrc(vp, ld_p, !ld_dead);
        rq = rsrc(qp, ld_q, !q_dead);
        rdead = rsrc(qp, ld_q, false);
        nk_off = tab[ld_row];
        if (SPLIT) nq_off = tab[ld_q.q0 + min(ld_row, ld_q.qn - 1)];
    }
    // the loader's next step: the next key block, the next query part of the
    // same problem (VRES), or the first block of the next item (true)
    auto advance = [&]() -> bool {
        if (++ld_b < NB) return false;
        ld_b = 0;
        if (VRES && ++ld_part < vparts) return false;
        ld_part = 0;
        ++ld_it;
        ld_dead = ld_it >= nmine;
        q_dead = ld_it + 1 >= nmine;
        ld_p = ld_q;
        if (!q_dead) ld_q = problem(ld_it + 1);
        return true;
    };
    auto issue_fast = [&](u32x4& dk, u32x4& dv, u32x4& dq) {
        const uint32_t o = nk_off + col_bytes;
        dk = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
        // VRES: value loads past the first query part return zeros unread
        dv = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(VRES && ld_part > 0 ? rdead : rv, o, 0, 0));
        if (QSTAGE) {
            if (SPLIT)
                dq = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   ld_b * BR >= ld_q.qn ? rdead : rq, nq_off + col_bytes, 0, 0));
            else
                dq = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
        }
        if (advance()) {
            rk = rsrc(kp, ld_p, !ld_dead);
            rv = rsrc(vp, ld_p, !ld_dead);
            rq = rsrc(qp, ld_q, !q_dead);
        }
        nk_off = tab[ld_b * BR + ld_row];
        if (SPLIT) nq_off = tab[ld_q.q0 + min(ld_b * BR + ld_row, ld_q.qn - 1)];
    };
    auto issue = [&](u32x4& dk, u32x4& dv, u32x4& dq) {
        if constexpr (FAST) {
            issue_fast(dk, dv, dq);
            return;
        }
        const uint32_t tv = tab[min(ld_b * BR + ld_row, L - 1)];
        const int64_t a = src_off(ld_p, tv) + ld_col;
        // the global pass's values are the local outputs: on a padded grid a
        // padded row's come from the side buffer
        const uint16_t* vb = vp;
        int64_t av = a;
        if (PAD && GP && !is_real(g, ld_p.base + (int)tv)) {
            vb = yp;
            av = ld_p.yoff + (int64_t)pad_index(g, ld_p.base + (int)tv) * row_stride + ld_col;
        }
        dk = *reinterpret_cast<const u32x4*>(kp + (ld_dead ? 0 : a));
        // VRES: value loads past the first query part read the tensor's first
        // 16 bytes (one cached line; never used)
        dv = *reinterpret_cast<const u32x4*>(vb + (ld_dead || (VRES && ld_part > 0) ? 0 : av));
        if (QSTAGE) {
            // row of the next item's query rows (unsplit: the key / value row)
            const uint32_t tq = SPLIT ? tab[ld_q.q0 + min(ld_b * BR + ld_row, ld_q.qn - 1)] : tv;
            const bool qd = q_dead || (SPLIT && ld_b * BR >= ld_q.qn);
            dq = *reinterpret_cast<const u32x4*>(qp + (qd ? 0 : src_off(ld_q, tq) + ld_col));
        }
        advance();
    };

    // swizzled position of this thread's V chunk (16-byte aligned); its two
    // 8-byte halves go to fixed addresses (swapped on alternate row groups)
    const int v_put = v_chunk_offset<D>(ld_row, ld_col / 8);
    const bool v_swap = v_halves_swapped<D>(ld_row);
    const int v_lo = v_put + (v_swap ? 4 : 0), v_hi = v_put + (v_swap ? 0 : 4);

    // VRES: value block blk goes to its own slot, in the first query part only
    auto put = [&](const u32x4& dk, const u32x4& dv, const u32x4& dq, int buf, int blk, int part) {
        if (stager) {
            *reinterpret_cast<u32x4*>(&kbuf[buf][ld_row * G::KSTR + ld_col]) = dk;
            if (!VRES || part == 0) {
                uint16_t* vd = vbuf[VRES ? blk : buf];
                *reinterpret_cast<u32x2*>(&vd[v_lo]) = u32x2{dv.x, dv.y};
                *reinterpret_cast<u32x2*>(&vd[v_hi]) = u32x2{dv.z, dv.w};
            }
            if (QSTAGE && (!SPLIT || blk * BR < QCAP))
                *reinterpret_cast<u32x4*>(&qstage[(blk * BR + ld_row) * G::KSTR + ld_col]) = dq;
        }
    };

    // ---- per-wave compute state --------------------------------------------
    bf16x8 qreg[QT][G::KS];
    f32x4 oacc[QT][G::DT];
    f32x4 osum[QT];  // every row: running sum of P for the lane's query
    bf16x8 pk[QT];
    float mrun[QT];
    // mrun + kRescaleHeadroom, kept for instances of up to two tiles per wave
    // (the 3- and 4-tile ones have no registers to spare and add it per block)
    constexpr bool KEEP_THR = QT <= 2;
    float mthr[KEEP_THR ? QT : 1];
    Prob cur_p{0, 0, 0, 0, 1};
    __amdgpu_buffer_rsrc_t ro;
    if constexpr (FAST) ro = rsrc(op, cur_p, false);
    int c_it = 0, c_part = 0;
    // the rows of query part `part` of item `it` (VRES), else the item's
    auto item_prob = [&](int it, int part) -> Prob {
        Prob p = problem(it);
        if (VRES) {
            p.q0 = part * prow;
            p.qn = min(L - p.q0, prow);
        }
        return p;
    };
    // waves past the item's last query tile only stage data; a wave's partial
    // tiles compute on clamped rows and are never stored (unsplit: the same
    // for every item)
    bool computes = wave * QT * 16 < L;

    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    // Q tiles of this wave (from the LDS stage, or straight from memory) into
    // MFMA B-operand registers
    auto read_q = [&]() {
        const Prob qprob = QSTAGE ? Prob{0, 0, 0, 0, 1} : item_prob(c_it, c_part);
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const int row = (wave * QT + t) * 16 + li;
#pragma unroll
            for (int s = 0; s < G::KS; ++s) {
                if (QSTAGE) {
                    qreg[t][s] = *reinterpret_cast<const bf16x8*>(&qstage[row * G::KSTR + (4 * s + lg) * 8]);
                } else {
                    const int64_t a = src_off(qprob, tab[qprob.q0 + min(row, qprob.qn - 1)]) + (4 * s + lg) * 8;
                    qreg[t][s] = *reinterpret_cast<const bf16x8*>(qp + a);
                }
            }
        }
    };

    auto start_problem = [&]() {
        cur_p = item_prob(c_it, c_part);
        if constexpr (FAST) ro = rsrc(op, cur_p, true);
        if (SPLIT || VRES) computes = wave * QT * 16 < cur_p.qn;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            mrun[t] = -INFINITY;
            if (KEEP_THR) mthr[KEEP_THR ? t : 0] = -INFINITY;
            osum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < G::DT; ++dt) oacc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // V operands of a step (instances whose K and V operands are read whole,
    // OPH == 1): read right after the score MFMAs are issued, before the
    // softmax, so that their LDS latency hides behind the softmax arithmetic
    // (a transposing fetch: lane (li, lg) addresses row 4*lg + li/4, and that
    // +16, at 4 consecutive d: column 4*(dt/2) + li%4, half dt%2; it receives 4
    // consecutive keys of one d column)
    bf16x8 vop[G::DT];
    auto read_v = [&](int buf) {
        const uint16_t* vb = vbuf[buf];
        const int vr = v_fetch_row(li, lg);
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) {
            const int off = v_half_offset<D>(vr, v_fetch_col(li, dt), v_fetch_half(dt));
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb[off]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb[off + 16 * G::VSTR]));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            vop[dt] = __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
        }
    };

    // max(a, b) of finite or -inf scores as med3(a, b, big) with big above any
    // score (|score| <= d * 448^2 in bf16 at d <= 128); big passes through an
    // empty asm statement so that the compiler cannot fold it into fmaxf
    float big = 3.0e38f;
    asm volatile("" : "+s"(big));
    auto max2 = [&](float a, float b) { return __builtin_amdgcn_fmed3f(a, b, big); };

    // K block: scores of this wave's tiles, online-softmax update, bf16 P.
    auto k_step = [&](int buf, int blk) {
        f32x4 s0[QT], s1[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            s0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            s1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const uint16_t* kb = kbuf[buf];
        // the K operands in OPH parts (instances of 3+ tiles per wave hold only
        // half of them at a time, a scheduling barrier between the halves)
#pragma unroll
        for (int h = 0; h < OPH; ++h) {
            constexpr int NS = G::KS / OPH;
            bf16x8 ka0[NS], ka1[NS];
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int s = h * NS + i;
                ka0[i] = *reinterpret_cast<const bf16x8*>(&kb[li * G::KSTR + (4 * s + lg) * 8]);
                ka1[i] = *reinterpret_cast<const bf16x8*>(&kb[(16 + li) * G::KSTR + (4 * s + lg) * 8]);
            }
#pragma unroll
            for (int i = 0; i < NS; ++i) {
#pragma unroll
                for (int t = 0; t < QT; ++t) {
                    const bf16x8 qs = qreg[t][h * NS + i];
                    s0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[i], qs, s0[t], 0, 0, 0);
                    s1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[i], qs, s1[t], 0, 0, 0);
                }
            }
            if (OPH > 1) __builtin_amdgcn_sched_barrier(0);
            if (OPH == 1) {
                // every K operand read ahead of the score MFMAs (one LDS round
                // trip per step instead of one per pair of MFMAs)
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * G::KS, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * G::KS * QT, 0);
            }
        }
        if constexpr (OPH == 1) {
            read_v(VRES ? blk : buf);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * G::DT, 1);
        }
        const bool mask = ragged && blk == NB - 1;
        const int kbase = blk * BR + 4 * lg;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            {
                if (mask) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (kbase + i >= L) s0[t][i] = -INFINITY;
                        if (kbase + 16 + i >= L) s1[t][i] = -INFINITY;
                    }
                }
                // the block maximum of the lane's 8 keys: med3 against a bound
                // above every score is the maximum, without the operand
                // canonicalisation fmaxf would add on MFMA results
                const float mx = max2(max2(max2(s0[t][0], s0[t][1]), max2(s0[t][2], s0[t][3])),
                                      max2(max2(s1[t][0], s1[t][1]), max2(s1[t][2], s1[t][3])));
                // a lane's own keys decide whether the row needs a new running
                // maximum (exactly when the row's keys do); only then is the
                // maximum reduced across the row's four lanes
                const float thr = KEEP_THR ? mthr[KEEP_THR ? t : 0] : mrun[t] + kRescaleHeadroom;
                if (__builtin_amdgcn_ballot_w64(mx * scale_log2 > thr) != 0) {
                    const float mnew = fmaxf(mrun[t], row_max4(mx) * scale_log2);
                    const float alpha = __builtin_amdgcn_exp2f(mrun[t] - mnew);
                    osum[t] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < G::DT; ++dt) oacc[t][dt] *= alpha;
                    mrun[t] = mnew;
                    if (KEEP_THR) mthr[KEEP_THR ? t : 0] = mnew + kRescaleHeadroom;
                }
                const float nm = -mrun[t];
                bf16x8 pv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s0[t][i], scale_log2, nm)));
                    pv[4 + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s1[t][i], scale_log2, nm)));
                }
                pk[t] = pv;
            }
        }
    };

    // V block: O^T += V^T P^T and the row sums.  Output d-tiles are used in
    // pairs (tile 2p row r holds d = 32p + 8(r/4) + r%4, tile 2p+1 the same
    // plus 4) so a lane's 4+4 accumulator rows are 8 consecutive d.
    auto v_step = [&](int buf) {
        uint16_t* vb = vbuf[buf];
        const int vr = v_fetch_row(li, lg);
#pragma unroll
        for (int t = 0; t < QT; ++t)
            osum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk[t], osum[t], 0, 0, 0);
        if constexpr (OPH == 1) {  // V operands already read (read_v)
#pragma unroll
            for (int t = 0; t < QT; ++t)
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt)
                    oacc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pk[t], oacc[t][dt], 0, 0, 0);
            return;
        }
        // the V operands in OPH parts, as the K operands above
#pragma unroll
        for (int h = 0; h < OPH; ++h) {
            constexpr int ND = G::DT / OPH;
            bf16x8 va[ND];
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                const int dt = h * ND + i;
                const int off = v_half_offset<D>(vr, v_fetch_col(li, dt), v_fetch_half(dt));
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb[off]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb[off + 16 * G::VSTR]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                va[i] = __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
            }
#pragma unroll
            for (int t = 0; t < QT; ++t)
#pragma unroll
                for (int i = 0; i < ND; ++i)
                    oacc[t][h * ND + i] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i], pk[t], oacc[t][h * ND + i], 0, 0, 0);
            if (OPH > 1) __builtin_amdgcn_sched_barrier(0);
        }
    };

    // after the last block: normalise and store this wave's rows of the problem
    auto finish_problem = [&]() {
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            // the row sum is >= 1 (the running maximum's own term), so the
            // hardware reciprocal (1 ulp) is exact enough for a bf16 output
            const float inv = __builtin_amdgcn_rcpf(osum[t][0]);
            const int row = (wave * QT + t) * 16 + li;
            // padded grids: real rows to out, padded rows of the local pass to
            // the side buffer, padded rows of the global pass nowhere (cropped)
            bool keep = row < cur_p.qn;
            if constexpr (FAST) {
                if (keep) {
                    const uint32_t tv = tab[cur_p.q0 + row];
#pragma unroll
                    for (int p = 0; p < G::DT / 2; ++p) {
                        bf16x8 o;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            o[i] = static_cast<__bf16>(oacc[t][2 * p][i] * inv);
                            o[4 + i] = static_cast<__bf16>(oacc[t][2 * p + 1][i] * inv);
                        }
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ro,
                                                               tv + 16u * lg + 64u * (uint32_t)p, 0, 0);
                    }
                    // optional row log-sum-exp (log2 units, scores scaled by
                    // log2(e)/sqrt(d)), [B, n, heads] float32
                    if (lse_out && lg == 0)
                        lse_out[(cur_p.off + (int64_t)(tv >> 1)) / D] = mrun[t] + __builtin_log2f(osum[t][0]);
                }
                continue;
            }
            uint16_t* dst = op;
            if (keep) {
                const uint32_t tv = tab[cur_p.q0 + row];
                if (!PAD) {
                    dst = op + cur_p.off + (int64_t)tv * row_stride + 8 * lg;
                } else if (is_real(g, cur_p.base + (int)tv)) {
                    dst = op + src_off(cur_p, tv) + 8 * lg;
                } else {
                    keep = !GP;
                    dst = yp + cur_p.yoff + (int64_t)pad_index(g, cur_p.base + (int)tv) * row_stride + 8 * lg;
                }
            }
            if (keep) {
#pragma unroll
                for (int p = 0; p < G::DT / 2; ++p) {
                    bf16x8 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o[i] = static_cast<__bf16>(oacc[t][2 * p][i] * inv);
                        o[4 + i] = static_cast<__bf16>(oacc[t][2 * p + 1][i] * inv);
                    }
                    *reinterpret_cast<bf16x8*>(dst + 32 * p) = o;
                }
                // optional row log-sum-exp (log2 units, scores scaled by
                // log2(e)/sqrt(d)) of unpadded grids, [B, n, heads] float32
                if (!PAD && lse_out && lg == 0)
                    lse_out[(dst - op) / D] = mrun[t] + __builtin_log2f(osum[t][0]);
            }
        }
    };

    // prologue: Q of the first item straight into the stage, then PD steps in
    // flight.  A wave copies 64 / KC rows per iteration (a 16-byte chunk per
    // lane), so the start-up waits for few memory round trips.
    if (QSTAGE && nmine > 0) {
        const Prob p0 = problem(0);
        constexpr int RPW = 64 / G::KC;
        const int c = lane % G::KC;
        for (int r = wave * RPW + lane / G::KC; r < QCAP; r += (blockDim.x >> 6) * RPW) {
            const int64_t a = src_off(p0, tab[p0.q0 + min(r, p0.qn - 1)]);
            *reinterpret_cast<u32x4*>(&qstage[r * G::KSTR + c * 8]) = *reinterpret_cast<const u32x4*>(qp + a + c * 8);
        }
    }
#pragma unroll
    for (int u = 0; u < PD; ++u) issue(sk[u], sv[u], sq[u]);
    __syncthreads();

    // Step e: (at a problem's first step: copy its Q tiles out of the stage and
    // wait for every wave to have done so), store the step's blocks into LDS
    // buffer e%2 and the Q stage, issue the loads of step e+PD, one barrier,
    // then the K and V work.  The K/V buffer written at step e was last read at
    // step e-2, which every wave finished before passing the barrier of step e-1.
    // (VRES: value slot b is written at step b of a problem's first part and
    // was last read by the previous problem's last part, at least NB steps
    // earlier; the problem's last part ends with the last value read.)
    // The loop runs whole groups of PD steps.  Loads and LDS stores happen on
    // every step, past the end too (clamped addresses, never consumed), so on
    // every path the staged loads are in issue order (slot 0 oldest) and each
    // wait only covers the slot being stored; only the compute is guarded.
    int blk = 0;
    for (int e0 = 0; e0 < total; e0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const bool live = e0 + u < total;
            if (live && blk == 0) {
                read_q();
                start_problem();
                __syncthreads();
            }
            put(sk[u], sv[u], sq[u], u & 1, blk, c_part);
            issue(sk[u], sv[u], sq[u]);
            __syncthreads();
            if (live) {
                if (computes) {
                    k_step(u & 1, blk);
                    v_step(VRES ? blk : (u & 1));
                }
                if (++blk == NB) {
                    if (computes) finish_problem();
                    blk = 0;
                    if (!VRES || ++c_part == vparts) {
                        c_part = 0;
                        ++c_it;
                    }
                }
            }
        }
    }
}

// The two passes as distinct kernels (so profiles tell them apart).
template <int D, int QT, int MAXW, int PD, int WPE, int LMAX, bool QSTAGE, bool PAD, bool SPLIT, bool FAST,
          bool VRES = false>
__global__ __launch_bounds__(64 * MAXW) __attribute__((amdgpu_waves_per_eu(WPE))) void squad_local_pass_bf16(
    PassGeom g, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp, const uint16_t* vp, uint16_t* op,
    uint16_t* yp, float* lse_out, float scale_log2) {
    pass_body<D, QT, PD, LMAX, QSTAGE, false, PAD, SPLIT, FAST, VRES>(g, qp, kp, vp, op, yp, lse_out, scale_log2);
}

template <int D, int QT, int MAXW, int PD, int WPE, int LMAX, bool QSTAGE, bool PAD, bool SPLIT, bool VRES = false>
__global__ __launch_bounds__(64 * MAXW) __attribute__((amdgpu_waves_per_eu(WPE))) void squad_global_pass_bf16(
    PassGeom g, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp, const uint16_t* vp, uint16_t* op,
    uint16_t* yp, float* lse_out, float scale_log2) {
    pass_body<D, QT, PD, LMAX, QSTAGE, true, PAD, SPLIT, false, VRES>(g, qp, kp, vp, op, yp, lse_out, scale_log2);
}

// Workgroups for a persistent launch over nprob items, a multiple of `mult`
// (when at least mult fit): as many as fit, less any that would only thin out
// the last round, so every workgroup walks the same number of items or one
// fewer.
// The FAST loader's 32-bit byte offsets: a row's offset from its problem's base
// row, plus a chunk's column, stays below 2^32 when a batch element of a
// tensor spans less than 4 GiB (minus a row).
template <int D>
bool fast_ok(const PassGeom& g) {
    return !g.pad && (int64_t)g.n * g.heads * D * 2 + (int64_t)g.heads * D * 2 <= (int64_t)0xffffffffu;
}

int grid_for(const void* kern, int threads, int nprob, int mult) {
    struct Entry {
        const void* k;
        int threads, dev, occ;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    int occ = -1;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].k == kern && cache[i].threads == threads && cache[i].dev == dev) occ = cache[i].occ;
    }
    if (occ < 0) {
        occ = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess || occ < 1) occ = 1;
        std::lock_guard<std::mutex> lock(mu);
        if (used < 64) cache[used++] = Entry{kern, threads, dev, occ};
    }
    long long want = (long long)occ * device_cu_count();
    if (want >= mult) want -= want % mult;
    if (want >= nprob) return nprob;
    const long long rounds = (nprob + want - 1) / want;
    long long grid = (nprob + rounds - 1) / rounds;
    if (want >= mult) grid = (grid + mult - 1) / mult * mult;  // still <= want
    return (int)grid;
}

// Launch menu.  A problem of length L needs ceil(L/16) query tiles spread over
// the waves of one workgroup; a workgroup has at least NCH/64 waves (8 at
// d = 128, 4 at d = 64) so that every thread stages one chunk per tensor.  The
// register budget follows the waves that share a SIMD (<= 12 waves: 168
// VGPRs; 8 waves: 256).  Problems of up to 12 tiles run one tile per wave
// with two steps in flight (four left fewer registers for the operand reads
// and ran slower), of 13-24 tiles 2 or 3 tiles per wave on 8 waves (each key
// and value read once).
// Longer ones are split into 2 parts of query rows (items) run by the 2-tile
// instance when the problem count is a multiple of 8 and the pass is not in
// place (a part writes its rows of `out` while another part of the problem
// may still be reading them as values otherwise): the parts of a problem are
// 8 items apart and the grid is a multiple of 8 * parts, so they run in the
// same round on workgroups 8 apart, which round-robin dispatch puts on the
// same XCD, and their repeated key / value reads are mostly served by its L2.
// Otherwise (in place, or a problem count not a multiple of 8) a workgroup
// takes a whole problem and its two query parts one after the other on the
// same 2-tile layout, keeping every value row in LDS from the first part
// (128 KB at L = 512, d = 128), so the second part reads only keys and
// queries from memory and the update stays in place.  With 24 heads on
// 21x68x120 and 21x4x5 windows the in-place 408-window global pass takes
// 1.46 ms this way, against 2.10 ms as two d-half items that each computed
// all scores, and 1.40 ms split into query parts out of place, which stays
// the choice where it applies.  The unpadded local pass takes the FAST
// loader when a batch element of a tensor spans less than 4 GiB.
template <int D, int QT, int MAXW, int PD, int WPE, int LMAX, bool QSTAGE, bool PAD, bool FAST, bool SPLIT = false,
          bool VRES = false>
hipError_t launch_one(const PassGeom& g, int waves, const void* q, const void* k, const void* v, void* o, void* y,
                      float* lse, hipStream_t st) {
    using KernelFn = void (*)(PassGeom, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*,
                              float*, float);
    KernelFn kfn;
    if constexpr (FAST)
        kfn = &squad_local_pass_bf16<D, QT, MAXW, PD, WPE, LMAX, QSTAGE, PAD, SPLIT, true, VRES>;
    else
        kfn = g.global ? &squad_global_pass_bf16<D, QT, MAXW, PD, WPE, LMAX, QSTAGE, PAD, SPLIT, VRES>
                       : &squad_local_pass_bf16<D, QT, MAXW, PD, WPE, LMAX, QSTAGE, PAD, SPLIT, false, VRES>;
    const void* kern = reinterpret_cast<const void*>(kfn);
    const int threads = 64 * waves;
    // resident values: at most two query parts of QT * 16 * waves rows
    const int tiles_max = VRES ? 2 * QT * waves : QT * waves;
    if (waves * 64 < Geo<D>::NCH || waves > MAXW || g.part_tiles * 16 > LMAX || g.part_tiles > tiles_max ||
        (g.parts > 1) != SPLIT || (SPLIT && g.nprob % 8 != 0) || (VRES && g.nitems != g.nprob) ||
        (FAST && (g.global || !fast_ok<D>(g))))
        return hipErrorInvalidConfiguration;  // the menu never asks for this
    // the query parts of one problem run in the same round, 8 apart
    const int mult = g.parts > 1 ? 8 * g.parts : 1;
    const int grid = grid_for(kern, threads, g.nitems, mult);
    const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf((float)D);
    hipLaunchKernelGGL(kfn, dim3(grid), dim3(threads), 0, st, g, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                       static_cast<uint16_t*>(y), lse, scale_log2);
    return hipGetLastError();
}

// Problems of more query tiles than this are split into query parts when the
// pass is not in place and the problem count is a multiple of 8.
constexpr int kSplitTiles = 24;

bool splits(const PassGeom& g) { return (g.L + 15) / 16 > kSplitTiles && g.nprob % 8 == 0; }

template <int D, bool PAD, bool FAST>
hipError_t launch_menu(const PassGeom& g0, const void* q, const void* k, const void* v, void* o, void* y, float* lse,
                       hipStream_t st) {
    constexpr int minw = Geo<D>::NCH / 64;
    const int tiles = (g0.L + 15) / 16;
    PassGeom g = g0;
    if (splits(g) && v != o) {
        g.parts = (tiles + 15) / 16;
        g.part_tiles = (tiles + g.parts - 1) / g.parts;
        g.nitems = g.nprob * g.parts;
        g.div_parts = make_fastdiv((uint32_t)g.parts);
    }
    const int waves = g.part_tiles > minw ? g.part_tiles : minw;
    if (g.parts > 1) return launch_one<D, 2, 8, 4, 2, 256, true, PAD, FAST, true>(g, 8, q, k, v, o, y, lse, st);
    if (tiles <= 12) return launch_one<D, 1, 12, 2, 3, 192, true, PAD, FAST>(g, waves, q, k, v, o, y, lse, st);
    if (tiles <= 16) return launch_one<D, 2, 8, 4, 2, 256, true, PAD, FAST>(g, 8, q, k, v, o, y, lse, st);
    if (tiles <= 24) return launch_one<D, 3, 8, 2, 2, 384, true, PAD, FAST>(g, 8, q, k, v, o, y, lse, st);
    // not split into query parts (in place, or a problem count not a multiple
    // of 8): whole problems, their query rows in two parts of 16 tiles on the
    // 2-tile layout, the value rows kept in LDS from the first part (Q
    // straight from memory: no LDS is left for a stage)
    return launch_one<D, 2, 8, 4, 2, 512, false, PAD, FAST, false, true>(g, 8, q, k, v, o, y, lse, st);
}

template <int D, bool PAD>
hipError_t launch_d(const PassGeom& g, const void* q, const void* k, const void* v, void* o, void* y, float* lse,
                    hipStream_t st) {
    if constexpr (!PAD)
        if (!g.global && fast_ok<D>(g)) return launch_menu<D, false, true>(g, q, k, v, o, y, lse, st);
    return launch_menu<D, PAD, false>(g, q, k, v, o, y, lse, st);
}

}  // namespace

bool pass_bf16_splits(const PassGeom& g) { return splits(g); }

hipError_t launch_pass_bf16(const PassGeom& g, int d, const void* q, const void* k, const void* vals, void* out,
                            void* ypad, float* lse_out, hipStream_t stream) {
    if (g.pad) {
        if (d == 128) return launch_d<128, true>(g, q, k, vals, out, ypad, nullptr, stream);
        return launch_d<64, true>(g, q, k, vals, out, ypad, nullptr, stream);
    }
    if (d == 128) return launch_d<128, false>(g, q, k, vals, out, nullptr, lse_out, stream);
    return launch_d<64, false>(g, q, k, vals, out, nullptr, lse_out, stream);
}

}  // namespace squad
