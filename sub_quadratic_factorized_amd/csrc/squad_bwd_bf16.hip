// bf16 MFMA backward of one SQuad-Attention pass on gfx950.
//
// A pass is a batch of independent softmax attentions O = P V with
// P = softmax(S), S = Q K^T / sqrt(d), over the rows of a problem (PassGeom).
// Given O and the upstream gradient dO (chain rule of softmax attention):
//     D = rowsum(dO * O),  dP = dO V^T,  dS = P * (dP - D),
//     dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO.
//
// One workgroup of 8 or 12 waves per problem; rows stream through LDS in
// blocks of 32 (clamped past the end) along one sequence of steps: per
// group of query tiles, NB steps over K and V; per group of key tiles, NB steps
// over Q and dO.  Every thread stages one 16-byte chunk of each of the step's
// two tensors in registers PD steps ahead of use, with unconditional loads,
// into double-buffered LDS, one barrier per step.  Two kinds of MFMA product
// occur, both on v_mfma_f32_16x16x32_bf16 with the operand layouts of the
// forward kernel:
//   * over d (S, dP): both operands are token rows, read as 16-byte row
//     chunks (the K/Q row layout in LDS, or registers loaded from memory);
//   * over tokens (dQ^T = K^T dS^T, dV^T = dO^T P, dK^T = Q^T dS): the A
//     operand is a block read transposed (the V layout and ds_read_b64_tr_b16
//     fetch of the forward kernel), the B operand is a 16x16 result tile pair
//     of the first kind packed to bf16 (its rows are the contracted tokens).
// Query sweep (waves own 16-query tiles): D from dO and O (or given per row:
// then O is not read), then one pass over K and V accumulating dQ^T; when the
// rows' log-sum-exp is given (HASLSE: the local pass, whose forward the
// backward has recomputed or the training forward kept) P is formed from it,
// otherwise dQ^T accumulates unnormalised probabilities under a running
// maximum and is divided by the row sum at the end of the pass, which also
// yields the log-sum-exp.  Key sweep (waves own 16-key tiles): a pass over Q
// and dO accumulating dV^T and dK^T from P and dS recomputed with the stored
// log-sum-exp and D, and optionally rowsum(dV * V) of the values rows (D of
// the backward of the pass that produced the values, which then need not read
// them again).  Rows past the end cost no per-element masks: keys there get a
// score of -inf in a problem's last block only, and query rows there a
// log-sum-exp of +inf and a D of 0, so their P and dS come out 0.  P and dS
// enter their MFMAs rounded to bf16, and the other pass's contributions to dQ
// and dK arrive in bf16; all sums are float32.  A problem whose keys fit one
// 16-key tile per wave and whose log-sum-exp and D are given (the local pass
// of windows up to 12 key tiles) takes the one-sweep variant further below
// instead: one pass over Q and dO, dQ reduced per block through LDS.
#include "squad_internal.h"
#include "squad_layout.h"
#include "squad_mfma.h"

namespace squad {
namespace {

constexpr int BR = kBlockRows;

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float (&lo)[4], const float (&hi)[4]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = static_cast<__bf16>(lo[i]);
        r[4 + i] = static_cast<__bf16>(hi[i]);
    }
    return r;
}

// NW: waves per workgroup (8: 256 VGPRs; 12: 168, so that problems of 9-12
// query tiles take one group per sweep instead of two); PD: steps in flight
// (even: the LDS buffers alternate by step parity).
template <int D, bool HASLSE, int NW, int PD>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW > 8 ? 3 : 2))) void squad_bwd_pass_bf16(
    PassGeom g, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const uint16_t* __restrict__ op, const uint16_t* __restrict__ dop, const uint16_t* __restrict__ addq,
    const uint16_t* __restrict__ addk, uint16_t* __restrict__ dqp, uint16_t* __restrict__ dkp,
    uint16_t* __restrict__ dvp, const float* __restrict__ lse_in, const float* __restrict__ dd_in,
    float* __restrict__ vdot, float c_log2, float scale) {
    using G = BlockGeo<D>;
    __shared__ __attribute__((aligned(16))) uint16_t rowA[2][BR * G::KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t rowB[2][BR * G::KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t trA[2][BR * G::VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t trB[2][BR * G::VSTR];
    __shared__ float lse[kMaxLen], dd[kMaxLen];
    __shared__ int tab[kMaxLen];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int L = g.L;
    const int NB = (L + BR - 1) / BR;
    const int ntiles = (L + 15) / 16;
    const int ngroups = (ntiles + NW - 1) / NW;
    const int row_stride = g.heads * D;

    const ProblemIndex pr = decode_problem(g, blockIdx.x);
    const int base = g.global ? slot_offset(g, pr.pi) : win_origin(g, pr.pi);
    const int64_t bh = (int64_t)pr.b * g.n * row_stride + (int64_t)pr.h * D;
    for (int r = tid; r < L; r += blockDim.x) tab[r] = g.global ? win_origin(g, r) : slot_offset(g, r);
    // rows past L up to the last block's end (NB * BR <= kMaxLen): log-sum-exp
    // +inf and D 0, so that the key sweep's probabilities and dS of such query
    // rows come out 0 without masking
    for (int r = L + tid; r < NB * BR; r += blockDim.x) {
        lse[r] = INFINITY;
        dd[r] = 0.0f;
    }
    __syncthreads();
    // element offset of row r of the problem (rows past the end clamped)
    auto row = [&](int r) -> int64_t { return bh + (int64_t)(base + tab[min(r, L - 1)]) * row_stride; };

    // ---- loader ---------------------------------------------------------------
    // Step kinds: the dQ pass over K and V (K -> row and transposed layouts,
    // V -> row layout), the dK / dV pass over Q and dO (both -> row and
    // transposed layouts).
    enum { kDq = 1, kDkv = 2 };
    // sweep A: per group NB dQ steps, padded to a multiple of PD so that
    // sweep B starts on slot 0
    const int live_a = ngroups * NB;
    const int nsteps_a = (live_a + PD - 1) / PD * PD;
    const int nsteps = nsteps_a + ngroups * NB;
    const bool stager = tid < G::NCH;
    const int ch = stager ? tid : G::NCH - 1;
    const int ld_row = ch / G::KC;
    const int ld_col = (ch % G::KC) * 8;
    int ld_s = 0, ld_blk = 0, ld_kind = kDq;
    u32x4 sx1[PD], sx2[PD];
    auto issue = [&](u32x4& x1, u32x4& x2) {
        const bool pad = ld_s >= live_a && ld_s < nsteps_a;  // the padding step of sweep A
        const bool dead = pad || ld_s >= nsteps;
        const int64_t a = row(ld_blk * BR + ld_row) + ld_col;
        const uint16_t* p1 = ld_kind == kDkv ? qp : kp;
        const uint16_t* p2 = ld_kind == kDkv ? dop : vp;
        x1 = *reinterpret_cast<const u32x4*>(p1 + (dead ? 0 : a));
        x2 = *reinterpret_cast<const u32x4*>(p2 + (dead ? 0 : a));
        ++ld_s;
        if (!pad && ++ld_blk == NB) {
            ld_blk = 0;
            ld_kind = ld_s >= live_a ? kDkv : kDq;
        }
    };
    const int t_put = v_chunk_offset<D>(ld_row, ld_col / 8);
    const bool t_swap = v_halves_swapped<D>(ld_row);
    auto put = [&](const u32x4& x1, const u32x4& x2, int buf, int kind) {
        if (!stager) return;
        *reinterpret_cast<u32x4*>(&rowA[buf][ld_row * G::KSTR + ld_col]) = x1;
        *reinterpret_cast<u32x4*>(&trA[buf][t_put]) = t_swap ? u32x4{x1.z, x1.w, x1.x, x1.y} : x1;
        *reinterpret_cast<u32x4*>(&rowB[buf][ld_row * G::KSTR + ld_col]) = x2;
        if (kind == kDkv)
            *reinterpret_cast<u32x4*>(&trB[buf][t_put]) = t_swap ? u32x4{x2.z, x2.w, x2.x, x2.y} : x2;
    };
    // a 16-row tile of x as the row operand (lane: row li, d = 32s + 8lg ..)
    auto load_tile = [&](const uint16_t* x, int tile, bf16x8 (&reg)[G::KS]) {
        const int64_t a = row(tile * 16 + li);
#pragma unroll
        for (int s = 0; s < G::KS; ++s) reg[s] = *reinterpret_cast<const bf16x8*>(x + a + (4 * s + lg) * 8);
    };
    auto row_op = [&](const uint16_t* rb, int half, int s) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(&rb[(half * 16 + li) * G::KSTR + (4 * s + lg) * 8]);
    };
    const int vr = v_fetch_row(li, lg);
    auto tr_op = [&](uint16_t* tb, int dt) -> bf16x8 {
        const int off = v_half_offset<D>(vr, v_fetch_col(li, dt), v_fetch_half(dt));
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&tb[off]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&tb[off + 16 * G::VSTR]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
    };
    // a transposed accumulator (rows d as the forward output tiles, column =
    // token li of `tile`) times `mul`, plus an optional bf16 addend, stored
    // to the token's row (8 consecutive d per lane and tile pair)
    auto store_rows = [&](const f32x4 (&acc)[G::DT], float mul, int tile, const uint16_t* add, uint16_t* dst) {
        const int r = tile * 16 + li;
        if (r >= L) return;
        const int64_t a = row(r) + 8 * lg;
#pragma unroll
        for (int p = 0; p < D / 32; ++p) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[i] = acc[2 * p][i] * mul;
                o[4 + i] = acc[2 * p + 1][i] * mul;
            }
            if (add) {
                const bf16x8 x = *reinterpret_cast<const bf16x8*>(add + a + 32 * p);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += (float)x[e];
            }
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = static_cast<__bf16>(o[e]);
            *reinterpret_cast<bf16x8*>(dst + a + 32 * p) = b;
        }
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < PD; ++u) issue(sx1[u], sx2[u]);

    // ---- sweep A: per query group, dQ over K and V ---------------------------
    // With the rows' log-sum-exp given, P = exp2(S c - lse) directly.  Without
    // it, the pass accumulates dQ from unnormalised probabilities exp2(S c - m)
    // under a running maximum m (refreshed, with dQ and the row sum rescaled,
    // only when some lane's keys exceed it by the headroom, as in the
    // forward), and divides by the row sum at the end, where the log-sum-exp
    // for the key sweep also becomes known: one pass over the keys instead of
    // two.
    constexpr float kHeadroom = 8.0f;  // log2 units
    bf16x8 qreg[G::KS], doreg[G::KS];
    float Dq = 0.0f, m = -INFINITY, lpart = 0.0f, lse2 = 0.0f;
    f32x4 dqacc[G::DT];
    // With one group of key tiles, the key tile of sweep B is this wave's own
    // (tile `wave`), and its K and V rows pass through LDS in sweep A's step
    // wave / 2: they are kept in registers from there instead of being read
    // from memory again at the start of sweep B (8-wave instances: the
    // 12-wave ones have no registers to spare).
    const bool kv_early = NW <= 8 && ngroups == 1;
    bf16x8 kreg[G::KS], vreg[G::KS];
    int st = 0;  // step of sweep A
    for (int s0 = 0; s0 < nsteps_a; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u, ++st) {
            const int grp = st / NB, blk = st - grp * NB;
            const int qt = grp * NW + wave;
            const bool active = st < live_a && qt < ntiles;
            put(sx1[u], sx2[u], u & 1, kDq);
            issue(sx1[u], sx2[u]);
            if (blk == 0 && active) {
                load_tile(qp, qt, qreg);
                load_tile(dop, qt, doreg);
                const int64_t a = row(qt * 16 + li);
                if (dd_in) {
                    Dq = dd_in[a / D];
                } else {
                    float part = 0.0f;
#pragma unroll
                    for (int s = 0; s < G::KS; ++s) {
                        const bf16x8 o = *reinterpret_cast<const bf16x8*>(op + a + (4 * s + lg) * 8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) part = fmaf((float)doreg[s][e], (float)o[e], part);
                    }
                    Dq = row_sum4(part);
                }
                if (HASLSE) {
                    lse2 = lse_in[a / D];
                    if (lg == 0 && qt * 16 + li < L) {
                        lse[qt * 16 + li] = lse2;
                        dd[qt * 16 + li] = Dq;
                    }
                } else {
                    m = -INFINITY;
                    lpart = 0.0f;
                }
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt) dqacc[dt] = zero;
            }
            __syncthreads();
            if (kv_early && st < live_a && blk == (wave >> 1) && wave < ntiles) {
#pragma unroll
                for (int s = 0; s < G::KS; ++s) {
                    kreg[s] = row_op(rowA[u & 1], wave & 1, s);
                    vreg[s] = row_op(rowB[u & 1], wave & 1, s);
                }
            }
            if (!active) continue;
            // dQ^T += K^T dS^T
            f32x4 sa = zero, sb = zero, pa = zero, pb = zero;
#pragma unroll
            for (int s = 0; s < G::KS; ++s) {
                sa = mfma(row_op(rowA[u & 1], 0, s), qreg[s], sa);
                sb = mfma(row_op(rowA[u & 1], 1, s), qreg[s], sb);
                pa = mfma(row_op(rowB[u & 1], 0, s), doreg[s], pa);  // dP^T
                pb = mfma(row_op(rowB[u & 1], 1, s), doreg[s], pb);
            }
            // keys past L (the last block only): score -inf, probability exp2(-inf) = 0
            if (blk == NB - 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (blk * BR + 4 * lg + i >= L) sa[i] = -INFINITY;
                    if (blk * BR + 16 + 4 * lg + i >= L) sb[i] = -INFINITY;
                }
            }
            if (!HASLSE) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(sa[i], sb[i]));
                if (__builtin_amdgcn_ballot_w64(mx * c_log2 > m + kHeadroom) != 0) {
                    const float mnew = fmaxf(m, row_max4(mx) * c_log2);
                    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
                    lpart *= alpha;
#pragma unroll
                    for (int dt = 0; dt < G::DT; ++dt) dqacc[dt] *= alpha;
                    m = mnew;
                }
            }
            const float sub = HASLSE ? lse2 : m;
            float ds0[4], ds1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(sa[i], c_log2, -sub));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(sb[i], c_log2, -sub));
                if (!HASLSE) lpart += e0 + e1;
                ds0[i] = e0 * (pa[i] - Dq);
                ds1[i] = e1 * (pb[i] - Dq);
            }
            const bf16x8 dsk = pack8(ds0, ds1);
#pragma unroll
            for (int dt = 0; dt < G::DT; ++dt) dqacc[dt] = mfma(tr_op(trA[u & 1], dt), dsk, dqacc[dt]);
            if (blk == NB - 1) {
                float mul = scale;
                if (!HASLSE) {
                    // the row's sum over its four lanes; every row has a key, so l >= 1
                    const float l = row_sum4(lpart);
                    lse2 = m + __builtin_log2f(l);
                    if (lg == 0 && qt * 16 + li < L) {
                        lse[qt * 16 + li] = lse2;
                        dd[qt * 16 + li] = Dq;
                    }
                    mul = scale / l;
                }
                store_rows(dqacc, mul, qt, addq, dqp);
            }
        }
    }

    // ---- sweep B: per key group, dV and dK over Q and dO --------------------
    // (every row's log-sum-exp and D reached LDS before the barriers since)
    f32x4 dkacc[G::DT], dvacc[G::DT];
    st = 0;  // step of sweep B
    for (int s0 = nsteps_a; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u, ++st) {
            const bool live = nsteps_a + st < nsteps;
            const int grp = st / NB, qb = st - grp * NB;
            const int kt = grp * NW + wave;
            const bool active = live && kt < ntiles;
            put(sx1[u], sx2[u], u & 1, kDkv);
            issue(sx1[u], sx2[u]);
            if (active && qb == 0) {
                if (!kv_early) {
                    load_tile(kp, kt, kreg);
                    load_tile(vp, kt, vreg);
                }
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt) dkacc[dt] = dvacc[dt] = zero;
            }
            __syncthreads();
            if (!active) continue;
            f32x4 sa = zero, sb = zero, pa = zero, pb = zero;
#pragma unroll
            for (int s = 0; s < G::KS; ++s) {
                sa = mfma(row_op(rowA[u & 1], 0, s), kreg[s], sa);  // S (queries x this wave's keys)
                sb = mfma(row_op(rowA[u & 1], 1, s), kreg[s], sb);
                pa = mfma(row_op(rowB[u & 1], 0, s), vreg[s], pa);  // dP
                pb = mfma(row_op(rowB[u & 1], 1, s), vreg[s], pb);
            }
            float pr0[4], pr1[4], ds0[4], ds1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // query rows past L: lse +inf and D 0 (set at the start), so P = 0, dS = 0
                const int q0 = qb * BR + 4 * lg + i, q1 = q0 + 16;
                const float e0 = __builtin_amdgcn_exp2f(fmaf(sa[i], c_log2, -lse[q0]));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(sb[i], c_log2, -lse[q1]));
                pr0[i] = e0;
                pr1[i] = e1;
                ds0[i] = e0 * (pa[i] - dd[q0]);
                ds1[i] = e1 * (pb[i] - dd[q1]);
            }
            const bf16x8 pp = pack8(pr0, pr1), dsp = pack8(ds0, ds1);
#pragma unroll
            for (int dt = 0; dt < G::DT; ++dt) {
                dvacc[dt] = mfma(tr_op(trB[u & 1], dt), pp, dvacc[dt]);
                dkacc[dt] = mfma(tr_op(trA[u & 1], dt), dsp, dkacc[dt]);
            }
            if (qb == NB - 1) {
                store_rows(dkacc, scale, kt, addk, dkp);
                store_rows(dvacc, 1.0f, kt, nullptr, dvp);
                if (vdot) {
                    // rowsum(dV * V) of the tile's rows, dV rounded as stored:
                    // accumulator pair p holds d = 32p + 8lg .. +7 of row li,
                    // the columns of vreg[p]
                    float part = 0.0f;
#pragma unroll
                    for (int p = 0; p < D / 32; ++p)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            part = fmaf((float)static_cast<__bf16>(dvacc[2 * p][i]), (float)vreg[p][i], part);
                            part = fmaf((float)static_cast<__bf16>(dvacc[2 * p + 1][i]), (float)vreg[p][4 + i], part);
                        }
                    const float dsum = row_sum4(part);
                    const int r = kt * 16 + li;
                    if (lg == 0 && r < L) vdot[row(r) / D] = dsum;
                }
            }
        }
    }
}

// One-sweep variant, for problems of at most NW key tiles whose rows'
// log-sum-exp and D are given (the local pass).  Every wave owns one 16-key
// tile: its V rows in registers, its K rows in LDS, where K is kept whole in
// the transposing layout.  One pass over Q and dO in 32-row blocks
// accumulates dK^T and dV^T as the key sweep above does.  Per block the
// waves' dS tiles meet in LDS (row-major over the block's queries, double
// buffered), and at the start of the next block's step the first D/16 waves
// form the block's dQ^T = K^T dS^T from them (one query half and one d-tile
// pair each) and store it, while the other waves begin that step's scores:
// every input row is read from memory once, and one barrier per block orders
// both the streamed rows and dS.  One step in flight (PD = 1) on 12 waves:
// with two, registers spill, and every reload of a spilled value waits for
// all loads in flight.
template <int D, int NW, int PD>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW > 8 ? 3 : 2))) void squad_bwd_onesweep_bf16(
    PassGeom g, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const uint16_t* __restrict__ dop, const uint16_t* __restrict__ addq, const uint16_t* __restrict__ addk,
    uint16_t* __restrict__ dqp, uint16_t* __restrict__ dkp, uint16_t* __restrict__ dvp,
    const float* __restrict__ lse_in, const float* __restrict__ dd_in, float c_log2, float scale) {
    using G = BlockGeo<D>;
    static_assert(NW % 2 == 0 && NW >= D / 16, "one key tile per wave, a dQ unit per wave");
    constexpr int KMAX = 16 * NW;     // keys (and query rows) a workgroup covers
    constexpr int KBLK = KMAX / BR;   // 32-row K blocks kept in LDS
    // dS rows (queries) padded by 16 bytes: the dQ operand fetch (16 rows, two
    // 8-byte pieces per 32 lanes) then covers every bank once
    constexpr int DSTR = KMAX + 8;
    constexpr int NU = D / 16;        // dQ units: 2 query halves x DT/2 d-tile pairs
    __shared__ __attribute__((aligned(16))) uint16_t rowA[2][BR * G::KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t rowB[2][BR * G::KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t trA[2][BR * G::VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t trB[2][BR * G::VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t ktr[KBLK * BR * G::VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t dsb[2][BR * DSTR];
    __shared__ float lse[KMAX], dd[KMAX];
    __shared__ int tab[KMAX];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int L = g.L;
    const int NB = (L + BR - 1) / BR;
    const int row_stride = g.heads * D;

    const ProblemIndex pr = decode_problem(g, blockIdx.x);
    const int base = g.global ? slot_offset(g, pr.pi) : win_origin(g, pr.pi);
    // the problem's (b, h) slice: rows are 32-bit element offsets from it
    // (the launcher requires n * heads * D < 2^31)
    const int64_t bh = (int64_t)pr.b * g.n * row_stride + (int64_t)pr.h * D;
    qp += bh;
    kp += bh;
    vp += bh;
    dop += bh;
    if (addq) addq += bh;
    if (addk) addk += bh;
    dqp += bh;
    dkp += bh;
    dvp += bh;
    const int64_t bh_row = bh / D;  // per-row arrays: [B, n, heads]
    lse_in += bh_row;
    dd_in += bh_row;
    for (int r = tid; r < L; r += blockDim.x) tab[r] = g.global ? win_origin(g, r) : slot_offset(g, r);
    // query rows past L up to the last block's end: log-sum-exp +inf and D 0
    for (int r = L + tid; r < NB * BR; r += blockDim.x) {
        lse[r] = INFINITY;
        dd[r] = 0.0f;
    }
    // K blocks and dS key columns past the last block: zero (the dQ product
    // runs over all KBLK blocks; no wave writes these)
    for (int i = NB * BR * G::VSTR + tid * 8; i < KBLK * BR * G::VSTR; i += blockDim.x * 8)
        *reinterpret_cast<u32x4*>(&ktr[i]) = u32x4{0u, 0u, 0u, 0u};
    for (int i = tid; i < 2 * BR * (KMAX - NB * BR); i += blockDim.x) {
        const int b = i / (BR * (KMAX - NB * BR)), j = i - b * (BR * (KMAX - NB * BR));
        const int q = j / (KMAX - NB * BR), c = NB * BR + j - q * (KMAX - NB * BR);
        dsb[b][q * DSTR + c] = 0;
    }
    __syncthreads();
    auto row = [&](int r) -> int { return (base + tab[min(r, L - 1)]) * row_stride; };

    // ---- loader: block st of Q (row and transposed layouts) and of dO (both)
    // PD steps in flight (staging registers); the step loop is unrolled by UN
    // (even, so that the LDS buffers alternate by step parity at compile time)
    // over NB live steps plus the dQ-only step
    constexpr int UN = PD < 2 ? 2 : PD;
    static_assert(UN % PD == 0 && UN % 2 == 0, "staging slots and buffer parity per unrolled step");
    const int nsteps = (NB + 1 + UN - 1) / UN * UN;
    const bool stager = tid < G::NCH;
    const int ch = stager ? tid : G::NCH - 1;
    const int ld_row = ch / G::KC;
    const int ld_col = (ch % G::KC) * 8;
    int ld_s = 0;
    u32x4 sx1[PD], sx2[PD];
    auto issue = [&](u32x4& x1, u32x4& x2) {
        const bool dead = ld_s >= NB;
        const int a = row(ld_s * BR + ld_row) + ld_col;
        x1 = *reinterpret_cast<const u32x4*>(qp + (dead ? 0 : a));
        x2 = *reinterpret_cast<const u32x4*>(dop + (dead ? 0 : a));
        ++ld_s;
    };
    const int t_put = v_chunk_offset<D>(ld_row, ld_col / 8);
    const bool t_swap = v_halves_swapped<D>(ld_row);
    auto put = [&](const u32x4& x1, const u32x4& x2, int buf) {
        if (!stager) return;
        *reinterpret_cast<u32x4*>(&rowA[buf][ld_row * G::KSTR + ld_col]) = x1;
        *reinterpret_cast<u32x4*>(&trA[buf][t_put]) = t_swap ? u32x4{x1.z, x1.w, x1.x, x1.y} : x1;
        *reinterpret_cast<u32x4*>(&rowB[buf][ld_row * G::KSTR + ld_col]) = x2;
        *reinterpret_cast<u32x4*>(&trB[buf][t_put]) = t_swap ? u32x4{x2.z, x2.w, x2.x, x2.y} : x2;
    };
    auto row_op = [&](const uint16_t* rb, int half, int s) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(&rb[(half * 16 + li) * G::KSTR + (4 * s + lg) * 8]);
    };
    const int vr = v_fetch_row(li, lg);
    auto tr_op = [&](const uint16_t* tb, int dt) -> bf16x8 {
        const int off = v_half_offset<D>(vr, v_fetch_col(li, dt), v_fetch_half(dt));
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&tb[off]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&tb[off + 16 * G::VSTR]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
    };
    // the same fetch at a given lane offset (rows off and off + 16 of block tb)
    auto tr_at = [&](uint16_t* tb, int off) -> bf16x8 {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&tb[off]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&tb[off + 16 * G::VSTR]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < PD; ++u) issue(sx1[u], sx2[u]);

    // ---- this wave's key tile: rows, whole-problem K in LDS, per-row sums --
    // Tiles past the last K block take no part; tiles inside it but past L
    // (clamped rows) take part with probabilities forced to 0.
    const int kt = wave;
    const bool kact = kt < 2 * NB;
    const bool kdead = kt * 16 + li >= L;
    for (int r = tid; r < L; r += blockDim.x) {
        const int ri = row(r) / D;
        lse[r] = lse_in[ri];
        dd[r] = dd_in[ri];
    }
    // The wave's K rows live only in LDS (the score operand is read back from
    // the transposing layout, halves restored): registers are kept for V.
    const int kr = 16 * (kt & 1) + li;
    const bool ksw = v_halves_swapped<D>(kr);
    uint16_t* const kblk = &ktr[(kt >> 1) * BR * G::VSTR];
    bf16x8 vreg[G::KS];
    if (kact) {
        const int a = row(kt * 16 + li);
        u32x4 kx[G::KS];
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            kx[s] = *reinterpret_cast<const u32x4*>(kp + a + (4 * s + lg) * 8);
            vreg[s] = *reinterpret_cast<const bf16x8*>(vp + a + (4 * s + lg) * 8);
        }
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            const u32x4 x = kx[s];
            *reinterpret_cast<u32x4*>(&kblk[v_chunk_offset<D>(kr, 4 * s + lg)]) = ksw ? u32x4{x.z, x.w, x.x, x.y} : x;
        }
    }
    auto k_op = [&](int s) -> bf16x8 {
        const u32x4 x = *reinterpret_cast<const u32x4*>(&kblk[v_chunk_offset<D>(kr, 4 * s + lg)]);
        return __builtin_bit_cast(bf16x8, ksw ? u32x4{x.z, x.w, x.x, x.y} : x);
    };
    f32x4 dkacc[G::DT], dvacc[G::DT];
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) dkacc[dt] = dvacc[dt] = zero;

    // dQ unit of this wave: query half uh, d tiles 2 up, 2 up + 1
    const bool dq_wave = wave < NU;
    const int uh = wave & 1, up = wave >> 1;
    // The dQ rows' addend load and store are buffer operations that every
    // wave issues at every step (lanes without a row use an offset past the
    // descriptor's end: the load returns zeros, the store is dropped), so the
    // count of memory operations between a step's loads and their use is the
    // same on every path: a wait for the streamed rows then need not also
    // wait for the previous step's dQ stores to complete.  The descriptors
    // cover the rest of the batch element from the (b, h) slice (under 2^31
    // bytes: the launcher requires n * heads * D < 2^30).
    const int slice_bytes = (int)((g.n * g.heads * D - (int64_t)pr.h * D) * 2);
    const __amdgpu_buffer_rsrc_t raq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(addq ? addq : dqp), 0, addq ? slice_bytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rdq = __builtin_amdgcn_make_buffer_rsrc(dqp, 0, slice_bytes, 0x00020000);
    constexpr uint32_t kNoRow = 0x80000000u;
    int st = 0;
    for (int s0 = 0; s0 < nsteps; s0 += UN) {
#pragma unroll
        for (int u = 0; u < UN; ++u, ++st) {
            if (st > NB) break;  // uniform
            // the other pass's contribution to the dQ rows formed in this step
            const int qr = (st - 1) * BR + 16 * uh + li;
            const bool qout = dq_wave && st >= 1 && qr < L;
            const uint32_t qoff = qout ? (uint32_t)(row(qr) + 32 * up + 8 * lg) * 2u : kNoRow;
            const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(raq, qoff, 0, 0));
            put(sx1[u % PD], sx2[u % PD], u & 1);
            issue(sx1[u % PD], sx2[u % PD]);
            __syncthreads();
            f32x4 a0 = zero, a1 = zero;
            if (st >= 1 && dq_wave) {
                // dQ^T of the previous block: contraction over its keys in 32-key steps.
                // The lane's LDS addresses are rebuilt here from a laundered lane
                // index, so that they are not held in registers across the step
                // loop (where they would be spilled and reloaded, and each reload
                // waits for every load in flight).
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int qli = ln & 15, qlg = ln >> 4;
                const uint16_t* db = &dsb[(u + 1) & 1][(16 * uh + qli) * DSTR + 4 * qlg];
                const int qvr = v_fetch_row(qli, qlg);
                const int o0 = v_half_offset<D>(qvr, v_fetch_col(qli, 2 * up), 0);
                const int o1 = v_half_offset<D>(qvr, v_fetch_col(qli, 2 * up + 1), 1);
                // all KBLK key blocks (those past the problem's last are zero), so
                // that the fetches of later blocks can be issued early
#pragma unroll
                for (int ks = 0; ks < KBLK; ++ks) {
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(db + 32 * ks);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(db + 32 * ks + 16);
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
                    uint16_t* kb = &ktr[ks * BR * G::VSTR];
                    a0 = mfma(tr_at(kb, o0), bop, a0);
                    a1 = mfma(tr_at(kb, o1), bop, a1);
                }
            }
            {
                bf16x8 b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    b[i] = static_cast<__bf16>(fmaf(a0[i], scale, (float)aq[i]));
                    b[4 + i] = static_cast<__bf16>(fmaf(a1[i], scale, (float)aq[4 + i]));
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), rdq, qoff, 0, 0);
            }
            if (st < NB && kact) {
                f32x4 sa = zero, sb = zero, pa = zero, pb = zero;
#pragma unroll
                for (int s = 0; s < G::KS; ++s) {
                    const bf16x8 kop = k_op(s);
                    sa = mfma(row_op(rowA[u & 1], 0, s), kop, sa);  // S (block queries x this wave's keys)
                    sb = mfma(row_op(rowA[u & 1], 1, s), kop, sb);
                    pa = mfma(row_op(rowB[u & 1], 0, s), vreg[s], pa);  // dP
                    pb = mfma(row_op(rowB[u & 1], 1, s), vreg[s], pb);
                }
                float pr0[4], pr1[4], ds0[4], ds1[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q0 = st * BR + 4 * lg + i, q1 = q0 + 16;
                    const float e0 = kdead ? 0.0f : __builtin_amdgcn_exp2f(fmaf(sa[i], c_log2, -lse[q0]));
                    const float e1 = kdead ? 0.0f : __builtin_amdgcn_exp2f(fmaf(sb[i], c_log2, -lse[q1]));
                    pr0[i] = e0;
                    pr1[i] = e1;
                    ds0[i] = e0 * (pa[i] - dd[q0]);
                    ds1[i] = e1 * (pb[i] - dd[q1]);
                }
                const bf16x8 pp = pack8(pr0, pr1), dsp = pack8(ds0, ds1);
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt) {
                    dvacc[dt] = mfma(tr_op(trB[u & 1], dt), pp, dvacc[dt]);
                    dkacc[dt] = mfma(tr_op(trA[u & 1], dt), dsp, dkacc[dt]);
                }
                // dS of this block: query rows 4lg + i and 16 + 4lg + i, key 16 kt + li
                // (the 16-bit halves of the packed words: a bit cast of one
                // bf16 element of the vector was compiled as element 0 for all)
                uint16_t* db = &dsb[u & 1][kt * 16 + li];
                const u32x4 w = __builtin_bit_cast(u32x4, dsp);
                const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    db[(4 * lg + i) * DSTR] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
                    db[(16 + 4 * lg + i) * DSTR] = (uint16_t)(wv[2 + (i >> 1)] >> (16 * (i & 1)));
                }
            }
        }
    }

    // ---- dK, dV of this wave's tile ------------------------------------------
    const int r = kt * 16 + li;
    if (!kact || r >= L) return;
    const int a = row(r) + 8 * lg;
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
        float ok[8], ov[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ok[i] = dkacc[2 * p][i] * scale;
            ok[4 + i] = dkacc[2 * p + 1][i] * scale;
            ov[i] = dvacc[2 * p][i];
            ov[4 + i] = dvacc[2 * p + 1][i];
        }
        if (addk) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(addk + a + 32 * p);
#pragma unroll
            for (int e = 0; e < 8; ++e) ok[e] += (float)x[e];
        }
        bf16x8 bk, bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bk[e] = static_cast<__bf16>(ok[e]);
            bv[e] = static_cast<__bf16>(ov[e]);
        }
        *reinterpret_cast<bf16x8*>(dkp + a + 32 * p) = bk;
        *reinterpret_cast<bf16x8*>(dvp + a + 32 * p) = bv;
    }
}

template <int D, int NW, int PD>
hipError_t launch_onesweep(const PassGeom& g, const BwdArgs& a, hipStream_t st) {
    const float scale = 1.0f / __builtin_sqrtf((float)D);
    const float c_log2 = 1.4426950408889634f * scale;
    hipLaunchKernelGGL((squad_bwd_onesweep_bf16<D, NW, PD>), dim3(g.nprob), dim3(64 * NW), 0, st, g,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.vals), static_cast<const uint16_t*>(a.dout),
                       static_cast<const uint16_t*>(a.addq), static_cast<const uint16_t*>(a.addk),
                       static_cast<uint16_t*>(a.dq), static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dvals),
                       a.lse, a.dd_in, c_log2, scale);
    return hipGetLastError();
}

template <int D, bool HASLSE, int NW, int PD>
hipError_t launch_nw(const PassGeom& g, const BwdArgs& a, hipStream_t st) {
    const float scale = 1.0f / __builtin_sqrtf((float)D);
    const float c_log2 = 1.4426950408889634f * scale;
    hipLaunchKernelGGL((squad_bwd_pass_bf16<D, HASLSE, NW, PD>), dim3(g.nprob), dim3(64 * NW), 0, st, g,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.vals), static_cast<const uint16_t*>(a.out),
                       static_cast<const uint16_t*>(a.dout), static_cast<const uint16_t*>(a.addq),
                       static_cast<const uint16_t*>(a.addk), static_cast<uint16_t*>(a.dq),
                       static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dvals), a.lse, a.dd_in, a.vdot,
                       c_log2, scale);
    return hipGetLastError();
}

// 12 waves when they save a group of query / key tiles over 8 waves (at the
// cost of a few spilled registers and two steps in flight), else 8 waves with
// four steps in flight
template <int D, bool HASLSE>
hipError_t launch_d(const PassGeom& g, const BwdArgs& a, hipStream_t st) {
    const int tiles = (g.L + 15) / 16;
    if ((tiles + 11) / 12 < (tiles + 7) / 8) return launch_nw<D, HASLSE, 12, 2>(g, a, st);
    return launch_nw<D, HASLSE, 8, 4>(g, a, st);
}

}  // namespace

hipError_t launch_bwd_pass_bf16(const PassGeom& g, int d, const BwdArgs& a, hipStream_t stream) {
    const int tiles = (g.L + 15) / 16;
    // the local pass (log-sum-exp and D given) of windows up to 12 key tiles:
    // the one-sweep kernel (32-bit row offsets within a batch element)
    if (a.lse && a.dd_in && !a.vdot && tiles <= 12 && g.n * g.heads * d < (int64_t(1) << 30)) {
        if (tiles <= 8)
            return d == 128 ? launch_onesweep<128, 8, 4>(g, a, stream) : launch_onesweep<64, 8, 4>(g, a, stream);
        return d == 128 ? launch_onesweep<128, 12, 1>(g, a, stream) : launch_onesweep<64, 12, 2>(g, a, stream);
    }
    if (a.lse) return d == 128 ? launch_d<128, true>(g, a, stream) : launch_d<64, true>(g, a, stream);
    return d == 128 ? launch_d<128, false>(g, a, stream) : launch_d<64, false>(g, a, stream);
}

}  // namespace squad
