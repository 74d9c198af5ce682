// bf16 MFMA kernel for one SQuad-Attention pass on gfx950 (CDNA4).
//
// A pass is a batch of independent softmax attentions ("problems", see
// PassGeom): softmax(Q K^T / sqrt(d)) V over the L rows of a window (local
// pass) or of a slot across all windows (global pass).  The re-indexing between
// the passes is nothing but the row-address map applied on load and store; no
// view is ever materialised.
//
// Workgroup organisation
//   * Persistent: a workgroup walks problems blockIdx.x, +gridDim.x, ...; one
//     problem is owned by one workgroup, so its rows are read completely before
//     any of them is written (this is what makes the in-place global pass safe).
//   * Each wave owns QT query tiles of 16 rows.  Q stays in registers as the
//     B operand of the 16x16x32 bf16 MFMA (prefetched one problem ahead).
//   * Keys and values stream through LDS in blocks of 32 rows: the item
//     sequence of a problem is K_0, V_0, K_1, V_1, ...  Every thread of the
//     workgroup stages CPL 16-byte chunks per item in registers, PD items ahead
//     of use, so ~PD*8 KB per workgroup are in flight while the MFMAs run.
//   * Scores are computed transposed, S^T = K Q^T: then each lane holds 4+4
//     keys of one query row, which is exactly the B-operand layout of
//     O^T = V^T P^T, so probabilities never leave registers.  V is written
//     transposed into LDS (V^T, keys contiguous) for the A operand.
//   * Softmax is online across key blocks with a lazily refreshed running
//     maximum (refreshed only when a block's maximum exceeds it by more than
//     2^8), so the accumulator rescale is rare; P <= 256 stays exact in range.
#include "squad_internal.h"

#include <mutex>

namespace squad {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int BR = 32;                  // keys per streamed block
constexpr float kRescaleHeadroom = 8.0f;  // log2 units

template <int D>
struct Geo {
    static constexpr int KC = D / 8;        // 16-byte chunks per row
    static constexpr int NCH = BR * KC;     // chunks per block
    static constexpr int KS = D / 32;       // k-steps of the score MFMA
    static constexpr int DT = D / 16;       // 16-row d tiles of the output
    static constexpr int KSTR = D + 8;      // K block row stride (elements)
    static constexpr int VSTR = BR + 4;     // V^T block row stride (elements)
};

// d index held by row r of output d-tile dt.  Tiles are used in pairs so that
// a lane's 4+4 accumulator rows cover 8 consecutive d (one 16-byte store).
__device__ __forceinline__ int dmap(int dt, int r) {
    return 32 * (dt >> 1) + 8 * (r >> 2) + 4 * (dt & 1) + (r & 3);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf16_value(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// D: head dim; QT: 16-row query tiles per wave; MAXW: waves per workgroup
// (upper bound); CPL, PD: 16-byte chunks per thread per item and items in
// flight; WPE: waves per SIMD the register budget is sized for; QPF: prefetch
// the next problem's Q one problem ahead (costs 4*QT*D/32 VGPRs).
template <int D, int QT, int MAXW, int CPL, int PD, int WPE, bool QPF>
__global__ __launch_bounds__(64 * MAXW) __attribute__((amdgpu_waves_per_eu(WPE))) void pass_bf16_kernel(
    PassGeom g, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* vp, uint16_t* op, float scale_log2) {
    using G = Geo<D>;
    __shared__ __attribute__((aligned(16))) uint16_t kblk[BR * G::KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vblk[D * G::VSTR];
    __shared__ int tab[kMaxLen];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int L = g.L;
    const int NB = (L + BR - 1) / BR;
    const int ipp = 2 * NB;  // items per problem
    const int ntiles = (L + 15) / 16;
    const int nmine = (g.nprob - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int total = nmine * ipp;
    const int row_stride = g.heads * D;

    // row r of any problem of this pass sits at a fixed token offset from the
    // problem's base token
    for (int r = tid; r < L; r += nthr) tab[r] = g.global ? win_origin(g, r) : slot_offset(g, r);
    __syncthreads();

    auto prob_offset = [&](int it) -> int64_t {
        const int p = (int)blockIdx.x + it * (int)gridDim.x;
        const int h = p % g.heads;
        const int t = p / g.heads;
        const int pi = t % g.P;
        const int b = t / g.P;
        const int base = g.global ? slot_offset(g, pi) : win_origin(g, pi);
        return ((int64_t)b * g.n + base) * row_stride + (int64_t)h * D;
    };

    // ---- loader: stage item (ld_it, ld_rem) in registers --------------------
    u32x4 stage[PD][CPL];
    int ld_it = 0, ld_rem = 0;
    int64_t ld_off = nmine > 0 ? prob_offset(0) : 0;

    auto issue = [&](u32x4(&dst)[CPL]) {
        const int blk = ld_rem >> 1;
        const uint16_t* src = (ld_rem & 1) ? vp : kp;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = tid + c * nthr;
            const int row = blk * BR + ch / G::KC;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (ch < G::NCH && ld_it < nmine && row < L) {
                val = *reinterpret_cast<const u32x4*>(src + ld_off + (int64_t)tab[row] * row_stride +
                                                      (ch % G::KC) * 8);
            }
            dst[c] = val;
        }
        if (++ld_rem == ipp) {
            ld_rem = 0;
            ++ld_it;
            if (ld_it < nmine) ld_off = prob_offset(ld_it);
        }
    };

    auto put = [&](const u32x4(&src)[CPL], bool is_v) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = tid + c * nthr;
            if (ch < G::NCH) {
                const int row = ch / G::KC;
                const int col = ch % G::KC;
                if (!is_v) {
                    *reinterpret_cast<u32x4*>(&kblk[row * G::KSTR + col * 8]) = src[c];
                } else {
                    uint16_t* dst = &vblk[(col * 8) * G::VSTR + row];
                    const u32x4 w = src[c];
                    dst[0 * G::VSTR] = (uint16_t)(w.x & 0xffffu);
                    dst[1 * G::VSTR] = (uint16_t)(w.x >> 16);
                    dst[2 * G::VSTR] = (uint16_t)(w.y & 0xffffu);
                    dst[3 * G::VSTR] = (uint16_t)(w.y >> 16);
                    dst[4 * G::VSTR] = (uint16_t)(w.z & 0xffffu);
                    dst[5 * G::VSTR] = (uint16_t)(w.z >> 16);
                    dst[6 * G::VSTR] = (uint16_t)(w.w & 0xffffu);
                    dst[7 * G::VSTR] = (uint16_t)(w.w >> 16);
                }
            }
        }
    };

    // ---- per-wave compute state --------------------------------------------
    bf16x8 qreg[QT][G::KS];
    bf16x8 qnext[QT][G::KS];
    f32x4 oacc[QT][G::DT];
    bf16x8 pk[QT];
    float mrun[QT], lsum[QT];
    int64_t cur_off = 0;

    auto load_q = [&](int it, bf16x8(&dst)[QT][G::KS]) {
        const bool live = it < nmine;
        const int64_t off = live ? prob_offset(it) : 0;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const int row = (wave * QT + t) * 16 + li;
            const bool ok = live && row < L;
            const uint16_t* src = qp + off + (ok ? (int64_t)tab[row] * row_stride : 0) + lg * 8;
#pragma unroll
            for (int s = 0; s < G::KS; ++s) {
                u32x4 val = {0u, 0u, 0u, 0u};
                if (ok) val = *reinterpret_cast<const u32x4*>(src + 32 * s);
                dst[t][s] = __builtin_bit_cast(bf16x8, val);
            }
        }
    };

    load_q(0, qnext);
#pragma unroll
    for (int u = 0; u < PD; ++u) issue(stage[u]);

    int c_it = 0, c_rem = 0;

    // K item: scores of this wave's query tiles against the 32 keys in LDS,
    // then the online-softmax update producing the bf16 P operand.
    auto k_step = [&](int blk) {
        if (blk == 0) {
            // a new problem starts: take the prefetched Q, prefetch the next
#pragma unroll
            for (int t = 0; t < QT; ++t)
#pragma unroll
                for (int s = 0; s < G::KS; ++s) qreg[t][s] = qnext[t][s];
            cur_off = prob_offset(c_it);
            if (QPF) load_q(c_it + 1, qnext);
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                mrun[t] = -INFINITY;
                lsum[t] = 0.0f;
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt) oacc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        f32x4 s0[QT], s1[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            s0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            s1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(&kblk[li * G::KSTR + (4 * s + lg) * 8]);
            const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(&kblk[(16 + li) * G::KSTR + (4 * s + lg) * 8]);
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                if (wave * QT + t < ntiles) {
                    s0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qreg[t][s], s0[t], 0, 0, 0);
                    s1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qreg[t][s], s1[t], 0, 0, 0);
                }
            }
        }
        const int kbase = blk * BR + 4 * lg;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            if (wave * QT + t < ntiles) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = (kbase + i < L) ? s0[t][i] * scale_log2 : -INFINITY;
                    x[4 + i] = (kbase + 16 + i < L) ? s1[t][i] * scale_log2 : -INFINITY;
                }
                float mx = x[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mnew = fmaxf(mrun[t], mx);
                if (__builtin_amdgcn_ballot_w64(mnew > mrun[t] + kRescaleHeadroom) != 0) {
                    const float alpha = __builtin_amdgcn_exp2f(mrun[t] - mnew);
                    lsum[t] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < G::DT; ++dt) oacc[t][dt] *= alpha;
                    mrun[t] = mnew;
                }
                bf16x8 pv;
                float ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint16_t pb = bf16_bits(__builtin_amdgcn_exp2f(x[i] - mrun[t]));
                    pv[i] = __builtin_bit_cast(__bf16, pb);
                    ps += bf16_value(pb);
                }
                lsum[t] += ps;
                pk[t] = pv;
            }
        }
    };

    // V item: O^T += V^T P^T for this wave's tiles; after the last block,
    // normalise and store the problem's rows.
    auto v_step = [&](int blk) {
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) {
            const int dr = dmap(dt, li);
            const u32x2 lo = *reinterpret_cast<const u32x2*>(&vblk[dr * G::VSTR + 4 * lg]);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(&vblk[dr * G::VSTR + 16 + 4 * lg]);
            const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
            for (int t = 0; t < QT; ++t)
                if (wave * QT + t < ntiles)
                    oacc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk[t], oacc[t][dt], 0, 0, 0);
        }
        if (blk == NB - 1) {
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                if (wave * QT + t < ntiles) {
                    float l = lsum[t];
                    l += __shfl_xor(l, 16);
                    l += __shfl_xor(l, 32);
                    const float inv = 1.0f / l;
                    const int row = (wave * QT + t) * 16 + li;
                    if (row < L) {
                        uint16_t* dst = op + cur_off + (int64_t)tab[row] * row_stride + 8 * lg;
#pragma unroll
                        for (int p = 0; p < D / 32; ++p) {
                            u32x4 w;
#pragma unroll
                            for (int i = 0; i < 4; i += 2) {
                                const uint32_t a0 = bf16_bits(oacc[t][2 * p][i] * inv);
                                const uint32_t a1 = bf16_bits(oacc[t][2 * p][i + 1] * inv);
                                const uint32_t b0 = bf16_bits(oacc[t][2 * p + 1][i] * inv);
                                const uint32_t b1 = bf16_bits(oacc[t][2 * p + 1][i + 1] * inv);
                                w[i / 2] = a0 | (a1 << 16);
                                w[2 + i / 2] = b0 | (b1 << 16);
                            }
                            *reinterpret_cast<u32x4*>(dst + 32 * p) = w;
                        }
                    }
                }
            }
            if (!QPF) load_q(c_it + 1, qnext);
        }
    };

    // Items alternate K_b, V_b and PD is even, so the kind of the item in
    // stage slot u is fixed: even slots carry keys, odd slots values.
    for (int e0 = 0; e0 < total; e0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int blk = c_rem >> 1;
            put(stage[u], (u & 1) != 0);
            issue(stage[u]);
            __syncthreads();
            if ((u & 1) == 0) {
                k_step(blk);
            } else {
                v_step(blk);
            }
            if (++c_rem == ipp) {
                c_rem = 0;
                ++c_it;
            }
        }
    }
}

int grid_for(const void* kern, int threads, int nprob) {
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
    const long long want = (long long)occ * device_cu_count();
    return (int)(want < nprob ? want : nprob);
}

// Launch menu.  Every problem of length L needs ceil(L/16) query tiles spread
// over the waves of one workgroup.  The register budget follows the waves that
// must share a SIMD: up to 8 waves per workgroup at 4 waves/SIMD (128 VGPRs)
// lets two workgroups share a CU; 9..12 waves take 168 VGPRs (one workgroup
// per CU); longer problems put 2 or 4 tiles on each wave.
template <int D, int QT, int MAXW, int CPL, int PD, int WPE, bool QPF>
hipError_t launch_one(const PassGeom& g, int waves, const void* q, const void* k, const void* v, void* o,
                      hipStream_t st) {
    auto kfn = &pass_bf16_kernel<D, QT, MAXW, CPL, PD, WPE, QPF>;
    const void* kern = reinterpret_cast<const void*>(kfn);
    const int threads = 64 * waves;
    const int grid = grid_for(kern, threads, g.nprob);
    const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf((float)D);
    hipLaunchKernelGGL(kfn, dim3(grid), dim3(threads), 0, st, g, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                       scale_log2);
    return hipGetLastError();
}

template <int D, int QT, int MAXW, int WPE, bool QPF, int MAXCPL>
hipError_t launch_cpl(const PassGeom& g, int waves, const void* q, const void* k, const void* v, void* o,
                      hipStream_t st) {
    const int nch = BR * D / 8;
    const int threads = 64 * waves;
    const int need = (nch + threads - 1) / threads;
    if (need > MAXCPL) return hipErrorInvalidConfiguration;  // the menu never asks for this
    if (need <= 1 || MAXCPL == 1) return launch_one<D, QT, MAXW, 1, 4, WPE, QPF>(g, waves, q, k, v, o, st);
    if (need <= 2 || MAXCPL == 2) return launch_one<D, QT, MAXW, (MAXCPL < 2 ? 1 : 2), 4, WPE, QPF>(g, waves, q, k, v, o, st);
    if (need <= 4 || MAXCPL == 4) return launch_one<D, QT, MAXW, (MAXCPL < 4 ? 1 : 4), 2, WPE, QPF>(g, waves, q, k, v, o, st);
    return launch_one<D, QT, MAXW, (MAXCPL < 8 ? 1 : 8), 2, WPE, QPF>(g, waves, q, k, v, o, st);
}

template <int D>
hipError_t launch_d(const PassGeom& g, const void* q, const void* k, const void* v, void* o, hipStream_t st) {
    // chunks per thread needed by W waves: ceil(32*D/8 / (64*W))
    const int tiles = (g.L + 15) / 16;
    if (tiles <= 8) return launch_cpl<D, 1, 8, 4, true, 8>(g, tiles, q, k, v, o, st);
    if (tiles <= 12) return launch_cpl<D, 1, 12, 3, true, 1>(g, tiles, q, k, v, o, st);
    if (tiles <= 16) return launch_cpl<D, 2, 8, 2, true, 2>(g, (tiles + 1) / 2, q, k, v, o, st);
    if (tiles <= 24) return launch_cpl<D, 3, 8, 2, false, 2>(g, (tiles + 2) / 3, q, k, v, o, st);
    return launch_cpl<D, 4, 8, 2, false, 2>(g, (tiles + 3) / 4, q, k, v, o, st);
}

}  // namespace

hipError_t launch_pass_bf16(const PassGeom& g, int d, const void* q, const void* k, const void* vals, void* out,
                            hipStream_t stream) {
    if (d == 128) return launch_d<128>(g, q, k, vals, out, stream);
    return launch_d<64>(g, q, k, vals, out, stream);
}

}  // namespace squad
