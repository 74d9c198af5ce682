// float32 kernel for one SQuad-Attention pass: the plain debug / reference
// path (fp32 storage and arithmetic, no MFMA).  Same problem decomposition and
// row-address maps as the bf16 kernel.
//
// One workgroup (4 waves) per problem.  The d axis is processed in chunks of
// DC columns: the chunk of V for all L rows of the problem is staged in LDS
// before any output of that chunk is written, and later chunks of V are never
// written before they are staged, so `vals == out` (in place) is safe.  Each
// wave handles query rows wave, wave+4, ...: scores one key per lane, exact
// softmax (max, exp, sum), then the weighted sum of the staged V chunk.
// Padded grids (g.pad) name rows by packed padded coordinates: q, k and the
// local pass's values are read through mirror images, the local outputs of
// padded rows go to the side buffer yp, and the global pass takes its values
// for padded rows from there and stores real rows only.
#include "squad_internal.h"

namespace squad {
namespace {

constexpr int DC = 32;      // d columns per staged chunk
constexpr int NWAVE = 4;

template <int D>
__global__ __launch_bounds__(64 * NWAVE) void pass_f32_kernel(PassGeom g, const float* __restrict__ qp,
                                                               const float* __restrict__ kp, const float* vp,
                                                               float* op, float* yp, float scale) {
    __shared__ float vs[kMaxLen * DC];
    __shared__ float ps[NWAVE][kMaxLen];
    __shared__ int tab[kMaxLen];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int L = g.L;
    const int row_stride = g.heads * D;

    const ProblemIndex pr = decode_problem(g, blockIdx.x);
    // run-time pass and padding selectors
    int base;
    if (g.pad) base = g.global ? slot_coords(g, pr.pi) : win_coords(g, pr.pi);
    else base = g.global ? slot_offset(g, pr.pi) : win_origin(g, pr.pi);
    const int64_t bh = (int64_t)pr.b * g.n * row_stride + (int64_t)pr.h * D;
    const int64_t bh_pad = (int64_t)pr.b * g.npad * row_stride + (int64_t)pr.h * D;

    for (int r = tid; r < L; r += blockDim.x) {
        if (g.pad) tab[r] = g.global ? win_coords(g, r) : slot_coords(g, r);
        else tab[r] = g.global ? win_origin(g, r) : slot_offset(g, r);
    }
    __syncthreads();

    // row r of q and k (and of the local pass's values)
    auto src = [&](int r) -> int64_t {
        return bh + (int64_t)(g.pad ? mirrored_token(g, base + tab[r]) : base + tab[r]) * row_stride;
    };
    // row r of Y, which is the global pass's values and either pass's output:
    // real rows in out (vals), padded rows in the side buffer; a padded row of
    // the global pass's output is not stored (nullptr)
    auto y_row = [&](float* real_base, int r, bool store) -> float* {
        if (!g.pad || is_real(g, base + tab[r])) return real_base + src(r);
        if (store && g.global) return nullptr;
        return yp + bh_pad + (int64_t)pad_index(g, base + tab[r]) * row_stride;
    };

    for (int c0 = 0; c0 < D; c0 += DC) {
        for (int x = tid; x < L * DC; x += blockDim.x) {
            const int r = x / DC, e = x % DC;
            vs[x] = g.global ? y_row(const_cast<float*>(vp), r, false)[c0 + e] : vp[src(r) + c0 + e];
        }
        __syncthreads();
        for (int r = wave; r < L; r += NWAVE) {
            const float* qrow = qp + src(r);
            float mx = -INFINITY;
            for (int kk = lane; kk < L; kk += 64) {
                const float* krow = kp + src(kk);
                float s = 0.0f;
                for (int e = 0; e < D; ++e) s = fmaf(qrow[e], krow[e], s);
                s *= scale;
                ps[wave][kk] = s;
                mx = fmaxf(mx, s);
            }
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            float sum = 0.0f;
            for (int kk = lane; kk < L; kk += 64) {
                const float e = expf(ps[wave][kk] - mx);
                ps[wave][kk] = e;
                sum += e;
            }
            for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            float* orow = y_row(op, r, true);
            if (lane < DC && orow) {
                float acc = 0.0f;
                for (int kk = 0; kk < L; ++kk) acc = fmaf(ps[wave][kk], vs[kk * DC + lane], acc);
                orow[c0 + lane] = acc / sum;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        __syncthreads();
    }
}

template <int D>
hipError_t launch_d(const PassGeom& g, const void* q, const void* k, const void* v, void* o, void* y,
                    hipStream_t st) {
    const float scale = 1.0f / sqrtf((float)D);
    hipLaunchKernelGGL(pass_f32_kernel<D>, dim3(g.nprob), dim3(64 * NWAVE), 0, st, g,
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<float*>(o), static_cast<float*>(y), scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pass_f32(const PassGeom& g, int d, const void* q, const void* k, const void* vals, void* out,
                           void* ypad, hipStream_t stream) {
    if (d == 128) return launch_d<128>(g, q, k, vals, out, ypad, stream);
    return launch_d<64>(g, q, k, vals, out, ypad, stream);
}

}  // namespace squad
