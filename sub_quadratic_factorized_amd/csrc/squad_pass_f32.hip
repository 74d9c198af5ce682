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
#include "squad_internal.h"

namespace squad {
namespace {

constexpr int DC = 32;      // d columns per staged chunk
constexpr int NWAVE = 4;

template <int D>
__global__ __launch_bounds__(64 * NWAVE) void pass_f32_kernel(PassGeom g, const float* __restrict__ qp,
                                                               const float* __restrict__ kp, const float* vp,
                                                               float* op, float scale) {
    __shared__ float vs[kMaxLen * DC];
    __shared__ float ps[NWAVE][kMaxLen];
    __shared__ int tab[kMaxLen];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int L = g.L;
    const int row_stride = g.heads * D;

    const ProblemIndex pr = decode_problem(g, blockIdx.x);
    const int base = g.global ? slot_offset(g, pr.pi) : win_origin(g, pr.pi);  // run-time pass selector
    const int64_t poff = ((int64_t)pr.b * g.n + base) * row_stride + (int64_t)pr.h * D;

    for (int r = tid; r < L; r += blockDim.x) tab[r] = g.global ? win_origin(g, r) : slot_offset(g, r);
    __syncthreads();

    for (int c0 = 0; c0 < D; c0 += DC) {
        for (int x = tid; x < L * DC; x += blockDim.x) {
            const int r = x / DC, e = x % DC;
            vs[x] = vp[poff + (int64_t)tab[r] * row_stride + c0 + e];
        }
        __syncthreads();
        for (int r = wave; r < L; r += NWAVE) {
            const float* qrow = qp + poff + (int64_t)tab[r] * row_stride;
            float mx = -INFINITY;
            for (int kk = lane; kk < L; kk += 64) {
                const float* krow = kp + poff + (int64_t)tab[kk] * row_stride;
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
            if (lane < DC) {
                float acc = 0.0f;
                for (int kk = 0; kk < L; ++kk) acc = fmaf(ps[wave][kk], vs[kk * DC + lane], acc);
                op[poff + (int64_t)tab[r] * row_stride + c0 + lane] = acc / sum;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        __syncthreads();
    }
}

template <int D>
hipError_t launch_d(const PassGeom& g, const void* q, const void* k, const void* v, void* o, hipStream_t st) {
    const float scale = 1.0f / sqrtf((float)D);
    hipLaunchKernelGGL(pass_f32_kernel<D>, dim3(g.nprob), dim3(64 * NWAVE), 0, st, g,
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<float*>(o), scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pass_f32(const PassGeom& g, int d, const void* q, const void* k, const void* vals, void* out,
                           hipStream_t stream) {
    if (d == 128) return launch_d<128>(g, q, k, vals, out, stream);
    return launch_d<64>(g, q, k, vals, out, stream);
}

}  // namespace squad
