// float32 backward of one SQuad-Attention pass: the plain debug / reference
// path of the gradients (fp32 storage and arithmetic, no MFMA).
//
// One pass is a batch of independent softmax attentions O = P V with
// P = softmax(Q K^T / sqrt(d)) over the rows of a problem (see PassGeom).
// Given the pass's output O and its upstream gradient dO, the chain rule
// gives, per problem,
//     D = rowsum(dO * O),  dP = dO V^T,  dS = P * (dP - D),
//     dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO.
// One workgroup (4 waves) per problem, two phases:
//   queries: each wave takes rows r, r+4, ...: scores against every key (one
//     key per lane), softmax, dP and dS for the row, then dQ of the row; the
//     row's log-sum-exp and D go to LDS;
//   keys: each wave takes key rows: P and dS of the key against every query
//     (recomputed from the stored log-sum-exp and D), then dK and dV of the key.
// dQ and dK may add a float32 addend (the other pass's contribution) before
// they are stored.
#include "squad_internal.h"

namespace squad {
namespace {

constexpr int NWAVE = 4;

__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

template <int D>
__device__ __forceinline__ float dot_rows(const float* a, const float* b) {
    float s = 0.0f;
#pragma unroll 8
    for (int e = 0; e < D; ++e) s = fmaf(a[e], b[e], s);
    return s;
}

template <int D>
__global__ __launch_bounds__(64 * NWAVE) void bwd_pass_f32_kernel(
    PassGeom g, const float* __restrict__ qp, const float* __restrict__ kp, const float* __restrict__ vp,
    const float* __restrict__ op, const float* __restrict__ dop, const float* __restrict__ addq,
    const float* __restrict__ addk, float* __restrict__ dqp, float* __restrict__ dkp, float* __restrict__ dvp,
    float scale) {
    __shared__ float lse[kMaxLen], dd[kMaxLen];
    __shared__ float pa[NWAVE][kMaxLen], pb[NWAVE][kMaxLen];
    __shared__ int tab[kMaxLen];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int L = g.L;
    const int row_stride = g.heads * D;

    const ProblemIndex pr = decode_problem(g, blockIdx.x);
    const int base = g.global ? slot_offset(g, pr.pi) : win_origin(g, pr.pi);
    const int64_t bh = (int64_t)pr.b * g.n * row_stride + (int64_t)pr.h * D;
    for (int r = tid; r < L; r += blockDim.x) tab[r] = g.global ? win_origin(g, r) : slot_offset(g, r);
    __syncthreads();
    auto row = [&](int r) -> int64_t { return bh + (int64_t)(base + tab[r]) * row_stride; };

    // ---- queries: log-sum-exp, D, dS and dQ of each row -------------------
    for (int r = wave; r < L; r += NWAVE) {
        const float* qr = qp + row(r);
        const float* dor = dop + row(r);
        float mx = -INFINITY;
        for (int j = lane; j < L; j += 64) {
            const float s = dot_rows<D>(qr, kp + row(j)) * scale;
            pa[wave][j] = s;
            mx = fmaxf(mx, s);
        }
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int j = lane; j < L; j += 64) {
            const float e = expf(pa[wave][j] - mx);
            pa[wave][j] = e;
            sum += e;
        }
        sum = wave_sum(sum);
        float dpart = 0.0f;
        for (int e = lane; e < D; e += 64) dpart = fmaf(dor[e], op[row(r) + e], dpart);
        const float Dr = wave_sum(dpart);
        const float inv = 1.0f / sum;
        for (int j = lane; j < L; j += 64) {
            const float p = pa[wave][j] * inv;
            pa[wave][j] = p * (dot_rows<D>(dor, vp + row(j)) - Dr);  // dS
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        for (int e = lane; e < D; e += 64) {
            float acc = 0.0f;
            for (int j = 0; j < L; ++j) acc = fmaf(pa[wave][j], kp[row(j) + e], acc);
            acc *= scale;
            if (addq) acc += addq[row(r) + e];
            dqp[row(r) + e] = acc;
        }
        if (lane == 0) {
            lse[r] = mx + logf(sum);
            dd[r] = Dr;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // ---- keys: dK and dV of each key row ----------------------------------
    for (int j = wave; j < L; j += NWAVE) {
        const float* kj = kp + row(j);
        const float* vj = vp + row(j);
        for (int r = lane; r < L; r += 64) {
            const float p = expf(dot_rows<D>(qp + row(r), kj) * scale - lse[r]);
            pa[wave][r] = p;
            pb[wave][r] = p * (dot_rows<D>(dop + row(r), vj) - dd[r]);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        for (int e = lane; e < D; e += 64) {
            float av = 0.0f, ak = 0.0f;
            for (int r = 0; r < L; ++r) {
                av = fmaf(pa[wave][r], dop[row(r) + e], av);
                ak = fmaf(pb[wave][r], qp[row(r) + e], ak);
            }
            ak *= scale;
            if (addk) ak += addk[row(j) + e];
            dvp[row(j) + e] = av;
            dkp[row(j) + e] = ak;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

template <int D>
hipError_t launch_d(const PassGeom& g, const BwdArgs& a, hipStream_t st) {
    const float scale = 1.0f / sqrtf((float)D);
    hipLaunchKernelGGL(bwd_pass_f32_kernel<D>, dim3(g.nprob), dim3(64 * NWAVE), 0, st, g,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.vals), static_cast<const float*>(a.out),
                       static_cast<const float*>(a.dout), static_cast<const float*>(a.addq),
                       static_cast<const float*>(a.addk), static_cast<float*>(a.dq), static_cast<float*>(a.dk),
                       static_cast<float*>(a.dvals), scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pass_f32(const PassGeom& g, int d, const BwdArgs& a, hipStream_t stream) {
    if (a.lse || a.dd_in || a.vdot) return hipErrorInvalidValue;  // bf16 kernels only
    if (d == 128) return launch_d<128>(g, a, stream);
    return launch_d<64>(g, a, stream);
}

}  // namespace squad
