// Internal declarations shared by the SQuad-Attention HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace squad {

// Longest attended sequence (m for the local pass, N_w for the global pass)
// any kernel instance accepts.
constexpr int kMaxLen = 512;

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
    int Hs, Ws;     // grid extents (T is implied)
    int wt, wh, ww; // window extents
    int Cy, Cx;     // windows along y and x
    int global;     // 0: local pass, 1: global pass
};

// Token index of slot 0 of window c (windows numbered row-major over their
// tile coordinates (ct, cy, cx)).
__host__ __device__ inline int win_origin(const PassGeom& g, int c) {
    const int per_t = g.Cy * g.Cx;
    const int ct = c / per_t;
    const int r = c - ct * per_t;
    const int cy = r / g.Cx;
    const int cx = r - cy * g.Cx;
    return ((ct * g.wt) * g.Hs + cy * g.wh) * g.Ws + cx * g.ww;
}

// Offset, in tokens, of in-window slot j (slots numbered row-major over the
// in-window offset (jt, jy, jx)).
__host__ __device__ inline int slot_offset(const PassGeom& g, int j) {
    const int per_t = g.wh * g.ww;
    const int jt = j / per_t;
    const int r = j - jt * per_t;
    const int jy = r / g.ww;
    const int jx = r - jy * g.ww;
    return (jt * g.Hs + jy) * g.Ws + jx;
}

// Kernel launchers.  Each validates nothing (the ABI layer did) and returns the
// launch status.  `vals` may equal `out` (in-place update, race-free because
// every workgroup reads all rows of its problems before writing them, and the
// problems of a pass partition the rows).
hipError_t launch_pass_bf16(const PassGeom& g, int d, const void* q, const void* k,
                            const void* vals, void* out, hipStream_t stream);
hipError_t launch_pass_f32(const PassGeom& g, int d, const void* q, const void* k,
                           const void* vals, void* out, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace squad
