// Vector types and lane reductions shared by the bf16 MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace squad {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Maximum and sum over the four lanes {l, l^16, l^32, l^48} that share a
// column of a 16x16 MFMA result.  Cross-lane exchange through __shfl_xor
// (ds_bpermute): the permlane swap builtins were tried here and the compiler
// treated the two results of a swap of a value with itself as equal, folding
// the reduction to a single lane.
__device__ __forceinline__ float row_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float row_sum4(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

}  // namespace squad
