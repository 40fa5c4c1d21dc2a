// Device helpers shared by the SparseStack apply kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// The zeta loop of the FP16 sketching page (§III-C): a compile-time zeta is
// fully unrolled; a run-time zeta runs eight guarded unrolled copies and a
// remainder loop for t >= 8.
template <int ZETA, typename F>
__device__ __forceinline__ void for_each_block(int zeta, F &&f) {
    if constexpr (ZETA > 0) {
#pragma unroll
        for (int t = 0; t < ZETA; ++t) f(t);
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            if (t < zeta) f(t);
        for (int t = 8; t < zeta; ++t) f(t);
    }
}

// No-return atomics: the results are never read, so the compiler emits the
// forms without a return path (global_atomic_add_f32, ds_add_f32,
// global_atomic_pk_add_f16, ds_pk_add_f16).
__device__ __forceinline__ void atomic_add_global_f32(float *p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_add_lds_f32(float *p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void atomic_add_global_h2(h2_t *p, h2_t v) {
    __builtin_amdgcn_global_atomic_fadd_v2f16((__attribute__((address_space(1))) h2_t *)p, v);
}
__device__ __forceinline__ void atomic_add_lds_h2(h2_t *p, h2_t v) {
    __builtin_amdgcn_ds_atomic_fadd_v2f16((__attribute__((address_space(3))) h2_t *)p, v);
}

// Two FP32 products rounded to nearest-even FP16 each (the page's
// __float2half contract), packed low = first column.
__device__ __forceinline__ h2_t cvt_rn_h2(float x, float y) {
    return h2_t{(_Float16)x, (_Float16)y};
}

inline hipError_t set_lds_limit(const void *kern, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace sk
