// Device helpers of the kernels that stream rows of A through LDS stages
// (the fused SparseStack sketch and the register BlockPerm apply).
#pragma once
#include "sk_stack_apply.hpp"

namespace sk {

// All LDS writes of this wavefront have landed, then a workgroup barrier.
// Unlike __syncthreads this leaves the wavefront's global loads in flight,
// which is what lets the next stage stream while this one is applied.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// K floats at global address base + off (base wave-uniform, off per lane),
// loaded through the global address space so the load takes its
// scalar-base form.  (The host pass of the compiler only parses kernel
// bodies; it sees a plain load.)
template <int K>
__device__ __forceinline__ FVec<K> load_row(uint64_t base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(1))) const char gchar;
    gchar *p = reinterpret_cast<gchar *>(base) + off;
    typedef __attribute__((address_space(1))) const float2 gfloat2;
    typedef __attribute__((address_space(1))) const float4 gfloat4;
#else
    const char *p = reinterpret_cast<const char *>(base) + off;
    typedef const float2 gfloat2;
    typedef const float4 gfloat4;
#endif
    FVec<K> r;
    if constexpr (K == 2) {
        const float2 v = *reinterpret_cast<gfloat2 *>(p);
        r.x[0] = v.x;
        r.x[1] = v.y;
    } else {
        const float4 v = *reinterpret_cast<gfloat4 *>(p);
        r.x[0] = v.x;
        r.x[1] = v.y;
        r.x[2] = v.z;
        r.x[3] = v.w;
    }
    return r;
}

// A wave-uniform 64-bit address, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_addr(uint64_t p) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
}

}  // namespace sk
