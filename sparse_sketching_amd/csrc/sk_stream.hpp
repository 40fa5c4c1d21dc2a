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
// scalar-base form.  Every element of A is read once per pass, so the load
// carries the nontemporal hint: the streamed rows do not displace what the
// caches hold for reuse, and the read rate rises (on gfx950 the fused FP16
// sketch of a 2^20 x 256 matrix ran 11 % faster with it, the register
// BlockPerm apply 18 %).  (The host pass of the compiler only parses kernel
// bodies; it sees a plain load.)
template <int K>
__device__ __forceinline__ FVec<K> load_row(uint64_t base, uint32_t off) {
    typedef float vk_t __attribute__((ext_vector_type(K)));
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(1))) const vk_t gvk_t;
    typedef __attribute__((address_space(1))) const char gchar;
    const vk_t v = __builtin_nontemporal_load(
        reinterpret_cast<gvk_t *>(reinterpret_cast<gchar *>(base) + off));
#else
    const vk_t v = *reinterpret_cast<const vk_t *>(reinterpret_cast<const char *>(base) + off);
#endif
    FVec<K> r;
#pragma unroll
    for (int i = 0; i < K; ++i) r.x[i] = v[i];
    return r;
}

// A wave-uniform 64-bit address, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_addr(uint64_t p) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
}

}  // namespace sk
