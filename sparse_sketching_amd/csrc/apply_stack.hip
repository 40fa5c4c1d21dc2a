// Launches of the LDS-privatized SparseStack apply (sk_stack_apply.hpp) for
// FP32 and FP16 accumulation, and of the workspace reduce that finishes the
// store-and-reduce flush.
#include "sk_internal.hpp"
#include "sk_stack_apply.hpp"

namespace sk {
namespace {

template <class T, int W, int ZG, bool NT>
const void *pick_kernel(bool full) {
    if constexpr (W == 2) {
        (void)full;
        return (const void *)k_stack_apply<T, 2, ZG, true, NT>;
    } else {
        return full ? (const void *)k_stack_apply<T, 1, ZG, true, NT>
                    : (const void *)k_stack_apply<T, 1, ZG, false, NT>;
    }
}

template <class T, int W, int ZG>
const void *pick_nt(bool full, bool nt) {
    return nt ? pick_kernel<T, W, ZG, true>(full) : pick_kernel<T, W, ZG, false>(full);
}

template <class T, int W>
const void *pick_zg(int zg, bool full, bool nt) {
    switch (zg) {
        case 1: return pick_nt<T, W, 1>(full, nt);
        case 2: return pick_nt<T, W, 2>(full, nt);
        case 4: return pick_nt<T, W, 4>(full, nt);
        case 8: return pick_nt<T, W, 8>(full, nt);
        default: return pick_nt<T, W, 0>(full, nt);
    }
}

template <class T>
hipError_t launch_stack(const LdsPlan &p, StackApplyArgs &a, int mode, hipStream_t s) {
    const bool full = p.slice == 64;
    // the kernel's slice width must match the plan the LDS and workspace
    // were sized for: two-word kernels exist for 64-lane slices only
    if ((p.words != 1 && p.words != 2) || (p.words == 2 && !full) || p.slice != a.sp ||
        p.slice < 8 || p.slice > 64)
        return hipErrorInvalidValue;
    // one block group reads each row of A once: nontemporal loads
    const bool nt = p.groups == 1;
    const void *kern = p.words == 2 ? pick_zg<T, 2>(p.zg, full, nt) : pick_zg<T, 1>(p.zg, full, nt);
    hipError_t e = set_lds_limit(kern, p.lds_bytes);
    if (e != hipSuccess) return e;
    void *params[] = {&a};
    e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3(p.threads), params, p.lds_bytes, s);
    if (e != hipSuccess) return e;
    if (a.ws == nullptr) return hipSuccess;
    return launch_stack_reduce<T>(a, a.sp * p.words, mode, s);
}

StackApplyArgs make_args(const LdsPlan &p, const float *A, int64_t m, int32_t units, int64_t lda,
                         const int32_t *ri, const float *v, int32_t zeta, void *B, int32_t d,
                         int64_t ldb_units, uint32_t *ws) {
    StackApplyArgs a;
    a.A = A;
    a.row_idx = ri;
    a.val = v;
    a.B = B;
    a.ws = ws;
    a.m = m;
    a.lda = lda;
    a.ldb = ldb_units;
    a.rows_per_chunk = p.rows_per_chunk;
    a.units = units;
    a.d = d;
    a.zeta = zeta;
    a.sp = p.slice;
    a.chunks = (int32_t)p.chunks;
    a.slices = (int32_t)p.slices;
    a.groups = p.groups;
    a.zg = p.zg;
    return a;
}

}  // namespace

hipError_t launch_f32_lds(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *ri, const float *v, int32_t zeta, float *B, int32_t d,
                          int64_t ldb, uint32_t *ws, int mode, hipStream_t s) {
    StackApplyArgs a = make_args(p, A, m, n, lda, ri, v, zeta, B, d, ldb, ws);
    return launch_stack<AccF32>(p, a, mode, s);
}

hipError_t launch_f16_lds(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *ri, const float *v, int32_t zeta, uint16_t *B, int32_t d,
                          int64_t ldb, uint32_t *ws, int mode, hipStream_t s) {
    StackApplyArgs a = make_args(p, A, m, n / 2, lda, ri, v, zeta, B, d, ldb / 2, ws);
    return launch_stack<AccF16>(p, a, mode, s);
}

}  // namespace sk
