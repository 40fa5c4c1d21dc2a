// Launches of the LDS-privatized SparseStack apply (sk_lock_apply.hpp) for
// FP32 and FP16 accumulation, and of the workspace reduce that finishes the
// store-and-reduce flush.
#include "sk_internal.hpp"
#include "sk_lock_apply.hpp"

namespace sk {
namespace {

template <class T>
hipError_t launch_lock(const LdsPlan &p, LockApplyArgs &a, int accumulate, hipStream_t s) {
    const dim3 grid((unsigned)p.slices, (unsigned)p.chunks);
    const dim3 block(p.threads);
#define SK_LAUNCH(Z)                                                                          \
    do {                                                                                      \
        auto kern = k_lock_apply<T, Z>;                                                       \
        hipError_t e = set_lds_limit((const void *)kern, p.lds_bytes);                        \
        if (e != hipSuccess) return e;                                                        \
        kern<<<grid, block, p.lds_bytes, s>>>(a);                                             \
    } while (0)
    switch (a.zeta) {
        case 1: SK_LAUNCH(1); break;
        case 2: SK_LAUNCH(2); break;
        case 4: SK_LAUNCH(4); break;
        case 8: SK_LAUNCH(8); break;
        default: SK_LAUNCH(0); break;
    }
#undef SK_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ws == nullptr) return e;
    const int64_t total = (int64_t)a.d * a.units;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65535) blocks = 65535;
    k_lock_reduce<T><<<dim3((unsigned)blocks), 256, 0, s>>>(a, (int32_t)p.slices, accumulate);
    return hipGetLastError();
}

LockApplyArgs make_args(const LdsPlan &p, const float *A, int64_t m, int32_t units, int64_t lda,
                        const int32_t *ri, const float *v, int32_t zeta, void *B, int32_t d,
                        int64_t ldb_units, uint32_t *ws) {
    LockApplyArgs a;
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
    return a;
}

}  // namespace

hipError_t launch_f32_lds(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *ri, const float *v, int32_t zeta, float *B, int32_t d,
                          int64_t ldb, uint32_t *ws, int accumulate, hipStream_t s) {
    LockApplyArgs a = make_args(p, A, m, n, lda, ri, v, zeta, B, d, ldb, ws);
    return launch_lock<AccF32>(p, a, accumulate, s);
}

hipError_t launch_f16_lds(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *ri, const float *v, int32_t zeta, uint16_t *B, int32_t d,
                          int64_t ldb, uint32_t *ws, int accumulate, hipStream_t s) {
    LockApplyArgs a = make_args(p, A, m, n / 2, lda, ri, v, zeta, B, d, ldb / 2, ws);
    return launch_lock<AccF16>(p, a, accumulate, s);
}

}  // namespace sk
