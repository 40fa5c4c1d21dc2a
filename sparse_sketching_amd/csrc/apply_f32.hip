// FP32 SparseStack flat scatter for gfx950 (wave64): the in-house FP32
// baseline.
//
// FP16 sketching page §III-A: every input row i contributes val*a to the
// zeta output rows row_idx[i*zeta + t]; A is read once and the loaded value
// is reused across the zeta loop.  §III-C: the zeta loop is peeled into
// eight guarded copies plus a remainder loop, so one kernel serves any zeta.
// One no-return global FP32 atomic add per contribution, laid out for
// wave64: 64 lanes on 64 consecutive columns of one row, so each atomic
// instruction touches 256 contiguous bytes and the row's metadata is a
// wave-uniform scalar load.  The LDS-privatized FP32 apply is in
// apply_lds.hip.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"

namespace sk {
namespace {

template <int ZETA>
__global__ __launch_bounds__(256) void k_f32_flat(const float *__restrict__ A, int64_t m, int32_t n,
                                                  int64_t lda, const int32_t *__restrict__ row_idx,
                                                  const float *__restrict__ val, int32_t zeta_rt,
                                                  float *__restrict__ B, int32_t d, int64_t ldb,
                                                  int64_t rows_per_wg) {
    constexpr int U = 4;        // rows in flight per wavefront
    const int zeta = ZETA ? ZETA : zeta_rt;
    const int32_t db = d / zeta;    // rows per stack block; entry t must lie in block t
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t col = blockIdx.x * 64 + lane;
    const bool active = col < n;
    for (int64_t r0 = (int64_t)blockIdx.y * rows_per_wg; r0 < m;
         r0 += (int64_t)gridDim.y * rows_per_wg) {
    const int64_t r1 = r0 + rows_per_wg < m ? r0 + rows_per_wg : m;
    for (int64_t base = r0 + wave; base < r1; base += 4 * U) {
        float a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 4 * u;
            a[u] = (active && i < r1) ? A[i * lda + col] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 4 * u;
            if (i >= r1) break;
            const int32_t *ri = row_idx + i * zeta;
            const float *vv = val + i * zeta;
            for_each_block<ZETA>(zeta, [&](int t) {
                const int32_t r = ri[t];
                if (active && (uint32_t)(r - t * db) < (uint32_t)db)
                    atomic_add_global_f32(B + (int64_t)r * ldb + col, a[u] * vv[t]);
            });
        }
    }
    }
}

}  // namespace

hipError_t launch_f32_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                           const int32_t *ri, const float *v, int32_t zeta, float *B, int32_t d,
                           int64_t ldb, hipStream_t s) {
    const int64_t rows_per_wg = 256;
    int64_t groups = (m + rows_per_wg - 1) / rows_per_wg;
    if (groups > 65535) groups = 65535;
    const dim3 grid((unsigned)((n + 63) / 64), (unsigned)groups);
    switch (zeta) {
        case 1: k_f32_flat<1><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        case 2: k_f32_flat<2><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        case 4: k_f32_flat<4><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        case 8: k_f32_flat<8><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        default: k_f32_flat<0><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
    }
    return hipGetLastError();
}

}  // namespace sk
