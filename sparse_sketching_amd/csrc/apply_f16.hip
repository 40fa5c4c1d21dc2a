// FP16-accumulate SparseStack flat scatter for gfx950 (wave64): the FP16
// sketching page's own design.
//
// §III-B/§III-D: inputs and signed products stay FP32; each contribution is
// rounded to FP16 with round-to-nearest-even; one lane owns a pair of
// adjacent columns, packs their two FP16 contributions into one 32-bit word
// and adds it with a packed f16x2 atomic whose result is discarded (§III-C),
// each half rounded to nearest-even, subnormals kept.  Here that is one
// no-return global_atomic_pk_add_f16 per (row, block, column pair), 64 lanes
// on 128 consecutive columns.  The LDS-privatized FP16 apply is in
// sk_stack_apply.hpp; the conversion variants are in apply_lowp.hip.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"

namespace sk {
namespace {

template <int ZETA>
__global__ __launch_bounds__(256) void k_f16_flat(const float *__restrict__ A, int64_t m,
                                                  int32_t npairs, int64_t lda,
                                                  const int32_t *__restrict__ row_idx,
                                                  const float *__restrict__ val, int32_t zeta_rt,
                                                  h2_t *__restrict__ B2, int32_t d, int64_t ldb2,
                                                  int64_t rows_per_wg) {
    constexpr int U = 4;
    const int zeta = ZETA ? ZETA : zeta_rt;
    const int32_t db = d / zeta;    // rows per stack block; entry t must lie in block t
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t pair = blockIdx.x * 64 + lane;
    const bool active = pair < npairs;
    for (int64_t r0 = (int64_t)blockIdx.y * rows_per_wg; r0 < m;
         r0 += (int64_t)gridDim.y * rows_per_wg) {
    const int64_t r1 = r0 + rows_per_wg < m ? r0 + rows_per_wg : m;
    for (int64_t base = r0 + wave; base < r1; base += 4 * U) {
        float2 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 4 * u;
            a[u] = (active && i < r1) ? *reinterpret_cast<const float2 *>(A + i * lda + 2 * pair)
                                      : float2{0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 4 * u;
            if (i >= r1) break;
            const int32_t *ri = row_idx + i * zeta;
            const float *vv = val + i * zeta;
            for_each_block<ZETA>(zeta, [&](int t) {
                const int32_t r = ri[t];
                const float v = vv[t];
                if (active && (uint32_t)(r - t * db) < (uint32_t)db)
                    atomic_add_global_h2(B2 + (int64_t)r * ldb2 + pair,
                                         cvt_rn_h2(a[u].x * v, a[u].y * v));
            });
        }
    }
    }
}

}  // namespace

hipError_t launch_f16_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                           const int32_t *ri, const float *v, int32_t zeta, uint16_t *B,
                           int32_t d, int64_t ldb, hipStream_t s) {
    const int32_t npairs = n / 2;
    h2_t *B2 = reinterpret_cast<h2_t *>(B);
    const int64_t ldb2 = ldb / 2;
    const int64_t rows_per_wg = 256;
    int64_t groups = (m + rows_per_wg - 1) / rows_per_wg;
    if (groups > 65535) groups = 65535;
    const dim3 grid((unsigned)((npairs + 63) / 64), (unsigned)groups);
    switch (zeta) {
        case 1: k_f16_flat<1><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        case 2: k_f16_flat<2><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        case 4: k_f16_flat<4><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        case 8: k_f16_flat<8><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        default: k_f16_flat<0><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
    }
    return hipGetLastError();
}

}  // namespace sk
