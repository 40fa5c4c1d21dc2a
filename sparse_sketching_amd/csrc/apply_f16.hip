// FP16-accumulate SparseStack apply kernels for gfx950 (wave64).
//
// FP16 sketching page §III-B/§III-D: inputs and signed products stay FP32;
// each contribution is rounded to FP16 with round-to-nearest-even; one lane
// owns a pair of adjacent columns, packs their two FP16 contributions into
// one 32-bit word and adds it with a packed f16x2 atomic whose result is
// discarded (§III-C), each half rounded to nearest-even, subnormals kept.
//
// Two variants:
//  * flat: one no-return global_atomic_pk_add_f16 per (row, block, column
//    pair) (the page's design; 64 lanes cover 128 consecutive columns);
//  * lds: a workgroup owns a slice of column pairs and a chunk of rows and
//    accumulates a private d x slice FP16 partial in LDS with ds_pk_add_f16;
//    at the end it adds the partial to B with packed global atomics.  The
//    arithmetic is the same RN conversion and RN FP16 additions, in a
//    two-level order; it cuts global atomic traffic by the chunk length and
//    shortens each FP16 running sum.
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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t pair = blockIdx.x * 64 + lane;
    const bool active = pair < npairs;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
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
                if (active && (uint32_t)r < (uint32_t)d)
                    atomic_add_global_h2(B2 + (int64_t)r * ldb2 + pair,
                                         cvt_rn_h2(a[u].x * v, a[u].y * v));
            });
        }
    }
}

template <int SP, int ZETA>
__global__ __launch_bounds__(1024) void k_f16_lds(const float *__restrict__ A, int64_t m,
                                                  int32_t npairs, int64_t lda,
                                                  const int32_t *__restrict__ row_idx,
                                                  const float *__restrict__ val, int32_t zeta_rt,
                                                  h2_t *__restrict__ B2, int32_t d, int64_t ldb2,
                                                  int64_t rows_per_chunk) {
    extern __shared__ uint32_t part_words[];   // d x SP packed f16x2, row-major
    h2_t *part = reinterpret_cast<h2_t *>(part_words);
    constexpr int RPW = 64 / SP;
    constexpr int U = 8;
    const int zeta = ZETA ? ZETA : zeta_rt;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pl = lane % SP;
    const int rsub = lane / SP;
    const int32_t pair = blockIdx.x * SP + pl;
    const bool active = pair < npairs;

    for (int k = threadIdx.x; k < d * SP; k += nthr) part_words[k] = 0u;
    __syncthreads();

    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < m ? r0 + rows_per_chunk : m;
    const int64_t step = (int64_t)nw * RPW;
    for (int64_t base = r0 + (int64_t)wave * RPW; base < r1; base += step * U) {
        float2 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + step * u + rsub;
            a[u] = (active && i < r1) ? *reinterpret_cast<const float2 *>(A + i * lda + 2 * pair)
                                      : float2{0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + step * u + rsub;
            if (i < r1) {
                const int32_t *ri = row_idx + i * zeta;
                const float *vv = val + i * zeta;
                for_each_block<ZETA>(zeta, [&](int t) {
                    const int32_t r = ri[t];
                    const float v = vv[t];
                    if (active && (uint32_t)r < (uint32_t)d)
                        atomic_add_lds_h2(part + r * SP + pl, cvt_rn_h2(a[u].x * v, a[u].y * v));
                });
            }
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < d * SP; k += nthr) {
        const int r = k / SP;
        const int32_t p = blockIdx.x * SP + (k - r * SP);
        const uint32_t w = part_words[k];
        if (p < npairs && w != 0u)
            atomic_add_global_h2(B2 + (int64_t)r * ldb2 + p, __builtin_bit_cast(h2_t, w));
    }
}

template <int SP>
hipError_t launch_f16_lds_sp(const LdsPlan &p, const float *A, int64_t m, int32_t npairs,
                             int64_t lda, const int32_t *ri, const float *v, int32_t zeta,
                             h2_t *B2, int32_t d, int64_t ldb2, hipStream_t s) {
    const dim3 grid((unsigned)p.slices, (unsigned)p.chunks);
    const dim3 block(p.threads);
#define SK_LAUNCH(Z)                                                                          \
    do {                                                                                      \
        auto kern = k_f16_lds<SP, Z>;                                                         \
        hipError_t e = set_lds_limit((const void *)kern, p.lds_bytes);                        \
        if (e != hipSuccess) return e;                                                        \
        kern<<<grid, block, p.lds_bytes, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2,    \
                                              p.rows_per_chunk);                              \
    } while (0)
    switch (zeta) {
        case 1: SK_LAUNCH(1); break;
        case 2: SK_LAUNCH(2); break;
        case 4: SK_LAUNCH(4); break;
        case 8: SK_LAUNCH(8); break;
        default: SK_LAUNCH(0); break;
    }
#undef SK_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_f16_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                           const int32_t *ri, const float *v, int32_t zeta, uint16_t *B,
                           int32_t d, int64_t ldb, hipStream_t s) {
    const int32_t npairs = n / 2;
    h2_t *B2 = reinterpret_cast<h2_t *>(B);
    const int64_t ldb2 = ldb / 2;
    const int64_t rows_per_wg = 256;
    const dim3 grid((unsigned)((npairs + 63) / 64), (unsigned)((m + rows_per_wg - 1) / rows_per_wg));
    switch (zeta) {
        case 1: k_f16_flat<1><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        case 2: k_f16_flat<2><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        case 4: k_f16_flat<4><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        case 8: k_f16_flat<8><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
        default: k_f16_flat<0><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, rows_per_wg); break;
    }
    return hipGetLastError();
}

hipError_t launch_f16_lds(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *ri, const float *v, int32_t zeta, uint16_t *B, int32_t d,
                          int64_t ldb, hipStream_t s) {
    const int32_t npairs = n / 2;
    h2_t *B2 = reinterpret_cast<h2_t *>(B);
    const int64_t ldb2 = ldb / 2;
    switch (p.slice) {
        case 64: return launch_f16_lds_sp<64>(p, A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, s);
        case 32: return launch_f16_lds_sp<32>(p, A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, s);
        case 16: return launch_f16_lds_sp<16>(p, A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, s);
        case 8: return launch_f16_lds_sp<8>(p, A, m, npairs, lda, ri, v, zeta, B2, d, ldb2, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sk
