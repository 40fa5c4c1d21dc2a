// FP32 SparseStack apply kernels for gfx950 (wave64).
//
// FP16 sketching page §III-A: every input row i contributes val*a to the
// zeta output rows row_idx[i*zeta + t]; A is read once and the loaded value
// is reused across the zeta loop.  §III-C: the zeta loop is peeled into
// eight guarded copies plus a remainder loop, so one kernel serves any zeta.
//
// Two variants:
//  * flat: one no-return global FP32 atomic add per contribution (the page's
//    scatter, laid out for wave64: 64 lanes on 64 consecutive columns of one
//    row, so each atomic instruction touches 256 contiguous bytes and the
//    row's metadata is a wave-uniform scalar load);
//  * lds: each workgroup owns a column slice and a chunk of rows, keeps a
//    private d x slice FP32 partial in LDS (LDS atomic adds), and adds the
//    partial to B with global atomics once at the end.
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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t col = blockIdx.x * 64 + lane;
    const bool active = col < n;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
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
                if (active && (uint32_t)r < (uint32_t)d)
                    atomic_add_global_f32(B + (int64_t)r * ldb + col, a[u] * vv[t]);
            });
        }
    }
}

template <int SP, int ZETA>
__global__ __launch_bounds__(1024) void k_f32_lds(const float *__restrict__ A, int64_t m, int32_t n,
                                                  int64_t lda, const int32_t *__restrict__ row_idx,
                                                  const float *__restrict__ val, int32_t zeta_rt,
                                                  float *__restrict__ B, int32_t d, int64_t ldb,
                                                  int64_t rows_per_chunk) {
    extern __shared__ float part[];  // d x SP, row-major
    constexpr int RPW = 64 / SP;     // rows per wavefront instruction
    constexpr int U = 8;             // row groups in flight per wavefront
    const int zeta = ZETA ? ZETA : zeta_rt;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cl = lane % SP;
    const int rsub = lane / SP;
    const int32_t col = blockIdx.x * SP + cl;
    const bool active = col < n;

    for (int k = threadIdx.x; k < d * SP; k += nthr) part[k] = 0.f;
    __syncthreads();

    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < m ? r0 + rows_per_chunk : m;
    const int64_t step = (int64_t)nw * RPW;
    for (int64_t base = r0 + (int64_t)wave * RPW; base < r1; base += step * U) {
        float a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + step * u + rsub;
            a[u] = (active && i < r1) ? A[i * lda + col] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + step * u + rsub;
            if (i < r1) {
                const int32_t *ri = row_idx + i * zeta;
                const float *vv = val + i * zeta;
                for_each_block<ZETA>(zeta, [&](int t) {
                    const int32_t r = ri[t];
                    if (active && (uint32_t)r < (uint32_t)d)
                        atomic_add_lds_f32(part + r * SP + cl, a[u] * vv[t]);
                });
            }
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < d * SP; k += nthr) {
        const int r = k / SP;
        const int32_t c = blockIdx.x * SP + (k - r * SP);
        const float x = part[k];
        if (c < n && x != 0.f) atomic_add_global_f32(B + (int64_t)r * ldb + c, x);
    }
}

template <int SP>
hipError_t launch_f32_lds_sp(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                             const int32_t *ri, const float *v, int32_t zeta, float *B, int32_t d,
                             int64_t ldb, hipStream_t s) {
    const dim3 grid((unsigned)p.slices, (unsigned)p.chunks);
    const dim3 block(p.threads);
#define SK_LAUNCH(Z)                                                                          \
    do {                                                                                      \
        auto kern = k_f32_lds<SP, Z>;                                                         \
        hipError_t e = set_lds_limit((const void *)kern, p.lds_bytes);                        \
        if (e != hipSuccess) return e;                                                        \
        kern<<<grid, block, p.lds_bytes, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb,           \
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

hipError_t launch_f32_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                           const int32_t *ri, const float *v, int32_t zeta, float *B, int32_t d,
                           int64_t ldb, hipStream_t s) {
    const int64_t rows_per_wg = 256;
    const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + rows_per_wg - 1) / rows_per_wg));
    switch (zeta) {
        case 1: k_f32_flat<1><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        case 2: k_f32_flat<2><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        case 4: k_f32_flat<4><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        case 8: k_f32_flat<8><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
        default: k_f32_flat<0><<<grid, 256, 0, s>>>(A, m, n, lda, ri, v, zeta, B, d, ldb, rows_per_wg); break;
    }
    return hipGetLastError();
}

hipError_t launch_f32_lds(const LdsPlan &p, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *ri, const float *v, int32_t zeta, float *B, int32_t d,
                          int64_t ldb, hipStream_t s) {
    switch (p.slice) {
        case 64: return launch_f32_lds_sp<64>(p, A, m, n, lda, ri, v, zeta, B, d, ldb, s);
        case 32: return launch_f32_lds_sp<32>(p, A, m, n, lda, ri, v, zeta, B, d, ldb, s);
        case 16: return launch_f32_lds_sp<16>(p, A, m, n, lda, ri, v, zeta, B, d, ldb, s);
        case 8: return launch_f32_lds_sp<8>(p, A, m, n, lda, ri, v, zeta, B, d, ldb, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sk
