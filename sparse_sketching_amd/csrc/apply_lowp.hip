// Reduced-precision SparseStack scatter with a choice of contribution
// conversion and accumulation format, for gfx950 (wave64).
//
// FP16 sketching page §III-D: the contribution (the FP32 product a*val) is
// converted by one of several rules and fed to the same packed
// nearest-even atomic accumulation; §V-E adds a BF16 variant.  Built here:
//  * FP16, round-to-nearest-even (the page's kernel);
//  * FP16, stochastic conversion: the magnitude rounds up to the upper FP16
//    neighbour v of l <= |q| < v when a 32-bit draw r is below
//    frac * 2^32, frac = (|q| - l) / (v - l), else down to l; representable
//    values are kept; past the largest finite value 65504 the upper
//    neighbour is 2^16, which stands for overflow to infinity.  The draw
//    for global row g, stack block t, column c is word c mod 4 of
//    Philox-4x32-10 with counter (g lo, g hi, c div 4, 3 + 4t) and key
//    (sr_seed lo, sr_seed hi);
//  * BF16, round-to-nearest-even conversion (v_cvt_pk_bf16_f32) and packed
//    BF16 atomics (global_atomic_pk_add_bf16).
// One lane owns a column pair: one no-return packed global atomic per
// (row, block, column pair), the page's flat design, 64 lanes on 128
// consecutive columns.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"
#include "sk_rng.hpp"

namespace sk {
namespace {

typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

// Stochastic conversion of one FP32 value with draw r.  The neighbour
// arithmetic is exact in FP64: |q|, l and v are FP32 values and v - l is a
// power of two.
__device__ __forceinline__ _Float16 sr_convert(float q, uint32_t r) {
    const float z = __builtin_fabsf(q);
    if (!(z <= 3.402823466e38f)) return (_Float16)q;    // inf, NaN: as nearest
    const _Float16 x = (_Float16)z;                      // nearest-even
    const float xf = (float)x;
    const uint16_t bits = __builtin_bit_cast(uint16_t, x);
    float l, v;
    if (bits == 0x7C00u) {                               // rounds to inf: z >= 65520
        l = 65504.f;
        v = 65536.f;
    } else if (xf <= z) {
        l = xf;
        v = bits == 0x7BFFu ? 65536.f : (float)__builtin_bit_cast(_Float16, (uint16_t)(bits + 1));
    } else {
        l = (float)__builtin_bit_cast(_Float16, (uint16_t)(bits - 1));
        v = xf;
    }
    if (z == l) return (_Float16)q;
    const double frac = ((double)z - (double)l) / ((double)v - (double)l);
    const float mag = (double)r < frac * 4294967296.0 ? v : l;
    const _Float16 h = mag >= 65536.f ? (_Float16)__builtin_inff() : (_Float16)mag;
    return __builtin_signbit(q) ? -h : h;
}

template <bool BF16, bool SR>
__global__ __launch_bounds__(256) void k_lowp_flat(const float *__restrict__ A, int64_t m,
                                                   int32_t npairs, int64_t lda,
                                                   const int32_t *__restrict__ row_idx,
                                                   const float *__restrict__ val, int32_t zeta,
                                                   uint32_t *__restrict__ Bw, int32_t d,
                                                   int64_t ldbw, int64_t rows_per_wg,
                                                   uint64_t sr_seed, int64_t row_offset) {
    const int32_t db = d / zeta;    // rows per stack block; entry t must lie in block t
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t pair = blockIdx.x * 64 + lane;
    const bool active = pair < npairs;
    for (int64_t r0 = (int64_t)blockIdx.y * rows_per_wg; r0 < m;
         r0 += (int64_t)gridDim.y * rows_per_wg) {
        const int64_t r1 = r0 + rows_per_wg < m ? r0 + rows_per_wg : m;
        for (int64_t i = r0 + wave; i < r1; i += 4) {
            const float2 a = active ? *reinterpret_cast<const float2 *>(A + i * lda + 2 * pair)
                                    : float2{0.f, 0.f};
            const int32_t *ri = row_idx + i * zeta;
            const float *vv = val + i * zeta;
            const uint64_t g = (uint64_t)row_offset + (uint64_t)i;
            for_each_block<0>(zeta, [&](int t) {
                const int32_t r = ri[t];
                const float v = vv[t];
                if (!active || (uint32_t)(r - t * db) >= (uint32_t)db) return;
                const float q0 = a.x * v, q1 = a.y * v;
                uint32_t *dst = Bw + (int64_t)r * ldbw + pair;
                if constexpr (BF16) {
                    const bf2_t c = {(__bf16)q0, (__bf16)q1};
                    __builtin_amdgcn_global_atomic_fadd_v2bf16(
                        (__attribute__((address_space(1))) bf2_t *)dst, c);
                } else if constexpr (SR) {
                    // columns 2*pair and 2*pair+1 share one Philox block
                    const u32x4 w = philox4x32_10(
                        u32x4{(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)pair >> 1,
                              3u + 4u * (uint32_t)t},
                        (uint32_t)sr_seed, (uint32_t)(sr_seed >> 32));
                    const bool hi = pair & 1;
                    const h2_t c = {sr_convert(q0, hi ? w.z : w.x), sr_convert(q1, hi ? w.w : w.y)};
                    atomic_add_global_h2(reinterpret_cast<h2_t *>(dst), c);
                } else {
                    atomic_add_global_h2(reinterpret_cast<h2_t *>(dst), cvt_rn_h2(q0, q1));
                }
            });
        }
    }
}

}  // namespace

hipError_t launch_lowp_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                            const int32_t *ri, const float *v, int32_t zeta, uint16_t *B,
                            int32_t d, int64_t ldb, bool bf16, bool sr, uint64_t sr_seed,
                            int64_t row_offset, hipStream_t s) {
    const int32_t npairs = n / 2;
    uint32_t *Bw = reinterpret_cast<uint32_t *>(B);
    const int64_t ldbw = ldb / 2;
    const int64_t rows_per_wg = 256;
    int64_t groups = (m + rows_per_wg - 1) / rows_per_wg;
    if (groups > 65535) groups = 65535;
    const dim3 grid((unsigned)((npairs + 63) / 64), (unsigned)groups);
    if (bf16 && sr) return hipErrorInvalidValue;
    if (bf16)
        k_lowp_flat<true, false><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, Bw, d, ldbw,
                                                      rows_per_wg, sr_seed, row_offset);
    else if (sr)
        k_lowp_flat<false, true><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, Bw, d, ldbw,
                                                      rows_per_wg, sr_seed, row_offset);
    else
        k_lowp_flat<false, false><<<grid, 256, 0, s>>>(A, m, npairs, lda, ri, v, zeta, Bw, d,
                                                       ldbw, rows_per_wg, sr_seed, row_offset);
    return hipGetLastError();
}

}  // namespace sk
