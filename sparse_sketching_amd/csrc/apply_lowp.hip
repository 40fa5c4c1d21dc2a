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
// Two designs:
//  * k_lowp_flat, the page's flat design: one lane owns a column pair, one
//    no-return packed global atomic per (row, block, column pair), 64 lanes
//    on 128 consecutive columns.
//  * k_lowp_reg, the two-level design of the FP16 fused sketch: a workgroup
//    owns a chunk of rows, a 128-column slice and 16 R output rows; each
//    wavefront keeps R output rows (inside one stack block) in registers
//    as packed FP16 or BF16 pairs.  Rows (FP32) and their metadata stream
//    through an LDS stage of 64 rows; every hit converts its own product
//    (SR needs its own draw per contribution) and adds it with a packed
//    nearest-even addition.  The chunk partials go to a workspace and the
//    reduce kernel adds them in a fixed order (in the accumulation format,
//    or in FP32 with one final rounding): reproducible, and no atomics.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"
#include "sk_rng.hpp"
#include "sk_stack_apply.hpp"

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

constexpr int kLW = 16;                 // wavefronts per workgroup
constexpr int kLS = 64;                 // input rows per stage
constexpr int kLD = kLS / kLW;          // rows each wavefront stages

// FMT: 0 FP16 nearest-even, 1 FP16 stochastic, 2 BF16 nearest-even.
template <int FMT, int R>
__global__ __launch_bounds__(kLW * 64) void k_lowp_reg(const LowpRegArgs a) {
    __shared__ float2 raw[kLS * 64];            // stage row j, lane l at j*64 + l
    __shared__ uint32_t me[kLowpMaxZeta * kLS]; // (t, j): bucket | sign << 31, 0x7FFFFFFF: none
    __shared__ float mv[kLowpMaxZeta * kLS];    // (t, j): the entry's value

    const int32_t G = a.groups;
    const int32_t wg = blockIdx.x;
    const int32_t slice = wg % a.slices;
    const int32_t cg = wg / a.slices;
    const int32_t grp = cg % G;
    const int32_t chunk = cg / G;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int zeta = a.zeta;
    const uint32_t db = (uint32_t)(a.d / zeta);
    const int32_t lo = (grp * kLW + wave) * R;      // the wave's first output row
    const int32_t t = lo / (int32_t)db;             // its stack block
    const uint32_t lob = (uint32_t)(lo - t * (int32_t)db);
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int32_t nrows = (int32_t)(r0 + a.rows_per_chunk < a.m ? a.rows_per_chunk : a.m - r0);
    const int32_t nst = (nrows + kLS - 1) / kLS;
    const int32_t pair = slice * 64 + lane;         // the lane's column pair
    const int32_t pc = pair < a.npairs ? pair : a.npairs - 1;
    const int64_t last_e = (r0 + nrows) * zeta - 1;

    uint32_t acc[R];
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k] = 0u;

    for (int32_t s = 0; s < nst; ++s) {
        // this wave's kLD rows of the stage and their entries (one per lane)
#pragma unroll
        for (int u = 0; u < kLD; ++u) {
            int32_t rel = s * kLS + wave * kLD + u;
            rel = rel < nrows ? rel : nrows - 1;
            raw[(wave * kLD + u) * 64 + lane] =
                *reinterpret_cast<const float2 *>(a.A + (r0 + rel) * a.lda + 2 * pc);
        }
        if (lane < kLD * zeta) {
            const int jj = lane / zeta, tt = lane - jj * zeta;
            const int32_t rel = s * kLS + wave * kLD + jj;
            int64_t e = (r0 + s * kLS + wave * kLD) * zeta + lane;
            e = e < last_e ? e : last_e;
            const int32_t ri = a.row_idx[e];
            const float v = a.val[e];
            const uint32_t bk = (uint32_t)(ri - tt * (int32_t)db);
            const bool ok = rel < nrows && bk < db;
            me[tt * kLS + wave * kLD + jj] = ok ? (bk | (__float_as_uint(v) & 0x80000000u))
                                                : 0x7FFFFFFFu;
            mv[tt * kLS + wave * kLD + jj] = v;
        }
        __syncthreads();
        // this wave's hits: ballot per owned row, then each hit's product,
        // converted and added
        const uint32_t e = me[t * kLS + lane];
        const float vl = mv[t * kLS + lane];
        const uint32_t rk = (e & 0x7FFFFFFFu) - lob;
        const int32_t rl = rk < (uint32_t)R ? (int32_t)rk : -1;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            uint64_t mk = __ballot(rl == k);
            while (mk) {
                const int i = __builtin_ctzll(mk);
                mk &= ~(1ull << i);
                const float2 x = raw[i * 64 + lane];
                const float v = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(vl), i));
                const float q0 = x.x * v, q1 = x.y * v;     // FP32 products
                uint32_t c;
                if constexpr (FMT == 2) {
                    c = AccBF16::pack(q0, q1);
                } else if constexpr (FMT == 1) {
                    const uint64_t g = (uint64_t)a.row_offset + (uint64_t)(r0 + s * kLS + i);
                    const u32x4 w = philox4x32_10(
                        u32x4{(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)pair >> 1,
                              3u + 4u * (uint32_t)t},
                        (uint32_t)a.sr_seed, (uint32_t)(a.sr_seed >> 32));
                    const bool hi = pair & 1;
                    const h2_t h = {sr_convert(q0, hi ? w.z : w.x), sr_convert(q1, hi ? w.w : w.y)};
                    c = __builtin_bit_cast(uint32_t, h);
                } else {
                    c = __builtin_bit_cast(uint32_t, cvt_rn_h2(q0, q1));
                }
                acc[k] = FMT == 2 ? AccBF16::sum(acc[k], c) : AccF16::sum(acc[k], c);
            }
        }
        __syncthreads();
    }
    // the wave's R partial rows of (slice, chunk): ws[slice][chunk][d][64]
    uint32_t *dst = a.ws + (((int64_t)slice * a.chunks + chunk) * a.d + lo) * 64 + lane;
#pragma unroll
    for (int k = 0; k < R; ++k) dst[k * 64] = acc[k];
}

template <int FMT>
const void *pick_lowp_reg(int R) {
    switch (R) {
        case 4: return (const void *)k_lowp_reg<FMT, 4>;
        case 8: return (const void *)k_lowp_reg<FMT, 8>;
        case 16: return (const void *)k_lowp_reg<FMT, 16>;
        case 32: return (const void *)k_lowp_reg<FMT, 32>;
    }
    return nullptr;
}

}  // namespace

// Plan: R = d / (16 G) output rows per wavefront for the fewest row groups
// G with R in {4, 8, 16, 32} dividing d / zeta (a wave's rows inside one
// block); chunks of whole 64-row stages so that about two workgroups per CU
// run; 128-column slices.
bool plan_lowp_reg(const DevInfo &di, int64_t m, int32_t n, int32_t d, int32_t zeta,
                   LowpRegPlan *p) {
    if (m < 1 || n < 2 || n % 2 != 0 || zeta < 1 || zeta > kLowpMaxZeta || d % 16 != 0) return false;
    if (d % zeta != 0 || di.num_cu < 1) return false;
    const int64_t db = d / zeta;
    int R = 0, G = 0;
    for (int g = 1; (int64_t)16 * g <= d; g *= 2) {
        if (d % (16 * g) != 0) break;
        const int64_t r = d / (16 * g);
        if (r > 32) continue;
        if (r < 4 || (r & (r - 1)) != 0) break;
        if (db % r == 0) {
            R = (int)r;
            G = g;
            break;
        }
    }
    if (R == 0) return false;
    const int64_t slices = (n / 2 + 63) / 64;
    const int64_t stages = (m + kLS - 1) / kLS;
    int64_t want = (2 * (int64_t)di.num_cu + slices * G - 1) / (slices * G);
    if (want > stages) want = stages;
    if (want > 65535) want = 65535;
    if (want < 1) want = 1;
    const int64_t spc = (stages + want - 1) / want;
    p->R = R;
    p->groups = G;
    p->slices = slices;
    p->rows_per_chunk = spc * kLS;
    p->chunks = (m + p->rows_per_chunk - 1) / p->rows_per_chunk;
    p->grid = slices * G * p->chunks;
    p->ws_bytes = (size_t)slices * (size_t)p->chunks * (size_t)d * 64 * 4;
    return p->grid <= ((int64_t)1 << 31) - 1 && p->rows_per_chunk < ((int64_t)1 << 30);
}

hipError_t launch_lowp_reg(const LowpRegPlan &p, const float *A, int64_t m, int32_t n,
                           int64_t lda, const int32_t *ri, const float *v, int32_t zeta,
                           uint16_t *B, int32_t d, int64_t ldb, bool bf16, bool sr,
                           uint64_t sr_seed, int64_t row_offset, uint32_t *ws, int mode,
                           hipStream_t s) {
    if (ws == nullptr || (bf16 && sr) || (int64_t)16 * p.R * p.groups != d ||
        zeta > kLowpMaxZeta || p.slices * 128 < n)
        return hipErrorInvalidValue;
    const int fmt = bf16 ? 2 : sr ? 1 : 0;
    const void *kern = fmt == 2 ? pick_lowp_reg<2>(p.R)
                       : fmt == 1 ? pick_lowp_reg<1>(p.R) : pick_lowp_reg<0>(p.R);
    if (kern == nullptr) return hipErrorInvalidValue;
    LowpRegArgs a{};
    a.A = A;
    a.row_idx = ri;
    a.val = v;
    a.ws = ws;
    a.m = m;
    a.lda = lda;
    a.rows_per_chunk = p.rows_per_chunk;
    a.row_offset = row_offset;
    a.sr_seed = sr_seed;
    a.npairs = n / 2;
    a.d = d;
    a.zeta = zeta;
    a.chunks = (int32_t)p.chunks;
    a.slices = (int32_t)p.slices;
    a.groups = p.groups;
    void *params[] = {&a};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3(kLW * 64), params, 0, s);
    if (e != hipSuccess) return e;
    StackApplyArgs r{};
    r.B = B;
    r.ws = ws;
    r.ldb = ldb / 2;
    r.units = n / 2;
    r.d = d;
    r.chunks = (int32_t)p.chunks;
    r.slices = (int32_t)p.slices;
    return bf16 ? launch_stack_reduce<AccBF16>(r, 64, mode, s)
                : launch_stack_reduce<AccF16>(r, 64, mode, s);
}

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
