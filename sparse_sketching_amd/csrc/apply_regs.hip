// SparseStack apply from stored metadata with the partial sketch in
// registers, for gfx950: the register variant of sk_apply_f32 and
// sk_apply_f16acc.
//
// What is computed (FP16 sketching page §III-A/§III-B): for every input row
// i and stack block t whose entry row_idx[i*zeta+t] lies in block t's rows
// [t*d/zeta, (t+1)*d/zeta), the contribution fl32(A[i, c] * val[i*zeta+t])
// is added to that output row; in the FP16 variant each contribution is
// rounded to FP16 (nearest-even) and added with FP16 nearest-even
// additions.  Entries outside their block contribute nothing.  Values may
// differ from entry to entry: the product is formed per hit.
//
// How (MI355X-specific): the ownership of the fused sketch (fused.hip) with
// the metadata read instead of drawn.
//  * A 1024-thread workgroup owns a chunk of input rows, a column slice (64
//    lanes x 4 FP32 columns for FP16, x 2 for FP32) and 16*R output rows
//    of one row group; wavefront w keeps R rows (inside one stack block) x
//    2 words per lane in registers.  No atomics, no LDS read-modify-write,
//    and a fixed order of additions: the result is reproducible.
//  * Rows stream through double-buffered LDS stages of 64 rows as raw FP32
//    (2 x 64 KiB for FP16); each wavefront loads 4 rows per stage, and with
//    them the metadata entries of those rows (lane q of the first 4*zeta
//    lanes loads entry q), into one of two register sets, so two stages are
//    in flight while one is applied.  Staging writes the rows and the
//    entries (row relative to its block, value) to LDS.
//  * A row whose zeta entries share one magnitude c (always so for
//    sk_meta_generate's metadata) is staged as its contributions
//    fl32(a*c), rounded to FP16 in the FP16 variant, once per row: the
//    products are exact in sign, fl32(a*-c) = -fl32(a*c), and nearest-even
//    rounding is odd, so a hit adds the staged word times the entry's sign,
//    a scalar +-1 FMA, bit for bit the per-hit product.  Other rows are
//    staged raw and each hit forms fl32(a*val) from the entry's value.
//  * After one barrier each wavefront reads its block's entries (one stage
//    row per lane), takes one ballot per owned row and adds each hit to
//    that row's registers.
//  * The partial goes to the workspace once; the reduce kernel writes B.
#include "sk_internal.hpp"
#include "sk_stack_apply.hpp"
#include "sk_stream.hpp"

namespace sk {
namespace {

constexpr int kStageR = 64;             // input rows per stage
constexpr int kWavesR = 16;
constexpr int kRowsR = kStageR / kWavesR;
constexpr int kSetsR = 2;               // register sets of loaded rows

template <int K> struct LdsRow;
template <> struct LdsRow<2> { typedef float2 type; };
template <> struct LdsRow<4> { typedef float4 type; };

template <int K>
__device__ __forceinline__ typename LdsRow<K>::type to_lds(const FVec<K> &v) {
    if constexpr (K == 2) return make_float2(v.x[0], v.x[1]);
    else return make_float4(v.x[0], v.x[1], v.x[2], v.x[3]);
}

template <int K>
__device__ __forceinline__ FVec<K> from_lds(const typename LdsRow<K>::type &w) {
    FVec<K> v;
    if constexpr (K == 2) {
        v.x[0] = w.x;
        v.x[1] = w.y;
    } else {
        v.x[0] = w.x;
        v.x[1] = w.y;
        v.x[2] = w.z;
        v.x[3] = w.w;
    }
    return v;
}

// One 32-bit word at global address base + off (base wave-uniform), in the
// scalar-base load form.
__device__ __forceinline__ uint32_t load_word(uint64_t base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(1))) const char gchar;
    typedef __attribute__((address_space(1))) const uint32_t gword;
    return *reinterpret_cast<gword *>(reinterpret_cast<gchar *>(base) + off);
#else
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + off);
#endif
}

template <class T, int R>
__global__ __launch_bounds__(kWavesR * 64) void k_stack_regs(const FusedArgs args) {
    constexpr int K = 2 * T::kCols;     // floats of A per lane per row
    constexpr int S = kStageR, D = kRowsR, P = kSetsR;
    typedef FVec<K> vec_t;
    typedef typename LdsRow<K>::type lrow_t;
    __shared__ lrow_t hs0[S * 64];      // stage rows, row j at [j*64, j*64+64)
    __shared__ lrow_t hs1[S * 64];
    __shared__ uint32_t ix0[kFusedMaxZeta * S];  // entry (t, j) at t*S + j: row_idx - t*db
    __shared__ uint32_t ix1[kFusedMaxZeta * S];
    __shared__ float vl0[kFusedMaxZeta * S];     // its value
    __shared__ float vl1[kFusedMaxZeta * S];
    __shared__ uint32_t uf0[S];                  // stage row j staged as contributions
    __shared__ uint32_t uf1[S];

    // workgroup -> (slice, chunk, row group), as the fused sketch
    const int32_t G = args.groups;
    const int32_t wg = blockIdx.x;
    const int32_t q = wg >> 3;
    const int32_t grp = q % G;
    const int32_t unit_id = (q / G) * 8 + (wg & 7);
    if (unit_id >= args.slices * args.chunks) return;
    const int32_t slice = unit_id % args.slices;
    const int32_t chunk = unit_id / args.slices;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int zeta = args.zeta;
    const uint32_t db = (uint32_t)(args.d / zeta);
    const int32_t lo = (grp * kWavesR + wave) * R;      // first output row of the wave
    const int32_t t = lo / (int32_t)db;                  // its stack block
    const uint32_t lob = (uint32_t)(lo - t * (int32_t)db);
    const int64_t r0 = (int64_t)chunk * args.rows_per_chunk;
    const int32_t nrows = (int32_t)((r0 + args.rows_per_chunk < args.m ? args.rows_per_chunk
                                                                        : args.m - r0));
    const int32_t nst = (nrows + S - 1) / S;
    const int64_t lda = args.lda;
    const int32_t col = slice * 64 * K + lane * K;
    const int32_t col_c = col <= args.n - K ? col : args.n - K;
    const uint32_t lane_off = (uint32_t)col_c * 4u;
    const char *__restrict__ A = reinterpret_cast<const char *>(args.A);
    // this lane's metadata entry within a wavefront's D rows (lanes past
    // D*zeta load none)
    const bool mlane = lane < D * zeta;
    const int32_t mrow = mlane ? lane / zeta : 0;
    const int32_t mblk = mlane ? lane - mrow * zeta : 0;

    uint32_t acc[R][2];
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k][0] = acc[k][1] = 0u;

    vec_t a[P][D];
    uint32_t mi[P];
    float mv[P];
    // rows and metadata of this wavefront's share of stage s, both loaded
    // from indexes clamped into the chunk and left untouched until staged.
    // Every call issues its loads, also past the last stage (the clamped
    // rows are L2 hits): a skipped load, or a loaded value used here, would
    // make the compiler wait for this stage's loads before the next ones.
    auto load = [&](int32_t s, vec_t (&av)[D], uint32_t &ri, float &rv) {
        const int32_t base = s * S + wave * D;
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int32_t rel = base + u < nrows ? base + u : nrows - 1;
            av[u] = load_row<K>(uniform_addr((uint64_t)(A + (r0 + rel) * lda * 4)), lane_off);
        }
        // the wavefront's entries are contiguous: a scalar base (its first
        // row, clamped into the chunk) and the lane's offset, clamped to the
        // chunk's last entry
        const int32_t rb = base < nrows ? base : nrows - 1;
        const int32_t left = (nrows - rb) * zeta - 1;
        const uint32_t eoff = (uint32_t)(lane < left ? lane : left) * 4u;
        const uint64_t eb = (uint64_t)(r0 + rb) * (uint64_t)zeta * 4u;
        ri = load_word(uniform_addr((uint64_t)args.row_idx + eb), eoff);
        rv = __builtin_bit_cast(float, load_word(uniform_addr((uint64_t)args.val + eb), eoff));
    };
    // stage s's rows and entries (the entry of a lane past D*zeta or of a
    // row past the chunk becomes "no hit", value 0)
    auto stage = [&](int32_t s, const vec_t (&av)[D], uint32_t ri_raw, float rv_raw, lrow_t *hs,
                     uint32_t *ix, float *vl, uint32_t *uf) {
        const bool live = mlane && s * S + wave * D + mrow < nrows;
        const uint32_t ri = live ? ri_raw - (uint32_t)mblk * db : 0xFFFFFFFFu;
        const float rv = live ? rv_raw : 0.f;
        const float amv = __builtin_fabsf(rv);
        uint32_t umask = 0u;
#pragma unroll
        for (int u = 0; u < D; ++u) {
            // row u's entries sit in lanes u*zeta .. u*zeta + zeta - 1
            const float c = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, amv), u * zeta));
            const bool uni = __ballot(mlane && mrow == u && amv != c) == 0;
            lrow_t *slot = hs + (wave * D + u) * 64 + lane;
            if (uni) {
                *reinterpret_cast<uint2 *>(slot) =
                    make_uint2(T::contrib(av[u].x, c), T::contrib(av[u].x + T::kCols, c));
                umask |= 1u << u;
            } else {
                *slot = to_lds<K>(av[u]);
            }
        }
        if (lane < D) uf[wave * D + lane] = (umask >> lane) & 1u;
        if (mlane) {
            ix[mblk * S + wave * D + mrow] = ri;
            vl[mblk * S + wave * D + mrow] = rv;
        }
    };
    // every hit of stage s on this wave's rows
    auto apply = [&](int32_t s, const lrow_t *hs, const uint32_t *ix, const float *vl,
                     const uint32_t *uf) {
        const uint32_t rk = ix[t * S + lane] - lob;
        const int32_t rl = s * S + lane < nrows && rk < (uint32_t)R ? (int32_t)rk : -1;
        const float v = vl[t * S + lane];
        const uint64_t uni = __ballot(uf[lane] != 0u);
        const uint64_t neg = __ballot(__builtin_signbit(v));
#pragma unroll
        for (int k = 0; k < R; ++k) {
            uint64_t mk = __ballot(rl == k);
            while (mk) {
                const int i = __builtin_ctzll(mk);
                mk &= mk - 1;
                // the contribution words and the sign to add them with (a
                // plain add, FMA by +1, for a product formed here)
                uint32_t c0, c1, un;
                if ((uni >> i) & 1u) {
                    const uint2 x = *reinterpret_cast<const uint2 *>(hs + i * 64 + lane);
                    c0 = x.x;
                    c1 = x.y;
                    un = T::unit((uint32_t)(neg >> i) & 1u);
                } else {
                    const float vi = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
                    const vec_t x = from_lds<K>(hs[i * 64 + lane]);
                    c0 = T::contrib(x.x, vi);
                    c1 = T::contrib(x.x + T::kCols, vi);
                    un = T::unit(0u);
                }
                acc[k][0] = T::fma_unit(c0, un, acc[k][0]);
                acc[k][1] = T::fma_unit(c1, un, acc[k][1]);
            }
        }
    };

    // stage 0 staged and stages 1..P loading; then per stage s: apply s,
    // stage s+1 from the register set it was loaded into, and reload that
    // set with stage s+1+P.  The reload and the barrier run on every path,
    // also for the odd stage past the end, so each staging step sees the
    // other set's loads issued after its own and the compiler's wait leaves
    // them in flight.
    load(0, a[0], mi[0], mv[0]);
    stage(0, a[0], mi[0], mv[0], hs0, ix0, vl0, uf0);
#pragma unroll
    for (int p = 1; p <= P; ++p) load(p, a[p % P], mi[p % P], mv[p % P]);
    __syncthreads();
    for (int32_t s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int32_t s = s0 + b;
            const int nb = (b + 1) % P;
            if (s < nst) {
                apply(s, b ? hs1 : hs0, b ? ix1 : ix0, b ? vl1 : vl0, b ? uf1 : uf0);
                stage(s + 1, a[nb], mi[nb], mv[nb], b ? hs0 : hs1, b ? ix0 : ix1,
                      b ? vl0 : vl1, b ? uf0 : uf1);
            }
            load(s + 1 + P, a[nb], mi[nb], mv[nb]);
            lds_barrier();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    // the wave's R partial rows of this (slice, chunk), as the fused sketch
    uint32_t *dst = args.ws + ((int64_t)slice * args.chunks + chunk) * (int64_t)args.d * 128 +
                    (int64_t)lo * 128 + lane * 2;
#pragma unroll
    for (int k = 0; k < R; ++k)
        *reinterpret_cast<uint2 *>(dst + k * 128) = make_uint2(acc[k][0], acc[k][1]);
}

template <class T>
const void *pick_regs(int R) {
    switch (R) {
        case 4: return (const void *)k_stack_regs<T, 4>;
        case 8: return (const void *)k_stack_regs<T, 8>;
        case 16: return (const void *)k_stack_regs<T, 16>;
        case 32: return (const void *)k_stack_regs<T, 32>;
    }
    return nullptr;
}

template <class T>
hipError_t launch_regs_t(const FusedPlan &p, const FusedArgs &fa, void *B, int64_t ldb_units,
                         int32_t units, int accumulate, hipStream_t s) {
    const void *kern = pick_regs<T>(p.rows_per_wave);
    // ownership and indexing must match the plan the workspace was sized
    // for: 16 waves x R rows x groups cover d; chunks are whole stages
    if (kern == nullptr || (int64_t)kWavesR * p.rows_per_wave * p.groups != fa.d ||
        fa.groups != p.groups || fa.zeta < 1 || fa.zeta > kFusedMaxZeta ||
        kRowsR * fa.zeta > 64 || fa.ws == nullptr || fa.row_idx == nullptr ||
        fa.val == nullptr || fa.rows_per_chunk % kStageR != 0 || (fa.d / fa.zeta) % p.rows_per_wave != 0)
        return hipErrorInvalidValue;
    FusedArgs a = fa;
    void *params[] = {&a};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3(kWavesR * 64), params, 0, s);
    if (e != hipSuccess) return e;
    StackApplyArgs r{};
    r.B = B;
    r.ws = fa.ws;
    r.ldb = ldb_units;
    r.units = units;
    r.d = fa.d;
    r.chunks = fa.chunks;
    r.slices = fa.slices;
    return launch_stack_reduce<T>(r, 128, accumulate, s);
}

}  // namespace

hipError_t launch_regs_apply(const FusedPlan &p, bool f16, const float *A, int64_t m, int32_t n,
                             int64_t lda, const int32_t *row_idx, const float *val, int32_t zeta,
                             int32_t d, void *B, int64_t ldb, uint32_t *ws, int accumulate,
                             hipStream_t s) {
    FusedArgs a{};
    a.A = A;
    a.ws = ws;
    a.row_idx = row_idx;
    a.val = val;
    a.m = m;
    a.lda = lda;
    a.rows_per_chunk = p.rows_per_chunk;
    a.n = n;
    a.d = d;
    a.zeta = zeta;
    a.chunks = (int32_t)p.chunks;
    a.slices = (int32_t)p.slices;
    a.groups = p.groups;
    if (f16) return launch_regs_t<AccF16>(p, a, B, ldb / 2, n / 2, accumulate, s);
    return launch_regs_t<AccF32>(p, a, B, ldb, n, accumulate, s);
}

}  // namespace sk
