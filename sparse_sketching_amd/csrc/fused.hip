// Fused SparseStack sketch for gfx950: the metadata is drawn inside the
// apply kernel instead of being stored (FP16 sketching page §III-C names a
// Philox metadata kernel; the FlashSketch page §5.2 makes a sketch's
// randomness on the fly and never stores S).  The same kernel, reading
// stored metadata instead (META), is the register variant of
// sk_apply_f32 / sk_apply_f16acc.
//
// What is computed: B (=|+=) S A for the SparseStack S whose entries are
// exactly those sk_meta_generate writes for (seed, row_offset): for global
// row g and stack block t, Philox-4x32-10 of counter (g lo, g hi, t div 4, 0)
// and key (seed lo, seed hi) gives word w = w_{t mod 4}; the row lands on
// output row t*db + mulhi(w, db) (db = d/zeta) with sign (w & 1 ? - : +)
// and magnitude c = float32(1/sqrt(zeta)).  Every contribution is the FP32
// product a*val (FP16 sketching page §III-A); in the FP16 variant it is
// rounded to FP16 nearest-even and added with FP16 nearest-even additions
// (§III-B).  All values share the magnitude c and nearest-even rounding is
// odd, so each row is multiplied (and rounded) once and every hit adds it or
// its negation: bit-identical to rounding a*val per hit.
//
// How (MI355X-specific):
//  * A workgroup (16 wavefronts) owns a chunk of input rows, a column slice
//    of 64 lanes x 2 words (256 columns for FP16 column pairs, 128 for FP32)
//    and a group of 16*R consecutive output rows; wavefront w keeps the
//    partial of its R output rows (inside one stack block) in registers:
//    no atomics of any kind, and no LDS read-modify-write.
//  * Rows stream through LDS in stages of 128: each wavefront loads 8 rows
//    (one coalesced 64-lane load per row), scales and rounds them once and
//    writes the two-word contributions to a double-buffered LDS stage; one
//    wavefront per stage draws the Philox words of the stage's 128 rows
//    (one row per lane) into LDS.  After one barrier every wavefront scans
//    the stage's entries of its block with a ballot per owned row and adds
//    each hit's contribution to that row's registers as a (packed) FMA by a
//    scalar +-1 word: exactly the add or subtract.
//    The next stage's rows are in flight from HBM while a stage is applied.
//  * The partial is written once to the workspace, and the reduce kernel of
//    the LDS apply (sk_stack_apply.hpp) sums the chunks in a fixed order
//    into B: deterministic, and B needs no separate zeroing.
//  * Rows of A are loaded with the nontemporal hint (read once).
#include "sk_internal.hpp"
#include "sk_rng.hpp"
#include "sk_stack_apply.hpp"
#include "sk_stream.hpp"

namespace sk {
namespace {

constexpr int kWaves = 16;              // wavefronts per workgroup

// W words of a lane's partial row in one LDS access (ds_read_b64 / _b128)
template <int W> struct WordVec;
template <> struct WordVec<1> { typedef uint32_t type; };
template <> struct WordVec<2> { typedef uint2 type; };
template <> struct WordVec<4> { typedef uint4 type; };
__device__ __forceinline__ uint32_t word(const uint32_t &x, int) { return x; }
__device__ __forceinline__ uint32_t word(const uint2 &x, int j) { return j == 0 ? x.x : x.y; }
__device__ __forceinline__ uint32_t word(const uint4 &x, int j) {
    return j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w;
}
__device__ __forceinline__ void set_words(uint32_t &x, const uint32_t *w) { x = w[0]; }
__device__ __forceinline__ void set_words(uint2 &x, const uint32_t *w) { x = make_uint2(w[0], w[1]); }
__device__ __forceinline__ void set_words(uint4 &x, const uint32_t *w) {
    x = make_uint4(w[0], w[1], w[2], w[3]);
}

// META: the metadata is read from row_idx / val (the stored-metadata
// apply, zeta <= kFusedMetaMaxZeta) instead of drawn: each wavefront loads
// the entries of the rows it stages, with them, one per lane.  Entries
// outside their own block are dropped.  The staged words hold a * scale,
// so the main loop assumes every |val| = scale (sk_meta_generate's
// values); a workgroup whose chunk holds any other value redoes the chunk
// afterwards with a per-hit product from raw rows.
// W: words per lane (2: 64-lane slices of 128 words; 4: slices of 256
// words, each hit covers twice the columns; 1: slices of 64 words (128
// FP16 / 64 FP32 columns) for narrow rows: half the accumulator registers
// per row, and 4-byte FP32 loads for any width or stride).  S: input rows per stage (128 at W = 2, 64 at W = 4: 128 KiB of
// stage buffers either way, one workgroup per CU; 64 at W = 1).  DUAL:
// the two-per-CU variant for few registers per lane (FP16 W = 2 with
// R <= 8, W = 1 with R <= 32; FP32 W = 2 with R <= 16, W = 1 with
// R <= 32): 64-row stages, at
// most 74 KiB of LDS and
// 64 VGPRs, so two workgroups share a CU (8 waves per SIMD) and each hides
// the other's per-hit LDS latency and stage barriers.
template <class T, int W, int S, int R, int P, bool META, bool DUAL>
__global__ __launch_bounds__(kWaves * 64, DUAL ? 8 : 4) void k_stack_fused(
    const FusedArgs args) {
    constexpr int K = W * T::kCols;     // floats of A per lane per row
    typedef FVec<K> vec_t;
    typedef typename WordVec<W>::type wv_t;
    constexpr int D = S / kWaves;           // rows each wave loads per stage
    constexpr int NL = S / 64;              // lane groups of a stage's entries
    static_assert(S == 64 || (S == 128 && W == 2), "stage shapes");
    static_assert(!DUAL || S == 64, "two-per-CU stages");
    // both stage buffers, contiguous: stage contributions, row j of buffer b
    // at [(b*S + j)*64, +64); the general redo holds one stage of raw rows
    __shared__ wv_t hs[2 * S * 64];
    wv_t *const hs0 = hs;
    wv_t *const hs1 = hs + S * 64;
    // entry (t, j) at t*S + j: bucket | sign << 31
    __shared__ uint32_t me0[kFusedMaxZeta * S];
    __shared__ uint32_t me1[kFusedMaxZeta * S];
    __shared__ uint32_t vote[kWaves];   // META: wave w saw a general value

    // workgroup -> (slice, chunk, row group); the groups of one (slice,
    // chunk) are 8 ids apart (same XCD under round-robin dispatch)
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
    const int32_t lo = (grp * kWaves + wave) * R;       // first output row of the wave
    const int32_t t = lo / (int32_t)db;                  // its stack block
    const uint32_t lob = (uint32_t)(lo - t * (int32_t)db);
    const int64_t r0 = (int64_t)chunk * args.rows_per_chunk;
    // rows of this chunk (the plan keeps chunks below 2^30 rows)
    const int32_t nrows = (int32_t)((r0 + args.rows_per_chunk < args.m ? args.rows_per_chunk
                                                                        : args.m - r0));
    const int32_t nst = (nrows + S - 1) / S;
    const int64_t lda = args.lda;
    // the lane's K columns, clamped into the row (lanes past the last column
    // load valid memory; their partial words are never reduced)
    const int32_t col = slice * 64 * K + lane * K;
    const int32_t col_c = col <= args.n - K ? col : args.n - K;
    const uint32_t lane_off = (uint32_t)col_c * 4u;        // bytes into a row
    const char *__restrict__ A = reinterpret_cast<const char *>(args.A);
    const float c = args.scale;
    const uint32_t cbits = __float_as_uint(c);
    bool gen = false;                   // META: this lane staged a general value

    uint32_t acc[R][W];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
        for (int j = 0; j < W; ++j) acc[k][j] = 0u;

    // rows [u0, u1) of this wave's share of stage s, clamped into the chunk
    vec_t a[P][D];
    // META: the entries of the wave's rows of a stage, D*zeta <= 64
    // consecutive ones, entry q on lane q (clamped into the chunk), loaded
    // with the rows
    int32_t mi[P];
    uint32_t mv[P];
    const int64_t last_e = (r0 + nrows) * zeta - 1;
    auto load_meta = [&](int32_t s, int32_t &ri, uint32_t &vb) {
        if constexpr (META) {
            const int64_t e0 = (r0 + (int64_t)s * S + wave * D) * zeta + lane;
            const int64_t e = e0 < last_e ? e0 : last_e;
            ri = args.row_idx[e];
            vb = __float_as_uint(args.val[e]);
        }
    };
    // (a row's address is wave-uniform: a scalar base plus the lane's
    // 32-bit offset, so the loads take the scalar-base form)
    auto load = [&](int32_t s, vec_t (&av)[D], int u0, int u1) {
        const int32_t base = s * S + wave * D;
#pragma unroll
        for (int u = u0; u < u1; ++u) {
            const int32_t rel = base + u < nrows ? base + u : nrows - 1;
            av[u] = load_row<K>(uniform_addr((uint64_t)(A + (r0 + rel) * lda * 4)), lane_off);
        }
    };
    // contributions of loaded rows [u0, u1) into stage buffer buf
    auto stage = [&](const vec_t (&av)[D], wv_t *buf, int u0, int u1) {
#pragma unroll
        for (int u = u0; u < u1; ++u) {
            uint32_t w[W];
#pragma unroll
            for (int j = 0; j < W; ++j) w[j] = T::contrib(av[u].x + j * T::kCols, c);
            set_words(buf[(wave * D + u) * 64 + lane], w);
        }
    };
    // META: this wave's entries of a stage into me (bucket | sign << 31;
    // 0x7FFFFFFF, which no wave owns, for an entry outside its block), and
    // in vb_out (if given) the values' bits at the same places
    auto stage_meta = [&](int32_t ri, uint32_t vb, uint32_t *me, uint32_t *vb_out) {
        if constexpr (META) {
            if (lane < D * zeta) {
                const int jj = lane / zeta, tt = lane - jj * zeta;
                const uint32_t bk = (uint32_t)(ri - tt * (int32_t)db);
                const bool ok = bk < db;
                gen |= ok && (vb & 0x7FFFFFFFu) != cbits;
                me[tt * S + wave * D + jj] = ok ? (bk | (vb & 0x80000000u)) : 0x7FFFFFFFu;
                if (vb_out != nullptr) vb_out[tt * S + wave * D + jj] = vb;
            }
        }
    };
    // the metadata of stage s into me: one wave per stage (rotating) draws
    // the Philox blocks of the stage's rows, one row per lane
    auto draw = [&](int32_t s, uint32_t *me) {
        if constexpr (META) return;
        if (wave != (s & (kWaves - 1))) return;
        const uint32_t k0 = (uint32_t)args.seed, k1 = (uint32_t)(args.seed >> 32);
        // one lane group at a time keeps the Philox temporaries few
#pragma unroll 1
        for (int h = 0; h < NL; ++h) {
            const uint64_t g = (uint64_t)args.row_offset +
                               (uint64_t)(r0 + (int64_t)s * S + h * 64 + lane);
            for (int gq = 0; gq * 4 < zeta; ++gq) {
                const u32x4 w4 = philox4x32_10(
                    u32x4{(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)gq, 0u}, k0, k1);
                const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (gq * 4 + j < zeta)
                        me[(gq * 4 + j) * S + h * 64 + lane] = mulhi32(ww[j], db) | (ww[j] << 31);
            }
        }
    };
    // this wave's entries of stage s: output row inside its range (-1:
    // none) and the +-1 word of its sign, lane j <-> stage row h*64 + j
    int32_t rl[NL];
    uint32_t su[NL];
    auto scan = [&](int32_t s, const uint32_t *me) {
#pragma unroll
        for (int h = 0; h < NL; ++h) {
            const uint32_t e = me[t * S + h * 64 + lane];
            const int32_t rel = s * S + h * 64 + lane;
            const uint32_t rk = (e & 0x7FFFFFFFu) - lob;
            rl[h] = rel < nrows && rk < (uint32_t)R ? (int32_t)rk : -1;
            su[h] = T::unit(e >> 31);
        }
    };
    // every hit of the scanned stage on this wave's rows [k0, k1); the +-1
    // word is read from the hit's lane into a scalar register (one VALU
    // readlane instead of three scalar shifts: the scalar unit, shared by
    // the CU's waves, is the busier one in this loop)
    auto process = [&](const wv_t *buf, int k0, int k1) {
#pragma unroll
        for (int k = k0; k < k1; ++k) {
#pragma unroll
            for (int h = 0; h < NL; ++h) {
                uint64_t mk = __ballot(rl[h] == k);
                while (mk) {
                    const int i = __builtin_ctzll(mk);
                    mk &= ~(1ull << i);     // two scalar ops (mk - 1 takes three)
                    const wv_t x = buf[(h * 64 + i) * 64 + lane];
                    const uint32_t u = __builtin_amdgcn_readlane(su[h], i);
#pragma unroll
                    for (int j = 0; j < W; ++j) acc[k][j] = T::fma_unit(word(x, j), u, acc[k][j]);
                }
            }
        }
    };

    // stage 0 staged and stages 1..P loading; then per stage s: apply s,
    // stage s+1 into the other buffer from the register set it was loaded
    // into, draw the metadata of s+1 (META: write the entries loaded with
    // its rows), and reload the set with stage s+1+P.
    // With P = 1 this is done in two halves (rows and output rows split at
    // the middle), so the next loads start half a stage earlier.
    constexpr int NH = (P == 1 && R < 32) ? 2 : 1;
    load(0, a[0], 0, D);
    load_meta(0, mi[0], mv[0]);
    stage(a[0], hs0, 0, D);
    stage_meta(mi[0], mv[0], me0, nullptr);
    draw(0, me0);
#pragma unroll
    for (int p = 1; p <= P; ++p) {
        load(p, a[p % P], 0, D);
        load_meta(p, mi[p % P], mv[p % P]);
    }
    __syncthreads();
    for (int32_t s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int32_t s = s0 + b;
            if (s < nst) scan(s, b ? me1 : me0);
#pragma unroll
            for (int j = 0; j < NH; ++j) {
                if (s < nst) {
                    process(b ? hs1 : hs0, j * R / NH, (j + 1) * R / NH);
                    stage(a[(b + 1) % P], b ? hs0 : hs1, j * D / NH, (j + 1) * D / NH);
                    // the Philox work runs while the staged registers are free
                    if (j == NH - 1) {
                        draw(s + 1, b ? me0 : me1);
                        stage_meta(mi[(b + 1) % P], mv[(b + 1) % P], b ? me0 : me1, nullptr);
                    }
                }
                // on every path (also for the odd stage past the end), so each
                // staging step finds the other set's loads issued after its
                // own and the compiler's wait leaves them in flight
                load(s + 1 + P, a[(b + 1) % P], j * D / NH, (j + 1) * D / NH);
                if (j == NH - 1) load_meta(s + 1 + P, mi[(b + 1) % P], mv[(b + 1) % P]);
            }
            lds_barrier();
        }
    }
    // the loads past the last stage (clamped rows) must land before exit
    __builtin_amdgcn_s_waitcnt(0);

    if constexpr (META) {
        // the waves' votes: does the chunk hold a value of another magnitude
        const bool mine = __ballot(gen) != 0;
        __syncthreads();
        if (lane == 0) vote[wave] = mine ? 1u : 0u;
        __syncthreads();
        if (__ballot(vote[lane & (kWaves - 1)] != 0u) != 0) {
            // redo the chunk: stage by stage, raw rows in LDS and the
            // values in me1, every hit adding the rounded product a * val
            float *raw = reinterpret_cast<float *>(hs);   // row j, lane l at (j*64 + l)*K
#pragma unroll
            for (int k = 0; k < R; ++k)
#pragma unroll
                for (int j = 0; j < W; ++j) acc[k][j] = 0u;
            for (int32_t s = 0; s < nst; ++s) {
                vec_t av[D];
                load(s, av, 0, D);
                int32_t ri;
                uint32_t vb;
                load_meta(s, ri, vb);
#pragma unroll
                for (int u = 0; u < D; ++u)
#pragma unroll
                    for (int i = 0; i < K; ++i) raw[((wave * D + u) * 64 + lane) * K + i] = av[u].x[i];
                stage_meta(ri, vb, me0, me1);
                __syncthreads();
                scan(s, me0);
                uint32_t vv[NL];
#pragma unroll
                for (int h = 0; h < NL; ++h) vv[h] = me1[t * S + h * 64 + lane];
#pragma unroll
                for (int k = 0; k < R; ++k) {
#pragma unroll
                    for (int h = 0; h < NL; ++h) {
                        uint64_t mk = __ballot(rl[h] == k);
                        while (mk) {
                            const int i = __builtin_ctzll(mk);
                            mk &= ~(1ull << i);
                            const float v = __uint_as_float(__builtin_amdgcn_readlane(vv[h], i));
                            const float *xr = raw + ((h * 64 + i) * 64 + lane) * K;
#pragma unroll
                            for (int j = 0; j < W; ++j)
                                acc[k][j] = T::fma_unit(T::contrib(xr + j * T::kCols, v), T::unit(0u),
                                                        acc[k][j]);
                        }
                    }
                }
                __syncthreads();
            }
        }
    }

    // the wave's R partial rows of this (slice, chunk), in the workspace's
    // 128-word slices: the lane's first word is word slice*64*W + lane*W of
    // the row (a W = 4 slice spans two workspace slices, two W = 1 slices
    // share one)
    const int32_t wcol = slice * 64 * W + lane * W;
    uint32_t *dst = args.ws + ((int64_t)(wcol >> 7) * args.chunks + chunk) * (int64_t)args.d * 128 +
                    (int64_t)lo * 128 + (wcol & 127);
#pragma unroll
    for (int k = 0; k < R; ++k) set_words(*reinterpret_cast<wv_t *>(dst + k * 128), acc[k]);
}

// The built (W, S, R, P, DUAL) shapes.  W = 2, S = 128: two register sets
// where the R rows leave room for them (R = 16), one set (loaded in two
// halves) otherwise; R = 4 and 8 are kept for devices where two workgroups
// do not share a CU.  W = 2 two per CU: R = 4, 8 (and 16 for FP32), one
// set in two halves.
// W = 1: R = 8, 16, 32 two per CU.  W = 4 (FP32 only): R = 8, 16 with two
// sets.
template <class T, bool META>
const void *pick_fused(int W, int S, int R, int P, bool dual) {
    if (W == 2 && S == 128 && !dual) {
        if (R == 4 && P == 1) return (const void *)k_stack_fused<T, 2, 128, 4, 1, META, false>;
        if (R == 8 && P == 2) return (const void *)k_stack_fused<T, 2, 128, 8, 2, META, false>;
        if (R == 16 && P == 2) return (const void *)k_stack_fused<T, 2, 128, 16, 2, META, false>;
        if (R == 32 && P == 1) return (const void *)k_stack_fused<T, 2, 128, 32, 1, META, false>;
    }
    if (W == 2 && S == 64 && dual) {
        if (R == 4 && P == 1) return (const void *)k_stack_fused<T, 2, 64, 4, 1, META, true>;
        if (R == 8 && P == 1) return (const void *)k_stack_fused<T, 2, 64, 8, 1, META, true>;
        if constexpr (T::kCols == 1)
            if (R == 16 && P == 1) return (const void *)k_stack_fused<T, 2, 64, 16, 1, META, true>;
    }
    {
        if (W == 1 && S == 64) {
            if (dual && R == 8 && P == 1) return (const void *)k_stack_fused<T, 1, 64, 8, 1, META, true>;
            if (dual && R == 16 && P == 1)
                return (const void *)k_stack_fused<T, 1, 64, 16, 1, META, true>;
            if (dual && R == 32 && P == 1)
                return (const void *)k_stack_fused<T, 1, 64, 32, 1, META, true>;
        }
    }
    if constexpr (T::kCols == 1) {
        if (W == 4 && S == 64 && !dual) {
            if (R == 8 && P == 2) return (const void *)k_stack_fused<T, 4, 64, 8, 2, META, false>;
            if (R == 16 && P == 2) return (const void *)k_stack_fused<T, 4, 64, 16, 2, META, false>;
        }
    }
    return nullptr;
}

template <class T>
hipError_t launch_fused_t(const FusedPlan &p, const FusedArgs &fa, void *B, int64_t ldb_units,
                          int32_t units, int mode, hipStream_t s) {
    const bool meta = fa.row_idx != nullptr;
    const void *kern =
        meta ? pick_fused<T, true>(p.words, p.stage_rows, p.rows_per_wave, p.load_sets, p.dual)
             : pick_fused<T, false>(p.words, p.stage_rows, p.rows_per_wave, p.load_sets, p.dual);
    // the kernel's row ownership must match the plan the workspace was
    // sized for: 16 waves x R rows x groups cover d exactly; with stored
    // metadata a wave's rows of a stage hold at most 64 entries
    if (kern == nullptr || (int64_t)kWaves * p.rows_per_wave * p.groups != fa.d ||
        fa.groups != p.groups || fa.slices != p.slices || fa.rows_per_chunk % p.stage_rows != 0 ||
        fa.zeta < 1 || fa.zeta > kFusedMaxZeta || fa.ws == nullptr ||
        (meta && (fa.val == nullptr || fa.zeta > kFusedMetaMaxZeta)))
        return hipErrorInvalidValue;
    FusedArgs a = fa;
    void *params[] = {&a};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3(kWaves * 64), params, 0, s);
    if (e != hipSuccess) return e;
    StackApplyArgs r{};
    r.B = B;
    r.ws = fa.ws;
    r.ldb = ldb_units;
    r.units = units;
    r.d = fa.d;
    r.chunks = fa.chunks;
    r.slices = (int32_t)((fa.slices * 64 * p.words + 127) / 128);   // 128-word workspace slices
    return launch_stack_reduce<T>(r, 128, mode, s);
}

}  // namespace

// Plan of the fused kernel.  Words per lane W: 4 (256 FP32 columns per
// slice) for FP32 matrices wider than 128 columns whose rows allow 16-byte
// lane loads: a hit then covers twice the columns, which halves the hit
// loop's instructions per byte (at the cost of more row groups, whose
// re-reads of A hit L2).  1 (128 FP16 / 64 FP32 columns) for FP16 matrices
// of at most 128 columns and FP32 matrices of at most 64: no idle half
// slice, half the accumulator registers per output row, so more rows per
// wave (fewer row groups) or two workgroups per CU, and for FP32 4-byte
// loads (any width, stride or base).  Else 2 (256 FP16 / 128 FP32 columns).  Rows per wave
// R = d / (16 G) for the fewest row groups G with R <= 32 (16 at W = 4)
// and R dividing d/zeta (a wave's rows inside
// one block); R must be one of the built sizes.  Few registers per lane
// (FP16 W = 2, R <= 8; W = 1, R <= 32; FP32 W = 2, R <= 16) take the
// two-per-CU shape where the LDS holds two of its workgroups.  Chunks are
// sized so the workgroups fill the device, in whole stages.  Narrow
// matrices (down to 2 FP16 / 1 FP32 columns: a right-hand side)
// run here too, most lanes of their slice idle: a narrow sketch is bound by
// the per-hit instructions, which do not depend on the active lanes, and
// the fused kernel's hits are cheaper than the LDS apply's.
namespace {
bool plan_rows(int32_t d, int32_t zeta, int W, int *R_out, int *G_out) {
    const int64_t db = d / zeta;
    // W = 1 stops at 32 rows per wavefront, two workgroups per CU: at d =
    // 1024 and 2048 two row groups of R = 32 (A read twice, mostly from L2)
    // beat one group of R = 64 at one workgroup per CU by 2-11% (FP16 128
    // and FP32 64 columns, fused and stored-metadata applies)
    const int rmax = W == 4 ? 16 : 32, rmin = W == 2 ? 4 : 8;
    for (int g = 1; (int64_t)kWaves * g <= d; g *= 2) {
        if (d % (kWaves * g) != 0) break;
        const int64_t r = d / (kWaves * g);
        if (r > rmax) continue;
        if (r < rmin || (r & (r - 1)) != 0) break;
        if (db % r == 0) {
            *R_out = (int)r;
            *G_out = g;
            return true;
        }
    }
    return false;
}
}  // namespace

bool plan_fused(const DevInfo &di, bool f16, int64_t m, int32_t n, int64_t lda, int a_align,
                int32_t d, int32_t zeta, FusedPlan *p) {
    if (m < 1 || zeta > kFusedMaxZeta || d % kWaves != 0) return false;
    if (n < (f16 ? 2 : 1)) return false;
    if (di.max_lds < kFusedLdsBytes) return false;
    // the kernel indexes rows inside a chunk with 32-bit integers
    if (m > (int64_t)65535 << 30) return false;
    // a lane loads K = W x (2 for FP16, 1 for FP32) floats of a row
    auto rows_ok = [&](int K) { return n % K == 0 && lda % K == 0 && a_align >= K * 4; };
    int W = 0, R = 0, G = 0;
    if (!f16 && n > 128 && rows_ok(4) && plan_rows(d, zeta, 4, &R, &G))
        W = 4;
    else if (f16 && n <= 128 && rows_ok(2) && plan_rows(d, zeta, 1, &R, &G))
        W = 1;
    else if (!f16 && n <= 64 && rows_ok(1) && plan_rows(d, zeta, 1, &R, &G))
        W = 1;
    else if (rows_ok(f16 ? 4 : 2) && plan_rows(d, zeta, 2, &R, &G))
        W = 2;
    else
        return false;
    const int K = W * (f16 ? 2 : 1);
    // two per CU where a lane's partial words (W x R) and one set of staged
    // rows (4 rows x K floats) take at most 40 registers: FP16 W = 2, R <= 8;
    // FP16 W = 1, R <= 32; FP32 W = 2, R <= 16 (all fit 64 VGPRs)
    const bool dual = W <= 2 && W * R + 4 * K <= 40 && di.max_lds >= 2 * kFusedDualLdsBytes;
    if (W == 1 && !dual) return false;              // W = 1 runs two per CU
    *p = FusedPlan{};
    p->kind = kFusedRegister;
    p->words = W;
    p->dual = dual ? 1 : 0;
    p->stage_rows = (W == 2 && !dual) ? 128 : 64;
    p->rows_per_wave = R;
    p->groups = G;
    p->load_sets = dual ? 1 : (R == 8 || R == 16) ? 2 : 1;
    p->slices = (n + 64 * K - 1) / (64 * K);
    const int64_t per_chunk = p->slices * G;
    int64_t want = ((int64_t)di.num_cu * (dual ? 2 : 1) + per_chunk - 1) / per_chunk;
    const int64_t stages = (m + p->stage_rows - 1) / p->stage_rows;
    if (want > stages) want = stages;
    if (want > 65535) want = 65535;
    if (want < 1) want = 1;
    const int64_t st_per_chunk = (stages + want - 1) / want;
    p->rows_per_chunk = st_per_chunk * p->stage_rows;
    p->chunks = (m + p->rows_per_chunk - 1) / p->rows_per_chunk;
    p->grid = (p->slices * p->chunks + 7) / 8 * 8 * G;
    // partial words per row: slices x 64 x W, stored in 128-word slices
    const size_t ws_slices = (size_t)((p->slices * 64 * W + 127) / 128);
    p->ws_bytes = ws_slices * (size_t)p->chunks * (size_t)d * 128 * 4;
    return true;
}

// Narrow rows go to the owner kernel where it covers them: rows of at most
// 32 words (FP16 up to 64 columns, FP32 up to 32), and rows of 64 words
// (FP16 128 columns, FP32 64) at no more than 8 words per lane (d <= 128).
// Measured on MI355X (2^20 rows unless noted, complete sketch): FP16
// 2 columns, d = 512: 35-42 us against 144 in the register kernel; FP16 64
// columns, 4,194,304 rows, d = 128: 225-235 us against 341; FP32 64 columns
// there: 244-250 us against 330; FP16 32 columns, d = 1024: 107 us against
// 181; but with 16 words per lane the register kernel stays faster: FP32 64
// columns at d = 256, 111 / 158 us against 102 / 140 (zeta = 4 / 8), FP16
// 128 columns at d = 256, 108 / 122 / 168 against 102 / 108 / 143 (zeta =
// 1 / 4 / 8).
bool plan_sketch(const DevInfo &di, bool f16, int64_t m, int32_t n, int64_t lda, int a_align,
                 int32_t d, int32_t zeta, FusedPlan *p) {
    FusedPlan q{};
    if (plan_owner(di, f16, m, n, lda, a_align, d, zeta, &q) && (q.row_words <= 32 || q.words <= 8)) {
        *p = q;
        return true;
    }
    return plan_fused(di, f16, m, n, lda, a_align, d, zeta, p);
}

hipError_t launch_sketch(const FusedPlan &p, bool f16, const float *A, int64_t m, int32_t n,
                         int64_t lda, uint64_t seed, int64_t row_offset, int32_t d, int32_t zeta,
                         float scale, void *B, int64_t ldb, uint32_t *ws, int mode,
                         hipStream_t s) {
    if (p.kind == kFusedOwner)
        return launch_owner(p, f16, A, m, n, lda, seed, row_offset, d, zeta, scale, B, ldb, ws,
                            mode, s);
    return launch_fused(p, f16, A, m, n, lda, seed, row_offset, nullptr, nullptr, d, zeta, scale,
                        B, ldb, ws, mode, s);
}

hipError_t launch_fused(const FusedPlan &p, bool f16, const float *A, int64_t m, int32_t n,
                        int64_t lda, uint64_t seed, int64_t row_offset, const int32_t *row_idx,
                        const float *val, int32_t d, int32_t zeta, float scale, void *B,
                        int64_t ldb, uint32_t *ws, int mode, hipStream_t s) {
    if (p.kind != kFusedRegister) return hipErrorInvalidValue;
    FusedArgs a{};
    a.A = A;
    a.ws = ws;
    a.row_idx = row_idx;
    a.val = val;
    a.m = m;
    a.lda = lda;
    a.rows_per_chunk = p.rows_per_chunk;
    a.row_offset = row_offset;
    a.seed = seed;
    a.n = n;
    a.d = d;
    a.zeta = zeta;
    a.chunks = (int32_t)p.chunks;
    a.slices = (int32_t)p.slices;
    a.groups = p.groups;
    a.scale = scale;
    if (f16) return launch_fused_t<AccF16>(p, a, B, ldb / 2, n / 2, mode, s);
    return launch_fused_t<AccF32>(p, a, B, ldb, n, mode, s);
}

}  // namespace sk
