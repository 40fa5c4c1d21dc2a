// LDS-privatized SparseStack apply for gfx950, shared by the FP32 and the
// FP16-accumulate entry points.
//
// What is computed (FP16 sketching page §III-A/§III-B): for every input row i
// and stack block t, the contribution val[i*zeta+t] * A[i, :] is added to
// output row row_idx[i*zeta+t], which lies in block t's rows
// [t*d/zeta, (t+1)*d/zeta) (entries outside their block contribute nothing);
// in the FP16 variant each FP32 product is rounded to FP16 (nearest-even) and
// added with FP16 nearest-even additions.
//
// How (MI355X-specific):
//  * A workgroup owns a column slice (SP lanes x W 32-bit words per lane:
//    one FP32 column or one FP16 column pair per word), a chunk of input rows
//    and a group of zg consecutive stack blocks, and keeps a private partial
//    sketch of those blocks' zg*d/zeta rows in LDS.  Splitting the blocks
//    lets a workgroup cover twice the columns with 64-bit words (half the
//    instructions per byte of A) at the cost of each row being read by each
//    group; the groups of one (slice, chunk) get workgroup ids 8 apart, so
//    they run on the same XCD and the second read is an L2 hit.
//  * Each wavefront streams whole rows of its slice: 64 lanes on
//    consecutive columns, so a row segment is one coalesced load.
//  * gfx950 executes floating-point LDS atomics (ds_add_f32, ds_pk_add_f16,
//    ds_pk_add_bf16) one lane at a time, about 3 clocks per active lane,
//    while integer LDS atomics and plain reads and writes take a few clocks
//    per 64-lane instruction.  So a partial word is updated by a plain read,
//    a register add and an integer compare-and-swap (ds_cmpst_rtn_b32/_b64)
//    that stores the sum only if the word(s) still hold what was read; a lane
//    whose swap failed (another wavefront updated the word in between)
//    retries with the value the swap returned.  A swap that succeeds always
//    applies the addition onto the latest sum, so every contribution is
//    added exactly once and no update is lost.  The hits of a row block are
//    issued straight-line (all reads, then all swaps) and failures are rare.
//  * Sketch metadata carries one magnitude per sketch with varying signs,
//    so a row's contribution is rounded once and each hit flips its sign
//    (nearest-even rounding is odd, so this equals rounding a*val itself);
//    a block whose values differ in magnitude is applied one hit at a time.
//  * At the end the partial is flushed once: either with packed/FP32 global
//    atomics into B, or with plain stores into a caller-supplied workspace
//    that a second kernel reduces in a fixed chunk order (no atomics, and no
//    separate zeroing of B).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sk_apply_common.hpp"
#include "sk_internal.hpp"

namespace sk {

// Per-precision word arithmetic.  A word is 32 bits of the partial sketch.
struct AccF32 {
    static constexpr int kCols = 1;     // columns per word
    typedef float out_t;                // B element (one word)
    // contribution word of x*v: the FP32 product, rounded to nearest-even
    __device__ static uint32_t contrib(const float *x, float v) {
        return __float_as_uint(__fmul_rn(x[0], v));
    }
    // the word's sign flip for a negative value (sign bit of s)
    __device__ static uint32_t signmask(uint32_t s) { return s & 0x80000000u; }
    __device__ static uint32_t sum(uint32_t x, uint32_t y) {
        return __float_as_uint(__fadd_rn(__uint_as_float(x), __uint_as_float(y)));
    }
    __device__ static void global_add(out_t *B, int64_t off, uint32_t w) {
        atomic_add_global_f32(B + off, __uint_as_float(w));
    }
    __device__ static uint32_t get(const out_t *B, int64_t off) { return __float_as_uint(B[off]); }
    __device__ static void put(out_t *B, int64_t off, uint32_t w) { B[off] = __uint_as_float(w); }
    // the reduce's accumulator: the word itself (FP32 partials add in FP32)
    typedef float wide_t;
    __device__ static wide_t widen(uint32_t w) { return __uint_as_float(w); }
    __device__ static wide_t wide_add(wide_t a, wide_t b) { return __fadd_rn(a, b); }
    __device__ static uint32_t narrow(wide_t a) { return __float_as_uint(a); }
    // the word +1 or -1 (b = 1): acc + x*unit is exactly acc + x or acc - x
    __device__ static uint32_t unit(uint32_t b) { return 0x3F800000u | (b << 31); }
    __device__ static uint32_t fma_unit(uint32_t x, uint32_t u, uint32_t acc) {
        return __float_as_uint(__builtin_fmaf(__uint_as_float(x), __uint_as_float(u),
                                              __uint_as_float(acc)));
    }
};

struct AccF16 {
    static constexpr int kCols = 2;     // a word is a column pair
    typedef h2_t out_t;
    // both FP32 products, each rounded to FP16 (RN), low half = first column
    __device__ static uint32_t contrib(const float *x, float v) {
        return __builtin_bit_cast(uint32_t, cvt_rn_h2(x[0] * v, x[1] * v));
    }
    __device__ static uint32_t signmask(uint32_t s) {
        const uint32_t m = s & 0x80000000u;
        return m | (m >> 16);
    }
    // per-half FP16 nearest-even additions (v_pk_add_f16, subnormals kept)
    __device__ static uint32_t sum(uint32_t x, uint32_t y) {
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, x) + __builtin_bit_cast(h2_t, y));
    }
    __device__ static void global_add(out_t *B, int64_t off, uint32_t w) {
        atomic_add_global_h2(B + off, __builtin_bit_cast(h2_t, w));
    }
    __device__ static uint32_t get(const out_t *B, int64_t off) {
        return __builtin_bit_cast(uint32_t, B[off]);
    }
    __device__ static void put(out_t *B, int64_t off, uint32_t w) { B[off] = __builtin_bit_cast(h2_t, w); }
    // the reduce's accumulator: the FP16 pair widened exactly to FP32; the
    // sum of the partials is rounded to FP16 (nearest-even) once
    typedef float2 wide_t;
    __device__ static wide_t widen(uint32_t w) {
        const h2_t h = __builtin_bit_cast(h2_t, w);
        return make_float2((float)h.x, (float)h.y);
    }
    __device__ static wide_t wide_add(wide_t a, wide_t b) {
        return make_float2(__fadd_rn(a.x, b.x), __fadd_rn(a.y, b.y));
    }
    __device__ static uint32_t narrow(wide_t a) {
        return __builtin_bit_cast(uint32_t, cvt_rn_h2(a.x, a.y));
    }
    // the pair (+1, +1) or (-1, -1) (b = 1): a packed FMA by it is exactly the
    // packed nearest-even add or subtract (the product is exact)
    __device__ static uint32_t unit(uint32_t b) { return 0x3C003C00u | (b << 31) | (b << 15); }
    __device__ static uint32_t fma_unit(uint32_t x, uint32_t u, uint32_t acc) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2_t, x),
                                                                      __builtin_bit_cast(h2_t, u),
                                                                      __builtin_bit_cast(h2_t, acc)));
    }
};

// BF16 pairs (8-bit exponent and significand): the word arithmetic of the
// two-level reduced-precision sketch's reduce.  A BF16 addition is the FP32
// sum of the two (exactly widened) values rounded to BF16 nearest-even once,
// which is the correctly rounded BF16 sum (FP32 has more than 2 x 8 + 2
// significand bits).
struct AccBF16 {
    static constexpr int kCols = 2;
    typedef uint32_t out_t;             // two BF16 values, low half = first column
    __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    __device__ static uint32_t pack(float x, float y) {
        typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
        const bf2_t b = {(__bf16)x, (__bf16)y};          // nearest-even
        return __builtin_bit_cast(uint32_t, b);
    }
    __device__ static uint32_t sum(uint32_t x, uint32_t y) {
        return pack(lo(x) + lo(y), hi(x) + hi(y));
    }
    __device__ static uint32_t get(const out_t *B, int64_t off) { return B[off]; }
    __device__ static void put(out_t *B, int64_t off, uint32_t w) { B[off] = w; }
    // the reduce's FP32 combine (one rounding of the total to BF16)
    typedef float2 wide_t;
    __device__ static wide_t widen(uint32_t w) { return make_float2(lo(w), hi(w)); }
    __device__ static wide_t wide_add(wide_t a, wide_t b) {
        return make_float2(__fadd_rn(a.x, b.x), __fadd_rn(a.y, b.y));
    }
    __device__ static uint32_t narrow(wide_t a) { return pack(a.x, a.y); }
};

// K consecutive floats of A, loaded as one vector; NT adds the nontemporal
// hint, for passes that read each element of A once.  (Where several
// workgroups read the same rows, the hint costs their shared L2 hits: on
// gfx950 the two block groups of the FP32 LDS apply of a 2^20 x 256 matrix
// ran 12 % slower with it.)
template <int K> struct FVec;
template <> struct FVec<1> { float x[1]; };
template <> struct FVec<2> { float x[2]; };
template <> struct FVec<4> { float x[4]; };
template <int K, bool NT>
__device__ __forceinline__ FVec<K> load_vec(const char *p) {
    typedef float vk_t __attribute__((ext_vector_type(K)));
    FVec<K> r;
    if constexpr (K == 1) {
        const float *q = reinterpret_cast<const float *>(p);
        r.x[0] = NT ? __builtin_nontemporal_load(q) : *q;
    } else {
        const vk_t *q = reinterpret_cast<const vk_t *>(p);
        const vk_t v = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
        for (int i = 0; i < K; ++i) r.x[i] = v[i];
    }
    return r;
}

// W 32-bit words of a lane, moved and swapped as one (64-bit for W = 2).
template <int W> struct WordT;
template <> struct WordT<1> { typedef uint32_t type; };
template <> struct WordT<2> { typedef uint64_t type; };

struct StackApplyArgs {
    const float *A;
    const int32_t *row_idx;
    const float *val;
    void *B;                // AccF32::out_t or AccF16::out_t, d x units, ldb units apart
    uint32_t *ws;           // NULL: flush with global atomics; else [slices][chunks][d][sp*W] words
    int64_t m, lda, ldb;    // lda in floats, ldb in B units (words)
    int64_t rows_per_chunk;
    int32_t units;          // words per row of B: columns (FP32) or column pairs (FP16)
    int32_t d, zeta, sp;    // sp: lanes per slice (power of two, <= 64)
    int32_t chunks, slices;
    int32_t groups, zg;     // block groups per (slice, chunk) and blocks per group
};

constexpr int kStackThreads = 1024;

// Rows a wave loads per block and hits issued together.  ZG = 0: run-time
// blocks per group (one row per block).
template <int ZG, int K, int W>
struct StackShape {
    static constexpr int ZU = ZG == 0 ? 1 : ZG;
    static constexpr int RB0 = 16 / K;                      // 32 VGPRs per register set
    static constexpr int RB = ZG == 0 ? 1 : (64 / ZU < RB0 ? 64 / ZU : RB0);
    static constexpr int NE = RB * ZU;                      // entries per block (<= 64)
    static constexpr int NHMAX = W == 1 ? 16 : 8;
    static constexpr int NH = NE < NHMAX ? NE : NHMAX;      // hits per group
    static constexpr int NSUB = NE / NH;
};

// word(s) <- word(s) + c with compare-and-swap retries; p is the value last
// seen in the word(s).
template <class T, int W>
__device__ __forceinline__ void cas_add(typename WordT<W>::type *lw, uint32_t idx,
                                        typename WordT<W>::type p, const uint32_t (&c)[W]) {
    typedef typename WordT<W>::type word_t;
    for (;;) {
        word_t nv;
        if constexpr (W == 1) {
            nv = T::sum(p, c[0]);
        } else {
            nv = (word_t)T::sum((uint32_t)p, c[0]) |
                 ((word_t)T::sum((uint32_t)(p >> 32), c[1]) << 32);
        }
        word_t expect = p;
        if (__hip_atomic_compare_exchange_strong(lw + idx, &expect, nv, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
            return;
        p = expect;
    }
}

// FULL: the slice is 64 lanes wide (sp == 64).  NT: one block group, so
// this workgroup is the only reader of its rows (nontemporal loads).
template <class T, int W, int ZG, bool FULL, bool NT>
__global__ __launch_bounds__(kStackThreads) void k_stack_apply(const StackApplyArgs args) {
    constexpr int K = W * T::kCols;             // floats of A per lane per row
    typedef FVec<K> vec_t;
    typedef typename WordT<W>::type word_t;
    typedef StackShape<ZG, K, W> Shape;
    constexpr int RB = Shape::RB;
    constexpr int NH = Shape::NH;
    constexpr int NSUB = Shape::NSUB;
    constexpr int ZU = Shape::ZU;

    // workgroup -> (slice, chunk, block group); the groups of one (slice,
    // chunk) are 8 ids apart (same XCD under round-robin dispatch)
    const int32_t G = args.groups;
    const int32_t wg = blockIdx.x;
    const int32_t q = wg >> 3;
    const int32_t grp = q % G;
    const int32_t unit_id = (q / G) * 8 + (wg & 7);
    if (unit_id >= args.slices * args.chunks) return;
    const int32_t slice = unit_id % args.slices;
    const int32_t chunk = unit_id / args.slices;

    extern __shared__ uint32_t lds[];
    word_t *lw = reinterpret_cast<word_t *>(lds);
    const int SP = FULL ? 64 : args.sp;
    const int zg = ZG ? ZG : args.zg;
    const int zeta = args.zeta;
    const int32_t db = args.d / zeta;           // rows per stack block
    const int32_t t0 = grp * zg;                // first block of the group
    const int32_t row0 = t0 * db;               // first output row of the group
    const int32_t dl = zg * db;                 // partial rows
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    // lw[]: dl x SP partial words, then nw x 64 dummy words (sinks of
    // masked updates)
    for (int k = threadIdx.x; k < dl * SP; k += nthr) lw[k] = 0;
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t lunits = args.units / W;      // lane positions per row
    const int32_t unit = slice * SP + lane;
    const int32_t unit_c = unit < lunits ? unit : lunits - 1;   // in-bounds address
    const int64_t r0 = (int64_t)chunk * args.rows_per_chunk;
    const int64_t r1 = r0 + args.rows_per_chunk < args.m ? r0 + args.rows_per_chunk : args.m;
    const float *__restrict__ A = args.A;
    const int64_t lda = args.lda;
    const uint32_t dummy_row = (uint32_t)(dl * SP + wave * 64);
    const uint32_t dummy_lane = dummy_row + (uint32_t)lane;
    const bool in_slice = FULL || lane < SP;

    // Block of RB rows starting at b: A values per lane, and the group's RB*zg
    // metadata entries (row u, block t0+k on lane u*zg+k), as the entry's
    // row inside the partial (-1: skipped) and its value.  Loads use
    // in-bounds addresses (rows clamped into the chunk, columns into the
    // matrix): no branches.  Values of rows past the chunk are never used
    // (their entries are -1); lanes past the last column only touch partial
    // words never flushed.  A row block is addressed from one 64-bit base
    // with 32-bit offsets (the host keeps RB rows within 2^31 bytes).
    const uint32_t row_bytes = (uint32_t)lda * 4u;
    const uint32_t lane_bytes = (uint32_t)unit_c * (uint32_t)(K * 4);
    auto load_block = [&](int64_t b, vec_t (&a)[RB], int32_t &rl, float &vl) {
        const int64_t bb = b < r1 ? b : r1 - 1;
        const int64_t left = r1 - 1 - bb;
        const int32_t lim = left < RB - 1 ? (int32_t)left : RB - 1;
        const char *base = reinterpret_cast<const char *>(A + bb * lda);
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const uint32_t off = (uint32_t)(u < lim ? u : lim) * row_bytes + lane_bytes;
            a[u] = load_vec<K, NT>(base + off);
        }
        const int u = lane / zg;
        const int k = lane - u * zg;
        const int64_t row = b + u;
        const bool ok = lane < RB * zg && row < r1;
        const int64_t e = (ok ? row : r0) * zeta + t0 + k;
        const int32_t rv = args.row_idx[e] - row0;
        const float vv = args.val[e];
        // inside its own block t0+k: [k*db, (k+1)*db) of the partial
        rl = ok && (uint32_t)(rv - k * db) < (uint32_t)db ? rv : -1;
        vl = vv;
    };

    auto words_of = [&](const vec_t &x, float v, uint32_t (&c)[W]) {
#pragma unroll
        for (int i = 0; i < W; ++i) c[i] = T::contrib(x.x + i * T::kCols, v);
    };

    // General values: hits one at a time (rows walked with compile-time
    // indices so a[] stays in registers).
    auto apply_general = [&](uint64_t all, int32_t rl, float vl, const vec_t (&a)[RB]) {
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const uint64_t rowbits = zg >= 64 ? ~0ull : (((1ull << zg) - 1) << (u * zg));
            uint64_t g = all & rowbits;
            while (g) {
                const int j = __builtin_ctzll(g);
                g &= g - 1;
                const uint32_t r = (uint32_t)__builtin_amdgcn_readlane(rl, j);
                const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vl), j));
                if (in_slice) {
                    uint32_t c[W];
                    words_of(a[u], v, c);
                    const uint32_t idx = r * (uint32_t)SP + (uint32_t)lane;
                    cas_add<T, W>(lw, idx, lw[idx], c);
                }
            }
        }
    };

    auto process_block = [&](const vec_t (&a)[RB], int32_t rl, float vl) {
        const bool valid = rl >= 0;
        const uint64_t all = __ballot(valid);
        if (all == 0) return;
        if constexpr (ZG == 0) {
            apply_general(all, rl, vl, a);
        } else {
            const float mag = __builtin_fabsf(
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vl), __builtin_ctzll(all))));
            if (__ballot(valid && __builtin_fabsf(vl) != mag) != 0) {
                apply_general(all, rl, vl, a);
                return;
            }
            // per lane: partial word index of its hit (the dummy row when
            // skipped), the value's sign in bit 31
            const uint32_t pk = (valid ? (uint32_t)rl * (uint32_t)SP : dummy_row) |
                                (__float_as_uint(vl) & 0x80000000u);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                constexpr int RPS = NH / ZU;        // rows per group of hits
                if (((all >> (s * NH)) & (NH >= 64 ? ~0ull : ((1ull << NH) - 1))) == 0) continue;
                uint32_t h[RPS][W];
#pragma unroll
                for (int qq = 0; qq < RPS; ++qq) words_of(a[s * RPS + qq], mag, h[qq]);
                // every hit of the group, straight-line: reads, then swaps;
                // word index and signed contribution are rebuilt from the
                // hit's scalar entry when needed
                uint32_t sj[NH];
                word_t p[NH], o[NH];
                auto widx = [&](uint32_t e) -> uint32_t {
                    return in_slice ? (e & 0x7FFFFFFFu) + (uint32_t)lane : dummy_lane;
                };
                auto newval = [&](int j, word_t old) -> word_t {
                    const uint32_t m = T::signmask(sj[j]);
                    if constexpr (W == 1) {
                        return T::sum(old, h[j / ZU][0] ^ m);
                    } else {
                        return (word_t)T::sum((uint32_t)old, h[j / ZU][0] ^ m) |
                               ((word_t)T::sum((uint32_t)(old >> 32), h[j / ZU][1] ^ m) << 32);
                    }
                };
#pragma unroll
                for (int j = 0; j < NH; ++j) {
                    sj[j] = (uint32_t)__builtin_amdgcn_readlane((int)pk, s * NH + j);
                    p[j] = lw[widx(sj[j])];
                }
#pragma unroll
                for (int j = 0; j < NH; ++j) {
                    o[j] = p[j];
                    __hip_atomic_compare_exchange_strong(lw + widx(sj[j]), &o[j], newval(j, p[j]),
                                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                bool lost = false;
#pragma unroll
                for (int j = 0; j < NH; ++j) lost |= o[j] != p[j];
                if (__ballot(lost) != 0) {
                    // another wavefront (or an earlier hit of this group)
                    // changed the word: add onto what the swap returned
#pragma unroll
                    for (int j = 0; j < NH; ++j) {
                        if (o[j] != p[j]) {
                            uint32_t c[W];
                            const uint32_t m = T::signmask(sj[j]);
#pragma unroll
                            for (int i = 0; i < W; ++i) c[i] = h[j / ZU][i] ^ m;
                            cas_add<T, W>(lw, widx(sj[j]), o[j], c);
                        }
                    }
                }
            }
        }
    };

    // Two register sets in ping-pong: the loads of the next block are in
    // flight while the current block's hits are applied.
    const int64_t stride = (int64_t)nw * RB;
    vec_t a0[RB], a1[RB];
    int32_t rl0, rl1;
    float vl0, vl1;
    int64_t b = r0 + (int64_t)wave * RB;
    if (b < r1) {
        load_block(b, a0, rl0, vl0);
        for (;;) {
            load_block(b + stride, a1, rl1, vl1);
            process_block(a0, rl0, vl0);
            b += stride;
            if (b >= r1) break;
            load_block(b + stride, a0, rl0, vl0);
            process_block(a1, rl1, vl1);
            b += stride;
            if (b >= r1) break;
        }
    }
    __syncthreads();

    // flush the partial once: rows row0 .. row0+dl-1 of the (slice, chunk)
    const int SPW = SP * W;                     // words per partial row
    const int total = dl * SPW;
    if (args.ws != nullptr) {
        uint32_t *dst = args.ws + ((int64_t)slice * args.chunks + chunk) * (int64_t)args.d * SPW +
                        (int64_t)row0 * SPW;
        for (int k = threadIdx.x; k < total; k += nthr) dst[k] = lds[k];
    } else {
        typename T::out_t *B = reinterpret_cast<typename T::out_t *>(args.B);
        for (int k = threadIdx.x; k < total; k += nthr) {
            const int r = k / SPW;
            const int32_t u = slice * SPW + (k - r * SPW);
            const uint32_t w = lds[k];
            if (u < args.units && w != 0u)
                T::global_add(B, (int64_t)(row0 + r) * args.ldb + u, w);
        }
    }
}

// How the reduce combines the chunk partials (the mode argument of
// launch_stack_reduce): bit 0 adds onto B's current words (B += ...), bit 1
// adds FP16 partials in FP32 and rounds the total once.
constexpr int kReduceAccumulate = kReduceModeAccumulate;
constexpr int kReduceCombineF32 = kReduceModeCombineF32;

// B[r, u] (=|+=) the sum over chunks p = 0..P-1 of the workspace partials.
// A 256-thread block takes 64 output words (one per lane).  Its 4
// wavefronts each sum a contiguous quarter of the chunks in chunk order,
// starting from +0, and the non-empty quarter sums are then added in
// quarter order onto the existing B word (accumulate) or onto +0: a fixed
// order, so the result is deterministic, with four times the loads in
// flight of one thread per word.
// WIDE = false: every addition is one of the partials' own (FP32, or FP16
// nearest-even per half for FP16 partials), so an FP16 sketch is accumulated
// in FP16 from its first contribution to its stored value.  WIDE = true
// (FP16 only): the FP16 partials are widened exactly to FP32, summed in
// FP32, and the total is rounded to FP16 once.
template <class T, bool WIDE>
__global__ __launch_bounds__(256) void k_stack_reduce(const StackApplyArgs args, int32_t spw,
                                                       int32_t accumulate) {
    struct Narrow {
        typedef uint32_t wide_t;
        __device__ static wide_t widen(uint32_t w) { return w; }
        __device__ static wide_t wide_add(wide_t a, wide_t b) { return T::sum(a, b); }
        __device__ static uint32_t narrow(wide_t a) { return a; }
    };
    typedef typename std::conditional<WIDE, T, Narrow>::type C;
    typedef typename C::wide_t wide_t;
    __shared__ wide_t part[4][64];
    typename T::out_t *B = reinterpret_cast<typename T::out_t *>(args.B);
    const int64_t total = (int64_t)args.d * args.units;
    const int64_t plane = (int64_t)args.d * spw;
    const int P = args.chunks;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int p0 = wave * P / 4, p1 = (wave + 1) * P / 4;
    for (int64_t k0 = (int64_t)blockIdx.x * 64; k0 < total; k0 += (int64_t)gridDim.x * 64) {
        const int64_t k = k0 + lane;
        const bool act = k < total;
        const int r = act ? (int)(k / args.units) : 0;
        const int32_t u = act ? (int32_t)(k - (int64_t)r * args.units) : 0;
        wide_t acc = C::widen(0u);
        if (act) {
            const int32_t s = u / spw;
            const int cl = u - s * spw;
            const uint32_t *src = args.ws + (int64_t)s * P * plane + (int64_t)r * spw + cl;
            int p = p0;
            for (; p + 8 <= p1; p += 8) {
                uint32_t w[8];
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) w[qq] = src[(int64_t)(p + qq) * plane];
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) acc = C::wide_add(acc, C::widen(w[qq]));
            }
            for (; p < p1; ++p) acc = C::wide_add(acc, C::widen(src[(int64_t)p * plane]));
        }
        part[wave][lane] = acc;
        __syncthreads();
        if (wave == 0 && act) {
            const int64_t off = (int64_t)r * args.ldb + u;
            wide_t sum = C::widen(accumulate ? T::get(B, off) : 0u);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                if ((w + 1) * P / 4 > w * P / 4) sum = C::wide_add(sum, part[w][lane]);
            T::put(B, off, C::narrow(sum));
        }
        __syncthreads();
    }
}

// Launch of k_stack_reduce over d x units output words; mode is a
// combination of kReduceAccumulate and kReduceCombineF32.
template <class T>
hipError_t launch_stack_reduce(const StackApplyArgs &a, int32_t spw, int mode, hipStream_t s) {
    const int64_t total = (int64_t)a.d * a.units;
    int64_t blocks = (total + 63) / 64;
    if (blocks > 65535) blocks = 65535;
    if (blocks < 1) return hipSuccess;
    const int32_t acc = (mode & kReduceAccumulate) ? 1 : 0;
    if ((mode & kReduceCombineF32) && T::kCols == 2)
        k_stack_reduce<T, true><<<dim3((unsigned)blocks), 256, 0, s>>>(a, spw, acc);
    else
        k_stack_reduce<T, false><<<dim3((unsigned)blocks), 256, 0, s>>>(a, spw, acc);
    return hipGetLastError();
}

}  // namespace sk
