// LDS-privatized SparseStack apply for gfx950, shared by the FP32 and the
// FP16-accumulate entry points.
//
// What is computed (FP16 sketching page §III-A/§III-B): for every input row i
// and stack block t, the contribution val[i*zeta+t] * A[i, :] is added to
// output row row_idx[i*zeta+t]; in the FP16 variant each FP32 product is
// rounded to FP16 (nearest-even) and added with FP16 nearest-even additions.
//
// How (MI355X-specific):
//  * A workgroup owns a slice of SP lanes (SP columns for FP32, SP column
//    pairs for FP16) and a chunk of input rows, and keeps a private d x SP
//    partial sketch in LDS (32-bit words: one FP32 value, or one packed f16x2
//    pair).  Each wavefront streams whole rows of its slice: 64 lanes on
//    consecutive columns, so a row segment is one coalesced load.
//  * gfx950 executes floating-point LDS atomics (ds_add_f32, ds_pk_add_f16,
//    ds_pk_add_bf16) one lane at a time, about 3 clocks per active lane,
//    while plain LDS reads and writes and integer LDS atomics take a few
//    clocks per 64-lane instruction.  So partial rows are updated with a
//    plain read-add-write under a per-row LDS lock: one ds_wrxchg_rtn_b32
//    instruction tries the locks of up to 16 (row, block) hits at once (lane j
//    holds hit j), the hits whose locks were won are read, added and written,
//    and one store releases them; lost hits retry.  A lane never waits while
//    holding a lock, so some wave always progresses and every hit is applied
//    exactly once.  LDS instructions of one wave are performed in issue order,
//    so the data written before a release is visible to the next owner.
//  * At the end the partial is flushed once: either with packed/FP32 global
//    atomics into B, or with plain stores into a caller-supplied workspace
//    that a second kernel reduces in a fixed chunk order (no atomics, and no
//    separate zeroing of B).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sk_apply_common.hpp"

namespace sk {

// Per-lane element types of the two accumulation precisions.
struct AccF32 {
    typedef float in_t;     // one A column per lane
    typedef float out_t;    // B element
    __device__ static in_t load(const float *A, int64_t i, int64_t lda, int32_t unit) {
        return A[i * lda + unit];
    }
    // partial word + val * a: FP32 product, then FP32 sum, each rounded to
    // nearest-even (no fused multiply-add)
    __device__ static uint32_t add(uint32_t p, in_t a, float v) {
        return __float_as_uint(__fadd_rn(__uint_as_float(p), __fmul_rn(a, v)));
    }
    __device__ static uint32_t sum(uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    }
    __device__ static void global_add(out_t *B, int64_t off, uint32_t w) {
        atomic_add_global_f32(B + off, __uint_as_float(w));
    }
    __device__ static uint32_t get(const out_t *B, int64_t off) { return __float_as_uint(B[off]); }
    __device__ static void put(out_t *B, int64_t off, uint32_t w) { B[off] = __uint_as_float(w); }
};

struct AccF16 {
    typedef float2 in_t;    // one column pair per lane
    typedef h2_t out_t;     // B column pair
    __device__ static in_t load(const float *A, int64_t i, int64_t lda, int32_t unit) {
        return *reinterpret_cast<const float2 *>(A + i * lda + 2 * unit);
    }
    // FP32 products, each rounded to FP16 (RN), added to the pair with
    // per-half FP16 RN additions (v_pk_add_f16, subnormals kept)
    __device__ static uint32_t add(uint32_t p, in_t a, float v) {
        const h2_t s = __builtin_bit_cast(h2_t, p) + cvt_rn_h2(a.x * v, a.y * v);
        return __builtin_bit_cast(uint32_t, s);
    }
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
};

struct LockApplyArgs {
    const float *A;
    const int32_t *row_idx;
    const float *val;
    void *B;                // AccF32::out_t or AccF16::out_t, d x units, ldb units apart
    uint32_t *ws;           // NULL: flush with global atomics; else [slices][chunks][d][sp] words
    int64_t m, lda, ldb;    // lda in floats, ldb in B units
    int64_t rows_per_chunk;
    int32_t units;          // columns (FP32) or column pairs (FP16)
    int32_t d, zeta, sp;    // sp: lanes per slice (power of two, <= 64)
    int32_t chunks;
};

constexpr int kLockBlockThreads = 1024;

// Rows a wave loads per block and rows whose hits share one lock instruction.
template <int ZETA>
struct LockShape {
    static constexpr int RB = ZETA == 0 ? 1 : (ZETA <= 8 ? 8 : 64 / ZETA);
    static constexpr int U = ZETA == 0 ? 1 : (16 / ZETA >= RB ? RB : (16 / ZETA > 0 ? 16 / ZETA : 1));
};

template <class T, int ZETA>
__global__ __launch_bounds__(kLockBlockThreads) void k_lock_apply(const LockApplyArgs args) {
    typedef typename T::in_t in_t;
    constexpr int RB = LockShape<ZETA>::RB;
    constexpr int U = LockShape<ZETA>::U;
    constexpr int NSUB = RB / U;
    extern __shared__ uint32_t lds[];
    const int SP = args.sp;
    const int32_t d = args.d;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    uint32_t *part = lds;                       // d x SP words
    uint32_t *locks = lds + (int64_t)d * SP;    // d words, 0 = free
    // then nw x 64 words: the waves' dummy rows, sinks of masked updates
    for (int k = threadIdx.x; k < d * (SP + 1); k += nthr) lds[k] = 0u;
    __syncthreads();

    const int zeta = ZETA ? ZETA : args.zeta;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t slice = blockIdx.x;
    const int32_t chunk = blockIdx.y;
    const int32_t unit = slice * SP + lane;
    const int32_t unit_c = unit < args.units ? unit : args.units - 1;   // in-bounds address
    const int64_t r0 = (int64_t)chunk * args.rows_per_chunk;
    const int64_t r1 = r0 + args.rows_per_chunk < args.m ? r0 + args.rows_per_chunk : args.m;
    const float *__restrict__ A = args.A;
    const int64_t lda = args.lda;
    const int64_t e_last = r1 * zeta - 1;       // last metadata entry of the chunk
    // word indices into lds[]: lanes >= SP always update the wave's dummy row
    const uint32_t dummy_row = (uint32_t)(d * (SP + 1) + wave * 64);
    const uint32_t dummy_lane = dummy_row + (uint32_t)lane;
    const bool in_slice = lane < SP;

    // Block of RB rows starting at b: A values per lane, and the block's
    // rows*zeta metadata entries with entry L on lane L (contiguous).  Every
    // load is issued with an in-bounds address (rows clamped into the chunk,
    // columns into the matrix), so the code is branch-free.  Values loaded
    // for rows past the chunk are never used: their entries are marked -1
    // and their updates go to the dummy row.  Lanes past the last column
    // only touch partial words that are never flushed.
    auto load_block = [&](int64_t b, in_t (&a)[RB], int32_t &rl, float &vl) {
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const int64_t i = b + u;
            const int64_t ic = i < r1 ? i : r1 - 1;
            a[u] = T::load(A, ic, lda, unit_c);
        }
        const int64_t e = b * zeta + lane;
        const bool ok = lane < RB * zeta && e <= e_last;
        const int64_t ec = e <= e_last ? e : e_last;
        const int32_t rv = args.row_idx[ec];
        const float vv = args.val[ec];
        rl = ok ? rv : -1;
        vl = vv;
    };

    // lds[] word of this lane for the hit on lane jj: its partial row if the
    // lock was won, else the dummy row.
    auto hit_word = [&](int32_t rl, uint64_t got, int jj) -> uint32_t {
        const uint32_t r = (uint32_t)__builtin_amdgcn_readlane(rl, jj);
        const uint32_t row = ((got >> jj) & 1u) ? r * (uint32_t)SP : dummy_row;
        return in_slice ? row + (uint32_t)lane : dummy_lane;
    };

    auto acquire = [&](uint64_t pending, int32_t rl) -> uint64_t {
        uint32_t old = 1u;
        if ((pending >> lane) & 1u)
            old = __hip_atomic_exchange(locks + rl, 1u, __ATOMIC_ACQUIRE,
                                        __HIP_MEMORY_SCOPE_WORKGROUP);
        return __ballot(((pending >> lane) & 1u) && old == 0u);
    };
    auto release = [&](uint64_t got, int32_t rl) {
        if ((got >> lane) & 1u)
            __hip_atomic_store(locks + rl, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // Slow path for hits that lost their lock: one hit at a time.  Rows are
    // walked with compile-time indices so a[] stays in registers.
    auto retry = [&](uint64_t pending, int32_t rl, float vl, const in_t (&a)[RB]) {
        while (pending) {
            const uint64_t got = acquire(pending, rl);
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const uint64_t rowbits =
                    zeta >= 64 ? ~0ull : (((1ull << zeta) - 1) << (u * zeta));
                uint64_t g = got & rowbits;
                while (g) {
                    const int j = __builtin_ctzll(g);
                    g &= g - 1;
                    const uint32_t r = (uint32_t)__builtin_amdgcn_readlane(rl, j);
                    const float v =
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vl), j));
                    if (in_slice) {
                        uint32_t *w = part + r * SP + lane;
                        *w = T::add(*w, a[u], v);
                    }
                }
            }
            release(got, rl);
            pending &= ~got;
        }
    };

    auto process_block = [&](const in_t (&a)[RB], int32_t rl, float vl) {
        // hits whose output row is in range; others contribute nothing
        const uint64_t all = __ballot((uint32_t)rl < (uint32_t)d);
        if constexpr (ZETA == 0) {
            retry(all, rl, vl, a);
        } else {
            constexpr int NH = U * ZETA;    // hits per lock instruction (<= 16)
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                const uint64_t smask = (NH >= 64 ? ~0ull : ((1ull << NH) - 1)) << (s * NH);
                const uint64_t pending = all & smask;
                if (pending == 0) continue;
                const uint64_t got = acquire(pending, rl);
                // every hit of the sub-batch, straight-line: reads, then adds
                // and writes (lost hits and idle lanes go to the dummy row)
                uint32_t w[NH], p[NH];
#pragma unroll
                for (int j = 0; j < NH; ++j) {
                    w[j] = hit_word(rl, got, s * NH + j);
                    p[j] = lds[w[j]];
                }
#pragma unroll
                for (int j = 0; j < NH; ++j) {
                    const float v =
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vl), s * NH + j));
                    lds[w[j]] = T::add(p[j], a[s * U + j / ZETA], v);
                }
                release(got, rl);
                if (pending & ~got) retry(pending & ~got, rl, vl, a);
            }
        }
    };

    // Two register sets in ping-pong: the loads of the next block are in
    // flight while the current block's hits are applied.
    const int64_t stride = (int64_t)nw * RB;
    in_t a0[RB], a1[RB];
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

    // flush the partial once
    const int total = d * SP;
    if (args.ws != nullptr) {
        uint32_t *dst = args.ws + ((int64_t)slice * args.chunks + chunk) * (int64_t)total;
        for (int k = threadIdx.x; k < total; k += nthr) dst[k] = part[k];
    } else {
        typename T::out_t *B = reinterpret_cast<typename T::out_t *>(args.B);
        for (int k = threadIdx.x; k < total; k += nthr) {
            const int r = k / SP;
            const int32_t u = slice * SP + (k - r * SP);
            const uint32_t w = part[k];
            if (u < args.units && w != 0u) T::global_add(B, (int64_t)r * args.ldb + u, w);
        }
    }
}

// B[r, u] (=|+=) sum over chunks p = 0..P-1, in that order, of the workspace
// partials: one thread per output unit, partials read coalesced.
template <class T>
__global__ __launch_bounds__(256) void k_lock_reduce(const LockApplyArgs args, int32_t slices,
                                                      int32_t accumulate) {
    typename T::out_t *B = reinterpret_cast<typename T::out_t *>(args.B);
    const int SP = args.sp;
    const int64_t total = (int64_t)args.d * args.units;
    const int64_t plane = (int64_t)args.d * SP;
    const int P = args.chunks;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * 256) {
        const int r = (int)(k / args.units);
        const int32_t u = (int32_t)(k - (int64_t)r * args.units);
        const int32_t s = u / SP;
        const int cl = u - s * SP;
        const uint32_t *src = args.ws + (int64_t)s * P * plane + (int64_t)r * SP + cl;
        const int64_t off = (int64_t)r * args.ldb + u;
        uint32_t acc = accumulate ? T::get(B, off) : 0u;
        int p = 0;
        for (; p + 8 <= P; p += 8) {
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) w[q] = src[(int64_t)(p + q) * plane];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc = T::sum(acc, w[q]);
        }
        for (; p < P; ++p) acc = T::sum(acc, src[(int64_t)p * plane]);
        T::put(B, off, acc);
    }
    (void)slices;
}

}  // namespace sk
