// BlockPerm-SJLT apply without a workspace for gfx950 (FlashSketch page §4,
// §5.1, §5.2, App. D): every output element is written once, by the one
// workgroup that accumulates it, with no global atomics.
//
// What is computed: Y (=|+=) S A for the shift wiring
// pi_j(g) = (sigma(g) + j C) mod M, C = M / kappa, so N(g) is the set of
// input blocks {rho + j C : j < kappa} with rho = sigma(g) mod C: the block
// graph is C disjoint complete bipartite components, each of kappa output
// blocks (g_l = sigma^-1(rho + l C)) and kappa input blocks (h_j = rho + j C).
// Row r of input block h adds +-A[r, :] / sqrt(kappa s) to the s rows
// (beta + i alpha) mod B_r of each output block g of its component, with
// v = fmix32(K(g, h) ^ r), beta = mulhi(v, B_r), alpha = 2 mulhi(fmix32(v +
// 0x9E3779B9), B_r / 2) + 1 (s > 1), sign negative when bit i of v is set.
//
// How (MI355X-specific):
//  * A workgroup (16 wavefronts) owns one component, one 32-column tile and
//    up to 64 of the component's kappa*B_r output rows (the tile rows).  It
//    reads the component's kappa*B_c input rows of its tile once (each
//    input element is read by one workgroup when kappa*B_r <= 64) in
//    stages of 128 rows, each 16-byte load two stages ahead of the stage
//    applied (a scalar stage base plus a fixed lane offset).
//  * Each tile row belongs to two 8-lane groups, one for the hits from the
//    stage's first 64 rows and one for the rest; a group's 8 lanes hold the
//    row's 32 columns as one float4 each, in registers.  No LDS
//    read-modify-write and no float atomics (gfx950 runs LDS float atomics
//    one lane at a time); the two sums of a row meet once, at the end.
//  * Per stage, every (row, output block, i) hit is hashed once and
//    bucketed by its group with an integer LDS atomic counter (a counting
//    sort: a few clocks per 64-lane instruction); a list entry is the staged
//    row's offset with the sign in bit 0.  Each group then walks its list
//    eight entries at a time (one LDS read of eight entries, eight
//    independent row reads, FMAs by +-1); slots past the count name a zero
//    row, so no lane branches, and each slot is reset to it after use.
//  * Staged rows are stored twice, once in each half of the LDS banks; the
//    two groups of a 16-lane LDS phase read opposite halves, so the row
//    reads of a phase never conflict (with one copy, two random rows of a
//    phase share banks about half the time).
//  * The loops step the stage with a cursor instead of dividing (64-bit
//    divisions per stage ran on the scalar unit and cost 10% of the time).
//    Within a stage the order in which a row's hits are added follows the
//    counter's slots, so the sums are not bitwise reproducible.
#include "sk_internal.hpp"
#include "sk_rng.hpp"
#include "sk_stream.hpp"

namespace sk {
namespace {

constexpr int kDW = 16;                 // wavefronts per workgroup
constexpr int kDThreads = kDW * 64;
constexpr int kDS = 128;                // input rows per stage
constexpr int kDRows = 64;              // tile rows per workgroup
constexpr int kDHalf = kDS / 2;         // stage rows per half: tile row r's hits from rows
                                        // u < kDHalf go to group r, the rest to group 64 + r
constexpr int kDCols = 32;              // columns per tile (8 lanes x float4)
constexpr int kDList = kDHalf + 8;      // u16 entries per group's list (+8: the lists of
                                        // groups k and k + 1 start 36 banks apart)
constexpr int kDMaxKappa = kBlockPermMaxM;
constexpr int kDMaxBlocks = kDRows + 1;  // output blocks one workgroup's tile rows touch
constexpr int kDLoads = kDS * 8 / kDThreads;   // float4 each lane loads per stage
static_assert(kDLoads * kDThreads == kDS * 8, "whole stages per load round");

struct Vec4 {
    float x, y, z, w;
};

// Nontemporal loads through the global address space (not flat: a flat load
// would also count against the LDS wait that each stage barrier does, and
// hold the barrier until the prefetched rows arrive).
__device__ __forceinline__ float load1_nt(const float *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_nontemporal_load(
        reinterpret_cast<__attribute__((address_space(1))) const float *>((uintptr_t)p));
#else
    return *p;
#endif
}
__device__ __forceinline__ Vec4 load4_nt(const float *p) {
    typedef float v4 __attribute__((ext_vector_type(4)));
#if defined(__HIP_DEVICE_COMPILE__)
    const v4 v = __builtin_nontemporal_load(
        reinterpret_cast<__attribute__((address_space(1))) const v4 *>((uintptr_t)p));
#else
    const v4 v = *reinterpret_cast<const v4 *>(p);
#endif
    return Vec4{v[0], v[1], v[2], v[3]};
}

// 4 floats of row `row` at columns col .. col+3 (VEC: one aligned 16-byte
// load; else 4 loads, columns past n clamped to n - 1).
template <bool VEC>
__device__ __forceinline__ Vec4 load4(const float *A, int64_t row, int64_t lda, int32_t col,
                                      int32_t n) {
    const float *p = A + row * lda;
    if constexpr (VEC) {
        // n % 4 == 0 here: a group past the last column reloads the last 4
        return load4_nt(p + (col < n ? col : n - 4));
    } else {
        const int32_t c0 = col < n ? col : n - 1;
        const int32_t c1 = col + 1 < n ? col + 1 : n - 1;
        const int32_t c2 = col + 2 < n ? col + 2 : n - 1;
        const int32_t c3 = col + 3 < n ? col + 3 : n - 1;
        return Vec4{load1_nt(p + c0), load1_nt(p + c1), load1_nt(p + c2), load1_nt(p + c3)};
    }
}

template <bool VEC, bool MULTI>
__global__ __launch_bounds__(kDThreads) void k_bp_direct(const BpDirectArgs args,
                                                         const BlockPermTable ginv) {
    // staged rows: row u (kDS: the zero row) at bytes [u*256, u*256 + 256),
    // stored twice, in the two 128-byte halves (LDS banks 0-31 and 32-63)
    __shared__ float4 data[2][(kDS + 1) * 16];
    // per tile row: kDList u16 entries u*256 | sign, the hits of the stage
    // in buffer b (slots past the stage's count hold the zero row)
    __shared__ uint32_t lists[2][2 * kDRows * kDList / 2];
    __shared__ uint32_t cnt[2][2 * kDRows];
    __shared__ uint32_t keys[2][kDMaxBlocks];          // K(g_l, h_j), l from l_lo; j by parity
    __shared__ int32_t gout[kDMaxBlocks];              // output block g_l, l from l_lo

    const int32_t kappa = args.kappa;
    const int32_t Br = args.Br;
    const int64_t Bc = args.Bc;
    // workgroup -> (column tile, component, row group)
    const int32_t wg = blockIdx.x;
    const int32_t tile = wg % args.tiles;
    const int32_t cg = wg / args.tiles;
    const int32_t grp = cg % args.groups;
    const int32_t rho = cg / args.groups;
    const int32_t tr0 = grp * kDRows;                   // first tile row of the workgroup
    const int32_t T = kappa * Br;
    const int32_t trn = T - tr0 < kDRows ? T - tr0 : kDRows;
    // output blocks whose rows this workgroup holds
    const int32_t l_lo = tr0 / Br, l_hi = (tr0 + trn - 1) / Br;
    const int32_t nl = l_hi - l_lo + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane & 7;                             // the lane's float4 of the tile
    const int k = wave * 8 + (lane >> 3);               // the lane's 8-lane group
    const int kr = k & (kDRows - 1);                    // its tile row (two groups per row)
    const int32_t col0 = tile * kDCols;
    // the half of each staged row this lane reads: 8-lane groups k and k + 1
    // share a 16-lane LDS phase and read opposite halves (no bank conflict)
    const uint32_t lane_off = (uint32_t)((k & 1) * 128 + q * 16);

    const int64_t spb = (Bc + kDS - 1) / kDS;           // stages per input block
    const int64_t nst = spb * kappa;
    const int s_rows = MULTI ? args.s : 1;
    constexpr uint32_t kZero = kDS * 256;               // entry of the zero row
    constexpr uint32_t kZeroPair = kZero | (kZero << 16);

    // keys of input block j (0 <= j < kappa) into keys[j & 1]
    auto make_keys = [&](int64_t j) {
        if (j >= kappa) return;
        const uint32_t h = (uint32_t)(rho + j * args.C);
        for (int l = tid; l < nl; l += kDThreads)
            keys[j & 1][l] = blockperm_key(args.seed, (uint32_t)gout[l], h);
    };
    for (int l = tid; l < nl; l += kDThreads) gout[l] = ginv.tab[rho + (l_lo + l) * args.C];
    for (int i = tid; i < 2 * 2 * kDRows; i += kDThreads) (&cnt[0][0])[i] = 0u;
    for (int i = tid; i < 2 * 2 * kDRows * kDList / 2; i += kDThreads)
        (&lists[0][0])[i] = kZeroPair;
    for (int i = tid; i < 16; i += kDThreads) {
        data[0][kDS * 16 + i] = make_float4(0.f, 0.f, 0.f, 0.f);
        data[1][kDS * 16 + i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();                                    // gout
    make_keys(0);
    make_keys(1);

    // A stage as (input block j of the component, first row r0 in it),
    // stepped without divisions (the stage loop would otherwise run 64-bit
    // divisions on the scalar unit every stage); past the last stage a
    // cursor stays on it
    struct Cursor {
        int32_t j;
        int64_t r0;
    };
    auto advance = [&](Cursor &c) {
        if (c.j == kappa - 1 && c.r0 + kDS >= Bc) return;
        c.r0 += kDS;
        if (c.r0 >= Bc) {
            c.r0 = 0;
            ++c.j;
        }
    };
    // loads of the cursor's stage (rows clamped into the block: every load
    // is in bounds)
    Vec4 regs[2][kDLoads];
    // full stages of 16-byte loads: a scalar stage base and a fixed 32-bit
    // offset per lane (rows of a stage span less than 2^32 bytes)
    const bool fast = VEC && args.lda <= ((int64_t)1 << 22);
    uint32_t loff[kDLoads];
#pragma unroll
    for (int i = 0; i < kDLoads; ++i) {
        const int f = tid + i * kDThreads;
        const int32_t col = col0 + (f & 7) * 4;
        const int32_t colc = col < args.n ? col : args.n - 4;
        loff[i] = fast ? (uint32_t)(((int64_t)(f >> 3) * args.lda + colc) * 4) : 0u;
    }
    auto load = [&](const Cursor &cur, Vec4 (&rv)[kDLoads]) {
        const int64_t r0 = cur.r0;
        const int64_t base = (rho + (int64_t)cur.j * args.C) * Bc;   // first row of block h_j
        if constexpr (VEC) {
            if (fast && r0 + kDS <= Bc) {
                const uint64_t sb = uniform_addr((uint64_t)(uintptr_t)(args.A + (base + r0) * args.lda));
#pragma unroll
                for (int i = 0; i < kDLoads; ++i) {
                    const FVec<4> v = load_row<4>(sb, loff[i]);
                    rv[i] = Vec4{v.x[0], v.x[1], v.x[2], v.x[3]};
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < kDLoads; ++i) {
            const int f = tid + i * kDThreads;
            int64_t r = r0 + (f >> 3);
            r = r < Bc ? r : Bc - 1;
            rv[i] = load4<VEC>(args.A, base + r, args.lda, col0 + (f & 7) * 4, args.n);
        }
    };
    // the stage's rows into both halves of their slots in data[b]; lanes
    // 8-15 of each 16-lane phase write the other half first, so the two rows
    // of a phase never share banks
    auto stage = [&](const Vec4 (&rv)[kDLoads], int b) {
#pragma unroll
        for (int i = 0; i < kDLoads; ++i) {
            const int f = tid + i * kDThreads;
            const int h = (f >> 3) & 1;
            const float4 v = make_float4(rv[i].x, rv[i].y, rv[i].z, rv[i].w);
            float4 *row = data[b] + (f >> 3) * 16 + (f & 7);
            row[h * 8] = v;
            row[(h ^ 1) * 8] = v;
        }
    };
    // the hits of the cursor's stage on this workgroup's tile rows into lists[b]
    auto build = [&](const Cursor &cur, int b) {
        const int64_t r0 = cur.r0;
        const int32_t nrows = (int32_t)(Bc - r0 < kDS ? Bc - r0 : kDS);
        const uint32_t *kk = keys[cur.j & 1];
        uint16_t *lb = reinterpret_cast<uint16_t *>(lists[b]);
        const int32_t E = kDS * nl;                     // (row, output block) pairs
        for (int e = tid; e < E; e += kDThreads) {
            const int u = e & (kDS - 1);
            const int li = e / kDS;
            if (u >= nrows) continue;
            const uint32_t v = fmix32(kk[li] ^ (uint32_t)(r0 + u));
            const uint32_t beta = mulhi32(v, (uint32_t)Br);
            uint32_t alpha = 0u;
            if constexpr (MULTI) alpha = 2u * mulhi32(fmix32(v + 0x9E3779B9u), (uint32_t)Br >> 1) + 1u;
            for (int i = 0; i < s_rows; ++i) {
                const uint32_t row = MULTI ? ((beta + (uint32_t)i * alpha) & ((uint32_t)Br - 1u)) : beta;
                const int32_t tr = (l_lo + li) * Br + (int32_t)row - tr0;
                if (tr < 0 || tr >= trn) continue;
                const int32_t g = (u >= kDHalf ? kDRows : 0) + tr;   // the row's group
                const uint32_t slot = atomicAdd(&cnt[b][g], 1u);
                lb[g * kDList + slot] = (uint16_t)((uint32_t)u * 256u | ((v >> i) & 1u));
            }
        }
    };

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const char *const dbytes[2] = {reinterpret_cast<const char *>(data[0]),
                                   reinterpret_cast<const char *>(data[1])};
    // a += x * (+1 or -1 by bit 0 of e): exactly a + x or a - x
    auto add_hit = [&](const float4 &x, uint32_t e) {
        const float sg = __uint_as_float(0x3F800000u | (e << 31));
        acc[0] = __builtin_fmaf(x.x, sg, acc[0]);
        acc[1] = __builtin_fmaf(x.y, sg, acc[1]);
        acc[2] = __builtin_fmaf(x.z, sg, acc[2]);
        acc[3] = __builtin_fmaf(x.w, sg, acc[3]);
    };
    // this group's hits of the stage in buffer b, eight at a time: one read
    // of eight entries, eight independent row reads (past the list's end
    // the entries name the zero row), then the slots are reset to it.  An
    // entry is u*256 | sign: its row address is (e & 0xFF00) | lane_off.
    auto process = [&](int b) {
        const uint32_t c = kr < trn ? cnt[b][k] : 0u;
        __builtin_amdgcn_wave_barrier();
        if (q == 0 && kr < trn) cnt[b][k] = 0u;         // ready for the stage after next
        uint4 *lw = reinterpret_cast<uint4 *>(lists[b] + k * (kDList / 2));
        const char *db = dbytes[b];
        for (uint32_t t0 = 0; __ballot(t0 < c) != 0; t0 += 8) {
            const uint4 ev = lw[t0 >> 3];
            const uint32_t w[4] = {ev.x, ev.y, ev.z, ev.w};
            float4 x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = *reinterpret_cast<const float4 *>(db + ((w[i] & 0xFF00u) | lane_off));
                x[2 * i + 1] =
                    *reinterpret_cast<const float4 *>(db + (((w[i] >> 16) & 0xFF00u) | lane_off));
            }
            if (q == 0) lw[t0 >> 3] = make_uint4(kZeroPair, kZeroPair, kZeroPair, kZeroPair);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                add_hit(x[2 * i], w[i]);
                add_hit(x[2 * i + 1], w[i] >> 16);
            }
        }
    };

    // stage 0 staged and built, stages 1 and 2 loading; then per stage st:
    // apply st, stage and build st+1 from the register set it was loaded
    // into, reload that set with stage st+3
    Cursor lc{0, 0}, bc{0, 0};                          // next load, next build
    load(lc, regs[0]);
    advance(lc);
    load(lc, regs[1]);
    advance(lc);
    stage(regs[0], 0);
    __syncthreads();                                    // keys of blocks 0 and 1
    build(bc, 0);
    advance(bc);
    load(lc, regs[0]);
    advance(lc);
    lds_barrier();
    for (int64_t s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t st = s0 + b;
            if (st < nst) {
                process(b);
                if (st + 1 < nst) {
                    stage(regs[b ^ 1], b ^ 1);
                    build(bc, b ^ 1);
                    // the first stage of block j is built here: the keys of
                    // block j + 1 go to the slot block j - 1's keys held
                    if (bc.r0 == 0) make_keys(bc.j + 1);
                    advance(bc);
                }
            }
            // on every path, so each staging step finds the other set's
            // loads issued after its own
            load(lc, regs[b ^ 1]);
            advance(lc);
            lds_barrier();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    // the second group of each tile row hands its sum to the first through
    // LDS (data[0] is free: the last stage barrier has passed), which adds
    // it and writes the row of Y, scaled once
    float4 *part = data[0];
    if (k >= kDRows) part[kr * 8 + q] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (k < kDRows && kr < trn) {
        const float4 o = part[kr * 8 + q];
        acc[0] += o.x;
        acc[1] += o.y;
        acc[2] += o.z;
        acc[3] += o.w;
        const int32_t tr = tr0 + kr;
        const int32_t l = tr / Br;
        const int64_t orow = (int64_t)gout[l - l_lo] * Br + (tr - l * Br);
        float *y = args.Y + orow * args.ldy;
        const float sc = args.scale;
        const float v[4] = {acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc};
        const int32_t c = col0 + q * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (c + i < args.n) y[c + i] = args.accumulate ? y[c + i] + v[i] : v[i];
    }
}

template <bool MULTI>
const void *pick_direct(bool vec) {
    return vec ? (const void *)k_bp_direct<true, MULTI> : (const void *)k_bp_direct<false, MULTI>;
}

}  // namespace

bool plan_bp_direct(int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa, int32_t s,
                    BpDirectPlan *p) {
    if (M < 1 || kappa < 1 || M % kappa != 0 || m % M != 0 || d % M != 0 || n < 1) return false;
    if (kappa > kDMaxKappa) return false;
    const int64_t Br = d / M, Bc = m / M;
    if (s < 1 || s > Br || (s > 1 && (Br & (Br - 1)) != 0)) return false;
    const int64_t T = (int64_t)kappa * Br;
    const int64_t tiles = (n + kDCols - 1) / kDCols;
    const int64_t groups = (T + kDRows - 1) / kDRows;
    const int64_t C = M / kappa;
    const int64_t grid = C * groups * tiles;
    if (grid < 1 || grid > ((int64_t)1 << 31) - 1) return false;
    if (Bc > ((int64_t)1 << 40)) return false;
    p->tiles = (int32_t)tiles;
    p->groups = (int32_t)groups;
    p->grid = grid;
    return true;
}

hipError_t launch_bp_direct(const BpDirectPlan &p, const BpDirectArgs &args,
                            const BlockPermTable &ginv, hipStream_t s) {
    // the launch must match the plan's ownership: every tile row of every
    // component and column tile belongs to exactly one workgroup
    const int64_t T = (int64_t)args.kappa * args.Br;
    if (args.kappa < 1 || args.kappa > kDMaxKappa || args.Br < 1 || args.s < 1 ||
        args.s > args.Br || (args.s > 1 && (args.Br & (args.Br - 1)) != 0) ||
        args.tiles != p.tiles || args.groups != p.groups ||
        (int64_t)p.groups * kDRows < T || (int64_t)p.tiles * kDCols < args.n ||
        (int64_t)args.C * args.kappa != args.M || p.grid != (int64_t)args.C * p.groups * p.tiles)
        return hipErrorInvalidValue;
    const bool vec = args.n % 4 == 0 && args.lda % 4 == 0 && (uintptr_t)args.A % 16 == 0;
    const void *kern = args.s > 1 ? pick_direct<true>(vec) : pick_direct<false>(vec);
    BpDirectArgs a = args;
    BlockPermTable t = ginv;
    void *params[] = {&a, &t};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3(kDThreads), params, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace sk
