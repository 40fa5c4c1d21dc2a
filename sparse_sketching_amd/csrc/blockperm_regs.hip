// Register-accumulating BlockPerm-SJLT apply for gfx950 (FlashSketch page
// §4, §5, App. B.1, App. D).
//
// What is computed: what the slice kernel (blockperm_general.hip) computes.
// Input block h is read by kappa output blocks, its readers (reader l is
// the output block whose l-th neighbour is h); row r of h, with
// v = fmix32(K(g_l, h) ^ r), adds +-A[r, :] to the s rows
// (beta + j alpha) mod B_r of reader l's block (beta = mulhi(v, B_r), alpha
// as in App. D; s = 1: beta alone), sign negative when bit j of v is set,
// every nonzero of magnitude 1/sqrt(kappa s).  The kappa*B_r partial rows of
// each (h, row slice) go to the workspace once and the reduce kernel sums
// them per output block in a fixed order (neighbour, then slice).
//
// How (MI355X-specific):
//  * A workgroup of 16 wavefronts owns (input block h, row slice, a
//    256-column slice, a row group): wavefront w keeps R consecutive
//    partial rows (all inside one reader's block) for its 64 lanes x 4
//    columns in registers.  No atomics and no LDS read-modify-write: the
//    LDS tiles of the component and slice kernels cost a read and a write
//    per contribution, this kernel a read per contribution.
//  * Rows stream through double-buffered LDS stages of 64 rows: each
//    wavefront loads 4 rows (one 1 KB float4 row segment each) and writes
//    them to the stage; one wavefront per stage (rotating) hashes the
//    stage's rows for every reader, one row per lane, into LDS.  After one
//    barrier each wavefront reads its reader's hashes, ballots the rows
//    that hit each of its R rows and adds each hit's stage row with a
//    scalar +-1 FMA (exactly an add or a subtract).  The scale multiplies
//    the partial once, at the end.
//  * Two register sets of loaded rows keep the next stages in flight from
//    HBM while a stage is applied; a barrier that waits for LDS only
//    (lds_barrier) leaves them in flight.
#include "sk_internal.hpp"
#include "sk_rng.hpp"
#include "sk_stream.hpp"
#include "sk_blockperm.hpp"

namespace sk {
namespace {

constexpr int kW = 16;                      // wavefronts per workgroup
constexpr int kS = kBpRegsStage;            // input rows per stage
constexpr int kD = kS / kW;                 // rows a wavefront loads per stage
constexpr int kP = 2;                       // register sets of loaded rows
constexpr int kK = kBlockPermGenMaxKappa;
static_assert(kS == 64, "one stage row per lane in the hash and ballot steps");
static_assert(kBpRegsCols == 64 * 4, "a slice is 64 lanes x one float4");

// +1.0f or -1.0f for bit i of the wave-uniform mask (built in scalar
// registers: the FMAs take it as their scalar operand).
__device__ __forceinline__ float sign_of(uint64_t neg, int i) {
    return __builtin_bit_cast(float, 0x3F800000u | ((uint32_t)(neg >> i) << 31));
}

// a += sg * x: exactly a + x or a - x.
__device__ __forceinline__ void add_signed(float (&a)[4], const float4 &x, float sg) {
    a[0] = __builtin_fmaf(x.x, sg, a[0]);
    a[1] = __builtin_fmaf(x.y, sg, a[1]);
    a[2] = __builtin_fmaf(x.z, sg, a[2]);
    a[3] = __builtin_fmaf(x.w, sg, a[3]);
}

template <int R, bool MULTI>
__global__ __launch_bounds__(kW * 64) void k_bp_regs(const BlockPermGenArgs args,
                                                     const BlockPermTable ginv) {
    __shared__ float4 hs0[kS * 64];         // stage rows, row j at [j*64, j*64+64)
    __shared__ float4 hs1[kS * 64];
    __shared__ uint32_t me0[kK * kS];       // hash v of (reader l, stage row j) at l*kS + j
    __shared__ uint32_t me1[kK * kS];
    __shared__ uint32_t keys[kK];           // K(reader l, h)

    // workgroup -> (unit, row group); the groups of one unit are 8 ids
    // apart (same XCD under round-robin dispatch, so their reads of the
    // same rows meet in one L2)
    const int32_t G = args.groups;
    const int32_t wg = blockIdx.x;
    const int32_t qq = wg >> 3;
    const int32_t grp = qq % G;
    const int32_t unit = (qq / G) * 8 + (wg & 7);
    if (unit >= args.M * args.Q * args.slices) return;
    const int32_t slice = unit % args.slices;
    const int32_t hq = unit / args.slices;  // h * Q + row slice
    const int32_t q = hq % args.Q;
    const uint32_t h = (uint32_t)(hq / args.Q);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kappa = args.kappa;
    const uint32_t Br = (uint32_t)args.Br;
    const int32_t lo = (grp * kW + wave) * R;           // first partial row of the wave
    const int32_t lw = lo / (int32_t)Br;                 // its reader
    const uint32_t lob = (uint32_t)(lo - lw * (int32_t)Br);
    const int64_t rb = (int64_t)q * args.rows_per_slice;  // first row of the slice in h
    const int32_t nrows =
        (int32_t)(rb + args.rows_per_slice < args.Bc ? args.rows_per_slice : args.Bc - rb);
    const int32_t nst = (nrows + kS - 1) / kS;
    // the lane's 4 columns, clamped into the row (lanes past the last column
    // load valid memory and write nothing)
    const int32_t col = slice * kBpRegsCols + lane * 4;
    const int32_t col_c = col <= args.n - 4 ? col : args.n - 4;
    const uint32_t lane_off = (uint32_t)col_c * 4u;
    const char *Ablk =
        reinterpret_cast<const char *>(args.A) + ((int64_t)h * args.Bc + rb) * args.lda * 4;
    const int64_t ldab = args.lda * 4;

    if ((int)threadIdx.x < kappa)
        keys[threadIdx.x] = blockperm_key(args.seed, bp_reader(args, ginv, h, threadIdx.x), h);

    float acc[R][4];
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k][0] = acc[k][1] = acc[k][2] = acc[k][3] = 0.f;

    typedef FVec<4> vec_t;
    vec_t a[kP][kD];
    // this wavefront's kD rows of stage st, clamped into the slice.  Every
    // call issues its loads, also past the last stage (the clamped rows are
    // L2 hits): a skipped load would make the compiler wait for the other
    // register set's loads at every staging step.
    auto load = [&](int32_t st, vec_t (&av)[kD]) {
#pragma unroll
        for (int u = 0; u < kD; ++u) {
            int32_t rel = st * kS + wave * kD + u;
            rel = rel < nrows ? rel : nrows - 1;
            av[u] = load_row<4>(uniform_addr((uint64_t)(Ablk + (int64_t)rel * ldab)), lane_off);
        }
    };
    auto stage = [&](const vec_t (&av)[kD], float4 *hs) {
#pragma unroll
        for (int u = 0; u < kD; ++u)
            hs[(wave * kD + u) * 64 + lane] = make_float4(av[u].x[0], av[u].x[1], av[u].x[2],
                                                          av[u].x[3]);
    };
    // the hashes of stage st's rows for every reader, lane j <-> row j
    auto draw = [&](int32_t st, uint32_t *me) {
        if (wave != (st & (kW - 1))) return;
        const uint32_t r = (uint32_t)(rb + (int64_t)st * kS + lane);
#pragma unroll 4
        for (int l = 0; l < kappa; ++l) me[l * kS + lane] = fmix32(keys[l] ^ r);
    };
    // every hit of stage st on this wavefront's rows
    auto apply = [&](int32_t st, const float4 *hs, const uint32_t *me) {
        const uint32_t v = me[lw * kS + lane];
        const bool valid = st * kS + lane < nrows;
        const uint32_t beta = mulhi32(v, Br);
        uint32_t alpha = 0u;
        if constexpr (MULTI) alpha = 2u * mulhi32(fmix32(v + 0x9E3779B9u), Br >> 1) + 1u;
        const int ns = MULTI ? args.s : 1;
        for (int j = 0; j < ns; ++j) {
            // B_r is a power of two when s > 1
            const uint32_t rk = (MULTI ? ((beta + (uint32_t)j * alpha) & (Br - 1u)) : beta) - lob;
            const uint64_t neg = __ballot((v >> j) & 1u);
#pragma unroll
            for (int k = 0; k < R; ++k) {
                // hits two at a time: both stage reads are in flight together
                uint64_t mk = __ballot(valid && rk == (uint32_t)k);
                while (mk & (mk - 1)) {
                    const int i0 = __builtin_ctzll(mk);
                    mk &= mk - 1;
                    const int i1 = __builtin_ctzll(mk);
                    mk &= mk - 1;
                    const float4 x0 = hs[i0 * 64 + lane];
                    const float4 x1 = hs[i1 * 64 + lane];
                    add_signed(acc[k], x0, sign_of(neg, i0));
                    add_signed(acc[k], x1, sign_of(neg, i1));
                }
                if (mk) {
                    const int i0 = __builtin_ctzll(mk);
                    add_signed(acc[k], hs[i0 * 64 + lane], sign_of(neg, i0));
                }
            }
        }
    };

    // stage 0 staged and stages 1..kP loading; then per stage st: apply st,
    // stage st+1 into the other buffer from the register set it was loaded
    // into, hash st+1, and reload the set with stage st+1+kP
    __syncthreads();                        // keys
    load(0, a[0]);
    stage(a[0], hs0);
    draw(0, me0);
#pragma unroll
    for (int p = 1; p <= kP; ++p) load(p, a[p % kP]);
    __syncthreads();
    for (int32_t s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int32_t st = s0 + b;
            if (st < nst) {
                apply(st, b ? hs1 : hs0, b ? me1 : me0);
                stage(a[(b + 1) % kP], b ? hs0 : hs1);
                draw(st + 1, b ? me0 : me1);
            }
            // on every path, so each staging step finds the other set's
            // loads issued after its own
            load(st + 1 + kP, a[(b + 1) % kP]);
            lds_barrier();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    // the wavefront's R partial rows of (h, row slice):
    // ws[(hq*kappa*B_r + lo + k)*n + col]
    if (col < args.n) {
        const float c = args.scale;
        float *dst = args.ws + ((int64_t)hq * kappa * (int64_t)Br + lo) * args.n + col;
#pragma unroll
        for (int k = 0; k < R; ++k)
            *reinterpret_cast<float4 *>(dst + (int64_t)k * args.n) =
                make_float4(acc[k][0] * c, acc[k][1] * c, acc[k][2] * c, acc[k][3] * c);
    }
}

template <bool MULTI>
const void *pick_bp_regs(int R) {
    switch (R) {
        case 1: return (const void *)k_bp_regs<1, MULTI>;
        case 2: return (const void *)k_bp_regs<2, MULTI>;
        case 4: return (const void *)k_bp_regs<4, MULTI>;
        case 8: return (const void *)k_bp_regs<8, MULTI>;
        case 16: return (const void *)k_bp_regs<16, MULTI>;
    }
    return nullptr;
}

}  // namespace

// Plan: R = kappa*B_r / (16 G) for the fewest row groups G (up to 8) with R
// one of the built 1, 2, 4, 8, 16 and R dividing B_r (a wavefront's rows
// inside one reader's block).  Row slices Q per input block: the fewest that
// keep at least 90% of a whole number of device-wide waves of workgroups
// busy (one workgroup per CU), each slice a whole number of stages.
bool plan_bp_regs(const DevInfo &di, int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa,
                  int32_t s, BpRegsPlan *p) {
    if (M < 1 || m % M != 0 || d % M != 0 || n < 4 || n % 4 != 0) return false;
    if (kappa < 1 || kappa > kK || s < 1 || s > 32) return false;
    if (di.max_lds < kBpRegsLdsBytes || di.num_cu < 1) return false;
    const int64_t Br = d / M, Bc = m / M;
    if (s > Br || (s > 1 && (Br & (Br - 1)) != 0)) return false;
    if (Bc > ((int64_t)1 << 31) - kS) return false;     // rows of a slice in 32 bits
    const int64_t T = (int64_t)kappa * Br;
    int R = 0, G = 0;
    for (int g = 1; g <= 8; g *= 2) {
        if (T % (16 * g) != 0) break;
        const int64_t r = T / (16 * g);
        if ((r == 1 || r == 2 || r == 4 || r == 8 || r == 16) && Br % r == 0) {
            R = (int)r;
            G = g;
            break;
        }
    }
    if (R == 0) return false;
    const int64_t slices = (n + kBpRegsCols - 1) / kBpRegsCols;
    const int64_t per = (int64_t)M * slices * G;        // workgroups per row slice
    const int64_t qmax_rows = (Bc + kS - 1) / kS;
    int64_t Q = 1;
    for (int64_t c = 1; c <= 64 && c <= qmax_rows; ++c) {
        const int64_t wgs = per * c;
        const int64_t waves = (wgs + di.num_cu - 1) / di.num_cu;
        Q = c;
        if (wgs * 10 >= waves * di.num_cu * 9) break;
    }
    int64_t rps = (Bc + Q - 1) / Q;
    rps = (rps + kS - 1) / kS * kS;
    Q = (Bc + rps - 1) / rps;
    const int64_t units = (int64_t)M * Q * slices;
    const int64_t grid = (units + 7) / 8 * 8 * G;
    if (grid > ((int64_t)1 << 31) - 1) return false;
    p->rows_per_wave = R;
    p->groups = G;
    p->slices = (int32_t)slices;
    p->Q = (int32_t)Q;
    p->rows_per_slice = rps;
    p->grid = grid;
    p->ws_bytes = (size_t)Q * (size_t)kappa * (size_t)d * (size_t)n * 4;
    return true;
}

hipError_t launch_bp_regs(const BpRegsPlan &p, const BlockPermGenArgs &args,
                          const BlockPermTable &ginv, const BlockPermTable &fwd, float *Y,
                          int64_t ldy, int accumulate, hipStream_t s) {
    // the kernel's row ownership and indexing must match the plan the
    // workspace was sized for
    const bool multi = args.s > 1;
    const void *kern = multi ? pick_bp_regs<true>(p.rows_per_wave)
                             : pick_bp_regs<false>(p.rows_per_wave);
    if (kern == nullptr || args.ws == nullptr || args.kappa < 1 || args.kappa > kK ||
        args.s < 1 || args.s > 32 || (int64_t)kW * p.rows_per_wave * p.groups !=
                                         (int64_t)args.kappa * args.Br ||
        args.Br % p.rows_per_wave != 0 || args.groups != p.groups || args.slices != p.slices ||
        args.Q != p.Q || args.rows_per_slice != p.rows_per_slice ||
        args.rows_per_slice % kS != 0 || (int64_t)args.Q * args.rows_per_slice < args.Bc ||
        (int64_t)args.slices * kBpRegsCols < args.n || args.n % 4 != 0 || args.lda % 4 != 0 ||
        (uintptr_t)args.A % 16 != 0 || (uintptr_t)args.ws % 16 != 0 ||
        (multi && (args.Br & (args.Br - 1)) != 0))
        return hipErrorInvalidValue;
    BlockPermGenArgs a = args;
    BlockPermTable t = ginv;
    void *params[] = {&a, &t};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3(kW * 64), params, 0, s);
    if (e != hipSuccess) return e;
    return launch_bp_reduce(args, fwd, Y, ldy, accumulate, s);
}

}  // namespace sk
