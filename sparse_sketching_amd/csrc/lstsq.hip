// Least squares on a small sketch: x = argmin ||SA x - Sb||_2 by an FP32
// Householder QR of SA, the projection Q^T Sb and a triangular solve (the
// reduced solve of the FP16 sketching page §V-A, §V-D: "FP32 QR,
// projection, and solve" on the d x n sketch; FlashSketch page App. F.1.4).
//
// How (MI355X-specific): the problem is a few hundred KiB, so it is bound by
// latency, not by bandwidth or flops; a vendor QR built from thousands of
// small launches spends its time launching.  Here two launches per panel:
//  * [SA | Sb] is copied into a column-major workspace (column j contiguous,
//    so every column access below is coalesced), Sb as column n, each column
//    scaled by a power of two that brings its largest magnitude into
//    [1/2, 1).  Householder QR commutes exactly with such scalings (every
//    rounding is scale-free away from overflow and underflow), so the
//    solution is unchanged bit for bit, but no norm or dot product can
//    overflow and no column of tiny entries loses its norm to underflow; x
//    is scaled back at the end.
//  * Panels of PB columns (32, 16 or 8 by d; the last columns in
//    power-of-two panels, so PB is a compile-time constant everywhere) are
//    factored by one workgroup with the panel held in registers: each lane
//    holds one or two columns on an interleaved set of rows.  Per column c,
//    one barrier: every lane forms its columns' partial dot products with
//    column c below row c, the partials are summed across the wavefront by
//    DPP and the gfx950 lane swaps and across wavefronts in LDS, and after
//    the barrier every lane has the norm of column c, its reflector
//    (LAPACK's larfg rule: beta = -sign(alpha) ||(alpha, x)||, tau = (beta -
//    alpha) / beta, v = x / (alpha - beta); tau = 0 when x = 0) and its
//    columns' dot products with it, and updates its registers.  Column c + 1
//    reaches the lanes of a row group by ds_bpermute while the barrier is
//    pending.  For the columns left of c the same dot products are the
//    entries of G = V^T V.
//  * The trailing columns, the right-hand side among them, are updated as
//    a <- (I - V T V^T)^T a = a - V (T^T (V^T a)) (H_1 ... H_PB = I - V T
//    V^T, T upper triangular, the forward column-wise accumulation) by as
//    many workgroups as they need (one column per wavefront), each with its
//    own LDS copy of V.  The PB dot products of a column are summed across
//    the wavefront by a transposing butterfly (each exchange halves the
//    values a lane holds), and u = T^T w is a forward substitution in G, so
//    T itself is never formed.
//  * R y = (Q^T Sb)[0:n] is solved by one workgroup in blocks of 32 rows
//    from the bottom: one wavefront solves a block's triangle in registers
//    with lane shuffles while the block's columns above it are in flight,
//    then every thread subtracts them from its rows of the right-hand side.
#include <cfloat>
#include <type_traits>

#include "sk_internal.hpp"

namespace sk {
namespace {

constexpr int kQrMaxNb = 32;
// panel widths by height: rows x (PB + 1) <= kQrPanelFloats (PB = 32 up to
// 775 rows, 16 up to 1505, 8 up to kQrMaxRows)
constexpr int kQrPanelFloats = 25600;
// the trailing update's V copy: rows x TrailShape<PB>::LS floats
constexpr int kQrTrailFloats = 30208;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// v + the value of lane l ^ 32 (l ^ 16): the gfx950 lane swaps exchange the
// two halves (the odd and even 16-lane rows) of a pair of registers; with
// the same register twice, the two results are v on the lane and on its
// partner, and their sum is the same on both lanes.
__device__ __forceinline__ float swap_sum32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float swap_sum16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over the lanes of a wavefront that agree in their lowest log2(LPG)
// bits (the lanes holding the same panel column); correct on lanes 0 ..
// LPG-1 at least.  Steps: xor 1, xor 2 (quad permutes), rotate by 4 and 8
// within the 16-lane row (after the earlier steps, or alone, the rotations
// sum the row's lanes of one residue class), xor 16, xor 32 (lane swaps).
template <int LPG>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPG <= 1) v += dpp_mov<0xB1>(v);          // quad_perm [1,0,3,2]
    if constexpr (LPG <= 2) v += dpp_mov<0x4E>(v);          // quad_perm [2,3,0,1]
    if constexpr (LPG <= 4) v += dpp_mov<0x124>(v);         // row_ror:4
    if constexpr (LPG <= 8) v += dpp_mov<0x128>(v);         // row_ror:8
    if constexpr (LPG <= 16) v = swap_sum16(v);
    return swap_sum32(v);
}

// Transposing sum over the 64 lanes of v[0 .. PB) (PB a power of two, at
// most 32; v is destroyed): at each exchange a lane keeps half of its values
// and sends the other half to its partner, so that PB values cost about
// 2 PB operations instead of PB full sums.  Lane l ends with the sum of
// v[l >> (6 - log2 PB)].  Partners: l ^ 32, l ^ 16 (lane swaps), l ^ 15
// (row mirror), l ^ 7 (half-row mirror), l ^ 3 (quad permute): each flips
// the bit being split and only bits not split yet, so partners hold the same
// indices; the bits left over are summed plainly.
template <int CTRL, int H>
__device__ __forceinline__ void split_dpp(float *v, bool upper) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float keep = upper ? v[i + H] : v[i];
        const float send = upper ? v[i] : v[i + H];
        v[i] = keep + dpp_mov<CTRL>(send);
    }
}

template <int PB>
__device__ __forceinline__ float transpose_sum(float *v) {
    const int lane = threadIdx.x & 63;
    if constexpr (PB >= 2) {
#pragma unroll
        for (int i = 0; i < PB / 2; ++i) {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                            __float_as_uint(v[i + PB / 2]), false,
                                                            false);
            v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    }
    if constexpr (PB >= 4) {
#pragma unroll
        for (int i = 0; i < PB / 4; ++i) {
            const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                            __float_as_uint(v[i + PB / 4]), false,
                                                            false);
            v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
    }
    if constexpr (PB >= 8) split_dpp<0x140, PB / 8>(v, lane & 8);     // row_mirror
    if constexpr (PB >= 16) split_dpp<0x141, PB / 16>(v, lane & 4);   // row_half_mirror
    if constexpr (PB >= 32) split_dpp<0x1B, PB / 32>(v, lane & 2);    // quad_perm [3,2,1,0]
    float r = v[0];
    r += dpp_mov<0xB1>(r);                                            // bit 0
    if constexpr (PB <= 16) r += dpp_mov<0x4E>(r);                    // bit 1
    if constexpr (PB <= 8) r += dpp_mov<0x141>(r);                    // bit 2
    if constexpr (PB <= 4) r += dpp_mov<0x140>(r);                    // bit 3
    if constexpr (PB <= 2) r = swap_sum16(r);                         // bit 4
    if constexpr (PB <= 1) r = swap_sum32(r);                         // bit 5
    return r;
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Workgroup barrier that orders LDS only: global loads issued before it stay
// in flight (__syncthreads also waits for them), so a load can be issued a
// phase ahead of its use.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float bperm(int byte_addr, float v) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(byte_addr, __float_as_int(v)));
}

struct QrArgs {
    const float *SA;            // d x n row-major, row stride ld
    const float *Sb;            // d
    float *x;                   // n
    float *W;                   // n + 1 columns of d floats
    float *G;                   // the current panel's V^T V, tau on the diagonal
    int *E;                     // n + 1 column exponents
    int64_t ld;
    int32_t d, n, nb;
};

// Workspace layout: W (n + 1 columns of d floats, column-major: [SA | Sb]
// scaled, then R, the reflectors and Q^T Sb), the panel's G (kQrMaxNb x
// kQrMaxNb floats: G[m][i] = v_m . v_i above the diagonal, tau_i on it),
// the n + 1 column exponents (int32).

// [SA | Sb] into column-major W, column j scaled by 2^-E[j] with E[j] the
// exponent of its largest magnitude (frexp convention: the largest
// magnitude becomes [1/2, 1); E = 0 for a zero or non-finite maximum).  One
// block of 1024 threads per 32 columns: each thread loads its column's rows
// rw, rw + 32, ... (all in flight at once), the maxima meet in LDS, and the
// scaled values leave through an LDS transpose (coalesced on both sides).
__global__ __launch_bounds__(1024) void k_qr_prep(const QrArgs args) {
    constexpr int RR = kQrMaxRows / 32;             // rows per thread at most
    __shared__ float tile[128][33];
    __shared__ float cmax[32][33];
    __shared__ int cexp[32];
    const int d = args.d, n = args.n;
    const int tid = threadIdx.x, cl = tid & 31, rw = tid >> 5;
    const int j0 = blockIdx.x * 32, j = j0 + cl;
    float t[RR];
#pragma unroll
    for (int u = 0; u < RR; ++u) {
        t[u] = 0.f;
        const int i = rw + 32 * u;
        if (32 * u < d && i < d)
            t[u] = j < n ? args.SA[(int64_t)i * args.ld + j] : j == n ? args.Sb[i] : 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < RR; ++u)
        if (32 * u < d) m = fmaxf(m, fabsf(t[u]));
    cmax[rw][cl] = m;
    __syncthreads();
    if (rw == 0) {
        float mm = cmax[0][cl];
#pragma unroll
        for (int q = 1; q < 32; ++q) mm = fmaxf(mm, cmax[q][cl]);
        int e = 0;
        if (mm > 0.f && mm <= FLT_MAX) (void)frexpf(mm, &e);
        cexp[cl] = e;
        if (j <= n) args.E[j] = e;
    }
    __syncthreads();
    const int e = cexp[cl];
#pragma unroll
    for (int ch = 0; ch < RR / 4; ++ch) {           // rows 128 ch .. 128 ch + 127
        if (128 * ch < d) {
#pragma unroll
            for (int v = 0; v < 4; ++v) tile[rw + 32 * v][cl] = ldexpf(t[4 * ch + v], -e);
            __syncthreads();
#pragma unroll
            for (int v = 0; v < 4; ++v) {           // column j0 + rw, row 128 ch + cl + 32 v
                const int i = 128 * ch + cl + 32 * v;
                if (j0 + rw <= n && i < d) args.W[(int64_t)(j0 + rw) * d + i] = tile[cl + 32 * v][rw];
            }
            __syncthreads();
        }
    }
}

// Register layout of a PB-column panel: NW wavefronts, CC columns per lane,
// LPG = PB / CC lanes per row group, NS = NW * 64 / LPG row groups (slices),
// slice s holding panel rows s, s + NS, s + 2 NS, ... (at most RMAX, a
// multiple of 8).
template <int PB, int NW> struct PanelShape;
template <> struct PanelShape<32, 4> { static constexpr int CC = 2, RMAX = 32; };   // <= 512 rows
template <> struct PanelShape<32, 8> { static constexpr int CC = 2, RMAX = 32; };   // <= 1024
template <> struct PanelShape<16, 8> { static constexpr int CC = 1, RMAX = 48; };   // <= 1536
template <> struct PanelShape<8, 8> { static constexpr int CC = 1, RMAX = 32; };    // <= 2048
template <> struct PanelShape<4, 4> { static constexpr int CC = 1, RMAX = 32; };
template <> struct PanelShape<2, 4> { static constexpr int CC = 1, RMAX = 16; };
template <> struct PanelShape<1, 4> { static constexpr int CC = 1, RMAX = 8; };

template <int PB, int NW>
constexpr int panel_slices() {
    return NW * 64 / (PB / PanelShape<PB, NW>::CC);
}

// f(k) for the row indices k < kcap (kcap a multiple of 8; whole 8-row
// chunks past it are skipped by a uniform branch)
template <int RMAX, typename F>
__device__ __forceinline__ void for_rows(int kcap, F &&f) {
#pragma unroll
    for (int kb = 0; kb < RMAX; kb += 8) {
        if (kb < kcap) {
#pragma unroll
            for (int k = kb; k < kb + 8; ++k) f(k);
        }
    }
}

// Factor panel columns p0 .. p0+PB-1 (one workgroup) in registers: R, beta
// on the diagonal and the reflectors to W, G (tau on its diagonal) to
// args.G.  Each lane also carries a copy of the next column on its rows:
// fetched from the column's lanes at the start of a step, it is in flight
// across the step's barrier and updated with the lane's own columns, so the
// next step starts on it without a cross-lane round trip.
template <int PB, int NW>
__global__ __launch_bounds__(NW * 64) void k_qr_panel(const QrArgs args, int p0) {
    constexpr int CC = PanelShape<PB, NW>::CC, RMAX = PanelShape<PB, NW>::RMAX;
    constexpr int NT = NW * 64, LPG = PB / CC, RG = 64 / LPG, NS = NW * RG;
    constexpr int KE = (PB + NS - 1) / NS;          // row indices that can hold rows < PB
    static_assert(NS == panel_slices<PB, NW>() && (NS & (NS - 1)) == 0, "slices");
    __shared__ __align__(16) float part[2][PB][NW]; // per column, per wavefront partial sums
    __shared__ float rowc[2][PB];                   // row c of every panel column
    __shared__ float G[kQrMaxNb * kQrMaxNb];        // G[m][i] = v_m . v_i, m < i; tau_i at [i][i]
    const int d = args.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cl = lane % LPG, rg = lane / LPG, s = wave * RG + rg;
    const int dp = d - p0;                          // panel rows p0 .. d-1
    const int kcap = ((dp + NS - 1) / NS + 7) & ~7;
    float *const P0 = args.W + (int64_t)p0 * d + p0;    // panel row 0, column 0
    float a[RMAX][CC];                              // rows s + NS k, columns cl * CC + j
#pragma unroll
    for (int k = 0; k < RMAX; ++k)
#pragma unroll
        for (int j = 0; j < CC; ++j) a[k][j] = 0.f;
    for_rows<RMAX>(kcap, [&](int k) {               // every load in flight at once
        const int r = s + NS * k;
#pragma unroll
        for (int j = 0; j < CC; ++j)
            if (r < dp) a[k][j] = P0[(int64_t)(cl * CC + j) * d + r];
    });
    float msc[CC];                                  // 1 / (alpha - beta) of the lane's columns
#pragma unroll
    for (int j = 0; j < CC; ++j) msc[j] = 1.f;
    const int gbase = (lane - cl) * 4;              // ds_bpermute address of the row group
    float xa[RMAX], xb[RMAX];                       // column c and column c + 1 on the lane's rows
    for_rows<RMAX>(kcap, [&](int k) { xa[k] = bperm(gbase, a[k][0]); });

    auto step = [&](const int c, auto jjc, float (&x)[RMAX], float (&z)[RMAX]) {
        constexpr int jj = decltype(jjc)::value;    // column c's slot in its lanes
        constexpr int nj = (jj + 1) % CC;           // column c + 1's
        const int buf = c & 1;
        const bool more = c + 1 < PB;
#pragma unroll
        for (int k = 0; k < KE; ++k)
            if (s + NS * k <= c) x[k] = 0.f;        // column c below row c
        float P[CC];
#pragma unroll
        for (int j = 0; j < CC; ++j) P[j] = 0.f;
        for_rows<RMAX>(kcap, [&](int k) {
#pragma unroll
            for (int j = 0; j < CC; ++j) P[j] = fmaf(x[k], a[k][j], P[j]);
        });
#pragma unroll
        for (int j = 0; j < CC; ++j) P[j] = group_sum<LPG>(P[j]);
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < CC; ++j) part[buf][cl * CC + j][wave] = P[j];
        }
        if (s == (c & (NS - 1))) {                  // the lanes holding row c
#pragma unroll
            for (int k = 0; k < KE; ++k)
                if (k == c / NS) {
#pragma unroll
                    for (int j = 0; j < CC; ++j) rowc[buf][cl * CC + j] = a[k][j];
                }
        }
        lds_barrier();
        // (part and rowc alternate between two buffers: a wavefront writes
        // step c + 1's only after every wavefront has passed this barrier,
        // that is, has finished reading step c - 1's)
        const int cn = more ? c + 1 : c;
        float pc[NW], pn[NW], pj[CC][NW], rj[CC];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            pc[w] = part[buf][c][w];
            pn[w] = part[buf][cn][w];
        }
        const float alpha = rowc[buf][c], rn = rowc[buf][cn];
#pragma unroll
        for (int j = 0; j < CC; ++j) {
#pragma unroll
            for (int w = 0; w < NW; ++w) pj[j][w] = part[buf][cl * CC + j][w];
            rj[j] = rowc[buf][cl * CC + j];
        }
        // column c + 1 as H_{c-1} left it, issued after this step's LDS reads
        // (so that neither they nor the barrier wait for it) and in flight
        // while the reflector is formed
        if (more) {
            const int src = gbase + ((c + 1) / CC) * 4;
            for_rows<RMAX>(kcap, [&](int k) { z[k] = bperm(src, a[k][nj]); });
        }
        float xn2 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) xn2 += pc[w];
        const float bt = -copysignf(sqrtf(alpha * alpha + xn2), alpha);
        const bool refl = xn2 != 0.f;               // x = 0: H_c = I
        const float beta = refl ? bt : alpha;
        const float tau = refl ? (bt - alpha) / bt : 0.f;
        const float scale = refl ? 1.f / (alpha - bt) : 1.f;
        // v_c . a_col with a_col's tail unscaled: a_col[c] + scale * sum
        auto vdot = [&](const float (&pw)[NW], float rv) {
            float q = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) q += pw[w];
            return rv + scale * q;
        };
        float wv[CC];
#pragma unroll
        for (int j = 0; j < CC; ++j) {
            const int col = cl * CC + j;
            const float u = vdot(pj[j], rj[j]);
            wv[j] = col > c ? tau * u : 0.f;
            // left of c the same sum is v_col . v_c / scale_col
            if (col < c && s == 0) G[col * kQrMaxNb + c] = msc[j] * u;
        }
        if (cl * CC + jj == c) msc[jj] = scale;
        if (tid == 0) G[c * kQrMaxNb + c] = tau;
        // the copy of column c + 1 takes the update its lanes take (same sum)
        const float wz = more ? tau * vdot(pn, rn) : 0.f;
        // a -= w v_c with v_c = scale * x below row c (x is zero on and
        // above row c) and 1 at row c
        float ws[CC];
#pragma unroll
        for (int j = 0; j < CC; ++j) ws[j] = wv[j] * scale;
        const float wzs = wz * scale;
        for_rows<RMAX>(kcap, [&](int k) {
#pragma unroll
            for (int j = 0; j < CC; ++j) a[k][j] = fmaf(-ws[j], x[k], a[k][j]);
            z[k] = fmaf(-wzs, x[k], z[k]);
        });
        if (s == (c & (NS - 1))) {                  // row c; beta on the diagonal
#pragma unroll
            for (int k = 0; k < KE; ++k)
                if (k == c / NS) {
#pragma unroll
                    for (int j = 0; j < CC; ++j) a[k][j] -= wv[j];
                    z[k] -= wz;
                    if (cl * CC + jj == c) a[k][jj] = beta;
                }
        }
    };
#pragma unroll 1
    for (int c0 = 0; c0 < PB; c0 += 2) {            // x and z trade places every step
        step(c0, std::integral_constant<int, 0>{}, xa, xb);
        if (c0 + 1 < PB) step(c0 + 1, std::integral_constant<int, 1 % CC>{}, xb, xa);
    }

    // R above the diagonal, beta on it, the reflector tails scaled below it
    for_rows<RMAX>(kcap, [&](int k) {
        const int r = s + NS * k;
        if (r < dp) {
#pragma unroll
            for (int j = 0; j < CC; ++j) {
                const int col = cl * CC + j;
                P0[(int64_t)col * d + r] = r > col ? a[k][j] * msc[j] : a[k][j];
            }
        }
    });
    lds_barrier();                                  // the last step's G entries
    for (int i = tid; i < PB * kQrMaxNb; i += NT) args.G[i] = G[i];
}

// Trailing update's V copy: row stride LS (a multiple of 4 with LS / 4 odd,
// so the float4 reads of 16 consecutive rows hit distinct banks), RT rows per
// lane at most.
template <int PB> struct TrailShape {
    static constexpr int LS = 4 * ((PB / 4) | 1);
    static constexpr int RT = PB == 32 ? 13 : PB == 16 ? 24 : 32;
};

// Trailing columns of panel p0 and the right-hand side (W's column n):
// a <- a - V u, u = T^T (V^T a) = T^T w, by forward substitution in G:
// u_i = tau_i (w_i - sum_{q<i} G[q][i] u_q) (T^-1 = diag(1/tau) +
// strictly-upper(G) for the forward recurrence; this form also holds for
// tau_i = 0).  Wavefront w of block b takes column p0 + PB + kTrailWaves b +
// w (one column per wavefront: the update is latency bound, and twice the
// blocks finish sooner than two columns per wavefront); V (unit lower
// trapezoid) from W.
constexpr int kTrailWaves = 8;                  // 512 threads: V staged in one round of loads
                                                // for up to 512 panel rows
template <int PB>
__global__ __launch_bounds__(kTrailWaves * 64) void k_qr_trail(const QrArgs args, int p0) {
    constexpr int LS = TrailShape<PB>::LS, RT = TrailShape<PB>::RT, NQ = (PB + 3) / 4;
    constexpr int SH = 6 - ilog2(PB);               // lane l holds dot product l >> SH
    __shared__ __align__(16) float V[kQrTrailFloats];
    const int d = args.d, n = args.n;
    float *const W = args.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dp = d - p0;
    const int k0 = p0 + PB + blockIdx.x * kTrailWaves + wave;
    const bool live = k0 <= n;
    float *const a0 = W + (int64_t)k0 * d + p0;
    // the wavefront's column and G's column (lane & (PB - 1)), in flight
    // while V is staged
    float x0[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int r = lane + 64 * i;
        x0[i] = live && r < dp ? a0[r] : 0.f;
    }
    const int ti = lane & (PB - 1);
    float gcol[PB], tq[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) {
        gcol[q] = q < ti ? args.G[q * kQrMaxNb + ti] : 0.f;
        tq[q] = args.G[q * (kQrMaxNb + 1)];
    }
    constexpr int CW = PB < 4 ? 4 : PB;             // columns written (zero padding read)
    for (int r0 = 0; r0 < dp; r0 += kTrailWaves * 64) {
        const int r = r0 + tid;
        float t[CW];
#pragma unroll
        for (int c = 0; c < CW; ++c)
            t[c] = c >= PB || r < c || r >= dp ? 0.f : r == c ? 1.f
                                                             : W[(int64_t)(p0 + c) * d + p0 + r];
        if (r < dp) {
#pragma unroll
            for (int c = 0; c < CW; ++c) V[r * LS + c] = t[c];
        }
    }
    lds_barrier();
    if (!live) return;                              // wave-uniform; no barrier follows
    float w0[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) w0[q] = 0.f;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        if (64 * i < dp) {
            const int r = lane + 64 * i, rr = r < dp ? r : 0;   // x = 0 past the panel
            const float4 *vr = reinterpret_cast<const float4 *>(V + rr * LS);
#pragma unroll
            for (int q4 = 0; q4 < NQ; ++q4) {
                const float4 v = vr[q4];
                const float ve[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (4 * q4 + e < PB) w0[4 * q4 + e] = fmaf(ve[e], x0[i], w0[4 * q4 + e]);
                }
            }
        }
    }
    // w_i onto lane i (and its copies), then the forward substitution
    float s0 = bperm((ti << SH) * 4, transpose_sum<PB>(w0));
    float su0[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) {
        su0[q] = tq[q] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s0), q));
        s0 = fmaf(-gcol[q], su0[q], s0);            // gcol[q] = 0 on lanes i <= q
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        if (64 * i < dp) {
            const int r = lane + 64 * i, rr = r < dp ? r : 0;
            const float4 *vr = reinterpret_cast<const float4 *>(V + rr * LS);
#pragma unroll
            for (int q4 = 0; q4 < NQ; ++q4) {
                const float4 v = vr[q4];
                const float ve[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (4 * q4 + e < PB) x0[i] = fmaf(-ve[e], su0[4 * q4 + e], x0[i]);
                }
            }
            if (r < dp) a0[r] = x0[i];
        }
    }
}

// R y = z, z = (Q^T Sb)[0:n], R(i, j) = W[j*d + i] for i <= j (one
// workgroup): 32-row blocks from the bottom.  A block's columns above it
// (and the next block's triangle) are loaded before its triangle is solved
// and stay in flight across the LDS-only barriers, so their latency
// overlaps the solve: one wave solves the triangle from registers (lane l
// holds row l) with lane shuffles, then every thread subtracts the block's
// columns from its rows of z.  x = y scaled back.
__global__ __launch_bounds__(1024) void k_qr_backsub(const QrArgs args) {
    __shared__ float zs[kQrMaxRows];
    __shared__ float xs[kQrMaxRows];
    __shared__ float Rb[32 * 33];                   // the block's triangle, row-major
    const int d = args.d, n = args.n;
    const float *const W = args.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bi = tid >> 5, bj = tid & 31;
    for (int i = tid; i < n; i += 1024) zs[i] = W[(int64_t)n * d + i];
    auto rload = [&](int b0, int bh) -> float {     // R(b0 + bi, b0 + bj), zero outside
        return b0 + bi < bh && b0 + bj < bh && bi <= bj ? W[(int64_t)(b0 + bj) * d + b0 + bi]
                                                          : 0.f;
    };
    const int top = (n + 31) / 32 * 32;
    float rnext = rload(top - 32, n);
    for (int b1 = top; b1 > 0; b1 -= 32) {
        const int b0 = b1 - 32, bh = b1 < n ? b1 : n;
        Rb[bi * 33 + bj] = rnext;
        float cv[2][32];                            // R(i, b0 + jj) for this thread's rows i < b0
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = tid + 1024 * t;
#pragma unroll
            for (int jj = 0; jj < 32; ++jj)
                cv[t][jj] = i < b0 && b0 + jj < bh ? W[(int64_t)(b0 + jj) * d + i] : 0.f;
        }
        if (b0 > 0) rnext = rload(b0 - 32, b0);
        lds_barrier();
        if (wave == 0) {
            const int l = lane & 31, nb = bh - b0;
            float rrow[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) rrow[j] = Rb[l * 33 + j];
            const float dg = Rb[l * 33 + l];
            float z = l < nb ? zs[b0 + l] : 0.f;
            float xl = 0.f;
#pragma unroll
            for (int j = 31; j >= 0; --j) {
                if (j < nb) {
                    const float zj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
                    const float rjj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dg), j));
                    const float xj = zj / rjj;
                    if (l == j) xl = xj;
                    z = fmaf(-xj, rrow[j], z);      // rows below j hold zero in column j
                }
            }
            if (lane < 32 && l < nb) xs[b0 + l] = xl;
        }
        lds_barrier();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = tid + 1024 * t;
            if (i < b0) {
                float zi = zs[i];
#pragma unroll
                for (int jj = 0; jj < 32; ++jj)
                    if (b0 + jj < bh) zi = fmaf(-cv[t][jj], xs[b0 + jj], zi);
                zs[i] = zi;
            }
        }
        lds_barrier();
    }
    const int en = args.E[n];
    for (int i = tid; i < n; i += 1024) args.x[i] = ldexpf(xs[i], en - args.E[i]);
}

template <int PB, int NW>
hipError_t qr_panel_step(const QrArgs &a, int p0, hipStream_t s) {
    const int dp = a.d - p0;
    // the register panel and the trailing update's LDS copy must hold the
    // panel's rows
    if ((dp + panel_slices<PB, NW>() - 1) / panel_slices<PB, NW>() > PanelShape<PB, NW>::RMAX ||
        (int64_t)dp * TrailShape<PB>::LS > kQrTrailFloats || (dp + 63) / 64 > TrailShape<PB>::RT)
        return hipErrorInvalidValue;
    k_qr_panel<PB, NW><<<dim3(1), dim3(NW * 64), 0, s>>>(a, p0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntrail = a.n + 1 - (p0 + PB);         // columns after the panel, rhs included
    const int blocks = (ntrail + kTrailWaves - 1) / kTrailWaves;
    k_qr_trail<PB><<<dim3(blocks), dim3(kTrailWaves * 64), 0, s>>>(a, p0);
    return hipGetLastError();
}

}  // namespace

// panel width by height: 32 columns up to 775 rows, 16 up to 1505, 8 above
int lstsq_panel_cols(int32_t d) {
    return (int64_t)d * 33 <= kQrPanelFloats ? 32 : (int64_t)d * 17 <= kQrPanelFloats ? 16 : 8;
}

size_t lstsq_workspace_floats(int32_t d, int32_t n) {
    return (size_t)(n + 1) * (size_t)d + (size_t)(kQrMaxNb * kQrMaxNb) + (size_t)(n + 1);
}

hipError_t launch_lstsq_qr(const float *SA, int32_t d, int32_t n, int64_t ld, const float *Sb,
                           float *x, float *W, hipStream_t s) {
    if (d < 1 || n < 1 || n > d || d > kQrMaxRows) return hipErrorInvalidValue;
    float *const G = W + (size_t)(n + 1) * (size_t)d;
    QrArgs a{SA, Sb, x, W, G, reinterpret_cast<int *>(G + kQrMaxNb * kQrMaxNb), ld, d, n,
             lstsq_panel_cols(d)};
    k_qr_prep<<<dim3((unsigned)((n + 1 + 31) / 32)), dim3(1024), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    // full panels of nb columns, then the rest in power-of-two panels
    for (int p0 = 0; p0 < n && e == hipSuccess;) {
        const int rem = n - p0;
        const int pb = rem >= a.nb ? a.nb : rem >= 16 ? 16 : rem >= 8 ? 8 : rem >= 4 ? 4
                                                                        : rem >= 2 ? 2 : 1;
        switch (pb) {
        case 32:
            e = d - p0 <= 512 ? qr_panel_step<32, 4>(a, p0, s) : qr_panel_step<32, 8>(a, p0, s);
            break;
        case 16: e = qr_panel_step<16, 8>(a, p0, s); break;
        case 8: e = qr_panel_step<8, 8>(a, p0, s); break;
        case 4: e = qr_panel_step<4, 4>(a, p0, s); break;
        case 2: e = qr_panel_step<2, 4>(a, p0, s); break;
        default: e = qr_panel_step<1, 4>(a, p0, s); break;
        }
        p0 += pb;
    }
    if (e != hipSuccess) return e;
    k_qr_backsub<<<dim3(1), dim3(1024), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sk
