// General BlockPerm-SJLT apply for gfx950: any kappa (<= 32), s unique rows
// per block pair (s <= 32), the shift or the affine full-cycle wiring, and
// input blocks split into row slices (FlashSketch page §4, §5, App. B.1,
// App. D).
//
// The shift-wiring kernel (blockperm.hip) relies on the shift family falling
// apart into disjoint K_{kappa,kappa} components.  The affine family
// pi_l = f^l does not, so here a workgroup owns one input block h (and one
// row slice of it, the page's split-B_c) and one 32-column tile: it reads
// its rows once, hashes each for the kappa output blocks that read h
// (the l-th reader of h is the output block whose l-th neighbour is h), and
// accumulates kappa partial output tiles in wavefront-private LDS tiles
// (plain read-add-write, no atomics, as in blockperm.hip).  The partial
// tiles go to a workspace once; a second kernel writes each output element
// once as the sum of its kappa x slices partials in a fixed order
// (neighbour j ascending, then slice): a deterministic two-pass reduction in
// place of the page's split-B_c global atomics.
//
// Hash (s unique rows, App. D): v = fmix32(K(g,h) ^ r) for row r of block
// h; beta = mulhi(v, B_r); for s > 1, w = fmix32(v + 0x9E3779B9) and
// alpha = 2 mulhi(w, B_r/2) + 1; row j is (beta + j alpha) mod B_r (B_r a
// power of two when s > 1) with sign bit j of v.  s = 1 is blockperm.hip's
// rule.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"
#include "sk_rng.hpp"
#include "sk_blockperm.hpp"

namespace sk {
namespace {

constexpr int kTileG = 32;          // columns per workgroup
constexpr int kBatchG = 64;         // rows per wavefront batch
constexpr int kMaxWavesG = 8;

__global__ __launch_bounds__(kMaxWavesG * 64) void k_bp_general(const BlockPermGenArgs args,
                                                                 const BlockPermTable ginv) {
    extern __shared__ float acc[];                  // nw x (kappa*B_r) x 64 floats
    __shared__ uint32_t keys[kBlockPermGenMaxKappa];
    const int32_t Br = args.Br;
    const int kappa = args.kappa;
    const int s = args.s;
    const uint32_t h = blockIdx.y / (uint32_t)args.Q;
    const int32_t slice = (int32_t)(blockIdx.y % (uint32_t)args.Q);
    const int64_t rb = (int64_t)slice * args.rows_per_slice;     // first row of the slice
    const int64_t re = rb + args.rows_per_slice < args.Bc ? rb + args.rows_per_slice : args.Bc;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int32_t col = blockIdx.x * kTileG + (lane & 31);
    const bool active = col < args.n;
    const int32_t col_c = active ? col : args.n - 1;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int trows = kappa * Br;
    float *tile = acc + (int64_t)wave * trows * 64 + lane;

    for (int k = threadIdx.x; k < nw * trows * 64; k += nthr) acc[k] = 0.f;
    if ((int)threadIdx.x < kappa)
        keys[threadIdx.x] = blockperm_key(args.seed, bp_reader(args, ginv, h, threadIdx.x), h);
    __syncthreads();

    const float scale = args.scale;
    const uint32_t brmask = (uint32_t)Br - 1;       // used only when s > 1 (B_r a power of two)
    const float *Ablk = args.A + (int64_t)h * args.Bc * args.lda;
    for (int64_t b = rb + (int64_t)wave * kBatchG; b < re; b += (int64_t)nw * kBatchG) {
        // rows clamped into the slice and columns into the matrix: every
        // load is in bounds; values past the slice or the row are zeroed
        float a[kBatchG / 2];
#pragma unroll
        for (int q = 0; q < kBatchG / 2; ++q) {
            const int64_t r = b + 2 * q + half;
            const int64_t rc = r < re ? r : re - 1;
            a[q] = Ablk[rc * args.lda + col_c];
        }
        for (int l = 0; l < kappa; ++l) {
            const uint32_t key = __builtin_amdgcn_readfirstlane(keys[l]);
            // lane k hashes row b + k of block h for reader l
            const uint32_t v = fmix32(key ^ (uint32_t)(b + lane));
            const uint32_t alpha =
                s > 1 ? 2u * mulhi32(fmix32(v + 0x9E3779B9u), (uint32_t)Br >> 1) + 1u : 0u;
            float *tl = tile + (int64_t)l * Br * 64;
#pragma unroll
            for (int q = 0; q < kBatchG / 2; ++q) {
                const uint32_t v0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 2 * q);
                const uint32_t v1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 2 * q + 1);
                const uint32_t vr = half ? v1 : v0;
                const int64_t r = b + 2 * q + half;
                const float x = (active && r < re) ? a[q] * scale : 0.f;
                const uint32_t beta = mulhi32(vr, (uint32_t)Br);
                if (s == 1) {
                    float *p = tl + (int)beta * 64;
                    *p += (vr & 1u) ? -x : x;
                } else {
                    const uint32_t a0 = (uint32_t)__builtin_amdgcn_readlane((int)alpha, 2 * q);
                    const uint32_t a1 = (uint32_t)__builtin_amdgcn_readlane((int)alpha, 2 * q + 1);
                    const uint32_t al = half ? a1 : a0;
                    // the s rows of this (row, reader) are distinct
                    for (int j = 0; j < s; ++j) {
                        const uint32_t row = (beta + (uint32_t)j * al) & brmask;
                        float *p = tl + (int)row * 64;
                        *p += ((vr >> j) & 1u) ? -x : x;
                    }
                }
            }
        }
    }
    __syncthreads();
    // partial tiles of (block h, slice): ws[((h*Q + slice)*kappa + l)*B_r + row][col]
    float *ws = args.ws + ((int64_t)h * args.Q + slice) * (int64_t)trows * args.n;
    for (int k = threadIdx.x; k < trows * kTileG; k += nthr) {
        const int tr = k / kTileG;
        const int cc = k - tr * kTileG;
        const int32_t c = blockIdx.x * kTileG + cc;
        if (c < args.n) {
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) {
                const float *t = acc + ((int64_t)w * trows + tr) * 64;
                sum += t[cc] + t[32 + cc];
            }
            ws[(int64_t)tr * args.n + c] = sum;
        }
    }
}

// Y[g*B_r + row, c] (=|+=) sum over neighbours j of g (h_j, reached as h_j's
// j-th reader) and slices q of the partials, in that order.
__global__ __launch_bounds__(256) void k_bp_reduce(const BlockPermGenArgs args,
                                                   const BlockPermTable fwd, float *Y, int64_t ldy,
                                                   int32_t accumulate) {
    const int64_t total = (int64_t)args.M * args.Br * args.n;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * 256) {
        const int64_t orow = k / args.n;
        const int32_t c = (int32_t)(k - orow * args.n);
        const uint32_t g = (uint32_t)(orow / args.Br);
        const int32_t row = (int32_t)(orow - (int64_t)g * args.Br);
        float sum = 0.f;
        uint32_t x = g;
        for (int j = 0; j < args.kappa; ++j) {
            uint32_t hj;
            if (args.wiring == 0) {
                hj = (uint32_t)(((int64_t)fwd.tab[g] + (int64_t)j * args.C) % args.M);
            } else {
                x = (uint32_t)(((uint64_t)args.a * x + args.b) % (uint64_t)args.M);
                hj = x;
            }
            const float *src = args.ws +
                               (((int64_t)hj * args.Q * args.kappa + j) * args.Br + row) * args.n + c;
            const int64_t qstride = (int64_t)args.kappa * args.Br * args.n;
            for (int q = 0; q < args.Q; ++q) sum += src[q * qstride];
        }
        float *p = Y + orow * ldy + c;
        *p = accumulate ? *p + sum : sum;
    }
}

}  // namespace

int blockperm_general_max_rows(const DevInfo &di) {
    return (di.max_lds - 1024) / (64 * (int)sizeof(float));
}

hipError_t launch_blockperm_general(const BlockPermGenArgs &args, const BlockPermTable &ginv,
                                    const BlockPermTable &fwd, float *Y, int64_t ldy,
                                    int accumulate, hipStream_t s) {
    DevInfo di;
    hipError_t e0 = dev_info(&di);
    if (e0 != hipSuccess) return e0;
    const int trows = args.kappa * args.Br;
    if (args.kappa < 1 || args.kappa > kBlockPermGenMaxKappa || args.s < 1 || args.s > 32 ||
        trows > blockperm_general_max_rows(di) || args.Q < 1 || args.ws == nullptr)
        return hipErrorInvalidValue;
    const size_t wave_bytes = (size_t)trows * 64 * sizeof(float);
    int nw = (int)((size_t)(di.max_lds - 1024) / wave_bytes);
    if (nw > kMaxWavesG) nw = kMaxWavesG;
    if (nw < 1) return hipErrorInvalidValue;
    const size_t lds = wave_bytes * nw;
    const dim3 grid((unsigned)((args.n + kTileG - 1) / kTileG), (unsigned)(args.M * args.Q));
    auto kern = k_bp_general;
    hipError_t e = set_lds_limit((const void *)kern, lds);
    if (e != hipSuccess) return e;
    kern<<<grid, dim3(nw * 64), lds, s>>>(args, ginv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bp_reduce(args, fwd, Y, ldy, accumulate, s);
}

hipError_t launch_bp_reduce(const BlockPermGenArgs &args, const BlockPermTable &fwd, float *Y,
                            int64_t ldy, int accumulate, hipStream_t s) {
    const int64_t total = (int64_t)args.M * args.Br * args.n;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65535) blocks = 65535;
    k_bp_reduce<<<dim3((unsigned)blocks), 256, 0, s>>>(args, fwd, Y, ldy, accumulate);
    return hipGetLastError();
}

}  // namespace sk
