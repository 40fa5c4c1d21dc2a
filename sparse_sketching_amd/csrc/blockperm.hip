// BlockPerm-SJLT apply kernel for gfx950 (FlashSketch page §4, §5, App. D).
//
// The shift wiring pi_j(g) = (sigma(g) + j*C) mod M with C = M/kappa makes
// N(g) = {rho + j*C : j < kappa} for rho = sigma(g) mod C, so the M x M block
// graph is C disjoint complete bipartite components of kappa output blocks
// and kappa input blocks.  One workgroup owns one component and one 32-column
// tile: it reads each input row of its kappa input blocks exactly once,
// hashes the row for each of the component's kappa output blocks on the fly
// (no stored S, §5.2), accumulates in LDS (§5.1), and writes every output
// element once with a plain store: no global atomics.  (The page's own grid
// gives each output block its own thread block, which reads each input block
// kappa times; the component grid reads A once.)
//
// LDS: gfx950 performs floating-point LDS atomics one lane at a time, so each
// wavefront owns a private kappa*B_r x 64 FP32 tile and updates it with plain
// read-add-write; the wave tiles are summed once at the end.  A wavefront
// covers two rows x 32 columns per load (two 128-byte segments); the two
// half-waves keep separate 32-word halves of each 64-word tile row, so the
// 64 lanes of one update always touch 64 different words (and banks).
// Hashes: lane k hashes row k of a 64-row batch for every output block of the
// component; the half-waves pick up the packed (row, sign) entries of their
// rows with v_readlane, leaving the LDS pipe to the tile updates.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"
#include "sk_rng.hpp"

namespace sk {
namespace {

constexpr int kTile = 32;   // columns per workgroup
constexpr int kBatch = 64;  // rows per wavefront batch
constexpr int kMaxWaves = 8;

template <int KAPPA>
__global__ __launch_bounds__(kMaxWaves * 64) void k_blockperm(const BlockPermArgs args) {
    extern __shared__ float acc[];            // nw x (KAPPA*B_r) x 64 floats
    __shared__ uint32_t keys[KAPPA * KAPPA];  // K(g_l, h_j) at [l*KAPPA + j]
    __shared__ int32_t gout[KAPPA];
    constexpr int NPW = (KAPPA + 1) / 2;      // packed 16-bit entries per lane
    const int32_t Br = args.Br;
    const int32_t C = args.C;
    const int64_t Bc = args.Bc;
    const int rho = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int32_t col = blockIdx.x * kTile + (lane & 31);
    const bool active = col < args.n;
    const int32_t col_c = active ? col : args.n - 1;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int trows = KAPPA * Br;
    float *tile = acc + (int64_t)wave * trows * 64 + lane;

    for (int k = threadIdx.x; k < nw * trows * 64; k += nthr) acc[k] = 0.f;
    if (threadIdx.x < KAPPA * KAPPA) {
        const int l = threadIdx.x / KAPPA, j = threadIdx.x % KAPPA;
        keys[threadIdx.x] = blockperm_key(args.seed, args.ginv[rho + l * C], (uint32_t)(rho + j * C));
    }
    if (threadIdx.x < KAPPA) gout[threadIdx.x] = args.ginv[rho + threadIdx.x * C];
    __syncthreads();

    const float scale = args.scale;
    for (int j = 0; j < KAPPA; ++j) {
        const float *Ablk = args.A + (int64_t)(rho + j * C) * Bc * args.lda;
        uint32_t kj[KAPPA];
#pragma unroll
        for (int l = 0; l < KAPPA; ++l) kj[l] = __builtin_amdgcn_readfirstlane(keys[l * KAPPA + j]);
        for (int64_t b = (int64_t)wave * kBatch; b < Bc; b += (int64_t)nw * kBatch) {
            // rows clamped into the block and columns into the matrix, so
            // every load is in bounds and the loop is branch-free; values of
            // rows past the block or columns past n are zeroed before use
            float a[kBatch / 2];
#pragma unroll
            for (int q = 0; q < kBatch / 2; ++q) {
                const int64_t r = b + 2 * q + half;
                const int64_t rc = r < Bc ? r : Bc - 1;
                a[q] = Ablk[rc * args.lda + col_c];
            }
            // lane k hashes row b + k for every output block of the component:
            // entry = tile row (l*B_r + bucket) | sign << 15
            const uint32_t rr = (uint32_t)(b + lane);
            uint32_t packed[NPW];
#pragma unroll
            for (int w = 0; w < NPW; ++w) packed[w] = 0u;
#pragma unroll
            for (int l = 0; l < KAPPA; ++l) {
                const uint32_t v = fmix32(kj[l] ^ rr);
                const uint32_t e = ((uint32_t)(l * Br) + mulhi32(v, (uint32_t)Br)) | ((v & 1u) << 15);
                packed[l / 2] |= e << (16 * (l & 1));
            }
#pragma unroll
            for (int q = 0; q < kBatch / 2; ++q) {
                uint32_t ev[NPW];
#pragma unroll
                for (int w = 0; w < NPW; ++w) {
                    const uint32_t e0 = (uint32_t)__builtin_amdgcn_readlane((int)packed[w], 2 * q);
                    const uint32_t e1 = (uint32_t)__builtin_amdgcn_readlane((int)packed[w], 2 * q + 1);
                    ev[w] = half ? e1 : e0;
                }
                const int64_t r = b + 2 * q + half;
                const float x = (active && r < Bc) ? a[q] * scale : 0.f;
                // the kappa updates of one row hit kappa different output
                // blocks, so their tile rows differ: all reads, then all writes
                float *p[KAPPA];
                float t[KAPPA];
#pragma unroll
                for (int l = 0; l < KAPPA; ++l) {
                    const uint32_t e = (ev[l / 2] >> (16 * (l & 1))) & 0xFFFFu;
                    p[l] = tile + (int)(e & 0x7FFFu) * 64;
                    t[l] = *p[l] + ((e >> 15) ? -x : x);
                }
#pragma unroll
                for (int l = 0; l < KAPPA; ++l) *p[l] = t[l];
            }
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < trows * kTile; k += nthr) {
        const int tr = k / kTile;
        const int cc = k - tr * kTile;
        const int32_t c = blockIdx.x * kTile + cc;
        if (c < args.n) {
            float s = 0.f;
            for (int w = 0; w < nw; ++w) {
                const float *t = acc + ((int64_t)w * trows + tr) * 64;
                s += t[cc] + t[32 + cc];
            }
            const int l = tr / Br;
            const int64_t orow = (int64_t)gout[l] * Br + (tr - l * Br);
            float *p = args.Y + orow * args.ldy + c;
            *p = args.accumulate ? *p + s : s;
        }
    }
}

}  // namespace

// LDS the kernel's static arrays (keys, gout) may take, kept out of the tiles.
constexpr int kStaticLds = 1024;

// One wave tile must fit: kappa*B_r rows of 64 floats.
int blockperm_max_rows(const DevInfo &di) {
    return (di.max_lds - kStaticLds) / (64 * (int)sizeof(float));
}

hipError_t launch_blockperm(const BlockPermArgs &args, int32_t kappa, hipStream_t s) {
    const size_t wave_bytes = (size_t)kappa * args.Br * 64 * sizeof(float);
    DevInfo di;
    hipError_t e0 = dev_info(&di);
    if (e0 != hipSuccess) return e0;
    int nw = (int)((size_t)(di.max_lds - kStaticLds) / wave_bytes);
    if (nw > kMaxWaves) nw = kMaxWaves;
    if (nw < 1) return hipErrorInvalidValue;
    const size_t lds = wave_bytes * nw;
    const dim3 grid((unsigned)((args.n + kTile - 1) / kTile), (unsigned)args.C);
    const dim3 block(nw * 64);
#define SK_LAUNCH(K)                                                                          \
    do {                                                                                      \
        auto kern = k_blockperm<K>;                                                           \
        hipError_t e = set_lds_limit((const void *)kern, lds);                                \
        if (e != hipSuccess) return e;                                                        \
        kern<<<grid, block, lds, s>>>(args);                                                  \
    } while (0)
    switch (kappa) {
        case 1: SK_LAUNCH(1); break;
        case 2: SK_LAUNCH(2); break;
        case 4: SK_LAUNCH(4); break;
        case 8: SK_LAUNCH(8); break;
        default: return hipErrorInvalidValue;
    }
#undef SK_LAUNCH
    return hipGetLastError();
}

}  // namespace sk
