// BlockPerm-SJLT apply kernel for gfx950 (FlashSketch page §4, §5, App. D).
//
// The shift wiring pi_j(g) = (sigma(g) + j*C) mod M with C = M/kappa makes
// N(g) = {rho + j*C : j < kappa} for rho = sigma(g) mod C, so the M x M block
// graph is C disjoint complete bipartite components of kappa output blocks
// and kappa input blocks.  One workgroup owns one component and one 32-column
// tile: it reads each input row of its kappa input blocks exactly once,
// hashes the row for each of the component's kappa output blocks on the fly
// (no stored S, §5.2), accumulates into a private kappa*B_r x 32 FP32 tile in
// LDS with LDS atomics (§5.1), and writes every output element once with a
// plain store: no global atomics.  (The page's own grid gives each output
// block its own thread block, which reads each input block kappa times; the
// component grid reads A once.)
//
// Wave layout: a wavefront covers two rows x 32 columns per load (two
// 128-byte segments); a batch is 64 rows, whose hashes lane k computes for
// row k and the other lanes fetch with ds_bpermute.  The LDS tile keeps the
// two half-waves in separate 32-word halves of a 64-word row, so the 64
// lanes of one LDS atomic always hit 64 different banks.
#include "sk_internal.hpp"
#include "sk_apply_common.hpp"
#include "sk_rng.hpp"

namespace sk {
namespace {

constexpr int kTile = 32;   // columns per workgroup
constexpr int kBatch = 64;  // rows per wavefront batch

template <int KAPPA>
__global__ __launch_bounds__(1024) void k_blockperm(const BlockPermArgs args) {
    extern __shared__ float acc[];           // (KAPPA*B_r) x 64 floats
    __shared__ uint32_t keys[KAPPA * KAPPA];  // K(g_l, h_j) at [l*KAPPA + j]
    __shared__ int32_t gout[KAPPA];
    constexpr int NPW = (KAPPA + 1) / 2;     // packed 16-bit entries per lane
    const int32_t Br = args.Br;
    const int32_t C = args.C;
    const int64_t Bc = args.Bc;
    const int rho = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int32_t col = blockIdx.x * kTile + (lane & 31);
    const bool active = col < args.n;
    const int nthr = blockDim.x;
    const int nw = nthr >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int trows = KAPPA * Br;

    for (int k = threadIdx.x; k < trows * 64; k += nthr) acc[k] = 0.f;
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
            // uniform row base per pair of rows + one 32-bit lane offset: the
            // loads take the scalar-base form and need no 64-bit addresses
            float a[kBatch / 2];
            const uint32_t off = (uint32_t)(half * args.lda + col);
#pragma unroll
            for (int q = 0; q < kBatch / 2; ++q) {
                const float *pq = Ablk + (b + 2 * q) * args.lda;
                const int64_t r = b + 2 * q + half;
                a[q] = (active && r < Bc) ? pq[off] : 0.f;
            }
            // lane k hashes row b + k for every output block of the component
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
                const int src = (2 * q + half) << 2;
                uint32_t ev[NPW];
#pragma unroll
                for (int w = 0; w < NPW; ++w)
                    ev[w] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)packed[w]);
                const int64_t r = b + 2 * q + half;
                if (active && r < Bc) {
                    const float x = a[q] * scale;
#pragma unroll
                    for (int l = 0; l < KAPPA; ++l) {
                        const uint32_t e = (ev[l / 2] >> (16 * (l & 1))) & 0xFFFFu;
                        atomic_add_lds_f32(acc + (int)(e & 0x7FFFu) * 64 + lane, (e >> 15) ? -x : x);
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < trows * kTile; k += nthr) {
        const int tr = k / kTile;
        const int cc = k - tr * kTile;
        const int32_t c = blockIdx.x * kTile + cc;
        if (c < args.n) {
            const float s = acc[tr * 64 + cc] + acc[tr * 64 + 32 + cc];
            const int l = tr / Br;
            const int64_t orow = (int64_t)gout[l] * Br + (tr - l * Br);
            float *p = args.Y + orow * args.ldy + c;
            *p = args.accumulate ? *p + s : s;
        }
    }
}

}  // namespace

int blockperm_max_rows(const DevInfo &di) { return di.max_lds / (64 * (int)sizeof(float)) - 1; }

hipError_t launch_blockperm(const BlockPermArgs &args, int32_t kappa, hipStream_t s) {
    const size_t lds = (size_t)kappa * args.Br * 64 * sizeof(float);
    const dim3 grid((unsigned)((args.n + kTile - 1) / kTile), (unsigned)args.C);
    const dim3 block(1024);
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
