// Least squares on a small sketch: x = argmin ||SA x - Sb||_2 by an FP32
// Householder QR of SA, the projection Q^T Sb and a triangular solve (the
// reduced solve of the FP16 sketching page §V-A, §V-D: "FP32 QR,
// projection, and solve" on the d x n sketch; FlashSketch page App. F.1.4).
//
// How (MI355X-specific): the problem is a few hundred KiB, so it is bound by
// latency, not by bandwidth or flops; a vendor QR built from many small
// launches spends its time launching.  Here one 1024-thread workgroup does
// the whole solve in one launch:
//  * [SA | Sb] is copied into a column-major workspace (column j contiguous,
//    so every column access below is coalesced), Sb as column n.
//  * Panels of PB columns (32, 16 or 8 by d, so the panel fits 100 KiB of
//    LDS; the last columns in power-of-two panels, so PB is a compile-time
//    constant everywhere) are factored in LDS with the reflector rule of
//    LAPACK's larfg (beta = -sign(alpha) ||(alpha, x)||, tau = (beta -
//    alpha) / beta, v = x / (alpha - beta); tau = 0 when x = 0), one column
//    after another.  The panel is row-major in LDS with an odd row stride
//    (PB + 1): a column is read without bank conflicts, a row by immediate
//    offsets from one address.
//  * Each panel's reflectors are combined as H_1 ... H_pb = I - V T V^T
//    (T upper triangular, the forward column-wise recurrence), and the
//    trailing columns, the right-hand side among them, are updated at once
//    as a <- a - V (T^T (V^T a)), one wavefront per column.
//  * R x = (Q^T Sb)[0:n] is solved by blocks of 32 rows from the bottom:
//    one wavefront solves the block's triangle with lane shuffles, then all
//    wavefronts subtract its columns from the remaining right-hand side.
#include "sk_internal.hpp"

namespace sk {
namespace {

constexpr int kQrThreads = 1024;
constexpr int kQrWaves = kQrThreads / 64;
constexpr int kQrMaxNb = 32;
// panel floats in LDS: rows x (PB + 1) <= kQrPanelFloats (PB = 32 up to 775
// rows, 16 up to 1505, 8 up to kQrMaxRows)
constexpr int kQrPanelFloats = 25600;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

struct QrArgs {
    const float *SA;            // d x n row-major, row stride ld
    const float *Sb;            // d
    float *x;                   // n
    float *W;                   // workspace: n + 1 columns of d floats
    int64_t ld;
    int32_t d, n, nb;
};

struct QrShared {
    float V[kQrPanelFloats];    // panel row r, column c at r * (PB + 1) + c
    float G[kQrMaxNb * kQrMaxNb];   // V^T V
    float T[kQrMaxNb * kQrMaxNb];   // row l at l * kQrMaxNb
    float tau[kQrMaxNb];
    float red[kQrWaves];
};

// One panel of PB columns starting at column p0: factor it, write R and the
// reflectors to W, and apply I - V T^T V^T to the trailing columns and the
// right-hand side (W's column n).
template <int PB>
__device__ __attribute__((noinline)) void qr_panel(QrShared &sh, float *W, int d, int n, int p0) {
    constexpr int LS = PB + 1;                      // LDS row stride
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dp = d - p0;                          // panel rows p0 .. d-1
    float *const V = sh.V;
    for (int idx = tid; idx < PB * dp; idx += kQrThreads) {
        const int c = idx / dp, r = idx - c * dp;
        V[r * LS + c] = W[(int64_t)(p0 + c) * d + p0 + r];
    }
    __syncthreads();
    for (int c = 0; c < PB; ++c) {
        float s = 0.f;
        for (int r = c + 1 + tid; r < dp; r += kQrThreads) s += V[r * LS + c] * V[r * LS + c];
        s = wave_sum(s);
        if (lane == 0) sh.red[wave] = s;
        __syncthreads();
        float xn2 = 0.f;
#pragma unroll
        for (int w = 0; w < kQrWaves; ++w) xn2 += sh.red[w];
        const float alpha = V[c * LS + c];
        float beta = alpha, tau = 0.f, scale = 1.f;
        if (xn2 != 0.f) {
            beta = -copysignf(sqrtf(alpha * alpha + xn2), alpha);
            tau = (beta - alpha) / beta;
            scale = 1.f / (alpha - beta);
        }
        __syncthreads();                            // every wave has read red and alpha
        for (int r = c + 1 + tid; r < dp; r += kQrThreads) V[r * LS + c] *= scale;
        if (tid == 0) {
            V[c * LS + c] = 1.f;                    // unit diagonal from here on
            sh.tau[c] = tau;
            W[(int64_t)(p0 + c) * d + p0 + c] = beta;   // R's diagonal entry
        }
        __syncthreads();
        // H_c on the panel's later columns, one wave per column
        for (int c2 = c + 1 + wave; c2 < PB; c2 += kQrWaves) {
            float w = 0.f;
            for (int r = c + lane; r < dp; r += 64) w += V[r * LS + c] * V[r * LS + c2];
            w = wave_sum(w) * tau;
            for (int r = c + lane; r < dp; r += 64) V[r * LS + c2] -= w * V[r * LS + c];
        }
        __syncthreads();
    }
    // write back R above the diagonal and the reflectors below it (the
    // diagonal already holds beta), then make V explicit: zeros above the
    // unit diagonal
    for (int idx = tid; idx < PB * dp; idx += kQrThreads) {
        const int c = idx / dp, r = idx - c * dp;
        if (r != c) W[(int64_t)(p0 + c) * d + p0 + r] = V[r * LS + c];
    }
    __syncthreads();
    for (int idx = tid; idx < PB * PB; idx += kQrThreads) {
        const int r = idx / PB, c = idx - r * PB;
        if (r < c) V[r * LS + c] = 0.f;
    }
    __syncthreads();
    // G = V^T V (entries m < i are used)
    for (int pr = wave; pr < PB * PB; pr += kQrWaves) {
        const int m = pr / PB, i = pr - m * PB;
        if (m >= i) continue;                       // wave-uniform
        float g = 0.f;
        for (int r = i + lane; r < dp; r += 64) g += V[r * LS + m] * V[r * LS + i];
        g = wave_sum(g);
        if (lane == 0) sh.G[m * kQrMaxNb + i] = g;
    }
    __syncthreads();
    // T: T[i][i] = tau_i, T[l][i] = -tau_i sum_{l<=q<i} T[l][q] G[q][i];
    // lane l of wave 0 writes row l and reads back only its own entries
    if (wave == 0 && lane < PB) {
        const int l = lane;
        for (int q = 0; q < PB; ++q) sh.T[l * kQrMaxNb + q] = q == l ? sh.tau[l] : 0.f;
        for (int i = 1; i < PB; ++i) {
            if (l < i) {
                float t = 0.f;
                for (int q = l; q < i; ++q) t += sh.T[l * kQrMaxNb + q] * sh.G[q * kQrMaxNb + i];
                sh.T[l * kQrMaxNb + i] = -sh.tau[i] * t;
            }
        }
    }
    __syncthreads();
    // trailing columns and the right-hand side: a <- a - V (T^T (V^T a)),
    // one wave per column
    for (int k = p0 + PB + wave; k <= n; k += kQrWaves) {
        float *const a = W + (int64_t)k * d + p0;
        float wv[PB];
#pragma unroll
        for (int c = 0; c < PB; ++c) wv[c] = 0.f;
        for (int r = lane; r < dp; r += 64) {
            const float ar = a[r];
            const float *vr = V + r * LS;
#pragma unroll
            for (int c = 0; c < PB; ++c) wv[c] += vr[c] * ar;
        }
#pragma unroll
        for (int c = 0; c < PB; ++c) wv[c] = wave_sum(wv[c]);
        // (T^T w)_i on lane i (column i of T, one entry per lane), then every
        // lane takes the PB entries back as wave-uniform values
        const int li = lane < PB ? lane : 0;
        float ui = 0.f;
#pragma unroll
        for (int q = 0; q < PB; ++q)
            if (q <= lane) ui += sh.T[q * kQrMaxNb + li] * wv[q];
        float u[PB];
#pragma unroll
        for (int c = 0; c < PB; ++c)
            u[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ui), c));
        for (int r = lane; r < dp; r += 64) {
            const float *vr = V + r * LS;
            float ar = a[r];
#pragma unroll
            for (int c = 0; c < PB; ++c) ar -= vr[c] * u[c];
            a[r] = ar;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kQrThreads) void k_lstsq_qr(const QrArgs args) {
    __shared__ QrShared sh;
    __shared__ float zs[kQrMaxRows];                // right-hand side of R x = z
    __shared__ float xs[kQrMaxRows];                // solution
    const int d = args.d, n = args.n, nb = args.nb;
    float *const W = args.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // [SA | Sb] into column-major W
    for (int64_t idx = tid; idx < (int64_t)d * n; idx += kQrThreads) {
        const int i = (int)(idx / n), j = (int)(idx - (int64_t)i * n);
        W[(int64_t)j * d + i] = args.SA[(int64_t)i * args.ld + j];
    }
    for (int i = tid; i < d; i += kQrThreads) W[(int64_t)n * d + i] = args.Sb[i];
    __syncthreads();

    // full panels of nb columns, then the rest in power-of-two panels
    int p0 = 0;
    while (p0 < n) {
        const int rem = n - p0;
        const int pb = rem >= nb ? nb : rem >= 16 ? 16 : rem >= 8 ? 8 : rem >= 4 ? 4
                                                                    : rem >= 2 ? 2 : 1;
        switch (pb) {
        case 32: qr_panel<32>(sh, W, d, n, p0); break;
        case 16: qr_panel<16>(sh, W, d, n, p0); break;
        case 8: qr_panel<8>(sh, W, d, n, p0); break;
        case 4: qr_panel<4>(sh, W, d, n, p0); break;
        case 2: qr_panel<2>(sh, W, d, n, p0); break;
        default: qr_panel<1>(sh, W, d, n, p0); break;
        }
        p0 += pb;
    }

    // R x = z, z = (Q^T Sb)[0:n]; R(i, j) = W[j*d + i] for i <= j
    for (int i = tid; i < n; i += kQrThreads) zs[i] = W[(int64_t)n * d + i];
    __syncthreads();
    const int top = (n + 31) / 32 * 32;
    for (int b1 = top; b1 > 0; b1 -= 32) {
        const int b0 = b1 - 32, bh = b1 < n ? b1 : n;
        if (wave == 0) {
            const int l = lane & 31;
            float z = b0 + l < bh ? zs[b0 + l] : 0.f;
            float xl = 0.f;
            for (int j = bh - 1; j >= b0; --j) {
                const float zj = __shfl(z, j - b0, 64);
                const float xj = zj / W[(int64_t)j * d + j];
                if (l == j - b0) xl = xj;
                if (l < j - b0) z -= xj * W[(int64_t)j * d + b0 + l];
            }
            if (lane < 32 && b0 + l < bh) xs[b0 + l] = xl;
        }
        __syncthreads();
        for (int i = tid; i < b0; i += kQrThreads) {
            float t = zs[i];
            for (int j = b0; j < bh; ++j) t -= W[(int64_t)j * d + i] * xs[j];
            zs[i] = t;
        }
        __syncthreads();
    }
    for (int i = tid; i < n; i += kQrThreads) args.x[i] = xs[i];
}

}  // namespace

// widest panel whose rows x (PB + 1) floats fit the LDS panel
int lstsq_panel_cols(int32_t d) {
    return (int64_t)d * 33 <= kQrPanelFloats ? 32 : (int64_t)d * 17 <= kQrPanelFloats ? 16 : 8;
}

hipError_t launch_lstsq_qr(const float *SA, int32_t d, int32_t n, int64_t ld, const float *Sb,
                           float *x, float *W, hipStream_t s) {
    if (d < 1 || n < 1 || n > d || d > kQrMaxRows) return hipErrorInvalidValue;
    QrArgs a{SA, Sb, x, W, ld, d, n, lstsq_panel_cols(d)};
    if ((int64_t)d * (a.nb + 1) > kQrPanelFloats) return hipErrorInvalidValue;
    k_lstsq_qr<<<dim3(1), dim3(kQrThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sk
