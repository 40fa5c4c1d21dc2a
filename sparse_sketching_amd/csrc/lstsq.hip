// Least squares on a small sketch: x = argmin ||SA x - Sb||_2 by an FP32
// Householder QR of SA, the projection Q^T Sb and a triangular solve (the
// reduced solve of the FP16 sketching page §V-A, §V-D: "FP32 QR,
// projection, and solve" on the d x n sketch; FlashSketch page App. F.1.4).
//
// How (MI355X-specific): the problem is a few hundred KiB, so it is bound by
// latency, not by bandwidth or flops; a vendor QR built from thousands of
// small launches spends its time launching.  Here a few launches per panel:
//  * [SA | Sb] is copied into a column-major workspace (column j contiguous,
//    so every column access below is coalesced), Sb as column n.
//  * Panels of PB columns (32, 16 or 8 by d, so the panel fits 100 KiB of
//    LDS; the last columns in power-of-two panels, so PB is a compile-time
//    constant everywhere) are factored by one workgroup in LDS with the
//    reflector rule of LAPACK's larfg (beta = -sign(alpha) ||(alpha, x)||,
//    tau = (beta - alpha) / beta, v = x / (alpha - beta); tau = 0 when
//    x = 0), one column after another.  The panel is row-major in LDS with
//    an odd row stride (PB + 1): a column is read without bank conflicts, a
//    row by immediate offsets from one address.  The reflectors are
//    combined as H_1 ... H_PB = I - V T V^T (T upper triangular, the forward
//    column-wise recurrence), T kept after W in the workspace.
//  * The trailing columns, the right-hand side among them, are updated as
//    a <- a - V (T^T (V^T a)) by as many workgroups as they need (16
//    columns each, one wavefront per column), each with its own LDS copy
//    of V: the update is spread over the device instead of one CU.
//  * R x = (Q^T Sb)[0:n] is solved by one workgroup in blocks of 32 rows
//    from the bottom: one wavefront solves a block's triangle from LDS with
//    lane shuffles, then all wavefronts subtract its columns from the rest.
#include "sk_internal.hpp"

namespace sk {
namespace {

constexpr int kQrThreads = 1024;
constexpr int kQrWaves = kQrThreads / 64;
constexpr int kQrMaxNb = 32;
// panel floats in LDS: rows x (PB + 1) <= kQrPanelFloats (PB = 32 up to 775
// rows, 16 up to 1505, 8 up to kQrMaxRows)
constexpr int kQrPanelFloats = 25600;

// Sum over the 64 lanes, the same value on every lane: within each 16-lane
// row by DPP moves (swap neighbours, swap pairs, mirror the half-row, mirror
// the row: each lane then holds its row's sum), then the four row sums by
// readlane.  VALU-only, no LDS round trip per step; the order is fixed.
template <int CTRL>
__device__ __forceinline__ float dpp_add_c(float v) {
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add_c<0xB1>(v);                         // quad_perm [1,0,3,2]
    v = dpp_add_c<0x4E>(v);                         // quad_perm [2,3,0,1]
    v = dpp_add_c<0x141>(v);                        // row_half_mirror
    v = dpp_add_c<0x140>(v);                        // row_mirror
    const int b = __float_as_int(v);
    return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
            __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
            __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

struct QrArgs {
    const float *SA;            // d x n row-major, row stride ld
    const float *Sb;            // d
    float *x;                   // n
    float *W;                   // workspace: n + 1 columns of d floats
    int64_t ld;
    int32_t d, n, nb;
};

// Workspace layout: W (n + 1 columns of d floats, column-major: [SA | Sb],
// then R, the reflectors and Q^T Sb) followed by the panel's T
// (kQrMaxNb x kQrMaxNb floats).

// [SA | Sb] into column-major W (grid-stride over the d x (n + 1) entries).
__global__ __launch_bounds__(256) void k_qr_copy(const QrArgs args) {
    const int64_t total = (int64_t)args.d * (args.n + 1);
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int i = (int)(idx / (args.n + 1)), j = (int)(idx - (int64_t)i * (args.n + 1));
        args.W[(int64_t)j * args.d + i] =
            j < args.n ? args.SA[(int64_t)i * args.ld + j] : args.Sb[i];
    }
}

// Factor panel columns p0 .. p0+PB-1 (one workgroup): R and the reflectors
// to W (the diagonal holds beta), T of I - V T V^T after W.
template <int PB>
__global__ __launch_bounds__(kQrThreads) void k_qr_panel(const QrArgs args, int p0) {
    constexpr int LS = PB + 1;                      // LDS row stride
    __shared__ float V[kQrPanelFloats];             // row r, column c at r * LS + c
    __shared__ float G[kQrMaxNb * kQrMaxNb];        // V^T V
    __shared__ float taus[kQrMaxNb];
    __shared__ float scales[kQrMaxNb];
    __shared__ float betas[kQrMaxNb];               // R's diagonal, written back with the panel
    // column c's ||x||^2 and alpha in slot c & 1 (read in step c; the next
    // column's are written into the other slot during step c)
    __shared__ float nrm[2][2];
    const int d = args.d;
    float *const W = args.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dp = d - p0;                          // panel rows p0 .. d-1
    for (int idx = tid; idx < PB * dp; idx += kQrThreads) {
        const int c = idx / dp, r = idx - c * dp;
        V[r * LS + c] = W[(int64_t)(p0 + c) * d + p0 + r];
    }
    __syncthreads();
    if (wave == 0) {                                // column 0's norm and alpha
        float q = 0.f;
        for (int r = 1 + lane; r < dp; r += 64) q += V[r * LS] * V[r * LS];
        q = wave_sum(q);
        if (lane == 0) {
            nrm[0][0] = q;
            nrm[0][1] = V[0];
        }
    }
    __syncthreads();
    // one barrier per column: the reflector's tail stays unscaled in LDS
    // while the panel is factored (every wave multiplies by scale when it
    // reads it), and wave 0, which updates column c + 1, also leaves that
    // column's norm for the next step
    for (int c = 0; c < PB; ++c) {
        const float xn2 = nrm[c & 1][0], alpha = nrm[c & 1][1];
        float beta = alpha, tau = 0.f, scale = 1.f;
        if (xn2 != 0.f) {
            beta = -copysignf(sqrtf(alpha * alpha + xn2), alpha);
            tau = (beta - alpha) / beta;
            scale = 1.f / (alpha - beta);
        }
        // (no global store inside the column loop: each barrier would wait
        // for it to land)
        if (tid == 0) {
            taus[c] = tau;
            scales[c] = scale;
            betas[c] = beta;
        }
        // H_c on the panel's later columns, one wave per column
        for (int c2 = c + 1 + wave; c2 < PB; c2 += kQrWaves) {
            float w = lane == 0 ? V[c * LS + c2] : 0.f;     // v_c = 1
            for (int r = c + 1 + lane; r < dp; r += 64) w += scale * V[r * LS + c] * V[r * LS + c2];
            w = wave_sum(w) * tau;
            if (lane == 0) V[c * LS + c2] -= w;
            float q = 0.f;
            for (int r = c + 1 + lane; r < dp; r += 64) {
                const float v = V[r * LS + c2] - w * (scale * V[r * LS + c]);
                V[r * LS + c2] = v;
                if (r > c + 1) q += v * v;
            }
            if (c2 == c + 1) {                      // wave 0: the next column's norm
                q = wave_sum(q);
                if (lane == 0) {
                    nrm[(c + 1) & 1][0] = q;
                    nrm[(c + 1) & 1][1] = V[(c + 1) * LS + c + 1];
                }
            }
        }
        __syncthreads();
    }
    // the reflectors scaled in place, unit diagonal
    for (int idx = tid; idx < PB * dp; idx += kQrThreads) {
        const int c = idx / dp, r = idx - c * dp;
        if (r > c) V[r * LS + c] *= scales[c];
        else if (r == c) V[r * LS + c] = 1.f;
    }
    __syncthreads();
    // R above the diagonal, beta on it and the reflectors below it to W
    for (int idx = tid; idx < PB * dp; idx += kQrThreads) {
        const int c = idx / dp, r = idx - c * dp;
        W[(int64_t)(p0 + c) * d + p0 + r] = r == c ? betas[c] : V[r * LS + c];
    }
    // G[m][i] = v_m . v_i for m < i (v_i: zero above row i, one at row i)
    for (int pr = wave; pr < PB * PB; pr += kQrWaves) {
        const int m = pr / PB, i = pr - m * PB;
        if (m >= i) continue;                       // wave-uniform
        float g = 0.f;
        for (int r = i + 1 + lane; r < dp; r += 64) g += V[r * LS + m] * V[r * LS + i];
        g = wave_sum(g);
        if (lane == 0) G[m * kQrMaxNb + i] = g + V[i * LS + m];
    }
    __syncthreads();
    // T: T[i][i] = tau_i, T[l][i] = -tau_i sum_{l<=q<i} T[l][q] G[q][i];
    // lane l of wave 0 builds row l in registers
    if (wave == 0 && lane < PB) {
        float trow[PB];
#pragma unroll
        for (int q = 0; q < PB; ++q) trow[q] = q == lane ? taus[q] : 0.f;
#pragma unroll
        for (int i = 1; i < PB; ++i) {
            if (lane < i) {
                float t = 0.f;
#pragma unroll
                for (int q = 0; q < i; ++q) t += trow[q] * G[q * kQrMaxNb + i];
                trow[i] = -taus[i] * t;
            }
        }
        float *const Tg = W + (int64_t)(args.n + 1) * d;
#pragma unroll
        for (int q = 0; q < PB; ++q) Tg[lane * kQrMaxNb + q] = trow[q];
    }
}

// Trailing columns of panel p0 and the right-hand side (W's column n):
// a <- a - V (T^T (V^T a)).  Workgroup b takes columns p0 + PB + 16 b ..
// +15, one wave per column; V (unit lower trapezoid) and T are read from W.
template <int PB>
__global__ __launch_bounds__(kQrThreads) void k_qr_trail(const QrArgs args, int p0) {
    constexpr int LS = PB + 1;
    __shared__ float V[kQrPanelFloats];
    __shared__ float T[kQrMaxNb * kQrMaxNb];
    const int d = args.d, n = args.n;
    float *const W = args.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dp = d - p0;
    for (int idx = tid; idx < PB * dp; idx += kQrThreads) {
        const int c = idx / dp, r = idx - c * dp;
        V[r * LS + c] = r < c ? 0.f : r == c ? 1.f : W[(int64_t)(p0 + c) * d + p0 + r];
    }
    const float *const Tg = W + (int64_t)(n + 1) * d;
    for (int idx = tid; idx < kQrMaxNb * kQrMaxNb; idx += kQrThreads) T[idx] = Tg[idx];
    __syncthreads();
    const int k = p0 + PB + blockIdx.x * kQrWaves + wave;
    if (k > n) return;                              // wave-uniform; no barrier follows
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
    // (T^T w)_i on lane i, then every lane takes the PB entries back
    const int li = lane < PB ? lane : 0;
    float ui = 0.f;
#pragma unroll
    for (int q = 0; q < PB; ++q)
        if (q <= lane) ui += T[q * kQrMaxNb + li] * wv[q];
    float u[PB];
#pragma unroll
    for (int c = 0; c < PB; ++c) u[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ui), c));
    for (int r = lane; r < dp; r += 64) {
        const float *vr = V + r * LS;
        float ar = a[r];
#pragma unroll
        for (int c = 0; c < PB; ++c) ar -= vr[c] * u[c];
        a[r] = ar;
    }
}

// R x = z, z = (Q^T Sb)[0:n], R(i, j) = W[j*d + i] for i <= j (one
// workgroup): 32-row blocks from the bottom, a block's triangle by one wave
// from LDS, then every wave subtracts its columns from the rest of z.
__global__ __launch_bounds__(kQrThreads) void k_qr_backsub(const QrArgs args) {
    __shared__ float zs[kQrMaxRows];
    __shared__ float xs[kQrMaxRows];
    __shared__ float Rb[32 * 33];                   // the block's triangle, row-major
    const int d = args.d, n = args.n;
    const float *const W = args.W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < n; i += kQrThreads) zs[i] = W[(int64_t)n * d + i];
    const int top = (n + 31) / 32 * 32;
    for (int b1 = top; b1 > 0; b1 -= 32) {
        const int b0 = b1 - 32, bh = b1 < n ? b1 : n;
        // R(b0 + i, b0 + j) for the block, zero outside it
        {
            const int i = tid >> 5, j = tid & 31;
            Rb[i * 33 + j] = (b0 + i < bh && b0 + j < bh && i <= j)
                                 ? W[(int64_t)(b0 + j) * d + b0 + i] : 0.f;
        }
        __syncthreads();
        if (wave == 0) {
            const int l = lane & 31;
            float z = b0 + l < bh ? zs[b0 + l] : 0.f;
            float xl = 0.f;
            for (int j = bh - b0 - 1; j >= 0; --j) {
                const float zj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
                const float xj = zj / Rb[j * 33 + j];
                if (l == j) xl = xj;
                if (l < j) z -= xj * Rb[l * 33 + j];
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

template <int PB>
hipError_t qr_panel_step(const QrArgs &a, int p0, hipStream_t s) {
    k_qr_panel<PB><<<dim3(1), dim3(kQrThreads), 0, s>>>(a, p0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntrail = a.n + 1 - (p0 + PB);         // columns after the panel, rhs included
    const int blocks = (ntrail + kQrWaves - 1) / kQrWaves;
    k_qr_trail<PB><<<dim3(blocks), dim3(kQrThreads), 0, s>>>(a, p0);
    return hipGetLastError();
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
    int64_t cb = ((int64_t)d * (n + 1) + 255) / 256;
    if (cb > 1024) cb = 1024;
    k_qr_copy<<<dim3((unsigned)cb), dim3(256), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    // full panels of nb columns, then the rest in power-of-two panels
    for (int p0 = 0; p0 < n && e == hipSuccess;) {
        const int rem = n - p0;
        const int pb = rem >= a.nb ? a.nb : rem >= 16 ? 16 : rem >= 8 ? 8 : rem >= 4 ? 4
                                                                        : rem >= 2 ? 2 : 1;
        switch (pb) {
        case 32: e = qr_panel_step<32>(a, p0, s); break;
        case 16: e = qr_panel_step<16>(a, p0, s); break;
        case 8: e = qr_panel_step<8>(a, p0, s); break;
        case 4: e = qr_panel_step<4>(a, p0, s); break;
        case 2: e = qr_panel_step<2>(a, p0, s); break;
        default: e = qr_panel_step<1>(a, p0, s); break;
        }
        p0 += pb;
    }
    if (e != hipSuccess) return e;
    k_qr_backsub<<<dim3(1), dim3(kQrThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sk
