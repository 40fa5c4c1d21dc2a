// C ABI of libsksketch: argument validation, variant choice, launch.
// Declarations and full contracts are in include/sk.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "sk.h"
#include "sk_internal.hpp"
#include "sk_rng.hpp"

namespace sk {

hipError_t dev_info(DevInfo *out) {
    constexpr int kMaxDev = 64;
    static DevInfo cache[kMaxDev];
    static bool have[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDev && have[dev]) {
        *out = cache[dev];
        return hipSuccess;
    }
    DevInfo di{};
    e = hipDeviceGetAttribute(&di.num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&di.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDev) {
        cache[dev] = di;
        have[dev] = true;
    }
    *out = di;
    return hipSuccess;
}

// Widest power-of-two slice (<= 64 lanes) whose d x slice partial of 4-byte
// words fits in LDS.  A partial that takes more than half the LDS runs one
// 1024-thread workgroup per CU; smaller partials run 512-thread workgroups,
// several per CU.  Row chunks are sized so the grid fills every CU.
bool plan_lds(const DevInfo &di, int64_t m, int64_t lanes_total, int32_t d, LdsPlan *p) {
    int slice = 64;
    while (slice > 8 && ((int64_t)d * slice * 4 > di.max_lds || slice / 2 >= lanes_total)) slice /= 2;
    if ((int64_t)d * slice * 4 > di.max_lds) return false;
    p->slice = slice;
    p->lds_bytes = (size_t)d * slice * 4;
    const int per_cu_lds = (int)(di.max_lds / (int64_t)p->lds_bytes);
    int per_cu;
    if (per_cu_lds < 2) {
        p->threads = 1024;
        per_cu = 1;
    } else {
        p->threads = 512;
        per_cu = per_cu_lds < 4 ? per_cu_lds : 4;
    }
    p->slices = (lanes_total + slice - 1) / slice;
    int64_t want = (int64_t)di.num_cu * per_cu / p->slices;
    if (want < 1) want = 1;
    int64_t rows = (m + want - 1) / want;
    if (rows < 1) rows = 1;
    p->rows_per_chunk = rows;
    p->chunks = (m + rows - 1) / rows;
    if (p->chunks < 1) p->chunks = 1;
    return true;
}

}  // namespace sk

namespace {

float scale_of(int64_t k) { return (float)(1.0 / sqrt((double)k)); }

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bbytes && y < x + abytes;
}

size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t elem) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)((rows - 1) * ld + cols) * elem;
}

sk_status hip_status(hipError_t e) { return e == hipSuccess ? SK_OK : SK_ERR_HIP; }

// Checks shared by the SparseStack apply calls (FP32 and FP16 output).
sk_status check_apply(const float *A, int64_t m, int32_t n, int64_t lda, const int32_t *row_idx,
                      const float *val, int32_t zeta, const void *B, size_t belem, int32_t d,
                      int64_t ldb, uint32_t flags) {
    if (m < 0 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0) return SK_ERR_SHAPE;
    if (lda < n || ldb < n) return SK_ERR_SHAPE;
    if (m > (INT64_MAX / 8) / (zeta > lda ? zeta : lda)) return SK_ERR_SHAPE;
    if (flags & ~(SK_ACCUMULATE | SK_VARIANT_FLAT | SK_VARIANT_LDS)) return SK_ERR_ARG;
    if ((flags & SK_VARIANT_FLAT) && (flags & SK_VARIANT_LDS)) return SK_ERR_ARG;
    if (B == nullptr) return SK_ERR_NULL;
    if (m > 0 && (A == nullptr || row_idx == nullptr || val == nullptr)) return SK_ERR_NULL;
    const size_t bspan = span_bytes(d, n, ldb, belem);
    if (m > 0) {
        if (overlaps(A, span_bytes(m, n, lda, 4), B, bspan)) return SK_ERR_ARG;
        if (overlaps(row_idx, (size_t)m * zeta * 4, B, bspan)) return SK_ERR_ARG;
        if (overlaps(val, (size_t)m * zeta * 4, B, bspan)) return SK_ERR_ARG;
    }
    return SK_OK;
}

}  // namespace

extern "C" {

const char *sk_status_string(sk_status s) {
    switch (s) {
        case SK_OK: return "ok";
        case SK_ERR_NULL: return "a required pointer is NULL";
        case SK_ERR_SHAPE: return "inconsistent sizes or leading dimensions";
        case SK_ERR_ALIGN: return "misaligned buffer or stride";
        case SK_ERR_UNSUPPORTED: return "unsupported configuration";
        case SK_ERR_HIP: return "HIP runtime error";
        case SK_ERR_ARG: return "invalid flags or overlapping buffers";
    }
    return "unknown status";
}

sk_status sk_meta_generate(uint64_t seed, int64_t row_offset, int64_t m, int32_t d, int32_t zeta,
                           int32_t *row_idx, float *val, void *stream) {
    if (m < 0 || row_offset < 0 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0)
        return SK_ERR_SHAPE;
    if (m > INT64_MAX / 8 / zeta) return SK_ERR_SHAPE;
    if (m == 0) return SK_OK;
    if (row_idx == nullptr || val == nullptr) return SK_ERR_NULL;
    if (overlaps(row_idx, (size_t)m * zeta * 4, val, (size_t)m * zeta * 4)) return SK_ERR_ARG;
    return hip_status(sk::launch_meta(seed, row_offset, m, d, zeta, scale_of(zeta), row_idx, val,
                                      (hipStream_t)stream));
}

sk_status sk_apply_f32(const float *A, int64_t m, int32_t n, int64_t lda, const int32_t *row_idx,
                       const float *val, int32_t zeta, float *B, int32_t d, int64_t ldb,
                       uint32_t flags, void *stream) {
    sk_status st = check_apply(A, m, n, lda, row_idx, val, zeta, B, 4, d, ldb, flags);
    if (st != SK_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    sk::DevInfo di;
    hipError_t e = sk::dev_info(&di);
    if (e != hipSuccess) return SK_ERR_HIP;
    sk::LdsPlan plan{};
    const bool lds_ok = m > 0 && sk::plan_lds(di, m, n, d, &plan);
    if ((flags & SK_VARIANT_LDS) && !lds_ok && m > 0) return SK_ERR_UNSUPPORTED;
    if (!(flags & SK_ACCUMULATE)) {
        e = sk::launch_zero_words(reinterpret_cast<uint32_t *>(B), d, n, ldb, s);
        if (e != hipSuccess) return SK_ERR_HIP;
    }
    if (m == 0) return SK_OK;
    if (!(flags & SK_VARIANT_FLAT) && lds_ok)
        return hip_status(sk::launch_f32_lds(plan, A, m, n, lda, row_idx, val, zeta, B, d, ldb, s));
    return hip_status(sk::launch_f32_flat(A, m, n, lda, row_idx, val, zeta, B, d, ldb, s));
}

sk_status sk_apply_f16acc(const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                          int32_t d, int64_t ldb, uint32_t flags, void *stream) {
    sk_status st = check_apply(A, m, n, lda, row_idx, val, zeta, B, 2, d, ldb, flags);
    if (st != SK_OK) return st;
    if (n % 2 != 0) return SK_ERR_SHAPE;
    if (ldb % 2 != 0 || (uintptr_t)B % 4 != 0) return SK_ERR_ALIGN;
    if (m > 0 && (lda % 2 != 0 || (uintptr_t)A % 8 != 0)) return SK_ERR_ALIGN;
    const hipStream_t s = (hipStream_t)stream;
    sk::DevInfo di;
    hipError_t e = sk::dev_info(&di);
    if (e != hipSuccess) return SK_ERR_HIP;
    sk::LdsPlan plan{};
    const bool lds_ok = m > 0 && sk::plan_lds(di, m, n / 2, d, &plan);
    if ((flags & SK_VARIANT_LDS) && !lds_ok && m > 0) return SK_ERR_UNSUPPORTED;
    if (!(flags & SK_ACCUMULATE)) {
        e = sk::launch_zero_words(reinterpret_cast<uint32_t *>(B), d, n / 2, ldb / 2, s);
        if (e != hipSuccess) return SK_ERR_HIP;
    }
    if (m == 0) return SK_OK;
    if (!(flags & SK_VARIANT_FLAT) && lds_ok)
        return hip_status(sk::launch_f16_lds(plan, A, m, n, lda, row_idx, val, zeta, B, d, ldb, s));
    return hip_status(sk::launch_f16_flat(A, m, n, lda, row_idx, val, zeta, B, d, ldb, s));
}

sk_status sk_apply_blockperm(const float *A, int64_t m, int32_t n, int64_t lda, int32_t d,
                             int32_t M, int32_t kappa, int32_t s, uint64_t seed, float *Y,
                             int64_t ldy, uint32_t flags, void *stream) {
    if (m < 1 || n < 1 || d < 1 || M < 1 || kappa < 1 || s < 1) return SK_ERR_SHAPE;
    if (M > sk::kBlockPermMaxM) return SK_ERR_UNSUPPORTED;
    if (m % M != 0 || d % M != 0 || M % kappa != 0 || lda < n || ldy < n) return SK_ERR_SHAPE;
    if (s > d / M) return SK_ERR_SHAPE;
    if (m > INT64_MAX / 8 / lda) return SK_ERR_SHAPE;
    if (flags & ~SK_ACCUMULATE) return SK_ERR_ARG;
    if (A == nullptr || Y == nullptr) return SK_ERR_NULL;
    if (overlaps(A, span_bytes(m, n, lda, 4), Y, span_bytes(d, n, ldy, 4))) return SK_ERR_ARG;
    if (s != 1) return SK_ERR_UNSUPPORTED;
    if (kappa != 1 && kappa != 2 && kappa != 4 && kappa != 8) return SK_ERR_UNSUPPORTED;
    const int32_t Br = d / M;
    sk::DevInfo di;
    if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
    if ((int64_t)kappa * Br > sk::blockperm_max_rows(di)) return SK_ERR_UNSUPPORTED;

    sk::BlockPermArgs args;
    memset(&args, 0, sizeof(args));
    args.A = A;
    args.Y = Y;
    args.lda = lda;
    args.ldy = ldy;
    args.Bc = m / M;
    args.n = n;
    args.Br = Br;
    args.C = M / kappa;
    args.accumulate = (flags & SK_ACCUMULATE) ? 1 : 0;
    args.scale = scale_of((int64_t)kappa * s);
    args.seed = seed;
    // sigma: Fisher-Yates over [M] with Philox draws (domain word 3 = 2).
    uint16_t sigma[sk::kBlockPermMaxM];
    for (int k = 0; k < M; ++k) sigma[k] = (uint16_t)k;
    for (int k = M - 1; k >= 1; --k) {
        const sk::u32x4 w = sk::philox4x32_10(sk::u32x4{(uint32_t)k, 0u, 0u, 2u}, (uint32_t)seed,
                                              (uint32_t)(seed >> 32));
        const uint32_t j = sk::mulhi32(w.x, (uint32_t)(k + 1));
        const uint16_t t = sigma[k];
        sigma[k] = sigma[j];
        sigma[j] = t;
    }
    for (int g = 0; g < M; ++g) args.ginv[sigma[g]] = (uint16_t)g;
    return hip_status(sk::launch_blockperm(args, kappa, (hipStream_t)stream));
}

}  // extern "C"
