// C ABI of libsksketch: argument validation, variant choice, launch.
// Declarations and full contracts are in include/sk.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "sk.h"
#include "sk_internal.hpp"
#include "sk_rng.hpp"

// The allocation-free sketch's scratch (sk_sketch_f16acc_noalloc): the
// fused kernel's partials live in this file-scope device array, of which
// each device holds its own copy while the library stays loaded.  Host code
// never passes `scratch` itself to a kernel (on the host the name stands for
// a host-side shadow, not a device address): it passes the device address
// hipGetSymbolAddress returns, taken once per device on that device's first
// call.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint32_t scratch[kStaticScratchBytes / 4];

namespace sk {

// The per-device attributes are read once and kept in atomics (0 = not yet
// read), so concurrent first calls from several host threads are safe: each
// stores the same values.
hipError_t dev_info(DevInfo *out) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache_cu[kMaxDev];
    static std::atomic<int> cache_lds[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDev;
    if (cached) {
        const int cu = cache_cu[dev].load(std::memory_order_relaxed);
        const int lds = cache_lds[dev].load(std::memory_order_relaxed);
        if (cu > 0 && lds > 0) {
            *out = DevInfo{cu, lds};
            return hipSuccess;
        }
    }
    DevInfo di{};
    e = hipDeviceGetAttribute(&di.num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&di.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    if (cached && di.num_cu > 0 && di.max_lds > 0) {
        cache_cu[dev].store(di.num_cu, std::memory_order_relaxed);
        cache_lds[dev].store(di.max_lds, std::memory_order_relaxed);
    }
    *out = di;
    return hipSuccess;
}

// LDS plan for k_stack_apply.  Preference order: two-word lanes (half the
// instructions per byte of A) with at most max_groups_wide block groups;
// then one-word lanes with all blocks in one group.  Extra groups re-read A
// through L2, which pays off for FP32 (twice the hits per byte of A) but not
// for FP16 (measured on MI355X: 2^20 x 256, d = 512).  For each, the slice is the widest
// power of two (at most 64 lanes, at least 8, no wider than the row needs)
// whose partial (plus the wavefronts' 64-lane dummy rows) fits in LDS.  A
// plan that takes more than half the LDS runs one 1024-thread workgroup per
// CU; smaller ones run 512-thread workgroups, several per CU.  Row chunks
// are sized so the grid fills every CU, with at least 256 rows per chunk so
// the one flush per workgroup stays small next to the rows it streams.
bool plan_lds(const DevInfo &di, int64_t m, int64_t units, bool wide_ok, int max_groups_wide,
              int32_t d, int32_t zeta, LdsPlan *p) {
    if (zeta > 64 || units < 1) return false;
    const int64_t db = d / zeta;
    bool found = false;
    for (int w = 2; w >= 1 && !found; --w) {
        if (w == 2 && (!wide_ok || units % 2 != 0 || units / 2 < 64)) continue;
        const int64_t lpos = units / w;
        for (int sp = 64; sp >= 8 && !found; sp /= 2) {
            if (sp > 8 && sp / 2 >= lpos) continue;
            // two-word lanes are built only for full 64-lane slices
            if (w == 2 && sp != 64) break;
            for (int g = 1; g <= zeta && !found; ++g) {
                if (zeta % g != 0) continue;
                if (w == 2 && g > max_groups_wide) break;
                if (w == 1 && g > 1) break;
                const int64_t zg = zeta / g;
                const int64_t need = (zg * db * sp + 16 * 64) * w * 4;
                if (need > di.max_lds) continue;
                p->words = w;
                p->slice = sp;
                p->groups = g;
                p->zg = (int)zg;
                p->lds_bytes = (size_t)need;
                p->slices = (lpos + sp - 1) / sp;
                found = true;
            }
        }
    }
    if (!found) return false;
    const int per_cu_lds = (int)(di.max_lds / (int64_t)p->lds_bytes);
    int per_cu;
    if (per_cu_lds < 2) {
        p->threads = 1024;
        per_cu = 1;
    } else {
        p->threads = 512;
        per_cu = per_cu_lds < 4 ? per_cu_lds : 4;
    }
    const int64_t per_chunk = p->slices * p->groups;
    int64_t want = ((int64_t)di.num_cu * per_cu + per_chunk - 1) / per_chunk;
    const int64_t max_chunks = (m + 255) / 256;
    if (want > max_chunks) want = max_chunks;
    if (want > 65535) want = 65535;
    if (want < 1) want = 1;
    int64_t rows = (m + want - 1) / want;
    if (rows < 1) rows = 1;
    p->rows_per_chunk = rows;
    p->chunks = (m + rows - 1) / rows;
    if (p->chunks < 1) p->chunks = 1;
    const int64_t units_sc = p->slices * p->chunks;      // (slice, chunk) pairs
    p->grid = (units_sc + 7) / 8 * 8 * p->groups;
    p->ws_bytes = (size_t)p->slices * (size_t)p->chunks * (size_t)d * (size_t)p->slice *
                  (size_t)p->words * 4;
    return true;
}

}  // namespace sk

namespace {

float scale_of(int64_t k) { return (float)(1.0 / sqrt((double)k)); }

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bbytes && y < x + abytes;
}

// alignment of a base address in bytes, capped at 16 (the widest lane load)
int base_align(const void *p) {
    const uintptr_t x = (uintptr_t)p;
    if (x % 16 == 0) return 16;
    return (int)(x & (~x + 1));
}

// The fused plan's workspace for rows of lda = n, the larger of the plans an
// A of 8- or 16-byte alignment gets (the word width depends on it); 0 if
// neither covers the shape.
size_t fused_ws_bytes(const sk::DevInfo &di, bool f16, int64_t m, int32_t n, int32_t d,
                      int32_t zeta) {
    size_t need = 0;
    for (int a = 8; a <= 16; a *= 2) {
        sk::FusedPlan fp{};
        if (sk::plan_fused(di, f16, m, n, n, a, d, zeta, &fp) && fp.ws_bytes > need)
            need = fp.ws_bytes;
    }
    return need;
}

size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t elem) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)((rows - 1) * ld + cols) * elem;
}

sk_status hip_status(hipError_t e) { return e == hipSuccess ? SK_OK : SK_ERR_HIP; }

int variant_count(uint32_t flags) {
    return ((flags & SK_VARIANT_FLAT) != 0) + ((flags & SK_VARIANT_LDS) != 0) +
           ((flags & SK_VARIANT_REG) != 0);
}

// Checks shared by the SparseStack apply calls (FP32 and FP16 output).
// extra_flags: the flags a precision adds to SK_ACCUMULATE and the variants
// (SK_COMBINE_F32 for FP16 output).
sk_status check_apply(const float *A, int64_t m, int32_t n, int64_t lda, const int32_t *row_idx,
                      const float *val, int32_t zeta, const void *B, size_t belem, int32_t d,
                      int64_t ldb, uint32_t flags, uint32_t extra_flags) {
    if (m < 0 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0) return SK_ERR_SHAPE;
    if (lda < n || ldb < n) return SK_ERR_SHAPE;
    if (m > (INT64_MAX / 8) / (zeta > lda ? zeta : lda)) return SK_ERR_SHAPE;
    if (flags & ~(SK_ACCUMULATE | SK_VARIANT_FLAT | SK_VARIANT_LDS | SK_VARIANT_REG | extra_flags))
        return SK_ERR_ARG;
    if (variant_count(flags) > 1) return SK_ERR_ARG;
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

// Variant choice and launch shared by the two SparseStack precisions.
sk_status apply_dispatch(bool f16, const float *A, int64_t m, int32_t n, int64_t lda,
                         const int32_t *row_idx, const float *val, int32_t zeta, void *B, int32_t d,
                         int64_t ldb, uint32_t flags, void *workspace, size_t workspace_bytes,
                         hipStream_t s) {
    sk::DevInfo di;
    hipError_t e = sk::dev_info(&di);
    if (e != hipSuccess) return SK_ERR_HIP;
    const bool accumulate = (flags & SK_ACCUMULATE) != 0;
    // the reduce's mode: accumulate, and the FP32 combine of FP16 partials
    const int mode = (accumulate ? sk::kReduceModeAccumulate : 0) |
                     ((f16 && (flags & SK_COMBINE_F32)) ? sk::kReduceModeCombineF32 : 0);
    // the register variant: asked for, or by default where it covers the
    // shape and the workspace holds its partials (reproducible, and the
    // faster one there)
    if (m > 0 && !(flags & (SK_VARIANT_FLAT | SK_VARIANT_LDS))) {
        const bool forced = (flags & SK_VARIANT_REG) != 0;
        sk::FusedPlan fp{};
        const bool covered =
            sk::plan_fused(di, f16, m, n, lda, base_align(A), d, zeta, &fp) &&
            zeta <= sk::kFusedMetaMaxZeta;
        if (forced) {
            if (!covered) return SK_ERR_UNSUPPORTED;
            if (workspace == nullptr) return SK_ERR_NULL;
            if ((uintptr_t)workspace % 16 != 0) return SK_ERR_ALIGN;
            if (workspace_bytes < fp.ws_bytes) return SK_ERR_ARG;
        }
        if (forced || (covered && workspace != nullptr && (uintptr_t)workspace % 16 == 0 &&
                       workspace_bytes >= fp.ws_bytes))
            return hip_status(sk::launch_fused(fp, f16, A, m, n, lda, 0, 0, row_idx, val, d,
                                               zeta, scale_of(zeta), B, ldb,
                                               static_cast<uint32_t *>(workspace), mode, s));
    }
    sk::LdsPlan plan{};
    const int64_t units = f16 ? n / 2 : n;
    // two-word lanes load 16 (FP16) or 8 (FP32) bytes per row
    const int64_t vec = f16 ? 4 : 2;
    const bool wide_ok = lda % vec == 0 && (uintptr_t)A % (vec * 4) == 0;
    // the LDS kernel addresses 16 rows of A from one base with 32-bit offsets
    const bool lds_ok = m > 0 && lda <= ((int64_t)1 << 24) &&
                        sk::plan_lds(di, m, units, wide_ok, f16 ? 1 : 2, d, zeta, &plan);
    if ((flags & SK_VARIANT_LDS) && !lds_ok && m > 0) return SK_ERR_UNSUPPORTED;
    const bool use_lds = m > 0 && !(flags & SK_VARIANT_FLAT) && lds_ok;
    uint32_t *ws = nullptr;
    if (use_lds && workspace != nullptr) {
        if (workspace_bytes < plan.ws_bytes) return SK_ERR_ARG;
        ws = static_cast<uint32_t *>(workspace);
    }
    // the store-and-reduce flush writes every element of B itself
    if (!accumulate && ws == nullptr) {
        e = f16 ? sk::launch_zero_words(reinterpret_cast<uint32_t *>(B), d, n / 2, ldb / 2, s)
                : sk::launch_zero_words(reinterpret_cast<uint32_t *>(B), d, n, ldb, s);
        if (e != hipSuccess) return SK_ERR_HIP;
    }
    if (m == 0) return SK_OK;
    if (f16) {
        uint16_t *B16 = static_cast<uint16_t *>(B);
        if (use_lds)
            return hip_status(sk::launch_f16_lds(plan, A, m, n, lda, row_idx, val, zeta, B16, d, ldb,
                                                 ws, mode, s));
        return hip_status(sk::launch_f16_flat(A, m, n, lda, row_idx, val, zeta, B16, d, ldb, s));
    }
    float *B32 = static_cast<float *>(B);
    if (use_lds)
        return hip_status(sk::launch_f32_lds(plan, A, m, n, lda, row_idx, val, zeta, B32, d, ldb, ws,
                                             mode, s));
    return hip_status(sk::launch_f32_flat(A, m, n, lda, row_idx, val, zeta, B32, d, ldb, s));
}

sk_status check_workspace(const void *ws, size_t bytes, const float *A, int64_t m, int32_t n,
                          int64_t lda, const int32_t *row_idx, const float *val, int32_t zeta,
                          const void *B, size_t bspan) {
    if (ws == nullptr) return SK_OK;
    if ((uintptr_t)ws % 4 != 0) return SK_ERR_ALIGN;
    if (overlaps(ws, bytes, B, bspan)) return SK_ERR_ARG;
    if (m > 0) {
        if (overlaps(ws, bytes, A, span_bytes(m, n, lda, 4))) return SK_ERR_ARG;
        if (overlaps(ws, bytes, row_idx, (size_t)m * zeta * 4)) return SK_ERR_ARG;
        if (overlaps(ws, bytes, val, (size_t)m * zeta * 4)) return SK_ERR_ARG;
    }
    return SK_OK;
}

// Fused sketch: workspace layout of the fallback (metadata + LDS apply):
// row_idx, then val, then the apply's workspace, each 256-byte aligned.
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t fallback_ws_bytes(const sk::DevInfo &di, bool f16, int64_t m, int32_t n, int32_t d,
                         int32_t zeta) {
    const size_t meta = align256((size_t)m * (size_t)zeta * 4);
    size_t apply = 0;
    sk::LdsPlan lp{};
    const int64_t units = f16 ? n / 2 : n;
    const int gw = f16 ? 1 : 2;
    if (sk::plan_lds(di, m, units, true, gw, d, zeta, &lp)) apply = lp.ws_bytes;
    if (sk::plan_lds(di, m, units, false, gw, d, zeta, &lp) && lp.ws_bytes > apply)
        apply = lp.ws_bytes;
    return 2 * meta + align256(apply);
}

// Bytes any sk_sketch_* call with these sizes may need, whatever lda and
// A's alignment: the larger of the fused plan and the fallback.
size_t sketch_ws_bytes(const sk::DevInfo &di, bool f16, int64_t m, int32_t n, int32_t d,
                       int32_t zeta) {
    if (m == 0) return 0;
    size_t need = fallback_ws_bytes(di, f16, m, n, d, zeta);
    const size_t fused = fused_ws_bytes(di, f16, m, n, d, zeta);
    if (fused > need) need = fused;
    // the owner kernel's plan (its load width follows lda and the alignment)
    for (int a = 4; a <= 16; a *= 2)
        for (int64_t lda = n; lda <= n + 1; ++lda) {
            sk::FusedPlan fp{};
            if (sk::plan_owner(di, f16, m, n, lda, a, d, zeta, &fp) && fp.ws_bytes > need)
                need = fp.ws_bytes;
        }
    return need;
}

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
uint32_t *scratch_dev[kMaxScratchDevices];     // guarded by scratch_mu

// The device address of `scratch` on the current device.
sk_status static_scratch(uint32_t **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SK_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return SK_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return SK_ERR_HIP;
        scratch_dev[dev] = static_cast<uint32_t *>(p);
    }
    *out = scratch_dev[dev];
    return SK_OK;
}

// use_static: the partials go to the device's static scratch (no
// workspace argument; only shapes the fused kernel covers within
// kStaticScratchBytes).
sk_status sketch_dispatch(bool f16, uint64_t seed, int64_t row_offset, const float *A, int64_t m,
                          int32_t n, int64_t lda, int32_t d, int32_t zeta, void *B,
                          int64_t ldb, uint32_t flags, void *workspace, size_t workspace_bytes,
                          hipStream_t s, bool use_static = false) {
    const size_t belem = f16 ? 2 : 4;
    if (m < 0 || row_offset < 0 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0)
        return SK_ERR_SHAPE;
    if (lda < n || ldb < n) return SK_ERR_SHAPE;
    if (m > (INT64_MAX / 8) / (zeta > lda ? zeta : lda)) return SK_ERR_SHAPE;
    if (f16 && n % 2 != 0) return SK_ERR_SHAPE;
    if (flags & ~(SK_ACCUMULATE | (f16 ? SK_COMBINE_F32 : 0u))) return SK_ERR_ARG;
    if (B == nullptr) return SK_ERR_NULL;
    if (f16 && (ldb % 2 != 0 || (uintptr_t)B % 4 != 0)) return SK_ERR_ALIGN;
    const size_t bspan = span_bytes(d, n, ldb, belem);
    const bool accumulate = (flags & SK_ACCUMULATE) != 0;
    const int mode = (accumulate ? sk::kReduceModeAccumulate : 0) |
                     ((flags & SK_COMBINE_F32) ? sk::kReduceModeCombineF32 : 0);
    if (m > 0) {
        if (A == nullptr || (!use_static && workspace == nullptr)) return SK_ERR_NULL;
        if (f16 && (lda % 2 != 0 || (uintptr_t)A % 8 != 0)) return SK_ERR_ALIGN;
        const size_t aspan = span_bytes(m, n, lda, 4);
        if (overlaps(A, aspan, B, bspan)) return SK_ERR_ARG;
        if (!use_static) {
            if ((uintptr_t)workspace % 16 != 0) return SK_ERR_ALIGN;
            if (overlaps(workspace, workspace_bytes, A, aspan) ||
                overlaps(workspace, workspace_bytes, B, bspan))
                return SK_ERR_ARG;
        }
    }
    sk::DevInfo di;
    if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
    if (m == 0) {
        if (accumulate) return SK_OK;
        const hipError_t e =
            f16 ? sk::launch_zero_words(static_cast<uint32_t *>(B), d, n / 2, ldb / 2, s)
                : sk::launch_zero_words(static_cast<uint32_t *>(B), d, n, ldb, s);
        return hip_status(e);
    }
    const float scale = scale_of(zeta);
    sk::FusedPlan fp{};
    if (use_static) {
        if (!sk::plan_sketch(di, f16, m, n, lda, base_align(A), d, zeta, &fp) ||
            fp.ws_bytes > kStaticScratchBytes)
            return SK_ERR_UNSUPPORTED;
        uint32_t *ws = nullptr;
        const sk_status st = static_scratch(&ws);
        if (st != SK_OK) return st;
        return hip_status(sk::launch_sketch(fp, f16, A, m, n, lda, seed, row_offset, d, zeta,
                                            scale, B, ldb, ws, mode, s));
    }
    if (workspace_bytes < sketch_ws_bytes(di, f16, m, n, d, zeta)) return SK_ERR_ARG;
    if (sk::plan_sketch(di, f16, m, n, lda, base_align(A), d, zeta, &fp))
        return hip_status(sk::launch_sketch(fp, f16, A, m, n, lda, seed, row_offset, d, zeta,
                                            scale, B, ldb, static_cast<uint32_t *>(workspace),
                                            mode, s));
    // not covered by the fused kernel: metadata into the workspace, then
    // the LDS (or flat) apply with the rest of it
    char *w = static_cast<char *>(workspace);
    const size_t meta = align256((size_t)m * (size_t)zeta * 4);
    int32_t *ri = reinterpret_cast<int32_t *>(w);
    float *v = reinterpret_cast<float *>(w + meta);
    hipError_t e = sk::launch_meta(seed, row_offset, m, d, zeta, scale, ri, v, s);
    if (e != hipSuccess) return SK_ERR_HIP;
    return apply_dispatch(f16, A, m, n, lda, ri, v, zeta, B, d, ldb,
                          flags & (SK_ACCUMULATE | SK_COMBINE_F32), w + 2 * meta,
                          workspace_bytes - 2 * meta, s);
}

// BlockPerm launch plan: the register kernel where its shape rules hold;
// else the component kernel (shift wiring: a workgroup per component,
// column tile and 64 output rows, no workspace) where its workgroups fill
// the device; else the slice kernel with Qs row slices; else the component
// kernel.  The register and slice kernels take a workspace of
// Q*kappa*d*n floats for their own Q; where the register kernel is planned
// the slice kernel stays the fallback for an unaligned A, so the workspace
// covers both.
struct BpPlan {
    int kernel;                 // SK_BLOCKPERM_KERNEL_*
    bool comp_ok;               // the component kernel applies (NULL workspace)
    sk::BpDirectPlan direct;    // its plan
    bool slice_ok;
    int32_t Qs;                 // slice kernel: row slices, rows per slice
    int64_t rps_s;
    size_t ws_s;
    sk::BpRegsPlan regs;        // register kernel (kernel == REGISTER)
    size_t ws_bytes;
    uint32_t a, ainv, b;        // affine wiring parameters
};

uint32_t gcd_u32(uint32_t x, uint32_t y) {
    while (y) {
        const uint32_t t = x % y;
        x = y;
        y = t;
    }
    return x;
}

// f(x) = (a x + b) mod M, a full cycle (Hull-Dobell), drawn from the seed:
// L = product of M's distinct primes (times 2 more when 4 | M and L is not
// already a multiple of 4), a = 1 + L*mulhi(w0, M/L) (1 when L >= M), b = the
// mulhi(w1, phi(M))-th unit below M; (w0, w1) = Philox(0, 0, 0, 1).
void affine_params(uint64_t seed, int32_t M, uint32_t *a, uint32_t *b, uint32_t *ainv) {
    if (M <= 1) {
        *a = 1;
        *b = 0;
        *ainv = 1;
        return;
    }
    const sk::u32x4 w = sk::philox4x32_10(sk::u32x4{0u, 0u, 0u, 1u}, (uint32_t)seed,
                                          (uint32_t)(seed >> 32));
    uint32_t L = 1, x = (uint32_t)M;
    for (uint32_t p = 2; p * p <= x; ++p) {
        if (x % p == 0) {
            L *= p;
            while (x % p == 0) x /= p;
        }
    }
    if (x > 1) L *= x;
    if (M % 4 == 0 && L % 4 != 0) L *= 2;
    *a = L < (uint32_t)M ? 1u + L * sk::mulhi32(w.x, (uint32_t)M / L) : 1u;
    uint32_t phi = 0;
    for (uint32_t u = 1; u < (uint32_t)M; ++u) phi += gcd_u32(u, (uint32_t)M) == 1;
    const uint32_t k = sk::mulhi32(w.y, phi);
    uint32_t seen = 0;
    *b = 1;
    for (uint32_t u = 1; u < (uint32_t)M; ++u) {
        if (gcd_u32(u, (uint32_t)M) != 1) continue;
        if (seen++ == k) {
            *b = u;
            break;
        }
    }
    *ainv = 1;
    for (uint32_t v = 1; v < (uint32_t)M; ++v)
        if ((uint64_t)*a * v % (uint32_t)M == 1) {
            *ainv = v;
            break;
        }
}

// Validation shared by the BlockPerm entry points.
sk_status check_blockperm(int64_t m, int32_t n, int64_t lda, int32_t d, int32_t M, int32_t kappa,
                          int32_t s, int32_t wiring, int64_t ldy) {
    if (m < 1 || n < 1 || d < 1 || M < 1 || kappa < 1 || s < 1) return SK_ERR_SHAPE;
    if (wiring != SK_WIRING_SHIFT && wiring != SK_WIRING_AFFINE) return SK_ERR_ARG;
    if (M > sk::kBlockPermMaxM) return SK_ERR_UNSUPPORTED;
    if (m % M != 0 || d % M != 0 || lda < n || ldy < n) return SK_ERR_SHAPE;
    if (wiring == SK_WIRING_SHIFT && M % kappa != 0) return SK_ERR_SHAPE;
    if (kappa > M) return SK_ERR_SHAPE;
    const int32_t Br = d / M;
    if (s > Br) return SK_ERR_SHAPE;
    if (m > INT64_MAX / 8 / lda) return SK_ERR_SHAPE;
    if (s > 1 && (Br & (Br - 1)) != 0) return SK_ERR_UNSUPPORTED;
    if (s > 32 || kappa > sk::kBlockPermGenMaxKappa) return SK_ERR_UNSUPPORTED;
    return SK_OK;
}

bool plan_blockperm(const sk::DevInfo &di, int64_t m, int32_t n, int32_t d, int32_t M,
                    int32_t kappa, int32_t s, int32_t wiring, uint64_t seed, BpPlan *p) {
    const int32_t Br = d / M;
    const int64_t Bc = m / M;
    const int64_t tiles = (n + 31) / 32;
    memset(p, 0, sizeof(*p));
    p->comp_ok = wiring == SK_WIRING_SHIFT && sk::plan_bp_direct(m, n, d, M, kappa, s, &p->direct);
    p->slice_ok = (int64_t)kappa * Br <= sk::blockperm_general_max_rows(di);
    if (p->slice_ok) {
        int64_t Q = (2 * (int64_t)di.num_cu + tiles * M - 1) / (tiles * M);
        const int64_t qmax = Bc / 64 > 1 ? Bc / 64 : 1;
        if (Q > qmax) Q = qmax;
        if (Q < 1) Q = 1;
        if (Q * M > 65535) Q = 65535 / M;
        p->Qs = (int32_t)Q;
        p->rps_s = (Bc + Q - 1) / Q;
        p->ws_s = (size_t)Q * (size_t)kappa * (size_t)d * (size_t)n * 4;
    }
    if (sk::plan_bp_regs(di, m, n, d, M, kappa, s, &p->regs)) {
        p->kernel = SK_BLOCKPERM_KERNEL_REGISTER;
        p->ws_bytes = p->regs.ws_bytes > p->ws_s ? p->regs.ws_bytes : p->ws_s;
    } else if (p->comp_ok && p->direct.grid >= di.num_cu) {
        p->kernel = SK_BLOCKPERM_KERNEL_COMPONENT;
    } else if (p->slice_ok) {
        p->kernel = SK_BLOCKPERM_KERNEL_SLICE;
        p->ws_bytes = p->ws_s;
    } else if (p->comp_ok) {
        p->kernel = SK_BLOCKPERM_KERNEL_COMPONENT;
    } else {
        return false;
    }
    if (wiring == SK_WIRING_AFFINE) affine_params(seed, M, &p->a, &p->b, &p->ainv);
    return true;
}

void sigma_table(uint64_t seed, int32_t M, uint16_t *sigma) {
    for (int k = 0; k < M; ++k) sigma[k] = (uint16_t)k;
    for (int k = M - 1; k >= 1; --k) {
        const sk::u32x4 w = sk::philox4x32_10(sk::u32x4{(uint32_t)k, 0u, 0u, 2u}, (uint32_t)seed,
                                              (uint32_t)(seed >> 32));
        const uint32_t j = sk::mulhi32(w.x, (uint32_t)(k + 1));
        const uint16_t t = sigma[k];
        sigma[k] = sigma[j];
        sigma[j] = t;
    }
}

// The component kernel (no workspace) for the shift wiring; arguments
// already validated.
sk_status run_direct(const float *A, int64_t m, int32_t n, int64_t lda, int32_t d, int32_t M,
                     int32_t kappa, int32_t s, uint64_t seed, float *Y, int64_t ldy,
                     uint32_t flags, hipStream_t stream) {
    sk::BpDirectPlan plan{};
    if (!sk::plan_bp_direct(m, n, d, M, kappa, s, &plan)) return SK_ERR_UNSUPPORTED;
    sk::BpDirectArgs args;
    memset(&args, 0, sizeof(args));
    args.A = A;
    args.Y = Y;
    args.lda = lda;
    args.ldy = ldy;
    args.Bc = m / M;
    args.n = n;
    args.Br = d / M;
    args.M = M;
    args.kappa = kappa;
    args.s = s;
    args.C = M / kappa;
    args.tiles = plan.tiles;
    args.groups = plan.groups;
    args.accumulate = (flags & SK_ACCUMULATE) ? 1 : 0;
    args.scale = scale_of((int64_t)kappa * s);
    args.seed = seed;
    sk::BlockPermTable fwd, ginv;
    memset(&ginv, 0, sizeof(ginv));
    sigma_table(seed, M, fwd.tab);
    for (int k = 0; k < M; ++k) ginv.tab[fwd.tab[k]] = (uint16_t)k;
    return hip_status(sk::launch_bp_direct(plan, args, ginv, stream));
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

sk_status sk_apply_f32_ws(const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, float *B,
                          int32_t d, int64_t ldb, uint32_t flags, void *workspace,
                          size_t workspace_bytes, void *stream) {
    sk_status st = check_apply(A, m, n, lda, row_idx, val, zeta, B, 4, d, ldb, flags, 0u);
    if (st != SK_OK) return st;
    st = check_workspace(workspace, workspace_bytes, A, m, n, lda, row_idx, val, zeta, B,
                         span_bytes(d, n, ldb, 4));
    if (st != SK_OK) return st;
    return apply_dispatch(false, A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags, workspace,
                          workspace_bytes, (hipStream_t)stream);
}

sk_status sk_apply_f32(const float *A, int64_t m, int32_t n, int64_t lda, const int32_t *row_idx,
                       const float *val, int32_t zeta, float *B, int32_t d, int64_t ldb,
                       uint32_t flags, void *stream) {
    return sk_apply_f32_ws(A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags, nullptr, 0, stream);
}

sk_status sk_apply_f16acc_ws(const float *A, int64_t m, int32_t n, int64_t lda,
                             const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                             int32_t d, int64_t ldb, uint32_t flags, void *workspace,
                             size_t workspace_bytes, void *stream) {
    sk_status st = check_apply(A, m, n, lda, row_idx, val, zeta, B, 2, d, ldb, flags,
                               SK_COMBINE_F32);
    if (st != SK_OK) return st;
    if (n % 2 != 0) return SK_ERR_SHAPE;
    if (ldb % 2 != 0 || (uintptr_t)B % 4 != 0) return SK_ERR_ALIGN;
    if (m > 0 && (lda % 2 != 0 || (uintptr_t)A % 8 != 0)) return SK_ERR_ALIGN;
    st = check_workspace(workspace, workspace_bytes, A, m, n, lda, row_idx, val, zeta, B,
                         span_bytes(d, n, ldb, 2));
    if (st != SK_OK) return st;
    return apply_dispatch(true, A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags, workspace,
                          workspace_bytes, (hipStream_t)stream);
}

sk_status sk_apply_f16acc(const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                          int32_t d, int64_t ldb, uint32_t flags, void *stream) {
    if (flags & SK_COMBINE_F32) return SK_ERR_ARG;
    return sk_apply_f16acc_ws(A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags, nullptr, 0,
                              stream);
}

sk_status sk_apply_workspace_size(int32_t precision, int64_t m, int32_t n, int32_t d,
                                  int32_t zeta, uint32_t flags, size_t *bytes) {
    if (bytes == nullptr) return SK_ERR_NULL;
    *bytes = 0;
    if (precision != SK_PRECISION_F32 && precision != SK_PRECISION_F16ACC &&
        precision != SK_PRECISION_LOWP)
        return SK_ERR_ARG;
    if (m < 0 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0) return SK_ERR_SHAPE;
    if (precision != SK_PRECISION_F32 && n % 2 != 0) return SK_ERR_SHAPE;
    if (precision == SK_PRECISION_LOWP) {
        // sk_apply_lowp with SK_VARIANT_REG; no workspace otherwise
        if (flags & ~(SK_ACCUMULATE | SK_VARIANT_FLAT | SK_VARIANT_REG | SK_COMBINE_F32))
            return SK_ERR_ARG;
        if (m == 0 || !(flags & SK_VARIANT_REG)) return SK_OK;
        sk::DevInfo di;
        if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
        sk::LowpRegPlan lp{};
        if (sk::plan_lowp_reg(di, m, n, d, zeta, &lp)) *bytes = lp.ws_bytes;
        return SK_OK;
    }
    const uint32_t extra = precision == SK_PRECISION_F16ACC ? SK_COMBINE_F32 : 0u;
    if (flags & ~(SK_ACCUMULATE | SK_VARIANT_FLAT | SK_VARIANT_LDS | SK_VARIANT_REG | extra))
        return SK_ERR_ARG;
    if (variant_count(flags) > 1) return SK_ERR_ARG;
    if (m == 0 || (flags & SK_VARIANT_FLAT)) return SK_OK;
    sk::DevInfo di;
    if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
    const bool f16 = precision == SK_PRECISION_F16ACC;
    size_t best = 0;
    // the register plans (lda = n, either alignment): SK_VARIANT_REG, and
    // the default, which takes it where it covers the shape
    if (!(flags & SK_VARIANT_LDS)) {
        if (zeta <= sk::kFusedMetaMaxZeta) best = fused_ws_bytes(di, f16, m, n, d, zeta);
        if (flags & SK_VARIANT_REG) {
            *bytes = best;
            return SK_OK;
        }
    }
    // the LDS plans a call may take (a two-word plan needs no more
    // workspace than the one-word plan)
    sk::LdsPlan plan{};
    const int64_t units = f16 ? n / 2 : n;
    const int gw = f16 ? 1 : 2;
    if (sk::plan_lds(di, m, units, true, gw, d, zeta, &plan) && plan.ws_bytes > best)
        best = plan.ws_bytes;
    if (sk::plan_lds(di, m, units, false, gw, d, zeta, &plan) && plan.ws_bytes > best)
        best = plan.ws_bytes;
    *bytes = best;
    return SK_OK;
}

sk_status sk_lds_plan_describe(int32_t precision, int64_t m, int32_t n, int64_t lda, int32_t d,
                               int32_t zeta, int32_t wide_ok, int32_t num_cu, int32_t max_lds,
                               int64_t *out) {
    if (out == nullptr) return SK_ERR_NULL;
    for (int i = 0; i < SK_PLAN_FIELDS; ++i) out[i] = 0;
    if (precision != SK_PRECISION_F32 && precision != SK_PRECISION_F16ACC) return SK_ERR_ARG;
    if (m < 1 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0 || lda < n)
        return SK_ERR_SHAPE;
    if (precision == SK_PRECISION_F16ACC && n % 2 != 0) return SK_ERR_SHAPE;
    if (num_cu < 1 || max_lds < 1) return SK_ERR_ARG;
    const bool f16 = precision == SK_PRECISION_F16ACC;
    const int64_t vec = f16 ? 4 : 2;
    sk::DevInfo di{num_cu, max_lds};
    sk::LdsPlan p{};
    if (lda > ((int64_t)1 << 24) ||
        !sk::plan_lds(di, m, f16 ? n / 2 : n, wide_ok != 0 && lda % vec == 0, f16 ? 1 : 2, d,
                      zeta, &p))
        return SK_OK;
    const int64_t v[SK_PLAN_FIELDS] = {1, p.words, p.slice, p.groups, p.zg, p.threads,
                                       p.rows_per_chunk, p.chunks, p.slices, p.grid,
                                       (int64_t)p.lds_bytes, (int64_t)p.ws_bytes};
    for (int i = 0; i < SK_PLAN_FIELDS; ++i) out[i] = v[i];
    return SK_OK;
}

sk_status sk_apply_lowp(const float *A, int64_t m, int32_t n, int64_t lda,
                        const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                        int32_t d, int64_t ldb, int32_t format, int32_t convert,
                        uint64_t sr_seed, int64_t row_offset, uint32_t flags, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (format != SK_FORMAT_F16 && format != SK_FORMAT_BF16) return SK_ERR_ARG;
    if (convert != SK_CONVERT_RN && convert != SK_CONVERT_SR) return SK_ERR_ARG;
    if (flags & ~(SK_ACCUMULATE | SK_VARIANT_FLAT | SK_VARIANT_REG | SK_COMBINE_F32))
        return SK_ERR_ARG;
    if ((flags & SK_VARIANT_FLAT) && (flags & SK_VARIANT_REG)) return SK_ERR_ARG;
    if (row_offset < 0) return SK_ERR_SHAPE;
    sk_status st = check_apply(A, m, n, lda, row_idx, val, zeta, B, 2, d, ldb,
                               flags & ~(SK_COMBINE_F32), 0u);
    if (st != SK_OK) return st;
    if (n % 2 != 0) return SK_ERR_SHAPE;
    if (ldb % 2 != 0 || (uintptr_t)B % 4 != 0) return SK_ERR_ALIGN;
    if (m > 0 && (lda % 2 != 0 || (uintptr_t)A % 8 != 0)) return SK_ERR_ALIGN;
    if (format == SK_FORMAT_BF16 && convert == SK_CONVERT_SR) return SK_ERR_UNSUPPORTED;
    const bool reg = (flags & SK_VARIANT_REG) != 0;
    if (!reg && (flags & SK_COMBINE_F32)) return SK_ERR_ARG;     // no reduce to combine in
    hipStream_t s = (hipStream_t)stream;
    const bool accumulate = (flags & SK_ACCUMULATE) != 0;
    if (reg) {
        if (m == 0) {
            if (accumulate) return SK_OK;
            return hip_status(
                sk::launch_zero_words(reinterpret_cast<uint32_t *>(B), d, n / 2, ldb / 2, s));
        }
        if (workspace == nullptr) return SK_ERR_NULL;
        if ((uintptr_t)workspace % 16 != 0) return SK_ERR_ALIGN;
        st = check_workspace(workspace, workspace_bytes, A, m, n, lda, row_idx, val, zeta, B,
                             span_bytes(d, n, ldb, 2));
        if (st != SK_OK) return st;
        sk::DevInfo di;
        if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
        sk::LowpRegPlan lp{};
        if (!sk::plan_lowp_reg(di, m, n, d, zeta, &lp)) return SK_ERR_UNSUPPORTED;
        if (workspace_bytes < lp.ws_bytes) return SK_ERR_ARG;
        const int mode = (accumulate ? sk::kReduceModeAccumulate : 0) |
                         ((flags & SK_COMBINE_F32) ? sk::kReduceModeCombineF32 : 0);
        return hip_status(sk::launch_lowp_reg(lp, A, m, n, lda, row_idx, val, zeta, B, d, ldb,
                                              format == SK_FORMAT_BF16,
                                              convert == SK_CONVERT_SR, sr_seed, row_offset,
                                              static_cast<uint32_t *>(workspace), mode, s));
    }
    if (!accumulate) {
        const hipError_t e =
            sk::launch_zero_words(reinterpret_cast<uint32_t *>(B), d, n / 2, ldb / 2, s);
        if (e != hipSuccess) return SK_ERR_HIP;
    }
    if (m == 0) return SK_OK;
    return hip_status(sk::launch_lowp_flat(A, m, n, lda, row_idx, val, zeta, B, d, ldb,
                                           format == SK_FORMAT_BF16, convert == SK_CONVERT_SR,
                                           sr_seed, row_offset, s));
}

sk_status sk_sketch_f32(uint64_t seed, int64_t row_offset, const float *A, int64_t m, int32_t n,
                        int64_t lda, int32_t d, int32_t zeta, float *B, int64_t ldb,
                        uint32_t flags, void *workspace, size_t workspace_bytes, void *stream) {
    return sketch_dispatch(false, seed, row_offset, A, m, n, lda, d, zeta, B, ldb, flags, workspace,
                           workspace_bytes, (hipStream_t)stream);
}

sk_status sk_sketch_f16acc(uint64_t seed, int64_t row_offset, const float *A, int64_t m,
                           int32_t n, int64_t lda, int32_t d, int32_t zeta, uint16_t *B,
                           int64_t ldb, uint32_t flags, void *workspace, size_t workspace_bytes,
                           void *stream) {
    return sketch_dispatch(true, seed, row_offset, A, m, n, lda, d, zeta, B, ldb, flags, workspace,
                           workspace_bytes, (hipStream_t)stream);
}

sk_status sk_sketch_f16acc_noalloc(uint64_t seed, int64_t row_offset, const float *A, int64_t m,
                                   int32_t n, int64_t lda, int32_t d, int32_t zeta, uint16_t *B,
                                   int64_t ldb, uint32_t flags, void *stream) {
    return sketch_dispatch(true, seed, row_offset, A, m, n, lda, d, zeta, B, ldb, flags, nullptr,
                           0, (hipStream_t)stream, true);
}

sk_status sk_sketch_workspace_size(int32_t precision, int64_t m, int32_t n, int32_t d,
                                   int32_t zeta, size_t *bytes) {
    if (bytes == nullptr) return SK_ERR_NULL;
    *bytes = 0;
    if (precision != SK_PRECISION_F32 && precision != SK_PRECISION_F16ACC) return SK_ERR_ARG;
    if (m < 0 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0) return SK_ERR_SHAPE;
    if (precision == SK_PRECISION_F16ACC && n % 2 != 0) return SK_ERR_SHAPE;
    sk::DevInfo di;
    if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
    *bytes = sketch_ws_bytes(di, precision == SK_PRECISION_F16ACC, m, n, d, zeta);
    return SK_OK;
}

sk_status sk_lstsq_workspace_size(int32_t d, int32_t n, size_t *bytes) {
    if (bytes == nullptr) return SK_ERR_NULL;
    *bytes = 0;
    if (n < 1 || d < n || d > sk::kQrMaxRows) return SK_ERR_SHAPE;
    *bytes = sk::lstsq_workspace_floats(d, n) * sizeof(float);
    return SK_OK;
}

sk_status sk_lstsq_qr_f32(const float *SA, int32_t d, int32_t n, int64_t ld, const float *Sb,
                          float *x, void *workspace, size_t workspace_bytes, void *stream) {
    if (n < 1 || d < n || d > sk::kQrMaxRows || ld < n) return SK_ERR_SHAPE;
    if (SA == nullptr || Sb == nullptr || x == nullptr || workspace == nullptr)
        return SK_ERR_NULL;
    if ((uintptr_t)workspace % 4 != 0) return SK_ERR_ALIGN;
    const size_t need = sk::lstsq_workspace_floats(d, n) * sizeof(float);
    if (workspace_bytes < need) return SK_ERR_ARG;
    const size_t aspan = span_bytes(d, n, ld, 4);
    if (overlaps(workspace, need, SA, aspan) || overlaps(workspace, need, Sb, (size_t)d * 4) ||
        overlaps(workspace, need, x, (size_t)n * 4) || overlaps(x, (size_t)n * 4, SA, aspan) ||
        overlaps(x, (size_t)n * 4, Sb, (size_t)d * 4))
        return SK_ERR_ARG;
    return hip_status(sk::launch_lstsq_qr(SA, d, n, ld, Sb, x, static_cast<float *>(workspace),
                                          (hipStream_t)stream));
}

sk_status sk_fused_plan_describe(int32_t precision, int64_t m, int32_t n, int64_t lda,
                                 int32_t a_align, int32_t d, int32_t zeta, int32_t num_cu,
                                 int32_t max_lds, int64_t *out) {
    if (out == nullptr) return SK_ERR_NULL;
    for (int i = 0; i < SK_FUSED_PLAN_FIELDS; ++i) out[i] = 0;
    if (precision != SK_PRECISION_F32 && precision != SK_PRECISION_F16ACC) return SK_ERR_ARG;
    if (m < 1 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0 || lda < n)
        return SK_ERR_SHAPE;
    if (precision == SK_PRECISION_F16ACC && n % 2 != 0) return SK_ERR_SHAPE;
    if (num_cu < 1 || max_lds < 1) return SK_ERR_ARG;
    sk::DevInfo di{num_cu, max_lds};
    sk::FusedPlan p{};
    if (!sk::plan_fused(di, precision == SK_PRECISION_F16ACC, m, n, lda, a_align, d, zeta, &p))
        return SK_OK;
    const int64_t v[SK_FUSED_PLAN_FIELDS] = {1, p.rows_per_wave, p.groups, p.slices,
                                             p.rows_per_chunk, p.chunks, p.grid,
                                             (int64_t)p.ws_bytes, p.words, p.stage_rows,
                                             p.dual ? 2 : 1};
    for (int i = 0; i < SK_FUSED_PLAN_FIELDS; ++i) out[i] = v[i];
    return SK_OK;
}

sk_status sk_sketch_plan_describe(int32_t precision, int64_t m, int32_t n, int64_t lda,
                                  int32_t a_align, int32_t d, int32_t zeta, int32_t num_cu,
                                  int32_t max_lds, int64_t *out) {
    if (out == nullptr) return SK_ERR_NULL;
    for (int i = 0; i < SK_SKETCH_PLAN_FIELDS; ++i) out[i] = 0;
    if (precision != SK_PRECISION_F32 && precision != SK_PRECISION_F16ACC) return SK_ERR_ARG;
    if (m < 1 || n < 1 || d < 1 || zeta < 1 || zeta > d || d % zeta != 0 || lda < n)
        return SK_ERR_SHAPE;
    if (precision == SK_PRECISION_F16ACC && n % 2 != 0) return SK_ERR_SHAPE;
    if (num_cu < 1 || max_lds < 1) return SK_ERR_ARG;
    sk::DevInfo di{num_cu, max_lds};
    sk::FusedPlan p{};
    if (!sk::plan_sketch(di, precision == SK_PRECISION_F16ACC, m, n, lda, a_align, d, zeta, &p))
        return SK_OK;
    const bool own = p.kind == sk::kFusedOwner;
    const int64_t v[SK_SKETCH_PLAN_FIELDS] = {own ? 2 : 1,
                                              p.words,
                                              own ? p.lanes_per_row : 0,
                                              own ? p.threads : 1024,
                                              own ? p.row_words : 0,
                                              p.stage_rows,
                                              own ? p.cap : 0,
                                              own ? p.load_words : 0,
                                              p.rows_per_chunk,
                                              p.chunks,
                                              p.grid,
                                              (int64_t)p.ws_bytes,
                                              own ? (int64_t)p.lds_bytes : 0,
                                              p.dual ? 2 : 1,
                                              own ? p.mask_stride : 0,
                                              own ? p.list_stride : 0,
                                              own ? p.barriers : 0,
                                              own ? p.load_slots : 0};
    for (int i = 0; i < SK_SKETCH_PLAN_FIELDS; ++i) out[i] = v[i];
    return SK_OK;
}

sk_status sk_apply_blockperm_ex(const float *A, int64_t m, int32_t n, int64_t lda, int32_t d,
                                int32_t M, int32_t kappa, int32_t s, int32_t wiring,
                                uint64_t seed, float *Y, int64_t ldy, uint32_t flags,
                                void *workspace, size_t workspace_bytes, void *stream) {
    sk_status st = check_blockperm(m, n, lda, d, M, kappa, s, wiring, ldy);
    if (st != SK_OK) return st;
    if (flags & ~SK_ACCUMULATE) return SK_ERR_ARG;
    if (A == nullptr || Y == nullptr) return SK_ERR_NULL;
    const size_t aspan = span_bytes(m, n, lda, 4), yspan = span_bytes(d, n, ldy, 4);
    if (overlaps(A, aspan, Y, yspan)) return SK_ERR_ARG;
    sk::DevInfo di;
    if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
    BpPlan p;
    if (!plan_blockperm(di, m, n, d, M, kappa, s, wiring, seed, &p)) return SK_ERR_UNSUPPORTED;
    if (p.kernel == SK_BLOCKPERM_KERNEL_COMPONENT || (workspace == nullptr && p.comp_ok))
        return run_direct(A, m, n, lda, d, M, kappa, s, seed, Y, ldy, flags,
                          (hipStream_t)stream);
    if (workspace == nullptr) return SK_ERR_NULL;
    if ((uintptr_t)workspace % 16 != 0) return SK_ERR_ALIGN;
    if (workspace_bytes < p.ws_bytes) return SK_ERR_ARG;
    if (overlaps(workspace, workspace_bytes, A, aspan) ||
        overlaps(workspace, workspace_bytes, Y, yspan))
        return SK_ERR_ARG;
    const bool regs = p.kernel == SK_BLOCKPERM_KERNEL_REGISTER && lda % 4 == 0 &&
                      (uintptr_t)A % 16 == 0;
    if (!regs && !p.slice_ok) return SK_ERR_ALIGN;
    sk::BlockPermGenArgs g;
    memset(&g, 0, sizeof(g));
    g.A = A;
    g.ws = static_cast<float *>(workspace);
    g.lda = lda;
    g.Bc = m / M;
    g.rows_per_slice = regs ? p.regs.rows_per_slice : p.rps_s;
    g.n = n;
    g.Br = d / M;
    g.M = M;
    g.kappa = kappa;
    g.s = s;
    g.Q = regs ? p.regs.Q : p.Qs;
    g.wiring = wiring;
    g.C = wiring == SK_WIRING_SHIFT ? M / kappa : 0;
    g.a = p.a;
    g.ainv = p.ainv;
    g.b = p.b;
    g.scale = scale_of((int64_t)kappa * s);
    g.seed = seed;
    g.slices = regs ? p.regs.slices : 0;
    g.groups = regs ? p.regs.groups : 0;
    sk::BlockPermTable ginv, fwd;
    memset(&ginv, 0, sizeof(ginv));
    memset(&fwd, 0, sizeof(fwd));
    if (wiring == SK_WIRING_SHIFT) {
        sigma_table(seed, M, fwd.tab);
        for (int k = 0; k < M; ++k) ginv.tab[fwd.tab[k]] = (uint16_t)k;
    }
    const int acc = (flags & SK_ACCUMULATE) ? 1 : 0;
    if (regs)
        return hip_status(sk::launch_bp_regs(p.regs, g, ginv, fwd, Y, ldy, acc,
                                             (hipStream_t)stream));
    return hip_status(sk::launch_blockperm_general(g, ginv, fwd, Y, ldy, acc,
                                                   (hipStream_t)stream));
}

sk_status sk_blockperm_workspace_size(int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa,
                                      int32_t s, int32_t wiring, size_t *bytes) {
    if (bytes == nullptr) return SK_ERR_NULL;
    *bytes = 0;
    sk_status st = check_blockperm(m, n, n, d, M, kappa, s, wiring, n);
    if (st != SK_OK) return st;
    sk::DevInfo di;
    if (sk::dev_info(&di) != hipSuccess) return SK_ERR_HIP;
    BpPlan p;
    if (!plan_blockperm(di, m, n, d, M, kappa, s, wiring, 0, &p)) return SK_ERR_UNSUPPORTED;
    *bytes = p.ws_bytes;
    return SK_OK;
}

sk_status sk_blockperm_plan_describe(int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa,
                                     int32_t s, int32_t wiring, uint64_t seed, int32_t num_cu,
                                     int32_t max_lds, int64_t *out) {
    if (out == nullptr) return SK_ERR_NULL;
    for (int i = 0; i < SK_BLOCKPERM_PLAN_FIELDS; ++i) out[i] = 0;
    sk_status st = check_blockperm(m, n, n, d, M, kappa, s, wiring, n);
    if (st != SK_OK) return st;
    if (num_cu < 1 || max_lds < 1) return SK_ERR_ARG;
    sk::DevInfo di{num_cu, max_lds};
    BpPlan p;
    if (!plan_blockperm(di, m, n, d, M, kappa, s, wiring, seed, &p)) return SK_ERR_UNSUPPORTED;
    const bool regs = p.kernel == SK_BLOCKPERM_KERNEL_REGISTER;
    const bool comp = p.kernel == SK_BLOCKPERM_KERNEL_COMPONENT;
    const int64_t v[SK_BLOCKPERM_PLAN_FIELDS] = {
        p.kernel, regs ? p.regs.Q : (comp ? 0 : p.Qs),
        regs ? p.regs.rows_per_slice : (comp ? 0 : p.rps_s), (int64_t)p.ws_bytes, p.a, p.b,
        p.ainv, regs ? p.regs.rows_per_wave : 0,
        regs ? p.regs.groups : (comp ? p.direct.groups : 0),
        regs ? p.regs.slices : (comp ? p.direct.tiles : 0)};
    for (int i = 0; i < SK_BLOCKPERM_PLAN_FIELDS; ++i) out[i] = v[i];
    return SK_OK;
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
    const int32_t Br = d / M;
    // s rows per block pair come from an odd stride modulo B_r
    if (s > 1 && (Br & (Br - 1)) != 0) return SK_ERR_UNSUPPORTED;
    return run_direct(A, m, n, lda, d, M, kappa, s, seed, Y, ldy, flags, (hipStream_t)stream);
}

}  // extern "C"
