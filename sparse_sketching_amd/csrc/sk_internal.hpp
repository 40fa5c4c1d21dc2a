// Internal launch interface of libsksketch: the C ABI in capi.hip validates
// arguments and picks variants; the per-family .hip files own the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

// Per-device facts the dispatch needs (queried once per device).
struct DevInfo {
    int num_cu;         // compute units
    int max_lds;        // bytes of LDS one workgroup may allocate
};
hipError_t dev_info(DevInfo *out);

// B[r, 0:words) = 0 for r < rows, rows ld_words apart (32-bit words).
hipError_t launch_zero_words(uint32_t *B, int64_t rows, int64_t words, int64_t ld_words,
                             hipStream_t stream);

hipError_t launch_meta(uint64_t seed, int64_t row_offset, int64_t m, int32_t d, int32_t zeta,
                       float scale, int32_t *row_idx, float *val, hipStream_t stream);

// Shape of an LDS-privatized SparseStack launch (k_stack_apply).
struct LdsPlan {
    int words;              // 32-bit words per lane (1, or 2 as one 64-bit word)
    int slice;              // lanes per column slice
    int groups;             // block groups: each row is read once per group
    int zg;                 // stack blocks per group
    int threads;            // workgroup size
    int64_t rows_per_chunk; // input rows per workgroup
    int64_t chunks;         // row chunks
    int64_t slices;         // column slices
    int64_t grid;           // workgroups (1-D, XCD-grouped)
    size_t lds_bytes;       // dynamic LDS per workgroup: partial + dummy rows
    size_t ws_bytes;        // workspace for the store-and-reduce flush
};
// Plan for `units` 32-bit words per row of B (columns, or column pairs for
// FP16).  wide_ok: rows of A allow two-word (8- or 16-byte) lane loads.
// Returns false when no slice fits in LDS, or zeta > 64 (the flat kernel
// runs then).
// max_groups_wide: block groups a two-word plan may use (each group reads
// every row of A once more through L2).
bool plan_lds(const DevInfo &di, int64_t m, int64_t units, bool wide_ok, int max_groups_wide,
              int32_t d, int32_t zeta, LdsPlan *plan);

hipError_t launch_f32_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                           const int32_t *row_idx, const float *val, int32_t zeta, float *B,
                           int32_t d, int64_t ldb, hipStream_t stream);
hipError_t launch_f16_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                           const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                           int32_t d, int64_t ldb, hipStream_t stream);
// LDS-privatized apply.  ws == NULL: the partials are added to B with global
// atomics (B must hold its start value).  ws != NULL: the partials are
// stored to ws (plan.ws_bytes) and a reduce kernel writes B (accumulate=0)
// or adds to it (accumulate=1) in chunk order.
hipError_t launch_f32_lds(const LdsPlan &plan, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, float *B,
                          int32_t d, int64_t ldb, uint32_t *ws, int accumulate,
                          hipStream_t stream);
hipError_t launch_f16_lds(const LdsPlan &plan, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                          int32_t d, int64_t ldb, uint32_t *ws, int accumulate,
                          hipStream_t stream);

constexpr int kBlockPermMaxM = 1024;
struct BlockPermArgs {
    const float *A;
    float *Y;
    int64_t lda, ldy;
    int64_t Bc;             // input rows per block
    int32_t n, Br;          // columns, output rows per block
    int32_t C;              // components = M / kappa
    int32_t accumulate;
    float scale;            // float32(1/sqrt(kappa*s))
    uint32_t pad_;
    uint64_t seed;
    uint16_t ginv[kBlockPermMaxM];  // sigma^{-1}
};
// Largest kappa*B_r the LDS tile allows.
int blockperm_max_rows(const DevInfo &di);
hipError_t launch_blockperm(const BlockPermArgs &args, int32_t kappa, hipStream_t stream);

}  // namespace sk
