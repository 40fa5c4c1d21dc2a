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
// Reduced-precision flat scatter: FP16 (nearest-even or stochastic
// conversion) or BF16 (nearest-even) contributions, packed global atomics.
hipError_t launch_lowp_flat(const float *A, int64_t m, int32_t n, int64_t lda,
                            const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                            int32_t d, int64_t ldb, bool bf16, bool sr, uint64_t sr_seed,
                            int64_t row_offset, hipStream_t stream);
// Two-level reduced-precision apply (apply_lowp.hip, k_lowp_reg): chunk
// partials in registers (FP16 or BF16 pairs), then the fixed-order reduce.
constexpr int kLowpMaxZeta = 16;
struct LowpRegArgs {
    const float *A;
    const int32_t *row_idx;
    const float *val;
    uint32_t *ws;               // [slices][chunks][d][64] partial words
    int64_t m, lda, rows_per_chunk, row_offset;
    uint64_t sr_seed;
    int32_t npairs, d, zeta, chunks, slices, groups;
};
struct LowpRegPlan {
    int R, groups;              // output rows per wavefront, row groups (16 R G = d)
    int64_t slices;             // 128-column slices
    int64_t rows_per_chunk, chunks, grid;
    size_t ws_bytes;
};
bool plan_lowp_reg(const DevInfo &di, int64_t m, int32_t n, int32_t d, int32_t zeta,
                   LowpRegPlan *p);
// mode: the reduce's kReduceMode* bits (below)
hipError_t launch_lowp_reg(const LowpRegPlan &p, const float *A, int64_t m, int32_t n,
                           int64_t lda, const int32_t *ri, const float *v, int32_t zeta,
                           uint16_t *B, int32_t d, int64_t ldb, bool bf16, bool sr,
                           uint64_t sr_seed, int64_t row_offset, uint32_t *ws, int mode,
                           hipStream_t stream);

// The reduce's mode (bits): kReduceModeAccumulate adds onto B's current
// words (B += ...); kReduceModeCombineF32 (FP16 only) sums the FP16 chunk
// partials in FP32 and rounds the total once, instead of FP16 nearest-even
// additions.
constexpr int kReduceModeAccumulate = 1;
constexpr int kReduceModeCombineF32 = 2;

// LDS-privatized apply.  ws == NULL: the partials are added to B with global
// atomics (B must hold its start value; mode is ignored).  ws != NULL: the
// partials are stored to ws (plan.ws_bytes) and a reduce kernel writes B
// (or adds to it, mode & kReduceModeAccumulate) in chunk order.
hipError_t launch_f32_lds(const LdsPlan &plan, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, float *B,
                          int32_t d, int64_t ldb, uint32_t *ws, int mode,
                          hipStream_t stream);
hipError_t launch_f16_lds(const LdsPlan &plan, const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                          int32_t d, int64_t ldb, uint32_t *ws, int mode,
                          hipStream_t stream);

// Fused SparseStack sketch (metadata drawn in the apply kernel, fused.hip).
constexpr int kFusedMaxZeta = 16;
// with stored metadata (8 rows x zeta entries per wavefront and stage, one
// per lane)
constexpr int kFusedMetaMaxZeta = 8;
// static LDS of the fused kernel (an upper bound over its word widths): two
// stages of 128 rows x 64 lanes x 8 bytes (or 64 rows x 64 lanes x 16
// bytes), two metadata stages of at most kFusedMaxZeta x 128 entries and 16
// per-wave votes
constexpr int kFusedLdsBytes = 2 * 128 * 64 * 8 + 2 * kFusedMaxZeta * 128 * 4 + 16 * 4;
// the two-per-CU shapes (one or two words per lane, 64-row stages)
constexpr int kFusedDualLdsBytes = 2 * 64 * 64 * 8 + 2 * kFusedMaxZeta * 64 * 4 + 16 * 4;
struct FusedArgs {
    const float *A;
    uint32_t *ws;               // [ceil(slices*64*words/128)][chunks][d][128] partial words
    const int32_t *row_idx;     // stored metadata (NULL: drawn in the kernel)
    const float *val;
    int64_t m, lda, rows_per_chunk, row_offset;
    uint64_t seed;
    int32_t n, d, zeta;
    int32_t chunks, slices, groups;
    float scale;                // float32(1/sqrt(zeta))
};
// The two fused kernels: output rows in wavefront registers over column
// slices (fused.hip), or output rows owned by lanes (fused_owner.hip).
constexpr int kFusedRegister = 0;
constexpr int kFusedOwner = 1;
struct FusedPlan {
    int kind;                   // kFusedRegister or kFusedOwner
    int words;                  // W: partial words per lane and output row (1, 2 or 4;
                                // owner kernel: V, 1 to 64)
    int dual;                   // 1: the two-workgroups-per-CU shape
    int stage_rows;             // input rows per LDS stage (128 at W = 2 one per CU,
                                // 64 otherwise)
    int rows_per_wave;          // R: output rows kept in one wavefront's registers
    int groups;                 // G: output row groups (each reads A once)
    int load_sets;              // P: stages of rows in flight in registers (1 or 2)
    int64_t slices;             // column slices of 64 lanes x W words (W = 2: 256 FP16 /
                                // 128 FP32 columns; W = 4: 256 FP32; W = 1: 128 FP16)
    int64_t rows_per_chunk;     // input rows per workgroup (whole stages)
    int64_t chunks;
    int64_t grid;               // workgroups (1-D, XCD-grouped)
    size_t ws_bytes;            // partial workspace
    // owner kernel only
    int threads;                // per workgroup: d x lanes_per_row
    int row_words;              // U: a row's words padded to a power of two
    int lanes_per_row;          // L = U / V
    int cap;                    // hits per output row and stage a list holds
    int mask_stride;            // LDS words between output rows' masks (and counts)
    int list_stride;            // LDS words between output rows' lists
    int load_words;             // words per lane load (1, 2 or 4)
    int barriers;               // workgroup barriers per stage (1 or 2)
    int load_slots;             // loads per thread and stage held in registers (2 or 4)
    size_t lds_bytes;           // dynamic LDS per workgroup
};
// a_align: the alignment of A's base in bytes (16 or more: any lane load;
// the kernel needs 16 for FP16 and for W = 4, 8 for FP32 at W = 2).  A plan
// the alignment does not allow returns false: the fused kernel does not
// cover the call.
bool plan_fused(const DevInfo &di, bool f16, int64_t m, int32_t n, int64_t lda, int a_align,
                int32_t d, int32_t zeta, FusedPlan *plan);
// Fused kernel into ws, then the chunk-order reduce into B (mode: the
// reduce's kReduceMode* bits).  B is float* (FP32) or FP16 bits (uint16_t*), ldb in elements.
// row_idx / val NULL: the metadata is drawn from (seed, row_offset) in the
// kernel; else it is read from them (the stored-metadata apply; seed and
// row_offset unused) and scale must be float32(1/sqrt(zeta)).
// The owner kernel's plan (false: it does not cover the shape) and launch
// (then the reduce, as launch_fused); drawn metadata only.
bool plan_owner(const DevInfo &di, bool f16, int64_t m, int32_t n, int64_t lda, int a_align,
                int32_t d, int32_t zeta, FusedPlan *plan);
hipError_t launch_owner(const FusedPlan &plan, bool f16, const float *A, int64_t m, int32_t n,
                        int64_t lda, uint64_t seed, int64_t row_offset, int32_t d, int32_t zeta,
                        float scale, void *B, int64_t ldb, uint32_t *ws, int mode,
                        hipStream_t stream);
// The plan of the complete fused sketch (metadata drawn in the kernel): the
// owner kernel for narrow rows where it covers the shape, else the register
// kernel; launch_sketch runs either.
bool plan_sketch(const DevInfo &di, bool f16, int64_t m, int32_t n, int64_t lda, int a_align,
                 int32_t d, int32_t zeta, FusedPlan *plan);
hipError_t launch_sketch(const FusedPlan &plan, bool f16, const float *A, int64_t m, int32_t n,
                         int64_t lda, uint64_t seed, int64_t row_offset, int32_t d, int32_t zeta,
                         float scale, void *B, int64_t ldb, uint32_t *ws, int mode,
                         hipStream_t stream);
hipError_t launch_fused(const FusedPlan &plan, bool f16, const float *A, int64_t m, int32_t n,
                        int64_t lda, uint64_t seed, int64_t row_offset, const int32_t *row_idx,
                        const float *val, int32_t d, int32_t zeta, float scale, void *B,
                        int64_t ldb, uint32_t *ws, int mode, hipStream_t stream);

constexpr int kBlockPermMaxM = 1024;

// BlockPerm without a workspace (blockperm_direct.hip): shift wiring, any
// kappa | M, s <= B_r (s > 1: B_r a power of two).  A workgroup per (shift
// component, 32-column tile, group of 64 of the component's kappa*B_r
// output rows) writes those rows of Y once.
struct BpDirectArgs {
    const float *A;
    float *Y;
    int64_t lda, ldy;
    int64_t Bc;                 // input rows per block
    int32_t n, Br, M, kappa, s;
    int32_t C;                  // components = M / kappa
    int32_t tiles, groups;      // column tiles, row groups per component
    int32_t accumulate;
    float scale;                // float32(1/sqrt(kappa*s))
    uint64_t seed;
};
struct BpDirectPlan {
    int32_t tiles, groups;
    int64_t grid;               // components x row groups x column tiles
};
bool plan_bp_direct(int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa, int32_t s,
                    BpDirectPlan *p);

// General BlockPerm (blockperm_general.hip): any kappa <= 32, s <= 32 unique
// rows, shift or affine wiring, input blocks in Q row slices; partial tiles
// to ws, then a fixed-order reduce into Y.
constexpr int kBlockPermGenMaxKappa = 32;
struct BlockPermTable {
    uint16_t tab[kBlockPermMaxM];
};
struct BlockPermGenArgs {
    const float *A;
    float *ws;                  // [M][Q][kappa][B_r][n] partials
    int64_t lda;
    int64_t Bc;                 // input rows per block
    int64_t rows_per_slice;     // rows per slice (the last may be short)
    int32_t n, Br, M, kappa, s, Q;
    int32_t wiring;             // 0: shift, 1: affine
    int32_t C;                  // shift: M / kappa
    uint32_t a, ainv, b;        // affine: f(x) = (a x + b) mod M, a^-1 mod M
    float scale;                // float32(1/sqrt(kappa*s))
    uint64_t seed;
    int32_t slices, groups;     // register kernel: column slices, row groups
};
int blockperm_general_max_rows(const DevInfo &di);
// ginv: shift wiring's sigma^-1 (readers); fwd: its sigma (neighbours).
hipError_t launch_blockperm_general(const BlockPermGenArgs &args, const BlockPermTable &ginv,
                                    const BlockPermTable &fwd, float *Y, int64_t ldy,
                                    int accumulate, hipStream_t stream);
// sigma^-1 of the shift wiring in ginv
hipError_t launch_bp_direct(const BpDirectPlan &p, const BpDirectArgs &args,
                            const BlockPermTable &ginv, hipStream_t stream);
// Y (=|+=) the fixed-order sum of the [M][Q][kappa][B_r][n] partials.
hipError_t launch_bp_reduce(const BlockPermGenArgs &args, const BlockPermTable &fwd, float *Y,
                            int64_t ldy, int accumulate, hipStream_t stream);

// Register BlockPerm apply (blockperm_regs.hip): a workgroup per (input
// block, row slice, 256-column slice, row group) keeps its share of the
// kappa*B_r partial rows in registers, rows streaming through LDS stages.
constexpr int kBpRegsCols = 256;            // columns per slice (64 lanes x 4)
constexpr int kBpRegsStage = 64;            // input rows per LDS stage
constexpr int kBpRegsLdsBytes = 2 * kBpRegsStage * kBpRegsCols * 4 +
                                2 * kBlockPermGenMaxKappa * kBpRegsStage * 4 +
                                kBlockPermGenMaxKappa * 4;
struct BpRegsPlan {
    int32_t rows_per_wave;      // R: partial rows a wavefront keeps
    int32_t groups;             // G: row groups (16 R G = kappa B_r)
    int32_t slices;             // column slices of 256
    int32_t Q;                  // row slices per input block
    int64_t rows_per_slice;     // a multiple of the stage (the last may be short)
    int64_t grid;               // workgroups
    size_t ws_bytes;            // partials: Q kappa d n floats
};
// Shape eligibility and plan; A must also have lda % 4 == 0 and a 16-byte
// aligned base (checked by the caller).
bool plan_bp_regs(const DevInfo &di, int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa,
                  int32_t s, BpRegsPlan *p);
hipError_t launch_bp_regs(const BpRegsPlan &p, const BlockPermGenArgs &args,
                          const BlockPermTable &ginv, const BlockPermTable &fwd, float *Y,
                          int64_t ldy, int accumulate, hipStream_t stream);

// Least squares on a small sketch (lstsq.hip): x = argmin ||SA x - Sb||_2 by
// an FP32 blocked Householder QR.  SA is d x n row-major (row stride ld),
// 1 <= n <= d <= kQrMaxRows; W is a workspace of lstsq_workspace_floats(d, n)
// floats.
constexpr int kQrMaxRows = 2048;
size_t lstsq_workspace_floats(int32_t d, int32_t n);
hipError_t launch_lstsq_qr(const float *SA, int32_t d, int32_t n, int64_t ld, const float *Sb,
                           float *x, float *W, hipStream_t stream);

}  // namespace sk
