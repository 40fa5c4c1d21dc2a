/*
 * sk.h: C ABI of the MI355X (gfx950) sparse-sketching library libsksketch.so.
 *
 * The library forms the sketch B = S A of a tall FP32 matrix A (m x n,
 * m >> n) for a sparse oblivious subspace embedding S (d x m):
 *
 *   - SparseStack: every input row is spread over zeta independent
 *     CountSketch blocks of d/zeta output rows each, with one signed nonzero
 *     of magnitude 1/sqrt(zeta) per block; zeta = 1 is CountSketch.
 *     ("On the Robustness of Sparse Randomized Sketching to FP16 Rounding
 *     on GPUs", §I, §II-A, §III-A, §IV-A.)
 *   - BlockPerm-SJLT: M x M blocks wired by a union of kappa edge-disjoint
 *     permutations, with a CountSketch-like hash inside each wired block.
 *     ("FlashSketch: Sketch-Kernel Co-Design for Fast Sparse Sketching on
 *     GPUs", §4, §5, App. D.)
 *
 * Conventions shared by every entry point:
 *   - Matrices are row-major.  A has leading dimension lda (elements) >= n,
 *     B has leading dimension ldb (elements) >= n.
 *   - Every pointer to matrix or metadata storage is a DEVICE pointer on the
 *     current HIP device.  The caller owns all memory; the library never
 *     allocates, frees or keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream and returns without
 *     synchronizing the host.
 *   - Arguments are validated before any HIP call; on failure nothing is
 *     enqueued and a non-zero sk_status is returned.  A failed launch
 *     returns SK_ERR_HIP.  Faults of enqueued work surface at the caller's
 *     next synchronization, as for any HIP kernel.
 *   - m = 0 is a valid empty input: B is zeroed (or left as is with
 *     SK_ACCUMULATE) and A / metadata pointers may then be NULL.
 *   - Output semantics: B = S A by default (the call zeroes B on the stream
 *     first, and that zeroing is part of the complete sketch time, FP16
 *     sketching page §V-A); with SK_ACCUMULATE it computes B += S A, so a
 *     matrix can be sketched in row chunks (see sk_meta_generate).
 *   - A and B must not overlap (SK_ERR_ARG).
 *   - Calls are reentrant.  The library keeps two kinds of state across
 *     calls: a per-device cache of device properties (compute-unit count
 *     and LDS size, filled on first use and read-only afterwards), and the
 *     per-device static scratch of sk_sketch_f16acc_noalloc (calls of it
 *     that overlap on one device race on that scratch).
 */
#ifndef SK_SKETCH_H
#define SK_SKETCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sk_status {
    SK_OK = 0,
    SK_ERR_NULL = 1,        /* a required pointer is NULL */
    SK_ERR_SHAPE = 2,       /* sizes or leading dimensions are inconsistent */
    SK_ERR_ALIGN = 3,       /* a buffer or stride breaks an alignment rule */
    SK_ERR_UNSUPPORTED = 4, /* a valid request this library does not build */
    SK_ERR_HIP = 5,         /* the HIP runtime reported an error */
    SK_ERR_ARG = 6          /* invalid flags, aliasing, or other argument */
} sk_status;

/* flags for the apply calls */
#define SK_ACCUMULATE   1u  /* B += S A instead of B = S A */
#define SK_VARIANT_FLAT 2u  /* one global atomic per contribution */
#define SK_VARIANT_LDS  4u  /* LDS-privatized partial sketches */
#define SK_VARIANT_REG  8u  /* partial sketches in registers, fixed order of
                               additions (reproducible) */
#define SK_COMBINE_F32 16u  /* FP16 output with a workspace: add the FP16
                               row-chunk partials in FP32 and round the total
                               to FP16 once (default: FP16 nearest-even
                               additions, as for every other contribution) */

/* wiring argument of sk_apply_blockperm_ex */
#define SK_WIRING_SHIFT  0
#define SK_WIRING_AFFINE 1

/* BlockPerm kernels, as sk_blockperm_plan_describe reports them */
#define SK_BLOCKPERM_KERNEL_COMPONENT 0  /* per component and column tile, no workspace */
#define SK_BLOCKPERM_KERNEL_SLICE     1  /* LDS tiles per (input block, row slice) */
#define SK_BLOCKPERM_KERNEL_REGISTER  2  /* partial rows in registers */

/* format and convert arguments of sk_apply_lowp */
#define SK_FORMAT_F16  0
#define SK_FORMAT_BF16 1
#define SK_CONVERT_RN  0
#define SK_CONVERT_SR  1

/* precision argument of sk_apply_workspace_size and sk_sketch_workspace_size */
#define SK_PRECISION_F32    0
#define SK_PRECISION_F16ACC 1
#define SK_PRECISION_LOWP   2   /* sk_apply_workspace_size: sk_apply_lowp */

/*
 * sk_meta_generate: routing and sign metadata of a SparseStack sketch.
 * (FP16 sketching page §III-C: the metadata is made once per sketch by a
 * coupled Philox kernel and stored as contiguous int32 and FP32 arrays of
 * length m*zeta; every apply kernel consumes it.)
 *
 * For global row g = row_offset + i (0 <= i < m) and stack block
 * t (0 <= t < zeta), let (w0, w1, w2, w3) = Philox-4x32-10 (Salmon et al.,
 * SC'11) of counter (g mod 2^32, g >> 32, t div 4, 0) and key
 * (seed mod 2^32, seed >> 32), and w = w_{t mod 4}.  Then
 *     row_idx[i*zeta + t] = t*(d/zeta) + floor(w * (d/zeta) / 2^32)
 *     val[i*zeta + t]     = (w & 1 ? -1 : +1) * float32(1/sqrt(zeta))
 * The counter is the GLOBAL row, so metadata for rows [r0, r0+m) equals
 * the slice of the whole matrix's metadata: a matrix sketched chunk by
 * chunk with SK_ACCUMULATE gives the same S as in one call.
 *
 *   seed       64-bit sketch seed.
 *   row_offset first global row (>= 0).
 *   m          rows (>= 0), d output rows (>= 1), 1 <= zeta <= d, d % zeta == 0.
 *   row_idx    device int32[m*zeta] (written).
 *   val        device float[m*zeta] (written).
 * Errors: SK_ERR_SHAPE on bad sizes, SK_ERR_NULL on NULL outputs with m > 0.
 */
sk_status sk_meta_generate(uint64_t seed, int64_t row_offset, int64_t m, int32_t d,
                           int32_t zeta, int32_t *row_idx, float *val, void *stream);

/*
 * sk_apply_f32: B = S A (or B += S A) in FP32 from the metadata above.
 * (FP16 sketching page §III-A: every input row contributes a*val to zeta
 * output rows; A is read once and reused over the zeta loop.)
 *
 *   A        device float, m x n, lda >= n.
 *   row_idx, val  device metadata of length m*zeta (sk_meta_generate's
 *            layout).  Entry i*zeta+t belongs to stack block t: it
 *            contributes only if row_idx lies in that block's rows
 *            [t*d/zeta, (t+1)*d/zeta); any other entry (outside [0, d), or in
 *            another block) contributes nothing.
 *   B        device float, d x n, ldb >= n.
 *   flags    SK_ACCUMULATE, and at most one of
 *              SK_VARIANT_FLAT: one no-return global FP32 atomic add per
 *                contribution (the page's scatter; the in-house baseline);
 *              SK_VARIANT_LDS: each workgroup keeps a private FP32 partial
 *                of a column slice (and a group of stack blocks) in LDS,
 *                updated by read, add and integer compare-and-swap, and
 *                adds it once to B with global atomics (B is zeroed first
 *                unless SK_ACCUMULATE).
 *            0 picks LDS when the partial fits in LDS and zeta <= 64, else
 *            FLAT.  The call allocates nothing and takes no workspace;
 *            sk_apply_f32_ws adds the workspace-based variants.
 * Order of additions: LDS follows which wavefront's compare-and-swap lands
 * first, FLAT the atomics' arrival, so neither is reproducible bit for bit.
 * Errors: SK_ERR_NULL (also SK_VARIANT_REG, which needs the workspace of
 * sk_apply_f32_ws), SK_ERR_SHAPE (n, d < 1, zeta range, d % zeta,
 * lda/ldb < n), SK_ERR_ARG (unknown flags, two variants, aliasing),
 * SK_ERR_UNSUPPORTED (SK_VARIANT_LDS forced where the partial cannot fit in
 * LDS or zeta > 64; SK_VARIANT_REG on a shape it does not cover), SK_ERR_HIP.
 */
sk_status sk_apply_f32(const float *A, int64_t m, int32_t n, int64_t lda,
                       const int32_t *row_idx, const float *val, int32_t zeta,
                       float *B, int32_t d, int64_t ldb, uint32_t flags, void *stream);

/*
 * sk_apply_f16acc: FP16-accumulated sketch.
 * (FP16 sketching page §III-B, §III-C, §III-D: inputs and signed products
 * stay FP32; each contribution is converted to FP16 with round-to-nearest-
 * even, subnormals kept; two adjacent columns are accumulated together by a
 * packed f16x2 addition, each half rounded to nearest-even; the sketch is
 * stored in FP16.)
 *
 *   A        device float, m x n; n even, lda even, A 8-byte aligned.
 *   B        device IEEE binary16 bits (uint16), d x n; ldb even, B 4-byte
 *            aligned.  Overflow gives +-inf, inf + -inf gives NaN.
 *   flags    as for sk_apply_f32.  SK_VARIANT_FLAT is the page's design: one
 *            no-return packed global atomic per contribution pair.
 *            SK_VARIANT_LDS accumulates FP16 partials of row chunks in LDS
 *            (packed f16x2 words, nearest-even additions) and adds them to
 *            B with packed FP16 nearest-even atomics.  Every addition is an
 *            FP16 nearest-even addition.
 * Errors: as sk_apply_f32, plus SK_ERR_SHAPE for odd n, SK_ERR_ALIGN for
 * odd lda/ldb or misaligned A/B, and SK_ERR_ARG for SK_COMBINE_F32 (there
 * is no reduce without a workspace).
 */
sk_status sk_apply_f16acc(const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta,
                          uint16_t *B, int32_t d, int64_t ldb, uint32_t flags, void *stream);

/*
 * sk_apply_f32_ws / sk_apply_f16acc_ws: sk_apply_f32 / sk_apply_f16acc with
 * a caller workspace, which adds the store-and-reduce flush and the register
 * variant (same sketch definition and argument rules as above).
 *
 *   flags    as above, plus
 *              SK_VARIANT_REG: each workgroup streams a chunk of rows (and
 *                their metadata) through LDS and each wavefront keeps its
 *                own output rows' partial in registers; the partials go to
 *                the workspace and a second kernel writes B as their sum.
 *                Needs a workspace, zeta <= 8, d % 16 == 0; FP32 up to 64
 *                columns any rows, wider: n and lda even and A 8-byte
 *                aligned; FP16: A 8-byte aligned, wider than 128 columns
 *                n and lda multiples of 4 and A 16-byte aligned: shapes
 *                sk_fused_plan_describe reports as covered, with zeta <= 8.  Its fast path
 *                assumes |val| = float32(1/sqrt(zeta)), as sk_meta_generate
 *                writes; a workgroup whose rows hold any other value redoes
 *                them with a per-hit product (about three times slower for
 *                that chunk, same result rules).
 *              SK_COMBINE_F32 (FP16 only): the reduce adds the FP16
 *                partials in FP32 and rounds the total to FP16 once (this
 *                library's option, more accurate than the FP16 additions of
 *                the default; ignored where no reduce runs: FLAT, or LDS
 *                without a workspace).  Without it every addition, the
 *                reduce's included, is an FP16 nearest-even addition.
 *            0 picks REG where it covers the shape and the workspace is
 *            large enough for it (16-byte aligned), else LDS when the
 *            partial fits in LDS and zeta <= 64, else FLAT.  At 2^20 x
 *            256, d = 512, zeta = 4 REG takes 0.20 ms and LDS 0.25 ms
 *            (FP16, with the reduce).
 *   workspace, workspace_bytes
 *            optional device scratch for the REG and LDS variants (4-byte
 *            aligned, 16 for REG; disjoint from every other buffer; size
 *            from sk_apply_workspace_size).  With a workspace the partials
 *            are stored there and a second kernel writes B as their sum, in
 *            a fixed order: four contiguous quarters of the row chunks,
 *            each summed in chunk order from +0, then the quarter sums added
 *            in order onto B (SK_ACCUMULATE) or +0 (no global atomics, no
 *            separate zeroing of B).  NULL: as sk_apply_f32 /
 *            sk_apply_f16acc.  Ignored by the FLAT variant.  The caller owns
 *            it; its contents on return are unspecified.  Calls that share a
 *            workspace must be ordered (same stream).
 * Order of additions: REG is fixed (reproducible bit for bit): each output
 * entry adds its contributions of a row chunk in ascending row order, from
 * +0, and the chunk partials in the reduce's order above.
 * Errors: as sk_apply_f32 / sk_apply_f16acc, plus SK_ERR_NULL
 * (SK_VARIANT_REG without a workspace), SK_ERR_ARG (SK_COMBINE_F32 on the
 * FP32 call, workspace smaller than required), SK_ERR_ALIGN (workspace not
 * 4-byte aligned, or not 16-byte aligned with SK_VARIANT_REG),
 * SK_ERR_UNSUPPORTED (SK_VARIANT_REG forced on a shape it does not cover).
 */
sk_status sk_apply_f32_ws(const float *A, int64_t m, int32_t n, int64_t lda,
                          const int32_t *row_idx, const float *val, int32_t zeta,
                          float *B, int32_t d, int64_t ldb, uint32_t flags,
                          void *workspace, size_t workspace_bytes, void *stream);
sk_status sk_apply_f16acc_ws(const float *A, int64_t m, int32_t n, int64_t lda,
                             const int32_t *row_idx, const float *val, int32_t zeta,
                             uint16_t *B, int32_t d, int64_t ldb, uint32_t flags,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * sk_apply_lowp: the reduced-precision sketch with a choice of contribution
 * conversion and accumulation format (FP16 sketching page §III-D: the
 * contribution is converted by one of several rules and fed to the same
 * packed nearest-even accumulation; §V-E: a BF16 variant).
 *
 *   A, row_idx, val, zeta, d, ldb  as for sk_apply_f16acc (n, lda, ldb
 *            even; A 8-byte and B 4-byte aligned).
 *   B        device uint16 bits, d x n: IEEE binary16 (SK_FORMAT_F16) or
 *            bfloat16 (SK_FORMAT_BF16, 8-bit exponent and significand).
 *   format, convert
 *            SK_FORMAT_F16 + SK_CONVERT_RN: nearest-even (the FP16 kernel's
 *              rule);
 *            SK_FORMAT_F16 + SK_CONVERT_SR: stochastic conversion.  For a
 *              contribution q with FP16 neighbours l <= |q| < v, the
 *              magnitude becomes v when the 32-bit draw r < frac * 2^32,
 *              frac = (|q| - l)/(v - l), else l; representable q are kept;
 *              past 65504 the upper neighbour is 2^16 and means +-inf.  The
 *              draw for global row g = row_offset + i, block t, column c is
 *              word c mod 4 of Philox-4x32-10 of counter (g lo, g hi,
 *              c div 4, 3 + 4t) and key (sr_seed lo, sr_seed hi);
 *            SK_FORMAT_BF16 + SK_CONVERT_RN: nearest-even conversion to
 *              BF16 and BF16 nearest-even additions.
 *            BF16 with SR is SK_ERR_UNSUPPORTED.
 *   sr_seed, row_offset  the SR draws' seed and A's first global row
 *            (ignored by the RN rules; row_offset >= 0).
 *   flags    SK_ACCUMULATE, and one of
 *              0 or SK_VARIANT_FLAT: the page's flat design, one packed
 *                global atomic per (row, block, column pair), additions in
 *                an unspecified order (B is zeroed first unless
 *                SK_ACCUMULATE); no workspace;
 *              SK_VARIANT_REG: the two-level design of the fused FP16
 *                sketch: each workgroup accumulates a chunk of rows in
 *                registers (packed pairs of the format, nearest-even
 *                additions, ascending rows) and a reduce adds the chunk
 *                partials in a fixed order (that of sk_apply_f16acc_ws's
 *                register variant), in the format, or in FP32 with one
 *                final rounding when SK_COMBINE_F32 is also given.
 *                Needs d % 16 == 0, zeta <= 16 and a workspace of
 *                sk_apply_workspace_size(SK_PRECISION_LOWP, ...,
 *                SK_VARIANT_REG) bytes (16-byte aligned, disjoint from the
 *                other buffers).  Reproducible bit for bit.
 *   workspace, workspace_bytes  SK_VARIANT_REG's scratch (else ignored).
 * Errors: as sk_apply_f16acc, plus SK_ERR_ARG for an unknown format,
 * conversion or flag (SK_COMBINE_F32 without SK_VARIANT_REG), SK_ERR_NULL
 * (SK_VARIANT_REG without a workspace) and SK_ERR_UNSUPPORTED for BF16 with
 * SR or a shape SK_VARIANT_REG does not cover.
 */
sk_status sk_apply_lowp(const float *A, int64_t m, int32_t n, int64_t lda,
                        const int32_t *row_idx, const float *val, int32_t zeta, uint16_t *B,
                        int32_t d, int64_t ldb, int32_t format, int32_t convert,
                        uint64_t sr_seed, int64_t row_offset, uint32_t flags,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * sk_apply_workspace_size: bytes of workspace that sk_apply_f32_ws
 * (precision SK_PRECISION_F32) or sk_apply_f16acc_ws (SK_PRECISION_F16ACC)
 * uses for these sizes and flags on the current device, whatever lda and
 * A's alignment: SK_VARIANT_REG the register plan (for A with lda = n and
 * an aligned base), SK_VARIANT_LDS the LDS plans, 0 the larger of the two.
 * SK_PRECISION_LOWP: the bytes sk_apply_lowp uses (SK_VARIANT_REG only).
 * 0 when the chosen variant uses none (FLAT, m = 0, or no plan fits).
 * Errors: SK_ERR_NULL (bytes NULL), SK_ERR_SHAPE, SK_ERR_ARG (precision or
 * flags), SK_ERR_HIP (device query failed).
 */
sk_status sk_apply_workspace_size(int32_t precision, int64_t m, int32_t n, int32_t d,
                                  int32_t zeta, uint32_t flags, size_t *bytes);

/*
 * sk_sketch_f32 / sk_sketch_f16acc: the complete SparseStack sketch in one
 * call, with the metadata drawn on the fly instead of stored.
 * (FP16 sketching page §III-C: the routing and signs come from a
 * counter-based Philox generator; FlashSketch page §5.2: a sketch's
 * randomness can be made inside the apply kernel, so S is never stored.)
 *
 * Computes exactly what sk_meta_generate(seed, row_offset, m, d, zeta)
 * followed by sk_apply_f32_ws / sk_apply_f16acc_ws (same flags) computes: the
 * same S, every contribution the FP32 product a*val, and for FP16 each
 * contribution rounded to FP16 nearest-even and accumulated with FP16
 * nearest-even additions.  The fused kernel keeps each workgroup's partial
 * in registers and writes it once to the workspace; a reduce kernel then
 * writes B as the sum of the partials in a fixed order (sk_apply_f16acc_ws's
 * register variant's order; no atomics, B needs no separate zeroing).  FP32 matrices wider than 128 columns whose rows
 * allow 16-byte loads (lda % 4 == 0, A 16-byte aligned) take four partial
 * words per lane (256 columns per workgroup) instead of two; the order of
 * each output word's additions is fixed either way.  Shapes the fused
 * kernel does not cover (zeta > 16, d not a multiple of 16, FP32 rows
 * wider than 64 columns without 8-byte lane loads (A 8-byte aligned, n and
 * lda even), FP16 rows wider than 128 columns without 16-byte lane loads,
 * row ownership that does not fit the registers) run sk_meta_generate into the
 * workspace and then the LDS (or flat) apply; the result is the same
 * sketch.
 *
 *   seed, row_offset  as for sk_meta_generate (row_offset >= 0 is the global
 *            index of A's first row, so row chunks with SK_ACCUMULATE give
 *            the sketch of the whole matrix).
 *   A        device float, m x n, lda >= n (FP16: n, lda even, A 8-byte
 *            aligned).
 *   B        device float (FP32) or IEEE binary16 bits (FP16: ldb even, B
 *            4-byte aligned), d x n, ldb >= n.
 *   flags    SK_ACCUMULATE, and for FP16 SK_COMBINE_F32 (the reduce adds
 *            the FP16 partials in FP32 and rounds once; by default every
 *            addition is an FP16 nearest-even addition).
 *   workspace, workspace_bytes
 *            device scratch, required when m > 0: 16-byte aligned, disjoint
 *            from A and B, at least sk_sketch_workspace_size bytes.  The
 *            caller owns it; its contents on return are unspecified; calls
 *            that share it must be ordered (same stream).
 * Errors: SK_ERR_NULL (A, B or workspace NULL when needed), SK_ERR_SHAPE
 * (sizes, zeta range, d % zeta, lda/ldb < n, odd n for FP16, row_offset < 0),
 * SK_ERR_ALIGN (workspace, or the FP16 alignment rules), SK_ERR_ARG (other
 * flags, overlapping buffers, workspace smaller than required), SK_ERR_HIP.
 */
sk_status sk_sketch_f32(uint64_t seed, int64_t row_offset, const float *A, int64_t m, int32_t n,
                        int64_t lda, int32_t d, int32_t zeta, float *B, int64_t ldb,
                        uint32_t flags, void *workspace, size_t workspace_bytes, void *stream);
sk_status sk_sketch_f16acc(uint64_t seed, int64_t row_offset, const float *A, int64_t m,
                           int32_t n, int64_t lda, int32_t d, int32_t zeta, uint16_t *B,
                           int64_t ldb, uint32_t flags, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * sk_sketch_f16acc_noalloc: sk_sketch_f16acc for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): no workspace argument, and the
 * call allocates nothing.  The fused kernel's partials go to a static
 * device scratch of 128 MiB that the library holds on every device it runs
 * on until the process ends; its device address is taken once per device,
 * on that device's first call.  Same sketch, arguments, flags and order of
 * additions as sk_sketch_f16acc.
 *   Only shapes the fused kernel covers run here (zeta <= 16, d % 16 == 0,
 *   the FP16 alignment rules of sk_sketch_f16acc, a plan whose partials fit
 *   the 128 MiB: every plan on a 256-CU device up to d = 2048 at 8192 FP16
 *   columns); any other shape returns SK_ERR_UNSUPPORTED and enqueues
 *   nothing.
 *   Every call on a device shares that device's scratch, and each call
 *   leaves its partials there: calls that overlap in time on one device
 *   (other streams, other host threads) race and give undefined results;
 *   order them on one stream.  The scratch needs no clearing: every word a
 *   call's reduce reads is first written by the same call.
 * Errors: as sk_sketch_f16acc (no workspace errors), plus
 * SK_ERR_UNSUPPORTED as above and SK_ERR_HIP when the scratch's device
 * address cannot be obtained.
 */
sk_status sk_sketch_f16acc_noalloc(uint64_t seed, int64_t row_offset, const float *A, int64_t m,
                                   int32_t n, int64_t lda, int32_t d, int32_t zeta,
                                   uint16_t *B, int64_t ldb, uint32_t flags, void *stream);

/*
 * sk_sketch_workspace_size: workspace bytes an sk_sketch_f32 (precision
 * SK_PRECISION_F32) or sk_sketch_f16acc (SK_PRECISION_F16ACC) call with
 * these sizes needs on the current device, whatever its lda and A's
 * alignment (the larger of the fused kernel's partials and the fallback's
 * metadata plus apply workspace); 0 for m = 0.
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_ARG (precision), SK_ERR_HIP.
 */
sk_status sk_sketch_workspace_size(int32_t precision, int64_t m, int32_t n, int32_t d,
                                   int32_t zeta, size_t *bytes);

/*
 * sk_fused_plan_describe: the launch plan of the fused kernel behind
 * sk_sketch_* (and SK_VARIANT_REG), for the given sizes, lda, the alignment
 * of A's base address in bytes (a_align: 16 or more allows every lane load;
 * FP32 needs 8, and 16 for four words per lane; FP16 needs 16), and the
 * device's compute units and per-workgroup LDS bytes.  Pure host
 * computation (no HIP call), for tests and tools that check a plan against
 * the kernel's index bounds.
 *   out  int64[SK_FUSED_PLAN_FIELDS], written: {fused kernel used (0: the
 *        fallback runs), output rows per wavefront, output row groups,
 *        column slices, rows per chunk, chunks, workgroups, workspace bytes,
 *        partial words per lane (1, 2 or 4), input rows per stage,
 *        workgroups per CU the plan is sized for (1 or 2)}.
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_ARG (precision, num_cu, max_lds).
 */
#define SK_FUSED_PLAN_FIELDS 11
sk_status sk_fused_plan_describe(int32_t precision, int64_t m, int32_t n, int64_t lda,
                                 int32_t a_align, int32_t d, int32_t zeta, int32_t num_cu,
                                 int32_t max_lds, int64_t *out);

/*
 * sk_sketch_plan_describe: the launch plan of sk_sketch_f32 /
 * sk_sketch_f16acc for the given sizes (arguments as for
 * sk_fused_plan_describe).  Narrow rows take the owner kernel where it
 * covers them (rows of at most 32 words: FP16 of at most 64 columns, FP32 of
 * at most 32; rows of 64 words with d <= 128): lanes own output rows, and
 * each stage's hits are counting-sorted into per-row lists walked in
 * ascending row order (the same order of additions as the register kernel);
 * other shapes take the register kernel sk_fused_plan_describe reports.  Pure host
 * computation, for tests and tools.
 *   out  int64[SK_SKETCH_PLAN_FIELDS], written: {kernel (0: the fallback,
 *        1: register kernel, 2: owner kernel), words per lane, lanes per
 *        output row (owner), threads per workgroup, a row's words padded to
 *        a power of two (owner), input rows per stage, list capacity per
 *        output row and stage (owner), words per lane load (owner), rows per
 *        chunk, chunks, workgroups, workspace bytes, dynamic LDS bytes per
 *        workgroup (owner), workgroups per CU the plan is sized for, LDS
 *        words between output rows' masks and between their lists (owner),
 *        workgroup barriers per stage (owner: 1 where the LDS holds three
 *        stage buffers at the same stage rows, else 2), loads per thread and
 *        stage held in registers (owner: 2 or 4)}.
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_ARG (precision, num_cu, max_lds).
 */
#define SK_SKETCH_PLAN_FIELDS 18
sk_status sk_sketch_plan_describe(int32_t precision, int64_t m, int32_t n, int64_t lda,
                                  int32_t a_align, int32_t d, int32_t zeta, int32_t num_cu,
                                  int32_t max_lds, int64_t *out);

/*
 * sk_apply_blockperm: Y = S A (or Y += S A) for S ~ BlockPerm-SJLT.
 * (FlashSketch page §4: input rows in M contiguous blocks of B_c = m/M,
 * output rows in M blocks of B_r = d/M; output block g reads the kappa input
 * blocks of N(g), a union of kappa edge-disjoint permutations; inside a
 * wired block pair each input row goes to s hashed output rows with
 * Rademacher signs; each block is scaled so each nonzero is
 * +-1/sqrt(kappa*s).  §5.1, §5.2: S is never stored; wiring and hashes are
 * made on the fly, accumulation is private to a workgroup, each output tile
 * is written once and there are no global atomics.)
 *
 * Wiring: pi_j(g) = (sigma(g) + j*M/kappa) mod M, j = 0..kappa-1, with sigma
 * the Fisher-Yates permutation of [M] whose swap partner for k = M-1..1 is
 * floor(w0*(k+1)/2^32), w0 the first word of Philox-4x32-10 of counter
 * (k, 0, 0, 2) and key (seed lo, seed hi).  The block graph is then M/kappa
 * disjoint complete bipartite components of kappa output and kappa input
 * blocks.
 * Hash: with fmix32 the MurmurHash3 32-bit finalizer and
 * c(H, x) = fmix32(H ^ x) + 0x9E3779B9, the block key is
 * K(g,h) = c(c(c(c(0x9E3779B9, seed lo), seed hi), g), h); input row r of
 * block h (0 <= r < B_c) has v = fmix32(K(g,h) ^ r) and
 * beta = floor(v*B_r/2^32); for s > 1, w = fmix32(v + 0x9E3779B9) and
 * alpha = 2*floor(w*(B_r/2)/2^32) + 1.  It goes to the s output rows
 * g*B_r + (beta + i*alpha) mod B_r, i < s (s = 1: beta), with sign
 * negative when bit i of v is set.
 *
 * One workgroup per (component, 32-column tile, group of 64 of the
 * component's kappa*B_r output rows) streams the component's input rows of
 * its tile, keeps its output rows in registers and writes them once: A is
 * read once when kappa*B_r <= 64 (ceil(kappa*B_r/64) times otherwise).
 * No workspace, no atomics, a fixed order of additions (reproducible).
 *
 *   A      device float, m x n, lda >= n (any alignment; 16-byte aligned A
 *          with n and lda multiples of 4 takes 16-byte loads).
 *   Y      device float, d x n, ldy >= n.
 *   M      blocks (1..1024), m % M == 0, d % M == 0, kappa | M.
 *   s      1 <= s <= B_r; s > 1 needs B_r a power of two (the odd stride
 *          alpha then gives s distinct rows).
 *   flags  SK_ACCUMULATE only.
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE (sizes, kappa not dividing M, s > B_r),
 * SK_ERR_UNSUPPORTED (M > 1024; s > 1 with B_r not a power of two),
 * SK_ERR_ARG (other flags, aliasing), SK_ERR_HIP.
 */
sk_status sk_apply_blockperm(const float *A, int64_t m, int32_t n, int64_t lda,
                             int32_t d, int32_t M, int32_t kappa, int32_t s,
                             uint64_t seed, float *Y, int64_t ldy, uint32_t flags,
                             void *stream);

/*
 * sk_apply_blockperm_ex: BlockPerm-SJLT with the general options.
 * (FlashSketch page §4, §5, App. B.1 split-B_c, App. D wiring and
 * within-block hashing.)
 *
 *   wiring  SK_WIRING_SHIFT: sk_apply_blockperm's family (kappa | M);
 *           SK_WIRING_AFFINE: pi_l = f^l, l = 1..kappa (kappa <= M), for the
 *           full-cycle map f(x) = (a x + b) mod M: with L the product of the
 *           distinct primes of M (times 2 when 4 | M and 4 does not divide
 *           it yet), a = 1 + L*floor(w0*(M/L)/2^32) (a = 1 when L >= M) and b
 *           the floor(w1*phi(M)/2^32)-th integer in [1, M) coprime to M,
 *           (w0, w1) the first words of Philox-4x32-10 of counter
 *           (0, 0, 0, 1) and key (seed lo, seed hi).
 *   s       nonzeros per column inside a block (1 <= s <= min(32, B_r);
 *           s > 1 needs B_r a power of two): with v and beta as for s = 1,
 *           w = fmix32(v + 0x9E3779B9) and alpha = 2*floor(w*(B_r/2)/2^32) + 1,
 *           row j = (beta + j*alpha) mod B_r, sign negative when bit j of v
 *           is set.  Each nonzero is +-1/sqrt(kappa*s).
 *   kappa   <= 32.
 *   workspace, workspace_bytes
 *           device scratch (16-byte aligned, disjoint from A and Y) of
 *           sk_blockperm_workspace_size bytes.  A kernel per (input block h,
 *           row slice, column slice) writes the kappa*B_r partial rows of h
 *           (its kappa readers' blocks) once, and a second kernel writes each
 *           Y element once as their sum in a fixed order (neighbour, then
 *           slice): no atomics, deterministic.  The partials are kept in
 *           registers (SK_BLOCKPERM_KERNEL_REGISTER) when n % 4 == 0,
 *           lda % 4 == 0, A is 16-byte aligned and kappa*B_r is 16 R G for
 *           some R in {1, 2, 4, 8, 16} dividing B_r and G <= 8; otherwise in
 *           LDS tiles of 32 columns (SK_BLOCKPERM_KERNEL_SLICE, kappa*B_r up
 *           to what one wavefront tile of LDS holds).  NULL is accepted for
 *           the shift wiring: sk_apply_blockperm's component kernel then
 *           runs (it also runs with a workspace where neither kernel above
 *           fills the device better).
 *   flags   SK_ACCUMULATE only.
 * Errors: as sk_apply_blockperm, plus SK_ERR_ARG (unknown wiring, small
 * workspace), SK_ERR_NULL (missing workspace), SK_ERR_ALIGN (workspace not
 * 16-byte aligned; A or lda unaligned where only the register kernel fits),
 * SK_ERR_UNSUPPORTED (s or kappa above 32, s > 1 with B_r not a power of
 * two, partial rows that neither kernel holds).
 */
sk_status sk_apply_blockperm_ex(const float *A, int64_t m, int32_t n, int64_t lda, int32_t d,
                                int32_t M, int32_t kappa, int32_t s, int32_t wiring,
                                uint64_t seed, float *Y, int64_t ldy, uint32_t flags,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * sk_blockperm_workspace_size: workspace bytes sk_apply_blockperm_ex needs
 * for these sizes on the current device, whatever A's alignment (the
 * larger of the register and slice kernels' needs where both apply).
 */
sk_status sk_blockperm_workspace_size(int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa,
                                      int32_t s, int32_t wiring, size_t *bytes);

/*
 * sk_blockperm_plan_describe: sk_apply_blockperm_ex's plan for A with
 * lda = n and a 16-byte aligned base, computed on the host (no HIP call):
 * out int64[SK_BLOCKPERM_PLAN_FIELDS] = {kernel (SK_BLOCKPERM_KERNEL_*), row
 * slices Q, rows per slice, workspace bytes, affine a, affine b, a^-1 mod M,
 * partial rows per wavefront R, row groups G, column slices} (a, b, a^-1 are
 * 0 for the shift wiring; R is 0 unless the register kernel runs; G and
 * the column slices are the register kernel's, or the component kernel's
 * groups of 64 output rows per component and 32-column tiles, else 0).
 */
#define SK_BLOCKPERM_PLAN_FIELDS 10
sk_status sk_blockperm_plan_describe(int64_t m, int32_t n, int32_t d, int32_t M, int32_t kappa,
                                     int32_t s, int32_t wiring, uint64_t seed, int32_t num_cu,
                                     int32_t max_lds, int64_t *out);

/*
 * sk_lds_plan_describe: the launch plan sk_apply_f32 (precision
 * SK_PRECISION_F32) or sk_apply_f16acc (SK_PRECISION_F16ACC) makes for its
 * LDS variant, for the given sizes, A's leading dimension lda, whether A's
 * base address allows two-word lane loads (wide_ok: 16-byte aligned for
 * FP16, 8-byte for FP32) and the device's compute units and per-workgroup
 * LDS bytes.  Pure host computation: no HIP call, no device needed.  For
 * tests and tools that check a plan against the kernels' index bounds.
 *   out  int64[SK_PLAN_FIELDS], written: {lds_variant_used (0: the flat
 *        kernel runs), words per lane, lanes per slice, block groups,
 *        blocks per group, threads per workgroup, rows per chunk, chunks,
 *        slices, workgroups, LDS bytes per workgroup, workspace bytes}.
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_ARG (precision, num_cu, max_lds).
 */
#define SK_PLAN_FIELDS 12
sk_status sk_lds_plan_describe(int32_t precision, int64_t m, int32_t n, int64_t lda, int32_t d,
                               int32_t zeta, int32_t wide_ok, int32_t num_cu, int32_t max_lds,
                               int64_t *out);

/*
 * sk_lstsq_qr_f32: x = argmin ||SA x - Sb||_2 for a small sketch, by an FP32
 * Householder QR of SA, the projection Q^T Sb and a triangular solve: the
 * reduced solve of sketch-and-solve least squares (FP16 sketching page
 * §V-A, §V-D: FP32 QR, projection and solve on the d x n sketch;
 * FlashSketch page App. F.1.4).  Two launches per panel of up to 32
 * columns: the panel factored by one workgroup (reflectors as in LAPACK's
 * larfg, combined as I - V T V^T), the trailing columns updated by several.
 * Every column of [SA | Sb] is first scaled by a power of two that brings
 * its largest magnitude into [1/2, 1), and x scaled back at the end: the QR
 * commutes exactly with such scalings, so x is the same bit for bit as
 * without them wherever no intermediate overflows or underflows, and no
 * norm or dot product overflows for any finite input.
 *   SA        device float, d x n row-major, row stride ld >= n; 1 <= n <= d
 *             <= 2048.  Not modified.
 *   Sb        device float[d].  Not modified.
 *   x         device float[n], written.
 *   workspace device scratch of at least sk_lstsq_workspace_size(d, n)
 *             bytes, 4-byte aligned, disjoint from SA, Sb and x; contents on
 *             return unspecified.  Calls sharing it must be ordered.
 * A zero diagonal entry of R (SA without full column rank) gives inf or NaN
 * entries of x, as a plain triangular solve would.
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE (n, d, ld), SK_ERR_ALIGN (workspace),
 * SK_ERR_ARG (workspace too small, or overlapping an argument), SK_ERR_HIP.
 */
sk_status sk_lstsq_qr_f32(const float *SA, int32_t d, int32_t n, int64_t ld, const float *Sb,
                          float *x, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of sk_lstsq_qr_f32 for these sizes ((n + 1) * (d + 1) +
 * 1024 floats).
 * Errors: SK_ERR_NULL, SK_ERR_SHAPE. */
sk_status sk_lstsq_workspace_size(int32_t d, int32_t n, size_t *bytes);

/* Static, NUL-terminated description of a status code. */
const char *sk_status_string(sk_status status);

#ifdef __cplusplus
}
#endif

#endif /* SK_SKETCH_H */
