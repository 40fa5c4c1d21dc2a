"""Sparse randomized sketching (SparseStack, CountSketch, BlockPerm-SJLT)
on AMD MI355X (gfx950).

The compute path is libsksketch.so (hand-written HIP kernels behind the C ABI
of include/sk.h); ``binding`` marshals torch tensors into it.  ``inputs``
draws the seeded synthetic workloads.
"""
from .binding import (SK_CONVERT_RN, SK_CONVERT_SR, SK_FORMAT_BF16, SK_FORMAT_F16, apply_lowp,
                      sk_apply_lowp, SK_ACCUMULATE, SK_PRECISION_F16ACC, SK_PRECISION_F32, SK_VARIANT_FLAT,
                      SK_VARIANT_LDS, SketchError, apply, blockperm, load, meta,
                      sk_apply_blockperm, sk_apply_f16acc, sk_apply_f32, sk_apply_workspace_size,
                      sk_meta_generate, sk_sketch_f16acc, sk_sketch_f32,
                      sk_sketch_workspace_size, sketch, sketch_fused, sketch_workspace,
                      status_string, workspace)

__all__ = ["SK_CONVERT_RN", "SK_CONVERT_SR", "SK_FORMAT_BF16", "SK_FORMAT_F16", "apply_lowp",
           "sk_apply_lowp", "SK_ACCUMULATE", "SK_PRECISION_F16ACC", "SK_PRECISION_F32", "SK_VARIANT_FLAT",
           "SK_VARIANT_LDS", "SketchError", "apply", "blockperm", "load", "meta",
           "sk_apply_blockperm", "sk_apply_f16acc", "sk_apply_f32", "sk_apply_workspace_size",
           "sk_meta_generate", "sk_sketch_f16acc", "sk_sketch_f32", "sk_sketch_workspace_size",
           "sketch", "sketch_fused", "sketch_workspace", "status_string", "workspace"]
