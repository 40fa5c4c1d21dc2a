"""CPU oracle for sparse sketching: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under this package: only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code, tables or
constants with the HIP library; each function here is written from the
definitions on the pages it cites:

* "On the Robustness of Sparse Randomized Sketching to FP16 Rounding on
  GPUs" (the FP16 sketching page): SparseStack / CountSketch, the coupled
  Philox metadata (§III-C), FP32 products with RN conversion to FP16 and
  FP16 accumulation (§III-B, §III-D), the error model (§IV-A, §IV-B).
* "FlashSketch: Sketch-Kernel Co-Design for Fast Sparse Sketching on GPUs"
  (the FlashSketch page): BlockPerm-SJLT (§4, Figure 2, App. A.1, App. D),
  the metrics of App. F.1.
* Sketch-and-solve least squares and ridge regression on a sketch (FP16
  sketching page §V-D, FlashSketch App. F.1.3-F.1.4) (``solve``).
* The FP16 sketching page's conversion variants (§III-D, §V-E):
  stochastic conversion to FP16 and BF16 accumulation (``lowp``).

Floating point is fp64 unless the page fixes the precision (the FP16
pipeline).  Every function is pinned by tests against something other than
itself; the one function without such a pin says so in its docstring
("parity unpinned").
"""
from .philox import philox4x32_10, philox_scalar, PHILOX4x32, PHILOX4x64
from .sparsestack import (scale_f32, meta_ref, sketch_matrix, dense_S, sketch_f64,
                          countsketch_f64, sketch_f16_rn_emul, rn_f16_add, in_block,
                          f16_erasures, f16_zero_subnormal_counts)
from .blockperm import (fmix32, perm_sigma, shift_wiring, blockperm_params,
                        blockperm_hash, blockperm_hash_s, blockperm_matrix, blockperm_dense_S,
                        blockperm_f64, affine_params, affine_wiring, wiring, prime_factors)
from .metrics import rel_frob, ose_error, sv_ratio, gram_rel_error
from .solve import residual, lstsq_qr, sketch_solve, ridge_solve, reference_solution
from .lowp import (sr_words, f16_neighbours, sr_f16, rn_bf16, rn_bf16_add,
                   sketch_lowp_emul)

__all__ = [
    "philox4x32_10", "philox_scalar", "PHILOX4x32", "PHILOX4x64",
    "scale_f32", "meta_ref", "sketch_matrix", "dense_S", "sketch_f64",
    "countsketch_f64", "sketch_f16_rn_emul", "rn_f16_add", "in_block", "f16_erasures",
    "f16_zero_subnormal_counts",
    "fmix32", "perm_sigma", "shift_wiring", "blockperm_params",
    "blockperm_hash", "blockperm_matrix", "blockperm_dense_S", "blockperm_f64",
    "blockperm_hash_s", "affine_params", "affine_wiring", "wiring", "prime_factors",
    "rel_frob", "ose_error", "sv_ratio", "gram_rel_error",
    "residual", "lstsq_qr", "sketch_solve", "ridge_solve", "reference_solution",
    "sr_words", "f16_neighbours", "sr_f16", "rn_bf16", "rn_bf16_add", "sketch_lowp_emul",
]
