"""Sketch-and-solve least squares, ridge regression and sketch-quality
metrics on top of the library's sketches.

* Sketch-and-solve (FP16 sketching page §V-A, §V-D): one map S is applied
  to A and to b ("shared map"), the d x n sketch SA gets an FP32 Householder
  QR, and x solves R x = Q^T Sb; residuals ||Ax - b|| / ||b|| are evaluated
  in FP64.  The sketches are libsksketch's fused calls (sk_sketch_f16acc or
  sk_sketch_f32): S depends only on (seed, row_offset, m, d, zeta), so the
  two calls apply the same S.
* Ridge regression on the sketch, argmin ||SA x - Sb||^2 + lam ||x||^2, and
  the same residual (FlashSketch page App. F.1.3, F.1.4).
* Gram approximation error, OSE spectral error and sigma_min/sigma_max of a
  sketched orthonormal basis (FlashSketch page App. F.1.1, F.1.2; FP16
  sketching page §V-C).

The sketches and the FP32 QR solve run in the library's kernels; torch
supplies device memory, stacks the ridge system and evaluates the FP64
residuals and metrics (measurement, not part of the solve).
"""
import torch

from . import binding as b


def sketch_pair(A, rhs, d, zeta, seed, precision="f16acc", row_offset=0, combine="f16"):
    """(SA, Sb) as float32 device tensors for the same S.  rhs is a length-m
    vector: the FP32 path sketches it as an m x 1 matrix; the FP16 path works
    on column pairs and sketches it as the first column of [b b] (columns
    are sketched independently; one copy builds the pair).  combine (FP16
    only): "f16" adds the row chunks' FP16 partials with FP16 additions
    (every addition in FP16, the page's arithmetic), "f32" in FP32 with one
    final rounding (SK_COMBINE_F32)."""
    m = A.shape[0]
    f16 = precision == "f16acc"
    Bv = rhs.reshape(m, 1).expand(m, 2).contiguous() if f16 else rhs.reshape(m, 1)
    flags = b.SK_COMBINE_F32 if (f16 and combine == "f32") else 0
    SA = b.sketch_fused(A, d, zeta, seed, precision, row_offset=row_offset, flags=flags)
    Sb = b.sketch_fused(Bv, d, zeta, seed, precision, row_offset=row_offset, flags=flags)[:, 0]
    return SA.float(), Sb.float().contiguous()


def solve_sketched(SA, Sb):
    """argmin ||SA x - Sb||_2 by the library's FP32 Householder QR, the
    projection Q^T Sb and a triangular solve (sk_lstsq_qr_f32, one launch);
    float32 result."""
    return b.lstsq_qr(SA.float().contiguous(), Sb.float().contiguous())


def ridge_sketched(SA, Sb, lam):
    """argmin ||SA x - Sb||^2 + lam ||x||^2 as the least-squares problem of
    [SA; sqrt(lam) I] and [Sb; 0] (FP32 QR)."""
    n = SA.shape[1]
    M = torch.cat([SA.float(), (lam ** 0.5) * torch.eye(n, dtype=torch.float32,
                                                        device=SA.device)])
    y = torch.cat([Sb.float(), torch.zeros(n, dtype=torch.float32, device=SA.device)])
    return solve_sketched(M, y)


def residual(A, x, rhs):
    """||Ax - b||_2 / ||b||_2 in FP64 (||Ax - b||_2 when b = 0)."""
    r = A.double() @ x.double() - rhs.double()
    nb = torch.linalg.norm(rhs.double())
    nr = torch.linalg.norm(r)
    return float(nr / nb) if float(nb) > 0 else float(nr)


def sketch_and_solve(A, rhs, d, zeta, seed, precision="f16acc", combine="f16"):
    """The complete sketch-and-solve: shared-map sketches, FP32 QR solve,
    FP64 residual.  Returns (x, residual)."""
    SA, Sb = sketch_pair(A, rhs, d, zeta, seed, precision, combine=combine)
    x = solve_sketched(SA, Sb)
    return x, residual(A, x, rhs)


def gram_rel_error(A, SA):
    """||A^T A - (SA)^T SA||_F / ||A^T A||_F in FP64 (the absolute error when
    A^T A = 0)."""
    A64, S64 = A.double(), SA.double()
    G = A64.T @ A64
    err = torch.linalg.norm(G - S64.T @ S64)
    nrm = torch.linalg.norm(G)
    return float(err / nrm) if float(nrm) > 0 else float(err)


def ose_error(SQ):
    """E_OSE = ||(SQ)^T SQ - I||_2 for the sketch of an orthonormal Q (FP64)."""
    Q = SQ.double()
    G = Q.T @ Q - torch.eye(Q.shape[1], dtype=torch.float64, device=Q.device)
    return float(torch.linalg.eigvalsh(G).abs().max())


def sv_ratio(SQ):
    """sigma_min(SQ) / sigma_max(SQ) (FP64)."""
    s = torch.linalg.svdvals(SQ.double())
    return float(s[-1] / s[0])
