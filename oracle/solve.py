"""Sketch-and-solve least squares and ridge regression on a sketch.
TEST INFRASTRUCTURE ONLY.

Follows the FP16 sketching page §V-A/§V-D (sketch-and-solve: the shared map
gives SA and Sb, an FP32 QR of SA, the projection Q^T Sb, a triangular
solve; residuals evaluated in FP64; the unsketched FP64 QR solution is the
reference) and the FlashSketch page App. F.1.3/F.1.4 (ridge regression on
the sketch, argmin ||SAx - Sb||^2 + lambda ||x||^2, and the residual
||Ax - b|| / ||b||, or ||Ax - b|| when b = 0).

Everything here is fp64 unless the page fixes FP32 (the QR of the sketch).
NumPy's LAPACK routines serve as the steps (QR, triangular and dense solves).
"""
import numpy as np


def residual(A, x, b):
    """||Ax - b||_2 / ||b||_2 in fp64 (||Ax - b||_2 when b = 0)."""
    A = np.asarray(A, dtype=np.float64)
    r = A @ np.asarray(x, dtype=np.float64) - np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(r) / nb) if nb > 0 else float(np.linalg.norm(r))


def lstsq_qr(M, y, dtype=np.float64):
    """argmin ||M x - y||_2 by a thin QR of M in `dtype`, the projection
    Q^T y and the triangular solve R x = Q^T y."""
    M = np.asarray(M, dtype=dtype)
    y = np.asarray(y, dtype=dtype)
    Q, R = np.linalg.qr(M, mode="reduced")
    z = Q.T @ y
    return np.linalg.solve(np.triu(R), z).astype(np.float64)


def sketch_solve(SA, Sb, dtype=np.float32):
    """The sketched least-squares solution: FP32 QR of SA (§V-A)."""
    return lstsq_qr(SA, Sb, dtype)


def ridge_solve(SA, Sb, lam):
    """argmin ||SA x - Sb||^2 + lam ||x||^2 (App. F.1.3), as the least-squares
    problem of the stacked matrix [SA; sqrt(lam) I] and right-hand side
    [Sb; 0], solved in fp64."""
    SA = np.asarray(SA, dtype=np.float64)
    n = SA.shape[1]
    M = np.vstack([SA, np.sqrt(lam) * np.eye(n)])
    y = np.concatenate([np.asarray(Sb, dtype=np.float64), np.zeros(n)])
    return lstsq_qr(M, y)


def reference_solution(A, b):
    """The unsketched minimizer x* by fp64 QR of A (§V-A reference)."""
    return lstsq_qr(A, b)
