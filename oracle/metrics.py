"""Sketch-quality metrics (fp64).  TEST INFRASTRUCTURE ONLY.

Definitions from "FlashSketch: Sketch-Kernel Co-Design for Fast Sparse
Sketching on GPUs", App. F.1 (Gram approximation, OSE spectral error) and
§3.2 (the OSE event ||U^T S^T S U - I||_2 <= eps), and the FP16 sketching
page's geometry study (§V-C: singular values of SU).
"""
import numpy as np


def rel_frob(B, B_ref):
    """||B - B_ref||_F / ||B_ref||_F in fp64."""
    B = np.asarray(B, dtype=np.float64)
    B_ref = np.asarray(B_ref, dtype=np.float64)
    return float(np.linalg.norm(B - B_ref) / np.linalg.norm(B_ref))


def ose_error(SU):
    """E_OSE = ||(SU)^T (SU) - I||_2 for the sketch of an orthonormal U."""
    Q = np.asarray(SU, dtype=np.float64)
    G = Q.T @ Q - np.eye(Q.shape[1])
    return float(np.max(np.abs(np.linalg.eigvalsh(G))))


def sv_ratio(SU):
    """sigma_min(SU) / sigma_max(SU)."""
    s = np.linalg.svd(np.asarray(SU, dtype=np.float64), compute_uv=False)
    return float(s[-1] / s[0])


def gram_rel_error(A, SA):
    """||A^T A - (SA)^T (SA)||_F / ||A^T A||_F (zero-safe as on the page)."""
    A = np.asarray(A, dtype=np.float64)
    SA = np.asarray(SA, dtype=np.float64)
    G = A.T @ A
    err = np.linalg.norm(G - SA.T @ SA)
    nrm = np.linalg.norm(G)
    return float(err / nrm) if nrm > 0 else float(err)
