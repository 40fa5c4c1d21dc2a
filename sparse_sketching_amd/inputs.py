"""Seeded synthetic inputs for the sketch workloads.

This module only draws input matrices; it holds none of the sketching
arithmetic.  It is shared by the test suite (both sides of every parity
check) and the benchmark.

Workloads (shapes and distributions of the FP16 sketching page's grids,
§V-B and §V-E, and of the FlashSketch page's dense-input study, §7.2):

* ``gaussian(m, n)``: i.i.d. N(0, 1) FP32, NumPy PCG64 seeded with 0.
* ``integer_matrix``: i.i.d. integers in [lo, hi] stored as FP32.
* ``coordinate(m, n)``: the coordinate input [I_n 0]^T of §V-B.
* ``coherent(m, n)``: N(0, 1) with n distinct rows p_j (drawn from the same
  generator after G) replaced by 1e3*e_j + G[p_j], so that a few rows carry
  most of the column-space energy (§V-C coherence study).
* ``range_stress(m, n, k)``: N(0, 1) rows times lognormal(0, 2) row scales
  (exp(2Z), Z ~ N(0, 1)), times the common factor 2^k (§V-E rescaling).
* ``orth(A)``: an orthonormal basis U of range(A) (fp64 Cholesky QR, two
  passes), stored as FP32.
* ``*_torch`` variants draw the same kind of input on the device with
  torch's seeded generator (used for the largest workloads, where host
  generation would dominate test time); their host copies feed the oracle.
"""
import numpy as np


def rng(seed=0):
    return np.random.default_rng(seed)


def gaussian(m, n, seed=0):
    return rng(seed).standard_normal((m, n), dtype=np.float32)


def integer_matrix(m, n, lo=-8, hi=8, seed=0):
    return rng(seed).integers(lo, hi + 1, size=(m, n)).astype(np.float32)


def coordinate(m, n):
    A = np.zeros((m, n), dtype=np.float32)
    A[np.arange(n), np.arange(n)] = 1.0
    return A


def coherent(m, n, seed=0, head=1e3):
    g = rng(seed)
    A = g.standard_normal((m, n), dtype=np.float32)
    p = g.choice(m, size=n, replace=False)
    A[p, np.arange(n)] += np.float32(head)
    return A


def range_stress(m, n, k, seed=0):
    g = rng(seed)
    A = g.standard_normal((m, n), dtype=np.float32)
    scale = np.exp(2.0 * g.standard_normal(m)).astype(np.float32)
    A *= scale[:, None]
    A *= np.float32(2.0) ** k          # exact power-of-two scaling
    return A


def orth(A):
    """Orthonormal basis of range(A): two passes of Cholesky QR in fp64
    (accurate for the well-conditioned workloads here), stored as FP32."""
    Q = np.asarray(A, dtype=np.float64)
    for _ in range(2):
        R = np.linalg.cholesky(Q.T @ Q).T
        Q = np.linalg.solve(R.T, Q.T).T
    return Q.astype(np.float32)


def orth_torch(A):
    """orth() on the device with torch (fp64 Cholesky QR, two passes)."""
    import torch
    Q = A.to(torch.float64)
    for _ in range(2):
        L = torch.linalg.cholesky(Q.T @ Q)          # n x n, Q^T Q = L L^T
        # Q <- Q L^{-T}: invert the small factor and multiply, so the tall
        # operand only meets a plain matrix product
        Q = Q @ torch.linalg.inv(L).T.contiguous()
    return Q.to(torch.float32).contiguous()


def coherent_torch(m, n, seed=0, head=1e3, device="cuda"):
    """coherent() drawn on the device with torch's seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    A = torch.randn((m, n), generator=g, device=device, dtype=torch.float32)
    p = torch.randperm(m, generator=g, device=device)[:n]
    A[p, torch.arange(n, device=device)] += head
    return A


def gaussian_torch(m, n, seed=0, device="cuda"):
    """N(0, 1) FP32 drawn on the device with torch's seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((m, n), generator=g, device=device, dtype=torch.float32)
