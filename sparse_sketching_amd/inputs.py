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
* ``orth(A)``: U = Q of the fp64 thin QR of A, stored as FP32.
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
    Q, _ = np.linalg.qr(np.asarray(A, dtype=np.float64), mode="reduced")
    return Q.astype(np.float32)


def gaussian_torch(m, n, seed=0, device="cuda"):
    """N(0, 1) FP32 drawn on the device with torch's seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((m, n), generator=g, device=device, dtype=torch.float32)
