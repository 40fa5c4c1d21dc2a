"""Pins of the sketch-and-solve / ridge oracle (oracle/solve.py) against
closed forms and independent routes: consistent systems are solved
exactly by any full-rank sketch, the QR route equals the normal equations,
ridge tends to least squares as lambda -> 0 and to x = 0 as lambda grows,
the identity sketch reproduces the unsketched problem, and the residual of
the unsketched minimizer is orthogonal to range(A)."""
import numpy as np

import oracle
from sparse_sketching_amd import inputs


def system(m=3000, n=20, seed=0, noise=0.1):
    g = np.random.default_rng(seed)
    A = g.standard_normal((m, n))
    x0 = g.standard_normal(n)
    b = A @ x0 + noise * g.standard_normal(m)
    return A, b, x0


def sketched(A, b, d, zeta, seed):
    ri, v = oracle.meta_ref(seed, A.shape[0], d, zeta)
    S = oracle.dense_S(ri, v, A.shape[0], d, zeta)
    return S @ A, S @ b


def test_consistent_system_is_solved_exactly():
    A, _, x0 = system(noise=0.0)
    b = A @ x0
    SA, Sb = sketched(A, b, 80, 4, 3)
    x = oracle.lstsq_qr(SA, Sb)
    assert np.allclose(x, x0, rtol=0, atol=1e-10)
    assert oracle.residual(A, x, b) < 1e-12


def test_qr_route_equals_normal_equations():
    A, b, _ = system()
    SA, Sb = sketched(A, b, 100, 4, 5)
    x_qr = oracle.lstsq_qr(SA, Sb)
    x_ne = np.linalg.solve(SA.T @ SA, SA.T @ Sb)
    assert np.allclose(x_qr, x_ne, rtol=1e-9, atol=1e-12)


def test_fp32_sketch_solve_close_to_fp64():
    A, b, _ = system()
    SA, Sb = sketched(A, b, 100, 4, 5)
    x32 = oracle.sketch_solve(SA, Sb)
    x64 = oracle.lstsq_qr(SA, Sb)
    assert np.linalg.norm(x32 - x64) / np.linalg.norm(x64) < 1e-4


def test_ridge_limits_and_closed_form():
    A, b, _ = system()
    SA, Sb = sketched(A, b, 100, 4, 7)
    x_ls = oracle.lstsq_qr(SA, Sb)
    assert np.allclose(oracle.ridge_solve(SA, Sb, 1e-12), x_ls, rtol=1e-8, atol=1e-10)
    lam = 37.5
    x_cf = np.linalg.solve(SA.T @ SA + lam * np.eye(SA.shape[1]), SA.T @ Sb)
    assert np.allclose(oracle.ridge_solve(SA, Sb, lam), x_cf, rtol=1e-9, atol=1e-12)
    x_big = oracle.ridge_solve(SA, Sb, 1e12)
    assert np.linalg.norm(x_big) < 1e-6 * np.linalg.norm(x_ls)
    assert abs(oracle.residual(A, x_big, b) - 1.0) < 1e-5


def test_identity_sketch_and_reference_optimality():
    A, b, _ = system(m=500, n=12)
    x_star = oracle.reference_solution(A, b)
    assert np.allclose(oracle.lstsq_qr(np.eye(500) @ A, b), x_star)
    r = A @ x_star - b
    assert np.linalg.norm(A.T @ r) < 1e-9 * np.linalg.norm(A) * np.linalg.norm(r)
    assert np.allclose(x_star, np.linalg.lstsq(A, b, rcond=None)[0])


def test_residual_definition():
    A = np.eye(3)
    assert oracle.residual(A, np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.residual(A, np.array([1.0, 0, 0]), np.zeros(3)) == 1.0
    assert oracle.residual(A, np.zeros(3), np.array([0, 3.0, 4.0])) == 1.0


def test_sketch_solve_residual_approaches_optimum_with_d():
    """Larger sketches give residuals closer to the unsketched optimum
    (the page's d/n sweep): d = 32 n is within 5% of optimal."""
    A, b, _ = system(m=8000, n=10, seed=4, noise=1.0)
    opt = oracle.residual(A, oracle.reference_solution(A, b), b)
    res = []
    for d in (20, 320):
        SA, Sb = sketched(A, b, d, 4, 11)
        res.append(oracle.residual(A, oracle.lstsq_qr(SA, Sb), b))
    assert res[1] <= res[0] and res[1] < 1.05 * opt and res[0] >= opt


def test_coherent_inputs_and_orth():
    U = inputs.orth(inputs.coherent(4096, 16, seed=1))
    SU, _ = sketched(U.astype(np.float64), np.zeros(4096), 64, 4, 2)
    assert oracle.ose_error(U.astype(np.float64)) < 1e-5       # U is orthonormal
    assert 0 < oracle.ose_error(SU) < 1.5
