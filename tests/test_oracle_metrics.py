"""Pins for the fp64 metrics (FlashSketch page App. F.1; FP16 sketching
page §V-C) against closed forms."""
import numpy as np

from oracle import gram_rel_error, ose_error, rel_frob, sv_ratio


def test_ose_error_closed_forms():
    Q = np.linalg.qr(np.random.default_rng(0).standard_normal((50, 6)))[0]
    assert ose_error(Q) < 1e-12                     # orthonormal: no distortion
    a = np.array([0.5, 1.0, 1.3, 0.9])
    D = np.zeros((7, 4))
    D[:4, :4] = np.diag(a)
    assert np.isclose(ose_error(D), np.max(np.abs(a**2 - 1)))
    assert np.isclose(ose_error(Q @ np.diag([1, 1, 1, 1, 1, 2.0])), 3.0)


def test_sv_ratio_and_rank_loss():
    assert np.isclose(sv_ratio(np.diag([4.0, 2.0, 1.0])), 0.25)
    M = np.ones((5, 2))
    assert sv_ratio(M) < 1e-12


def test_gram_and_frob():
    A = np.random.default_rng(1).standard_normal((40, 5))
    Q = np.linalg.qr(np.random.default_rng(2).standard_normal((40, 40)))[0]
    assert gram_rel_error(A, Q @ A) < 1e-12          # orthogonal S keeps the Gram
    assert np.isclose(gram_rel_error(A, 2 * A), 3.0)
    assert np.isclose(rel_frob(1.5 * A, A), 0.5)
