"""Sizes past 2^31 elements of A: every address and offset the kernels form
from (row, lda) must be 64-bit.  A is 2^22 x 544 FP32 (2.28e9 elements,
9.1 GB), drawn on the device; each path's sketch is checked against the
fp64 oracle on sampled columns spread over every column slice (FP16
sketching page §III; FlashSketch page §4, §5)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync

pytestmark = pytest.mark.gpu

M_ROWS, N_COLS = 1 << 22, 544
COLS = [0, 1, 63, 255, 256, 300, 511, 512, 543]
D, ZETA, SEED = 512, 4, 3
BP_D, BP_M, BP_KAPPA, BP_SEED = 1024, 64, 4, 5


@pytest.fixture(scope="module")
def big():
    assert M_ROWS * N_COLS > 1 << 31
    say(f"large: drawing A {M_ROWS} x {N_COLS} on the device and the oracle's metadata")
    A = inputs.gaussian_torch(M_ROWS, N_COLS, seed=0)
    Ac = A[:, torch.tensor(COLS, device=A.device)].cpu().numpy()
    ri, v = oracle.meta_ref(SEED, M_ROWS, D, ZETA)
    return A, Ac, oracle.sketch_f64(Ac, ri, v, D, ZETA)


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_fused_past_2g_elements(big, precision, tol):
    A, _, ref = big
    say(f"large fused {precision}")
    B = b.sketch_fused(A, D, ZETA, SEED, precision)
    sync()
    err = oracle.rel_frob(B[:, COLS].float().cpu().numpy().astype(np.float64), ref)
    say(f"  rel err {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_lds_apply_past_2g_elements(big, precision, tol):
    A, _, ref = big
    say(f"large LDS apply {precision}")
    ri, v = b.meta(SEED, M_ROWS, D, ZETA, device=dev())
    B = b.apply(A, ri, v, ZETA, D, precision=precision, flags=b.SK_VARIANT_LDS)
    sync()
    err = oracle.rel_frob(B[:, COLS].float().cpu().numpy().astype(np.float64), ref)
    say(f"  rel err {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_register_apply_past_2g_elements(big, precision, tol):
    """The stored-metadata apply on the fused kernel (the default with a
    workspace)."""
    A, _, ref = big
    say(f"large register apply {precision}")
    ri, v = b.meta(SEED, M_ROWS, D, ZETA, device=dev())
    B = b.apply(A, ri, v, ZETA, D, precision=precision, flags=b.SK_VARIANT_REG)
    sync()
    err = oracle.rel_frob(B[:, COLS].float().cpu().numpy().astype(np.float64), ref)
    say(f"  rel err {err:.3e}")
    assert err <= tol


def test_blockperm_register_past_2g_elements(big):
    A, Ac, _ = big
    say("large BlockPerm (register kernel)")
    p = b.sk_blockperm_plan_describe(M_ROWS, N_COLS, BP_D, BP_M, BP_KAPPA, 1, b.SK_WIRING_SHIFT,
                                     BP_SEED, num_cu=256, max_lds=160 * 1024)
    assert p["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
    Y = b.blockperm(A, BP_D, BP_M, BP_KAPPA, BP_SEED)
    sync()
    ref = oracle.blockperm_matrix(M_ROWS, BP_D, BP_M, BP_KAPPA, 1, BP_SEED) @ Ac.astype(np.float64)
    err = oracle.rel_frob(Y[:, COLS].cpu().numpy().astype(np.float64), ref)
    say(f"  rel err {err:.3e}")
    assert err <= 1e-5
