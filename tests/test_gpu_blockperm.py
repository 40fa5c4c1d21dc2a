"""GPU parity for sk_apply_blockperm against the BlockPerm-SJLT oracle
(FlashSketch page §4, §5, App. D): dense brute force on tiny instances,
exact integer inputs, and the full 2^21 x 512 configuration on sampled
columns."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,d,M,kappa,seed", [
    (256, 5, 32, 4, 2, 9),          # B_c = 64, B_r = 8, ragged column tile
    (512, 33, 64, 8, 4, 1),         # two column tiles
    (512, 32, 64, 8, 1, 2),         # kappa = 1: localized block-diagonal
    (1024, 40, 128, 16, 8, 3),      # kappa = 8
    (6 * 100, 7, 6 * 3, 6, 2, 4),   # B_c = 100 (partial row batch), B_r = 3
])
def test_small_vs_dense(m, n, d, M, kappa, seed):
    say(f"blockperm m={m} n={n} d={d} M={M} kappa={kappa}")
    A = inputs.gaussian(m, n, seed=seed)
    Y = b.blockperm(to_dev(A), d, M, kappa, seed)
    sync()
    ref = oracle.blockperm_dense_S(m, d, M, kappa, 1, seed) @ A.astype(np.float64)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


def test_integer_exact_and_accumulate():
    m, n, d, M, kappa = 4096, 64, 256, 16, 4
    A = inputs.integer_matrix(m, n, -8, 8, seed=1)
    Ad = to_dev(A)
    ref = oracle.blockperm_f64(A, d, M, kappa, 1, 77)
    Y = b.blockperm(Ad, d, M, kappa, 77)
    sync()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)
    b.blockperm(Ad, d, M, kappa, 77, out=Y, flags=b.SK_ACCUMULATE)
    sync()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), 2 * ref)


def test_padded_strides():
    m, n, d, M, kappa = 2048, 45, 128, 8, 2
    A = inputs.gaussian(m, 64, seed=3)
    Ad = to_dev(A)[:, :n]
    out = torch.full((d, 50), 5.0, device=dev())
    b.blockperm(Ad, d, M, kappa, 5, out=out[:, :n])
    sync()
    Y = out.cpu().numpy()
    assert np.all(Y[:, n:] == 5.0)
    ref = oracle.blockperm_f64(np.ascontiguousarray(A[:, :n]), d, M, kappa, 1, 5)
    assert oracle.rel_frob(Y[:, :n], ref) <= 1e-5


def test_full_configuration_sampled_columns():
    """A 2^21 x 512 N(0,1) (drawn on the device, seeded), d = 1024, M = 64,
    kappa = 4, s = 1.  Every output row is checked on 24 columns spread over
    all 16 column tiles, against the fp64 oracle on those columns."""
    m, n, d, M, kappa, seed = 1 << 21, 512, 1024, 64, 4, 1
    say("blockperm full configuration")
    Ad = inputs.gaussian_torch(m, n, seed=0)
    Y = b.blockperm(Ad, d, M, kappa, seed)
    sync()
    cols = np.unique(np.concatenate([np.arange(0, n, 23), [1, 31, 32, 255, 480, 511]]))
    A_cols = Ad[:, torch.from_numpy(cols).to(Ad.device)].cpu().numpy()
    ref = oracle.blockperm_f64(A_cols, d, M, kappa, 1, seed)
    got = Y.cpu().numpy()[:, cols]
    err = oracle.rel_frob(got, ref)
    say(f"  rel err {err:.3e} on {len(cols)} columns")
    assert err <= 1e-5
    # unbiased norm: E||Sx||^2 = ||x||^2 holds for the whole output
    assert abs(float((Y.double() ** 2).sum() / (Ad.double() ** 2).sum()) - 1) < 0.05
