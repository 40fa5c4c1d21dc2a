"""Pins for the BlockPerm-SJLT oracle (FlashSketch page §4, Figure 2,
§6.3, App. A.2, A.7, App. D)."""
import math
import os

import numpy as np
import pytest

from oracle import (blockperm_dense_S, blockperm_f64, blockperm_hash, blockperm_matrix,
                    blockperm_params, fmix32, perm_sigma, shift_wiring)
from oracle.blockperm import block_key
from sparse_sketching_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "figure2_shapes.txt")


def _golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=")
            out[k.strip()] = int(v)
    return out


def test_figure2_shape_arithmetic():
    g = _golden()
    m, d = g["input_dim"], g["output_dim"]
    B_c, B_r = blockperm_params(m, d, g["M"], g["kappa"], g["s"])
    assert (B_c, B_r) == (g["B_c"], g["B_r"])
    assert g["kappa"] * g["s"] == g["nnz_per_column"]
    # with s = 1 (the case built here) every column holds kappa nonzeros
    S = blockperm_matrix(m, d, g["M"], g["kappa"], 1, seed=4)
    assert np.all(np.diff(S.tocsc().indptr) == g["kappa"])


def _fmix32_inverse(h):
    """Inverse of the MurmurHash3 finalizer from modular inverses."""
    h = np.asarray(h, dtype=np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(16)
    h = (h * np.uint64(pow(0xC2B2AE35, -1, 2**32))) & m32
    h ^= (h >> np.uint64(13)) ^ (h >> np.uint64(26))
    h = (h * np.uint64(pow(0x85EBCA6B, -1, 2**32))) & m32
    h ^= h >> np.uint64(16)
    return h.astype(np.uint32)


def test_fmix32_is_a_bijection():
    x = np.random.default_rng(0).integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(_fmix32_inverse(fmix32(x)), x)
    assert int(fmix32(0)) == 0 and int(fmix32(1)) != 1


def test_fmix32_avalanche():
    """Flipping one input bit flips each output bit with probability ~1/2."""
    x = np.random.default_rng(2).integers(0, 2**32, 20000, dtype=np.uint64)
    h0 = fmix32(x).astype(np.uint64)
    for b in (0, 5, 15, 31):
        h1 = fmix32(x ^ np.uint64(1 << b)).astype(np.uint64)
        diff = h0 ^ h1
        frac = np.array([((diff >> np.uint64(k)) & np.uint64(1)).mean() for k in range(32)])
        assert np.all(np.abs(frac - 0.5) < 0.05)


def test_sigma_is_permutation_and_seeded():
    for M in (1, 2, 16, 64, 100):
        s = perm_sigma(7, M)
        assert sorted(s.tolist()) == list(range(M))
    assert not np.array_equal(perm_sigma(1, 64), perm_sigma(2, 64))


@pytest.mark.parametrize("M,kappa", [(64, 4), (16, 4), (8, 2), (12, 3), (5, 1)])
def test_wiring_biregular_edge_disjoint(M, kappa):
    N = shift_wiring(perm_sigma(3, M), M, kappa)
    for g in range(M):
        assert len(set(N[g].tolist())) == kappa             # distinct neighbours
    cnt = np.bincount(N.ravel(), minlength=M)
    assert np.all(cnt == kappa)                             # each h used kappa times
    for j in range(kappa):
        assert sorted(N[:, j].tolist()) == list(range(M))   # each pi_j a permutation
    edges = {(g, int(h)) for g in range(M) for h in N[g]}
    assert len(edges) == M * kappa                          # edge-disjoint


def test_energy_identity_and_coherence_bounds():
    """App. A.2: sum_g ||x_N(g)||^2 = kappa ||x||^2; App. A.7:
    mu_blk/kappa <= mu_nbr <= mu_blk for an orthonormal U."""
    M, kappa, B = 64, 4, 8
    N = shift_wiring(perm_sigma(11, M), M, kappa)
    x = np.random.default_rng(0).standard_normal(M * B)
    xb = x.reshape(M, B)
    lhs = sum(float((xb[N[g]] ** 2).sum()) for g in range(M))
    assert math.isclose(lhs, kappa * float((x**2).sum()), rel_tol=1e-12)
    U = np.linalg.qr(np.random.default_rng(1).standard_normal((M * B, 6)) *
                     np.repeat(np.random.default_rng(2).uniform(0.1, 3, M), B)[:, None])[0]
    Ub = U.reshape(M, B, 6)
    mu_blk = M * max(np.linalg.norm(Ub[h], 2) ** 2 for h in range(M))
    mu_nbr = M / kappa * max(np.linalg.norm(Ub[N[g]].reshape(-1, 6), 2) ** 2 for g in range(M))
    assert mu_blk / kappa - 1e-12 <= mu_nbr <= mu_blk + 1e-12


def test_shift_family_components():
    """The shift family splits the block graph into M/kappa complete
    bipartite components: g and g' share N(g) iff sigma(g) = sigma(g') mod M/kappa."""
    M, kappa = 64, 4
    sigma = perm_sigma(5, M)
    N = shift_wiring(sigma, M, kappa)
    comps = {}
    for g in range(M):
        comps.setdefault(frozenset(N[g].tolist()), []).append(g)
    assert len(comps) == M // kappa
    for hs, gs in comps.items():
        assert len(gs) == kappa and len(hs) == kappa
        assert len({int(sigma[g]) % (M // kappa) for g in gs}) == 1


def test_dense_brute_force_tiny():
    m, n, d, M, kappa = 256, 5, 32, 4, 2          # B_c = 64, B_r = 8
    A = inputs.gaussian(m, n, seed=4)
    S = blockperm_dense_S(m, d, M, kappa, 1, seed=9)
    assert np.allclose(blockperm_f64(A, d, M, kappa, 1, 9), S @ A.astype(np.float64),
                       rtol=1e-13, atol=1e-12)
    assert np.allclose(blockperm_matrix(m, d, M, kappa, 1, 9).toarray(), S, rtol=0, atol=0)
    # column structure: kappa nonzeros of magnitude 1/sqrt(kappa), in distinct output blocks
    c = np.float32(1 / math.sqrt(kappa))
    for col in range(m):
        nz = np.nonzero(S[:, col])[0]
        assert len(nz) == kappa and np.all(np.abs(S[nz, col]) == np.float64(c))
        assert len(set((nz // (d // M)).tolist())) == kappa


def test_kappa1_is_localized_block_diagonal():
    """kappa = 1 gives the localized (block-diagonal up to a block
    permutation) SJLT: output block g reads only input block sigma(g)."""
    m, d, M = 512, 64, 8
    S = blockperm_dense_S(m, d, M, 1, 1, seed=2)
    sigma = perm_sigma(2, M)
    B_c, B_r = m // M, d // M
    for g in range(M):
        for h in range(M):
            blk = S[g * B_r:(g + 1) * B_r, h * B_c:(h + 1) * B_c]
            if h == sigma[g]:
                assert np.all(np.count_nonzero(blk, axis=0) == 1)
            else:
                assert not blk.any()


def test_hash_statistics():
    B_r, B_c = 16, 1 << 15
    r = np.arange(B_c)
    for (g, h) in [(0, 0), (3, 17), (63, 48)]:
        b, s = blockperm_hash(1, g, h, r, B_r)
        cnt = np.bincount(b, minlength=B_r)
        chi2 = float(((cnt - B_c / B_r) ** 2 / (B_c / B_r)).sum())
        assert chi2 < (B_r - 1) + 6 * math.sqrt(2 * (B_r - 1))
        assert abs(s.sum()) < 6 * math.sqrt(B_c)
    # different block pairs get different keys
    keys = {block_key(1, g, h) for g in range(64) for h in range(64)}
    assert len(keys) == 64 * 64


def test_unbiased_norm_over_seeds():
    """E ||S x||^2 = ||x||^2 (the scale 1/sqrt(kappa s) makes S isotropic)."""
    m, d, M, kappa = 1024, 64, 8, 4
    x = np.random.default_rng(3).standard_normal((m, 1))
    r = []
    for seed in range(400):
        y = blockperm_f64(x, d, M, kappa, 1, seed)
        r.append(float((y**2).sum() / (x**2).sum()))
    r = np.array(r)
    assert abs(r.mean() - 1) < 5 * r.std(ddof=1) / math.sqrt(r.size)


def test_invalid_shapes():
    with pytest.raises(ValueError):
        blockperm_params(1000, 64, 64, 4, 1)
    with pytest.raises(ValueError):
        blockperm_params(1024, 64, 64, 3, 1)
    with pytest.raises(NotImplementedError):
        blockperm_matrix(1024, 64, 8, 4, 2, 1)
