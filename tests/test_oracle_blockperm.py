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
    with pytest.raises(ValueError):
        blockperm_params(1024, 96, 8, 4, 2)        # s > 1 needs a power-of-two B_r
    with pytest.raises(ValueError):
        blockperm_params(1024, 64, 8, 9, 1, "affine")   # kappa > M


# --------------------------------------------- affine wiring and s > 1

@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 12, 60, 64, 97, 100, 128, 1024])
@pytest.mark.parametrize("seed", [0, 1, 12345678901])
def test_affine_map_is_a_full_cycle(M, seed):
    """Hull-Dobell: the drawn (a, b) make f(x) = (a x + b) mod M visit all of
    [M] from any start (checked by walking the orbit)."""
    import oracle
    a, b = oracle.affine_params(seed, M)
    assert 0 <= a < max(M, 2) and 0 <= b < max(M, 1)
    x, seen = 0, set()
    for _ in range(M):
        seen.add(x)
        x = (a * x + b) % M
    assert len(seen) == M and x == 0
    if M > 1:
        assert math.gcd(b, M) == 1
        for p in oracle.prime_factors(M):
            assert (a - 1) % p == 0
        if M % 4 == 0:
            assert (a - 1) % 4 == 0


@pytest.mark.parametrize("M,kappa", [(64, 4), (60, 7), (12, 12), (97, 3), (8, 1)])
def test_affine_wiring_biregular_edge_disjoint(M, kappa):
    import oracle
    N = oracle.wiring(5, M, kappa, "affine")
    for l in range(kappa):
        assert sorted(N[:, l].tolist()) == list(range(M))      # each pi_l a permutation
    assert all(len(set(N[g].tolist())) == kappa for g in range(M))   # edge-disjoint
    counts = np.bincount(N.ravel(), minlength=M)
    assert np.all(counts == kappa)


def test_affine_wiring_is_powers_of_f():
    import oracle
    a, b = oracle.affine_params(3, 64)
    N = oracle.affine_wiring(a, b, 64, 5)
    for g in (0, 17, 63):
        x = g
        for l in range(5):
            x = (a * x + b) % 64
            assert N[g, l] == x


@pytest.mark.parametrize("B_r,s", [(16, 1), (16, 2), (16, 4), (8, 8), (64, 3), (1, 1)])
def test_s_rows_distinct_and_s1_unchanged(B_r, s):
    import oracle
    r = np.arange(3000)
    rows, signs = oracle.blockperm_hash_s(9, 3, 5, r, B_r, s)
    assert rows.shape == (3000, s) and np.all((rows >= 0) & (rows < B_r))
    assert all(len(set(rows[i].tolist())) == s for i in range(0, 3000, 7))
    assert set(np.unique(signs).tolist()) <= {-1.0, 1.0}
    b1, s1 = blockperm_hash(9, 3, 5, r, B_r)
    assert np.array_equal(rows[:, 0], b1) and np.array_equal(signs[:, 0], s1)


@pytest.mark.parametrize("kind,kappa,s", [("affine", 3, 1), ("affine", 4, 2), ("shift", 4, 4),
                                          ("shift", 2, 2)])
def test_dense_brute_force_general(kind, kappa, s):
    """S built nonzero by nonzero equals the sparse construction; every
    column holds exactly kappa*s nonzeros of magnitude float32(1/sqrt(kappa s))."""
    import oracle
    m, d, M = 96, 64, 8
    Sd = oracle.blockperm_dense_S(m, d, M, kappa, s, 7, kind)
    Ss = oracle.blockperm_matrix(m, d, M, kappa, s, 7, kind=kind).toarray()
    assert np.array_equal(Sd, Ss)
    c = float(np.float32(1 / math.sqrt(kappa * s)))
    nnz = (Sd != 0).sum(axis=0)
    assert np.all(nnz == kappa * s)
    assert np.allclose(np.abs(Sd[Sd != 0]), c)
    A = np.random.default_rng(1).standard_normal((m, 5))
    assert np.allclose(oracle.blockperm_f64(A, d, M, kappa, s, 7, kind), Sd @ A, rtol=1e-12,
                       atol=1e-12)


def test_unbiased_norm_affine_s2():
    import oracle
    m, d, M, kappa, s = 256, 64, 8, 3, 2
    x = np.random.default_rng(2).standard_normal((m, 1))
    r = np.array([float((oracle.blockperm_f64(x, d, M, kappa, s, seed, "affine") ** 2).sum()
                        / (x ** 2).sum()) for seed in range(300)])
    assert abs(r.mean() - 1) < 5 * r.std(ddof=1) / math.sqrt(r.size)
