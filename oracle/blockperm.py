"""BlockPerm-SJLT oracle.  TEST INFRASTRUCTURE ONLY.

Follows "FlashSketch: Sketch-Kernel Co-Design for Fast Sparse Sketching on
GPUs", written in the FP16 sketching page's letters (A is m x n, S is d x m,
Y = SA is d x n; the FlashSketch page calls these d, k and k x n):

* §4 (block model): the m input rows form M contiguous blocks of
  B_c = m/M rows, the d output rows form M blocks of B_r = d/M rows;
  output block g reads the input blocks of its neighbourhood N(g).
* §4 and App. D: N(g) is the union of kappa edge-disjoint permutations.
  The family used here is the shift family pi_j(g) = (sigma(g) + j*M/kappa)
  mod M, j = 0..kappa-1, with sigma a seeded permutation of [M]; for a fixed
  g the kappa shifts are distinct, so the permutations are edge-disjoint.
* §4 (intra-block mixing) and App. A.1: block (g, h) with h in N(g) is an
  SJLT Phi_{g,h} with s nonzeros +-1/sqrt(s) per column, and the block is
  scaled by 1/sqrt(kappa) (the squared-norm identity of App. A.5 has the
  factor 1/kappa in front of the sum of ||Phi_g x_N(g)||^2, so the
  per-block scale is 1/sqrt(kappa); the extracted text of §4 lost the
  square root).  Each nonzero is therefore +-1/sqrt(kappa*s).
* §5.2 and App. D (within-block hashing): each input row of block h is
  combined with (g, h) and a seed by a fast 32-bit mixing hash to give its
  output row in [B_r] and an independent Rademacher sign.

Readings where the page is silent (each listed in the design notes):
* sigma: Fisher-Yates over [M]; for k = M-1 down to 1 the swap partner is
  floor(w0 * (k+1) / 2^32) with w0 the first word of
  Philox-4x32-10(counter = (k, 0, 0, 2), key = (seed lo, seed hi));
* the 32-bit mixing hash is MurmurHash3's 32-bit finalizer (Appleby),
  fmix32; the block key is K(g,h) = c(c(c(c(0x9E3779B9, seed lo), seed hi),
  g), h) with c(H, x) = fmix32(H ^ x) + 0x9E3779B9 mod 2^32; the row value
  is v = fmix32(K(g,h) ^ r) with r the row index inside block h; the output
  row is floor(v * B_r / 2^32) and the sign is negative when bit 0 of v is
  set.
* s > 1 (App. D: s unique rows from an affine map whose scale and shift come
  from the hash): with beta = floor(v * B_r / 2^32) and
  w = fmix32(v + 0x9E3779B9), alpha = 2 * floor(w * (B_r/2) / 2^32) + 1
  (odd, so a unit modulo B_r when B_r is a power of two, which s > 1
  requires); the rows are (beta + j*alpha) mod B_r for j = 0..s-1 (distinct)
  and the sign of row j is negative when bit j of v is set.  s = 1 reduces
  to the rule above.
* The affine full-cycle wiring (App. D: f(x) = (a x + b) mod M with
  pi_l = f^l, l = 1..kappa, parameters meeting the Hull-Dobell conditions
  so f visits all of [M]): with L = the product of the distinct primes of
  M, times 2 more when 4 | M, a = 1 + L * floor(w0 * (M/L) / 2^32) (a = 1
  when L >= M) and b the floor(w1 * phi(M) / 2^32)-th unit modulo M in
  ascending order, where (w0, w1) are the first two words of
  Philox-4x32-10(counter = (0, 0, 0, 1), key = (seed lo, seed hi)).
"""
import numpy as np
import scipy.sparse as sp

from .philox import philox4x32_10

_U32 = 0xFFFFFFFF
_GOLD = 0x9E3779B9


def fmix32(x):
    """MurmurHash3 32-bit finalizer on uint32 arrays (or scalars)."""
    x = np.asarray(x, dtype=np.uint64) & np.uint64(_U32)
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x85EBCA6B)) & np.uint64(_U32)
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(0xC2B2AE35)) & np.uint64(_U32)
    x ^= x >> np.uint64(16)
    return x.astype(np.uint32)


def _combine(h, x):
    return (int(fmix32(int(h) ^ (int(x) & _U32))) + _GOLD) & _U32


def block_key(seed, g, h):
    """K(g, h): the per-block-pair key of the within-block hash."""
    seed = int(seed)
    k = _combine(_GOLD, seed & _U32)
    k = _combine(k, (seed >> 32) & _U32)
    k = _combine(k, g)
    return _combine(k, h)


def perm_sigma(seed, M):
    """Seeded permutation sigma of [M] (Fisher-Yates, Philox draws)."""
    seed = int(seed)
    sigma = list(range(M))
    for k in range(M - 1, 0, -1):
        w0 = int(philox4x32_10(k, 0, 0, 2, seed & _U32, (seed >> 32) & _U32)[0])
        j = (w0 * (k + 1)) >> 32
        sigma[k], sigma[j] = sigma[j], sigma[k]
    return np.array(sigma, dtype=np.int64)


def prime_factors(M):
    """Distinct primes of M (trial division)."""
    out, p, x = [], 2, int(M)
    while p * p <= x:
        if x % p == 0:
            out.append(p)
            while x % p == 0:
                x //= p
        p += 1
    if x > 1:
        out.append(x)
    return out


def affine_params(seed, M):
    """(a, b) of the full-cycle map f(x) = (a x + b) mod M drawn from the seed
    (Hull-Dobell: gcd(b, M) = 1, a - 1 divisible by every prime of M, and by
    4 when 4 | M)."""
    seed = int(seed)
    if M == 1:
        return 1, 0
    w = philox4x32_10(0, 0, 0, 1, seed & _U32, (seed >> 32) & _U32)
    w0, w1 = int(w[0]), int(w[1])
    L = 1
    for p in prime_factors(M):
        L *= p
    if M % 4 == 0:
        L *= 2 if L % 4 else 1
    a = 1 + L * ((w0 * (M // L)) >> 32) if L < M else 1
    units = [u for u in range(1, M) if np.gcd(u, M) == 1]
    b = units[(w1 * len(units)) >> 32]
    return a, b


def affine_wiring(a, b, M, kappa):
    """N[g, l-1] = f^l(g), l = 1..kappa, for f(x) = (a x + b) mod M."""
    if not 1 <= kappa <= M:
        raise ValueError("the affine family needs 1 <= kappa <= M")
    N = np.zeros((M, kappa), dtype=np.int64)
    x = np.arange(M, dtype=np.int64)
    for l in range(kappa):
        x = (a * x + b) % M
        N[:, l] = x
    return N


def wiring(seed, M, kappa, kind="shift"):
    """The kappa neighbours of every output block: N[g] (M x kappa)."""
    if kind == "shift":
        return shift_wiring(perm_sigma(seed, M), M, kappa)
    if kind == "affine":
        a, b = affine_params(seed, M)
        return affine_wiring(a, b, M, kappa)
    raise ValueError(kind)


def shift_wiring(sigma, M, kappa):
    """N[g, j] = (sigma[g] + j*M/kappa) mod M: kappa edge-disjoint permutations."""
    if M % kappa:
        raise ValueError("the shift family needs kappa | M")
    j = np.arange(kappa, dtype=np.int64)
    return (np.asarray(sigma, dtype=np.int64)[:, None] + j[None, :] * (M // kappa)) % M


def blockperm_params(m, d, M, kappa, s, kind="shift"):
    """(B_c, B_r) = (m/M, d/M) for the block model of §4."""
    if m % M or d % M:
        raise ValueError("m and d must be multiples of M")
    if kind == "shift" and M % kappa:
        raise ValueError("the shift family needs kappa | M")
    if not 1 <= kappa <= M or not 1 <= s <= d // M:
        raise ValueError("need 1 <= kappa <= M and 1 <= s <= B_r")
    B_r = d // M
    if s > 1 and (B_r & (B_r - 1)):
        raise ValueError("s > 1 needs a power-of-two B_r")
    if s > 32:
        raise ValueError("s <= 32 (one sign bit per row)")
    return m // M, B_r


def blockperm_hash(seed, g, h, r, B_r):
    """(output row in [B_r], sign) for rows r (array) of input block h in
    output block g (s = 1)."""
    v = fmix32(np.uint64(block_key(seed, g, h)) ^ np.asarray(r, dtype=np.uint64)).astype(np.uint64)
    bucket = ((v * np.uint64(B_r)) >> np.uint64(32)).astype(np.int64)
    sign = np.where((v & np.uint64(1)).astype(bool), -1.0, 1.0)
    return bucket, sign


def blockperm_hash_s(seed, g, h, r, B_r, s):
    """(rows, signs), each len(r) x s: the s distinct output rows in [B_r]
    of rows r of input block h in output block g, and their signs."""
    r = np.asarray(r, dtype=np.uint64)
    v = fmix32(np.uint64(block_key(seed, g, h)) ^ r).astype(np.uint64)
    beta = ((v * np.uint64(B_r)) >> np.uint64(32)).astype(np.int64)
    if s == 1:
        alpha = np.zeros_like(beta)
    else:
        w = fmix32((v + np.uint64(_GOLD)) & np.uint64(_U32)).astype(np.uint64)
        alpha = 2 * ((w * np.uint64(B_r // 2)) >> np.uint64(32)).astype(np.int64) + 1
    j = np.arange(s, dtype=np.int64)
    rows = (beta[:, None] + j[None, :] * alpha[:, None]) % B_r
    bits = (v[:, None] >> j[None, :].astype(np.uint64)) & np.uint64(1)
    signs = np.where(bits.astype(bool), -1.0, 1.0)
    return rows, signs


def _scale(kappa, s):
    return np.float64(np.float32(1.0 / np.sqrt(np.float64(kappa * s))))


def blockperm_matrix(m, d, M, kappa, s, seed, blocks=None, kind="shift"):
    """S (d x m, sparse) restricted to the columns of the listed input blocks
    (all blocks when blocks is None)."""
    B_c, B_r = blockperm_params(m, d, M, kappa, s, kind)
    N = wiring(seed, M, kappa, kind)
    want = set(range(M)) if blocks is None else set(int(b) for b in blocks)
    c = _scale(kappa, s)
    rows, cols, vals = [], [], []
    r = np.arange(B_c, dtype=np.int64)
    for g in range(M):
        for h in N[g]:
            h = int(h)
            if h not in want:
                continue
            rr, sg = blockperm_hash_s(seed, g, h, r, B_r, s)
            rows.append((g * B_r + rr).ravel())
            cols.append(np.repeat(h * B_c + r, s))
            vals.append((sg * c).ravel())
    if not rows:
        return sp.csr_matrix((d, m))
    return sp.csr_matrix((np.concatenate(vals), (np.concatenate(rows), np.concatenate(cols))),
                         shape=(d, m))


def blockperm_dense_S(m, d, M, kappa, s, seed, kind="shift"):
    """Dense S built block pair by block pair, row by row and nonzero by
    nonzero (tiny inputs)."""
    B_c, B_r = blockperm_params(m, d, M, kappa, s, kind)
    N = wiring(seed, M, kappa, kind)
    c = _scale(kappa, s)
    S = np.zeros((d, m), dtype=np.float64)
    for g in range(M):
        for h in N[g]:
            for r in range(B_c):
                rr, sg = blockperm_hash_s(seed, g, int(h), np.array([r]), B_r, s)
                for j in range(s):
                    S[g * B_r + int(rr[0, j]), int(h) * B_c + r] += float(sg[0, j]) * c
    return S


def blockperm_f64(A, d, M, kappa, s, seed, kind="shift"):
    """Y = S A in fp64, one input block at a time."""
    m, n = A.shape
    B_c, _ = blockperm_params(m, d, M, kappa, s, kind)
    Y = np.zeros((d, n), dtype=np.float64)
    for h in range(M):
        S = blockperm_matrix(m, d, M, kappa, s, seed, blocks=[h], kind=kind)
        Y += S[:, h * B_c:(h + 1) * B_c] @ np.asarray(A[h * B_c:(h + 1) * B_c], dtype=np.float64)
    return Y
