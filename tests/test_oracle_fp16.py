"""Pins for the oracle's FP16 pipeline: RN conversion of one contribution
and FP16 RN accumulation (FP16 sketching page §III-B, §III-D, §IV-A/B,
§V-C, §V-E).  The reference rounding here is exact rational arithmetic,
written independently of NumPy's float16 cast."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (dense_S, f16_erasures, f16_zero_subnormal_counts, meta_ref, rn_f16_add, scale_f32, sketch_f16_rn_emul,
                    sketch_f64, sketch_lowp_emul, sketch_matrix)
from sparse_sketching_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp16_rn_values.txt")
H = Fraction(1, 2**24)                    # binary16 subnormal spacing


def rn_binary16_exact(x):
    """Nearest-even binary16 of a rational x, returned as a Python float."""
    x = Fraction(x)
    if x == 0:
        return 0.0
    sgn = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                              # 2^e <= a < 2^(e+1)
    q = Fraction(2) ** (max(e, -14) - 10)   # spacing of the binade (or h)
    k = a / q
    f = math.floor(k)
    rem = k - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    v = f * q
    if v >= 2**16:
        return sgn * math.inf
    if v > 65504:
        return sgn * math.inf
    return sgn * float(v)


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            a, b, _ = [p.strip() for p in line.split("|")]
            rows.append((eval(a), float(eval(b.replace("inf", "float('inf')")))))
    return rows


@pytest.mark.parametrize("x,expect", _golden_rows())
def test_printed_rn_values(x, expect):
    got = np.float32(x).astype(np.float16)          # the oracle's conversion
    assert float(got) == expect and math.copysign(1, float(got)) == math.copysign(1, expect)
    assert rn_binary16_exact(Fraction(float(np.float32(x)))) == expect


def test_unit_roundoff_from_page():
    # u * sqrt(n) = 1/64 at n = 1024 (§V-C)  =>  u = 2^-11 = eps(binary16)/2.
    u = (1 / 64) / math.sqrt(1024)
    assert u == 2.0**-11 == float(np.finfo(np.float16).eps) / 2
    assert float(np.finfo(np.float16).smallest_subnormal) == float(H)


def test_conversion_matches_exact_rounding():
    g = np.random.default_rng(11)
    x = np.concatenate([
        g.standard_normal(4000).astype(np.float32),
        (g.standard_normal(2000) * 2.0**-20).astype(np.float32),   # subnormal range
        (g.standard_normal(2000) * 2.0**-26).astype(np.float32),   # below h/2
        (g.uniform(6.0e4, 6.6e4, 1000) * g.choice([-1, 1], 1000)).astype(np.float32),
        # exact ties: odd multiples of half a spacing
        (np.float32(2.0**-25) * (2 * g.integers(0, 2**10, 1000) + 1)).astype(np.float32),
    ])
    conv = x.astype(np.float16)
    for xi, ci in zip(x, conv):
        assert float(ci) == rn_binary16_exact(Fraction(float(xi))), xi


def test_rn_f16_add_is_correctly_rounded():
    g = np.random.default_rng(5)
    bits = g.integers(0, 2**16, size=(2, 20000), dtype=np.uint16)
    a, b = bits[0].view(np.float16), bits[1].view(np.float16)
    ok = np.isfinite(a) & np.isfinite(b)
    a, b = a[ok], b[ok]
    s = rn_f16_add(a, b)
    for ai, bi, si in zip(a, b, s):
        ref = rn_binary16_exact(Fraction(float(ai)) + Fraction(float(bi)))
        assert float(si) == ref or (ref == 0.0 and float(si) == 0.0), (ai, bi, si)


def test_flat_emulation_matches_scalar_loop():
    """Tiny case: the vectorised rank-by-rank emulation equals a plain loop
    over contributions in ascending (i, t) order with exact rounding."""
    m, n, d, zeta = 96, 3, 8, 2
    A = (inputs.gaussian(m, n, seed=3) * np.float32(37.0)).astype(np.float32)
    ri, v = meta_ref(9, m, d, zeta)
    B = [[0.0] * n for _ in range(d)]
    for e in range(m * zeta):
        i = e // zeta
        for j in range(n):
            q = float(np.float32(A[i, j]) * np.float32(v[e]))       # FP32 product
            c = rn_binary16_exact(Fraction(q))                       # RN to FP16
            B[ri[e]][j] = rn_binary16_exact(Fraction(B[ri[e]][j]) + Fraction(c))
    got = sketch_f16_rn_emul(A, ri, v, d, zeta)
    assert np.array_equal(got.astype(np.float64), np.array(B))


def test_two_level_orders():
    m, n, d, zeta = 512, 4, 16, 4
    A = inputs.gaussian(m, n, seed=1)
    ri, v = meta_ref(2, m, d, zeta)
    flat = sketch_f16_rn_emul(A, ri, v, d, zeta)
    assert np.array_equal(sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=m), flat)
    # chunk of one row: each partial holds one contribution per bucket at most
    # (zeta blocks of distinct rows), so partial = contribution exactly.
    one = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=1)
    assert np.array_equal(one, flat)
    two = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=64)
    B64 = sketch_f64(A, ri, v, d, zeta)
    assert np.linalg.norm(two - B64) / np.linalg.norm(B64) < 4e-3


def test_exact_case_half_integers():
    """A in {-1,0,1}, zeta=4: every contribution is +-1/2 or 0 and every
    partial sum is a half-integer of magnitude < 1024, exact in binary16."""
    m, n, d, zeta = 4096, 32, 64, 4
    A = inputs.integer_matrix(m, n, -1, 1, seed=0)
    ri, v = meta_ref(1, m, d, zeta)
    load = np.bincount(ri, minlength=d).max()
    assert 0.5 * load < 1024
    B16 = sketch_f16_rn_emul(A, ri, v, d, zeta)
    assert np.array_equal(B16.astype(np.float64), sketch_f64(A, ri, v, d, zeta))


def test_conversion_error_bound_and_sign_cancellation():
    """§IV-B: sum of squared conversion errors <= u^2 ||A||_F^2 in the normal
    range (each contribution has |e| <= u|q| and sum q^2 = ||A||_F^2), and
    the signed error averages to zero over sketch seeds."""
    m, n, d, zeta = 2048, 16, 64, 4
    g = np.random.default_rng(4)
    A = (g.uniform(1.0, 2.0, (m, n)) * g.choice([-1, 1], (m, n))).astype(np.float32)
    u = 2.0**-11
    tot = []
    for seed in range(40):
        ri, v = meta_ref(seed, m, d, zeta)
        i = np.arange(m * zeta) // zeta
        q = (A[i] * v[:, None]).astype(np.float32)
        e = q.astype(np.float16).astype(np.float64) - q.astype(np.float64)
        assert float((e**2).sum()) <= u**2 * float((A.astype(np.float64) ** 2).sum())
        # signed error summed into each bucket: E over signs is zero
        Be = np.zeros((d, n))
        np.add.at(Be, ri, e)
        tot.append(Be.sum())
    tot = np.array(tot)
    assert abs(tot.mean()) < 5 * tot.std(ddof=1) / np.sqrt(tot.size)


def test_fp16_flat_vs_fp64_error_model():
    """Flat FP16 accumulation of K contributions per entry loses accuracy
    like u*sqrt(K/12); a 64-row-chunk two-level order keeps it near 1e-3."""
    m, n, d, zeta = 8192, 16, 16, 4          # K = m*zeta/d = 2048
    A = inputs.gaussian(m, n)
    ri, v = meta_ref(3, m, d, zeta)
    B64 = sketch_f64(A, ri, v, d, zeta)
    flat = np.linalg.norm(sketch_f16_rn_emul(A, ri, v, d, zeta) - B64) / np.linalg.norm(B64)
    pred = 2.0**-11 * math.sqrt(2048 / 12)
    assert 0.25 * pred < flat < 4 * pred
    two = np.linalg.norm(sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=256) - B64) / np.linalg.norm(B64)
    assert two < flat


def test_scale_is_exact_at_zeta4():
    assert scale_f32(4) == np.float32(0.5) and scale_f32(1) == np.float32(1.0)


def _scalar_two_level(A, ri, v, d, zeta, chunk_rows, B0=None):
    """Plain loop with exact rational rounding: each chunk of rows summed in
    ascending (i, t) order from +0 into its own partial, the partials then
    added in chunk order, every addition rounded to binary16."""
    m, n = A.shape
    B = [[0.0] * n for _ in range(d)] if B0 is None else [list(map(float, r)) for r in B0]
    for r0 in range(0, m, chunk_rows):
        P = [[0.0] * n for _ in range(d)]
        for e in range(r0 * zeta, min(m, r0 + chunk_rows) * zeta):
            i = e // zeta
            for j in range(n):
                q = float(np.float32(A[i, j]) * np.float32(v[e]))
                c = rn_binary16_exact(Fraction(q))
                P[ri[e]][j] = rn_binary16_exact(Fraction(P[ri[e]][j]) + Fraction(c))
        for r in range(d):
            for j in range(n):
                B[r][j] = rn_binary16_exact(Fraction(B[r][j]) + Fraction(P[r][j]))
    return np.array(B)


def _scalar_grouped(A, ri, v, d, zeta, chunk_rows, groups, B0=None):
    """Plain loop with exact rational rounding for the grouped combine:
    chunk partials as above, then G contiguous groups of them (group w:
    chunks [w*P//G, (w+1)*P//G)), each summed from +0 in chunk order, and
    the non-empty group sums added in group order onto B0 or +0; every
    addition rounded to binary16."""
    m, n = A.shape
    parts = []
    for r0 in range(0, m, chunk_rows):
        P = [[0.0] * n for _ in range(d)]
        for e in range(r0 * zeta, min(m, r0 + chunk_rows) * zeta):
            i = e // zeta
            for j in range(n):
                q = float(np.float32(A[i, j]) * np.float32(v[e]))
                c = rn_binary16_exact(Fraction(q))
                P[ri[e]][j] = rn_binary16_exact(Fraction(P[ri[e]][j]) + Fraction(c))
        parts.append(P)
    B = [[0.0] * n for _ in range(d)] if B0 is None else [list(map(float, r)) for r in B0]
    npart = len(parts)
    for w in range(groups):
        lo, hi = w * npart // groups, (w + 1) * npart // groups
        if hi == lo:
            continue
        Q = [[0.0] * n for _ in range(d)]
        for P in parts[lo:hi]:
            for r in range(d):
                for j in range(n):
                    Q[r][j] = rn_binary16_exact(Fraction(Q[r][j]) + Fraction(P[r][j]))
        for r in range(d):
            for j in range(n):
                B[r][j] = rn_binary16_exact(Fraction(B[r][j]) + Fraction(Q[r][j]))
    return np.array(B)


@pytest.mark.parametrize("chunk_rows,groups", [(1, 4), (7, 4), (32, 3), (10, 64)])
def test_grouped_combine_matches_scalar_loop(chunk_rows, groups):
    """The grouped chunk combine equals a plain loop with exact rounding,
    from +0 and from an existing sketch B0 (more groups than chunks leave
    groups empty)."""
    m, n, d, zeta = 160, 3, 8, 2
    A = (inputs.gaussian(m, n, seed=15) * np.float32(91.0)).astype(np.float32)
    ri, v = meta_ref(14, m, d, zeta)
    got = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=chunk_rows, groups=groups)
    assert np.array_equal(got.astype(np.float64),
                          _scalar_grouped(A, ri, v, d, zeta, chunk_rows, groups))
    B0 = (inputs.gaussian(d, n, seed=16) * np.float32(300.0)).astype(np.float16)
    got0 = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=chunk_rows, groups=groups, B0=B0)
    assert np.array_equal(got0.astype(np.float64),
                          _scalar_grouped(A, ri, v, d, zeta, chunk_rows, groups, B0=B0))


def test_grouped_combine_association():
    """One output entry, one-row chunks with partials 2048, 0, 1, 1 (d = 1,
    zeta = 1, values +1).  Added one after another each +1 is a tie at 2048
    (spacing 2) and rounds back to 2048; in two groups (2048 + 0) and
    (1 + 1) = 2 the total is 2048 + 2 = 2050, exact.  Groups of one chunk
    each, or one group, give the sequential order."""
    A = np.array([[2048.0], [0.0], [1.0], [1.0]], dtype=np.float32)
    ri = np.zeros(4, dtype=np.int32)
    v = np.ones(4, dtype=np.float32)
    seq = sketch_f16_rn_emul(A, ri, v, 1, 1, chunk_rows=1)
    assert float(seq[0, 0]) == 2048.0
    assert float(sketch_f16_rn_emul(A, ri, v, 1, 1, chunk_rows=1, groups=2)[0, 0]) == 2050.0
    for g in (1, 4, 8):
        assert float(sketch_f16_rn_emul(A, ri, v, 1, 1, chunk_rows=1, groups=g)[0, 0]) == 2048.0
    # FP32 combine: (2048 + 0) + (1 + 1) and the sequential FP32 sum are both
    # exact, 2050 rounded once
    for g in (None, 2, 4):
        assert float(sketch_f16_rn_emul(A, ri, v, 1, 1, chunk_rows=1, combine="f32",
                                        groups=g)[0, 0]) == 2050.0


@pytest.mark.parametrize("chunk_rows", [1, 7, 32, 200])
def test_two_level_matches_scalar_loop(chunk_rows):
    """The chunked (two-level) FP16 order equals a plain loop with exact
    rounding, also when it starts from an existing sketch B0."""
    m, n, d, zeta = 160, 3, 8, 2
    A = (inputs.gaussian(m, n, seed=5) * np.float32(91.0)).astype(np.float32)
    ri, v = meta_ref(4, m, d, zeta)
    got = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=chunk_rows)
    assert np.array_equal(got.astype(np.float64), _scalar_two_level(A, ri, v, d, zeta, chunk_rows))
    B0 = (inputs.gaussian(d, n, seed=6) * np.float32(300.0)).astype(np.float16)
    got0 = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=chunk_rows, B0=B0)
    assert np.array_equal(got0.astype(np.float64),
                          _scalar_two_level(A, ri, v, d, zeta, chunk_rows, B0=B0))


def test_combine_f32_overflow_between_chunks():
    """Partials 60000, 30000, -50000 on one entry: FP16 additions overflow
    after the second partial (90000 > 65504) and stay infinite; an FP32
    combine rounds the finite total 40000 (exact in binary16) once."""
    d, zeta = 1, 1
    ri, v = meta_ref(1, 3, d, zeta)
    want = np.array([60000.0, 30000.0, -50000.0])
    A = (want / v.astype(np.float64)).astype(np.float32)[:, None]
    f16 = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=1, combine="f16")
    f32 = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=1, combine="f32")
    assert np.isinf(f16[0, 0]) and f16[0, 0] > 0
    assert float(f32[0, 0]) == 40000.0
    # one chunk: nothing to combine, both equal the flat order
    flat = sketch_f16_rn_emul(A, ri, v, d, zeta)
    for c in ("f16", "f32"):
        assert np.array_equal(sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=3, combine=c), flat)


def test_combine_f32_rounds_the_exact_sum_once():
    """One-row chunks: each partial is RN_f16(k 2^-10), a multiple of 2^-10
    below 2^4, so 64 of them add exactly in FP32 and the FP32 combine is the
    exactly rounded binary16 of the partials' sum."""
    m, n, d, zeta = 64, 4, 4, 1
    g = np.random.default_rng(3)
    ri, v = meta_ref(2, m, d, zeta)
    k = g.integers(-2**14, 2**14, size=(m, n))
    A = (k * 2.0**-10 / v.astype(np.float64)[:, None]).astype(np.float32)   # q = k 2^-10
    got = sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=1, combine="f32")
    for r in range(d):
        for j in range(n):
            parts = [Fraction(rn_binary16_exact(Fraction(int(k[i, j]), 2**10)))
                     for i in range(m) if ri[i] == r]
            assert float(got[r, j]) == rn_binary16_exact(sum(parts, Fraction(0)))


def test_out_of_block_entries_contribute_nothing():
    """Every oracle function applies the same rule: entry i*zeta + t counts
    only if its row lies in block t.  Planting rows outside [0, d) or in
    another block gives the sketch of the metadata with those entries'
    values set to zero."""
    m, n, d, zeta = 300, 4, 16, 4
    A = inputs.gaussian(m, n, seed=2)
    ri, v = meta_ref(5, m, d, zeta)
    bad = ri.copy()
    g = np.random.default_rng(0)
    sel = g.choice(m * zeta, size=60, replace=False)
    t = sel % zeta
    bad[sel[:20]] = ((t[:20] + 1) % zeta) * (d // zeta)        # another block
    bad[sel[20:40]] = d + 3                                       # past the end
    bad[sel[40:]] = -1                                            # negative
    zeroed = v.copy()
    zeroed[sel] = 0.0
    assert np.array_equal(sketch_f64(A, bad, v, d, zeta), sketch_f64(A, ri, zeroed, d, zeta))
    assert np.array_equal(dense_S(bad, v, m, d, zeta), dense_S(ri, zeroed, m, d, zeta))
    assert np.array_equal(sketch_matrix(bad, v, m, d, zeta).toarray(),
                          sketch_matrix(ri, zeroed, m, d, zeta).toarray())
    for ch in (None, 64):
        assert np.array_equal(sketch_f16_rn_emul(A, bad, v, d, zeta, chunk_rows=ch),
                              sketch_f16_rn_emul(A, ri, zeroed, d, zeta, chunk_rows=ch))
    for fmt, conv in (("f16", "rn"), ("f16", "sr"), ("bf16", "rn")):
        assert np.array_equal(sketch_lowp_emul(A, bad, v, d, zeta, fmt, conv, sr_seed=3),
                              sketch_lowp_emul(A, ri, zeroed, d, zeta, fmt, conv, sr_seed=3))


def test_f16_erasures_closed_form():
    """Coordinate-like input whose entries are placed around h/2 = 2^-25
    after the 1/2 scale (FP16 page §V-E: RN erases contributions below h/2,
    the tie at h/2 included): the counts follow from each entry's value."""
    m, n, d, zeta = 64, 8, 16, 4
    row = np.array([2.0**-24,                 # q = h/2: a tie, rounds to 0
                    2.0**-24 * (1 + 2.0**-20),  # just above h/2: rounds to h
                    2.0**-30,                 # far below: 0
                    -(2.0**-25),              # q = -h/4: -0
                    1.0,                      # normal
                    0.0,                      # zero: not a contribution
                    2.0**-13,                 # q = 2^-14, the smallest normal
                    3 * 2.0**-15],            # q = 1.5 * 2^-15: subnormal
                   dtype=np.float32)
    A = np.tile(row, (m, 1)).astype(np.float32)
    ri, v = meta_ref(3, m, d, zeta)
    erased, sub, total = f16_erasures(A, ri, v, d, zeta)
    per_row = m * zeta
    assert total == 7 * per_row
    assert erased == 3 * per_row
    assert sub == 2 * per_row
    # the entry-by-entry count, with one entry's value of magnitude 3/4:
    # its products of 2^-24 (3h/4 -> h) and 3 * 2^-15 (1.125 * 2^-14,
    # normal) move, so one erasure less and one subnormal in, one out
    v2 = v.copy()
    v2[1] = np.float32(np.sign(v[1]) * 0.75)
    assert f16_erasures(A, ri, v2, d, zeta) == (erased - 1, sub, total)


def test_zero_subnormal_thresholds_match_the_conversion():
    """The threshold classification of f16_zero_subnormal_counts equals the
    nearest-even cast itself on values around h/2 and 2^-14 - h/2 (every
    FP32 value in a window around each threshold) and on random magnitudes
    across the subnormal range."""
    def by_cast(q):
        c = q.astype(np.float16).astype(np.float64)
        nz = q != 0
        return int((nz & (c == 0)).sum()), int(((c > 0) & (c < 2.0**-14)).sum()), int(nz.sum())
    for t in (2.0**-25, 2.0**-14 - 2.0**-25):
        bits = np.float32(t).view(np.uint32)
        q = (np.arange(-4096, 4097, dtype=np.int64) + int(bits)).astype(np.uint32).view(np.float32)
        assert f16_zero_subnormal_counts(q) == by_cast(q)
    g = np.random.default_rng(1)
    q = (2.0 ** g.uniform(-30, -12, 200000)).astype(np.float32)
    q[::7] = 0
    assert f16_zero_subnormal_counts(q) == by_cast(q)
