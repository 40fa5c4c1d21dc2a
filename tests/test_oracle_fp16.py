"""Pins for the oracle's FP16 pipeline: RN conversion of one contribution
and FP16 RN accumulation (FP16 sketching page §III-B, §III-D, §IV-A/B,
§V-C, §V-E).  The reference rounding here is exact rational arithmetic,
written independently of NumPy's float16 cast."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import meta_ref, rn_f16_add, scale_f32, sketch_f16_rn_emul, sketch_f64
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
