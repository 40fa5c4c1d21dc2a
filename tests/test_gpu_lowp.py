"""GPU parity of the conversion variants (sk_apply_lowp: FP16 with
nearest-even or stochastic conversion, BF16 with nearest-even conversion)
against the CPU oracle (FP16 sketching page §III-D, §V-E).

Bars: one contribution per output entry (coordinate inputs) makes B the
converted contribution itself, compared bit for bit, SR draws included;
sums that stay exact (integers for BF16, multiples of the FP16 subnormal
step for SR) are compared bit for bit in any order; otherwise relative
Frobenius error against fp64 within the random-walk bar of the format."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu

U_BF16 = 2.0**-8


def as_f64(B):
    return B.float().cpu().numpy().astype(np.float64)


VARIANT = {"flat": 0, "reg": b.SK_VARIANT_REG}


def run(A, d, zeta, seed, fmt, conv, sr_seed=0, row_offset=0, meta=None, variant="flat"):
    Ad = A if isinstance(A, torch.Tensor) else to_dev(A)
    m = Ad.shape[0]
    ri, v = meta if meta is not None else b.meta(seed, m, d, zeta, row_offset=row_offset,
                                                 device=dev())
    B = b.apply_lowp(Ad, ri, v, zeta, d, fmt, conv, sr_seed=sr_seed, row_offset=row_offset,
                     flags=VARIANT[variant])
    sync()
    return as_f64(B)


@pytest.mark.parametrize("variant", ["flat", "reg"])
@pytest.mark.parametrize("fmt,conv", [("f16", "rn"), ("f16", "sr"), ("bf16", "rn")])
def test_one_conversion_per_entry(fmt, conv, variant):
    """Coordinate input times values spanning ties, subnormals and
    overflow: every output entry receives exactly one contribution q, so B
    is the oracle's conversion of q (with that entry's SR draw)."""
    say(f"lowp coordinate {fmt} {conv} {variant}")
    m, n, d, zeta, seed, sr_seed, off = 4096, 64, 64, 4, 3, 77, 5000
    specials = np.array([2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-20 * 3, 2.0**16, 65504 * 2,
                         65520 * 2, 70000 * 2, -(2.0**-23), 1 + 2.0**-10, 1 + 3 * 2.0**-11,
                         2.0**-14, 1e-9, -7.0e4 * 2, 12345.678, 1e-40, 3.0e38, 1 + 2.0**-7,
                         1 + 3 * 2.0**-8, 0.1, -0.3, 2.0**-133, 1e30, 7.25],
                        dtype=np.float32)
    vals = np.resize(specials, n)
    A = inputs.coordinate(m, n) * vals[None, :]
    B = run(A, d, zeta, seed, fmt, conv, sr_seed=sr_seed, row_offset=off, variant=variant)
    ri, v = oracle.meta_ref(seed, m, d, zeta, row_offset=off)
    expect = oracle.sketch_lowp_emul(A, ri, v, d, zeta, fmt, conv, sr_seed=sr_seed,
                                     row_offset=off).astype(np.float64)
    assert np.array_equal(B, expect, equal_nan=True)
    assert np.array_equal(np.signbit(B), np.signbit(expect))


@pytest.mark.parametrize("variant", ["flat", "reg"])
def test_sr_exact_sums_match_oracle_draw_for_draw(variant):
    """Contributions below the FP16 normal range: SR turns each into a
    multiple of h = 2^-24, and the sums (|sum| <= K h < 2^-13) stay exact
    multiples of h, so the GPU result must equal the oracle's SR sketch bit
    for bit: same draws, same decisions, whatever the atomic order."""
    m, n, d, zeta, seed, sr_seed, off = 4096, 64, 64, 4, 11, 2024, 123
    A = (inputs.gaussian(m, n, seed=5) * np.float32(2.0**-25)).astype(np.float32)
    ri, v = oracle.meta_ref(seed, m, d, zeta, row_offset=off)
    B = run(A, d, zeta, seed, "f16", "sr", sr_seed=sr_seed, row_offset=off, variant=variant)
    expect = oracle.sketch_lowp_emul(A, ri, v, d, zeta, "f16", "sr", sr_seed=sr_seed,
                                     row_offset=off).astype(np.float64)
    assert np.abs(expect).max() < 2.0**-13
    assert np.array_equal(B, expect)


@pytest.mark.parametrize("variant", ["flat", "reg"])
def test_bf16_exact_inputs_bit_exact(variant):
    m, n, d, zeta = 4096, 64, 64, 4
    A = inputs.integer_matrix(m, n, -3, 3, seed=8)
    ri, v = oracle.meta_ref(2, m, d, zeta)
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    assert np.abs(ref).max() <= 256                 # every partial sum exact in BF16
    assert np.array_equal(run(A, d, zeta, 2, "bf16", "rn", variant=variant), ref)


@pytest.mark.parametrize("variant", ["flat", "reg"])
@pytest.mark.parametrize("fmt,conv,u", [("f16", "rn", 2.0**-11), ("f16", "sr", 2.0**-11),
                                        ("bf16", "rn", U_BF16)])
def test_gaussian_within_random_walk_bar(fmt, conv, u, variant):
    """N(0,1) input: relative Frobenius error against fp64 within four times
    the random-walk estimate u*sqrt(K/12) of a K-term running sum (SR adds
    its conversion variance, at most u per term in relative terms)."""
    m, n, d, zeta = 8192, 64, 64, 4
    A = inputs.gaussian(m, n, seed=9)
    ri, v = oracle.meta_ref(4, m, d, zeta)
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    K = m * zeta // d
    err = oracle.rel_frob(run(A, d, zeta, 4, fmt, conv, sr_seed=1, variant=variant), ref)
    say(f"  {fmt} {conv} {variant} rel err {err:.3e} (bar {4 * u * math.sqrt(K / 12):.3e})")
    assert err <= 4 * u * math.sqrt(K / 12)


def test_rn_f16_variant_equals_flat_f16_kernel_on_exact_inputs():
    m, n, d, zeta = 4096, 64, 64, 4
    A = inputs.integer_matrix(m, n, -1, 1, seed=10)
    Ad = to_dev(A)
    ri, v = b.meta(6, m, d, zeta, device=dev())
    B1 = b.apply_lowp(Ad, ri, v, zeta, d, "f16", "rn")
    B2 = b.apply(Ad, ri, v, zeta, d, precision="f16acc", flags=b.SK_VARIANT_FLAT, ws=None)
    sync()
    assert torch.equal(B1, B2)


@pytest.mark.parametrize("variant", ["flat", "reg"])
@pytest.mark.parametrize("fmt,conv", [("f16", "sr"), ("bf16", "rn")])
def test_accumulate_and_empty(fmt, conv, variant):
    d, n = 64, 32
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    out = torch.full((d, n), 3.0, dtype=dt, device=dev())
    A = torch.empty((0, n), dtype=torch.float32, device=dev())
    b.apply_lowp(A, None, None, 4, d, fmt, conv, out=out,
                 flags=b.SK_ACCUMULATE | VARIANT[variant])
    sync()
    assert torch.all(out == 3.0)
    b.apply_lowp(A, None, None, 4, d, fmt, conv, out=out, flags=VARIANT[variant])
    sync()
    assert torch.all(out == 0.0)


@pytest.mark.parametrize("combine", [0, b.SK_COMBINE_F32])
@pytest.mark.parametrize("fmt,conv", [("f16", "rn"), ("f16", "sr"), ("bf16", "rn")])
def test_two_level_fixed_order(fmt, conv, combine):
    """The two-level variant in 64-row calls (one row chunk each, rows in
    ascending order from +0, SR draws keyed by the global row) chained with
    SK_ACCUMULATE: each call adds its chunk partial to B with one addition
    (in the format; FP32 then one rounding is the same for a single
    addition), so the result equals the oracle's chunked emulation with the
    same draws bit for bit.  N(0,1) x 37 inputs make nearly every addition
    round."""
    rows, calls, n, d, zeta, seed, sr_seed = 64, 40, 96, 128, 8, 17, 99
    m = rows * calls
    A = (inputs.gaussian(m, n, seed=14) * np.float32(37.0)).astype(np.float32)
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    expect = oracle.sketch_lowp_emul(A, ri, v, d, zeta, fmt, conv, sr_seed=sr_seed,
                                     chunk_rows=rows).astype(np.float64)
    flat = oracle.sketch_lowp_emul(A, ri, v, d, zeta, fmt, conv, sr_seed=sr_seed)
    assert (flat.astype(np.float64) != expect).mean() > 0.1     # the order shows
    Ad = to_dev(A)
    rid, vd = b.meta(seed, m, d, zeta, device=dev())
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    out = torch.empty((d, n), dtype=dt, device=dev())
    say(f"two-level order {fmt} {conv} combine={combine}")
    for c in range(calls):
        r0 = c * rows
        b.apply_lowp(Ad[r0:r0 + rows], rid[r0 * zeta:(r0 + rows) * zeta],
                     vd[r0 * zeta:(r0 + rows) * zeta], zeta, d, fmt, conv, sr_seed=sr_seed,
                     row_offset=r0, out=out,
                     flags=b.SK_VARIANT_REG | combine | (b.SK_ACCUMULATE if c else 0))
    sync()
    assert np.array_equal(as_f64(out), expect)


def test_two_level_more_accurate_than_flat():
    """At K = 2048 contributions per entry the two-level FP16 order (chunk
    partials of about 32 rows per entry) beats the flat running sum, for RN
    and SR, and BF16 two-level stays within its own random-walk bar."""
    m, n, d, zeta = 1 << 16, 128, 128, 4
    A = inputs.gaussian(m, n, seed=15)
    ri, v = oracle.meta_ref(5, m, d, zeta)
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    errs = {}
    for fmt, conv in (("f16", "rn"), ("f16", "sr"), ("bf16", "rn")):
        for var in ("flat", "reg"):
            errs[(fmt, conv, var)] = oracle.rel_frob(
                run(A, d, zeta, 5, fmt, conv, sr_seed=3, variant=var), ref)
    say(f"  rel errors {errs}")
    assert errs[("f16", "rn", "reg")] < errs[("f16", "rn", "flat")]
    assert errs[("f16", "sr", "reg")] < errs[("f16", "sr", "flat")]
    assert errs[("bf16", "rn", "reg")] < 4 * U_BF16 * math.sqrt(2048 / 12)


def test_sr_draws_depend_on_seed_and_global_row():
    """Different SR seeds give different sketches; the same seed and global
    rows give the same one (deterministic draws)."""
    m, n, d, zeta = 2048, 64, 64, 4
    A = (inputs.gaussian(m, n, seed=12) * np.float32(2.0**-20)).astype(np.float32)
    B1 = run(A, d, zeta, 1, "f16", "sr", sr_seed=1)
    B2 = run(A, d, zeta, 1, "f16", "sr", sr_seed=2)
    B1b = run(A, d, zeta, 1, "f16", "sr", sr_seed=1)
    assert not np.array_equal(B1, B2)
    ri, v = oracle.meta_ref(1, m, d, zeta)
    # exact-sum regime is not guaranteed here (|q| up to ~2^-17), so compare
    # the two runs with each other only up to the atomic order
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    assert abs(oracle.rel_frob(B1, ref) - oracle.rel_frob(B1b, ref)) < 1e-2


# --------------------------------- range stress (A 4,194,304 x 64, d = 128)

@pytest.fixture(scope="module")
def range_case():
    """A 4,194,304 x 64: N(0,1) rows times exp(2Z) row scales (seed 0);
    zeta = 4, d = 128; metadata seed 1; fp64 oracle sketch of the unscaled A
    (scaling A by 2^k scales the exact sketch by 2^k)."""
    m, n, d, zeta, seed = 4194304, 64, 128, 4, 1
    say("range case: drawing A and the fp64 oracle sketch")
    A = inputs.range_stress(m, n, 0, seed=0)
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    Ad = to_dev(A)
    rid, vd = b.meta(seed, m, d, zeta, device=dev())
    return Ad, A, ri, v, rid, vd, d, zeta, seed, oracle.sketch_f64(A, ri, v, d, zeta)


def _measure(B, k, ref):
    """(non-finite entries, relative Frobenius error after undoing 2^k,
    entries that are zero although the exact sketch is not: underflow, or a
    sum that cancels to zero in the format)."""
    x = as_f64(B) * 2.0 ** (-k)
    fin = np.isfinite(x)
    err = oracle.rel_frob(x, ref) if fin.all() else float("nan")
    return int((~fin).sum()), err, int(((x == 0) & (ref != 0)).sum())


@pytest.mark.parametrize("k", [-24, -16, -8, 0, 8, 12])
def test_range_stress(range_case, k):
    """Common rescaling by 2^k (FP16 sketching page §V-E, Corollary 3):
    FP32 is unaffected; BF16 stays finite over the whole range; the FP16
    variants are finite while the sums fit FP16 and overflow (+-inf) when
    they do not; at the bottom of the range RN conversion erases the
    contributions of magnitude at most h/2 (the oracle counts them) and
    output entries underflow to zero; at ordinary scale the two-level FP16
    sketch is the most accurate FP16 variant.  The range stress is a
    measurement, not a parity gate: the bars here are properties, and the
    printed table is the result."""
    Ad0, A, ri_h, v_h, ri, v, d, zeta, seed, ref = range_case
    Ad = Ad0 * (2.0**k)
    r32 = _measure(b.sketch_fused(Ad, d, zeta, seed, "f32"), k, ref)
    r16 = _measure(b.sketch_fused(Ad, d, zeta, seed, "f16acc"), k, ref)
    r16c = _measure(b.sketch_fused(Ad, d, zeta, seed, "f16acc", flags=b.SK_COMBINE_F32), k, ref)
    rfl = _measure(b.apply_lowp(Ad, ri, v, zeta, d, "f16", "rn"), k, ref)
    rsr = _measure(b.apply_lowp(Ad, ri, v, zeta, d, "f16", "sr", sr_seed=1), k, ref)
    rbf = _measure(b.apply_lowp(Ad, ri, v, zeta, d, "bf16", "rn"), k, ref)
    reg = b.SK_VARIANT_REG
    r2sr = _measure(b.apply_lowp(Ad, ri, v, zeta, d, "f16", "sr", sr_seed=1, flags=reg), k, ref)
    r2bf = _measure(b.apply_lowp(Ad, ri, v, zeta, d, "bf16", "rn", flags=reg), k, ref)
    sync()
    Ak = (A * np.float32(2.0**k)).astype(np.float32)
    erased, sub, total = oracle.f16_erasures(Ak, ri_h, v_h, d, zeta)
    say(f"  k={k:4d} (non-finite, rel err, zero outputs)  fp32 {r32}  "
        f"f16 rn two-level {r16}  f16 rn two-level fp32 combine {r16c}  f16 rn flat {rfl}  "
        f"f16 sr flat {rsr}  bf16 rn flat {rbf}  f16 sr two-level {r2sr}  "
        f"bf16 rn two-level {r2bf}  | oracle: erased contributions "
        f"{erased}/{total} ({erased / total:.3e}), subnormal {sub}")
    assert r32[0] == 0 and r32[1] <= 1e-5 and r32[2] == 0
    # BF16 is finite over the whole range (§V-E); its zero outputs are
    # cancellations of 8-bit sums, not underflow (same count at every k)
    assert rbf[0] == 0 and rbf[1] <= 0.2
    assert r2bf[0] == 0 and r2bf[1] <= rbf[1]
    fits = np.abs(ref).max() * 2.0**k < 32768           # every exact sum far inside FP16
    past = int((np.abs(ref) * 2.0**k > 2 * 65520).sum())  # sums far past the FP16 range
    for nonfin, err, _ in (r16, r16c, rfl, rsr, r2sr):
        if fits:
            assert nonfin == 0
        assert nonfin >= past
    if fits:
        assert r16[1] < rfl[1] and r16[1] < 2e-2 and r16c[1] <= r16[1]
    # erasure grows toward the bottom of the range (the smallest lognormal
    # row scales already lose a few hundred contributions at k = 0)
    if k <= -16:
        assert erased > 0.01 * total
