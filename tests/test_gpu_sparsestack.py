"""GPU parity for the SparseStack apply kernels (FP32 and FP16-accumulate)
against the CPU oracle (FP16 sketching page §III, §IV, §V).

Bars: integer, half-integer and coordinate inputs are exact in any
accumulation order, so there the GPU must equal the fp64 oracle bit for
bit; FP32 sketches are within relative Frobenius error 1e-5 of fp64;
FP16-accumulated sketches are within 4e-3 of fp64 and their subspace
distortion at d = 2n is within 1e-2 of the RN-emulation oracle's."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu

# (flags, workspace): the page's flat scatter; the LDS-privatized apply with
# the store-and-reduce flush (workspace); the same with the atomic flush;
# the register apply (workspace; the shapes the fused kernel covers)
VARIANTS = {"flat": (b.SK_VARIANT_FLAT, None), "lds": (b.SK_VARIANT_LDS, True),
            "lds_atomic": (b.SK_VARIANT_LDS, None), "reg": (b.SK_VARIANT_REG, True)}
ALL = ["flat", "lds", "lds_atomic"]
WIDE = ALL + ["reg"]
U16 = 2.0**-11          # unit roundoff of binary16


def f16_tolerance(K):
    """Relative Frobenius bar for an FP16-accumulated sketch whose output
    entries each receive K contributions.  4e-3 is the bar at the sketch
    sizes the FP16 sketching page's study uses (d = 2n, K in the thousands);
    a degenerate shape (d = zeta: every input row hits every output row)
    piles K = m contributions on each entry, and a running FP16 sum of K
    random-sign terms then carries a relative error of about u*sqrt(K/12)
    whatever the order, so the bar there is four times that estimate."""
    return max(4e-3, 4 * U16 * math.sqrt(K / 12))


def run(A, d, zeta, seed, precision, variant="lds", meta=None):
    """Metadata (GPU) + apply (GPU); returns (B on host as fp64, ri, v host)."""
    Ad = A if isinstance(A, torch.Tensor) else to_dev(A)
    m = Ad.shape[0]
    ri, v = meta if meta is not None else b.meta(seed, m, d, zeta, device=dev())
    flags, ws = VARIANTS[variant]
    B = b.apply(Ad, ri, v, zeta, d, precision=precision, flags=flags, ws=ws)
    sync()
    return B.cpu().numpy().astype(np.float64), ri, v


# ---------------------------------------------------------------- tiny config

@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("zeta", [1, 4])
def test_tiny_f32_vs_dense(variant, zeta):
    """A 4096 x 32 N(0,1) seed 0, d = 64: against the dense S*A brute force."""
    say(f"tiny f32 {variant} zeta={zeta}")
    m, n, d = 4096, 32, 64
    A = inputs.gaussian(m, n)
    B, _, _ = run(A, d, zeta, 1, "f32", variant)
    ri, v = oracle.meta_ref(1, m, d, zeta)
    ref = oracle.dense_S(ri, v, m, d, zeta) @ A.astype(np.float64)
    assert oracle.rel_frob(B, ref) <= 1e-5


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("variant", ALL)
def test_exact_inputs_bit_exact(precision, variant):
    """Integer inputs (FP32, |A| <= 8) and {-1,0,1} inputs (FP16): every
    partial sum is exactly representable, so the order of atomics cannot
    matter and a lost or doubled update changes the result."""
    say(f"exact {precision} {variant}")
    m, n, d, zeta = 4096, 32, 64, 4
    lo, hi = (-8, 8) if precision == "f32" else (-1, 1)
    A = inputs.integer_matrix(m, n, lo, hi)
    B, _, _ = run(A, d, zeta, 1, precision, variant)
    ri, v = oracle.meta_ref(1, m, d, zeta)
    if precision == "f16acc":
        assert 0.5 * np.bincount(ri, minlength=d).max() < 1024
    assert np.array_equal(B, oracle.sketch_f64(A, ri, v, d, zeta))


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("zeta", [1, 4, 8])
def test_coordinate_input(precision, variant, zeta):
    """A = [I_n 0]^T: SA equals the first n columns of S exactly."""
    m, n, d = 4096, 32, 64
    A = inputs.coordinate(m, n)
    B, _, _ = run(A, d, zeta, 8, precision, variant)
    ri, v = oracle.meta_ref(8, m, d, zeta)
    S_n = oracle.dense_S(ri[:n * zeta], v[:n * zeta], n, d, zeta)
    if precision == "f16acc":
        # one contribution per entry: B = +0 + RN_f16(val), e.g. 1/sqrt(8)
        S_n = S_n.astype(np.float32).astype(np.float16).astype(np.float64)
    assert np.array_equal(B, S_n)


@pytest.mark.parametrize("variant", ALL)
def test_tiny_f16_vs_fp64(variant):
    m, n, d, zeta = 4096, 32, 64, 4
    A = inputs.gaussian(m, n)
    B, _, _ = run(A, d, zeta, 1, "f16acc", variant)
    ri, v = oracle.meta_ref(1, m, d, zeta)
    assert oracle.rel_frob(B, oracle.sketch_f64(A, ri, v, d, zeta)) <= 4e-3


# ------------------------------------------------------- FP16 number format

@pytest.mark.parametrize("variant", ALL)
def test_f16_conversion_ties_subnormals_overflow(variant):
    """Coordinate input, zeta = 4 (scale 1/2): each output entry receives one
    contribution q = a/2, so B = RN_f16(q) for every a.  Covers the page's
    printed cases (h/2 -> 0, 32768 finite), ties to even, subnormals kept
    (no flush to zero) and overflow to infinity (§III-C, §V-E)."""
    n, d, zeta = 32, 64, 4
    specials = np.array([2.0**-24, 2.0**-23, 3 * 2.0**-24, 2.0**-20 * 3, 2.0**16, 65504 * 2,
                         65520 * 2, 2.0**-26 * 2, -(2.0**-23), 1 + 2.0**-10, 1 + 3 * 2.0**-11,
                         2.0**-14, 2.0**-15 * 3, 1e-9, -7.0e4 * 2, 12345.678],
                        dtype=np.float32)
    vals = np.resize(specials, n)
    A = inputs.coordinate(4096, n) * vals[None, :]
    B, _, _ = run(A, d, zeta, 3, "f16acc", variant)
    ri, v = oracle.meta_ref(3, 4096, d, zeta)
    # one contribution per entry: B = +0 + RN(q), so the order is irrelevant
    expect = oracle.sketch_f16_rn_emul(A, ri, v, d, zeta)
    assert np.isinf(expect).sum() >= 2 and (expect == 0).sum() > 0
    assert np.array_equal(B, expect.astype(np.float64), equal_nan=True)
    assert np.array_equal(np.signbit(B), np.signbit(expect))


@pytest.mark.parametrize("variant", ALL)
def test_f16_subnormal_accumulation(variant):
    """Sums that stay in the FP16 subnormal range are exact multiples of
    h = 2^-24: the atomics must keep subnormals (§III-C) and equal fp64."""
    m, n, d, zeta = 4096, 32, 64, 4
    A = inputs.integer_matrix(m, n, -3, 3, seed=5) * np.float32(2.0**-23)   # q = k * 2^-24
    B, _, _ = run(A, d, zeta, 4, "f16acc", variant)
    ri, v = oracle.meta_ref(4, m, d, zeta)
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    assert np.abs(ref).max() < 2.0**-14            # whole computation subnormal
    assert np.array_equal(B, ref)


# ---------------------------------------------------- ragged and edge cases

@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("m,n,d,zeta,pad", [
    (1000, 38, 96, 3, 6),       # ragged rows / columns, zeta = 3, padded strides
    (777, 130, 40, 8, 2),       # more columns than one slice, zeta = 8
    (5, 2, 16, 16, 0),          # tiny, zeta = d
    (3001, 64, 5, 5, 0),        # d = zeta: every row hits every block
    (2048, 66, 88, 11, 0),      # run-time zeta above the peeled eight
])
def test_ragged_shapes(precision, variant, m, n, d, zeta, pad):
    say(f"ragged {precision} {variant} m={m} n={n} d={d} zeta={zeta} pad={pad}")
    if d % zeta:
        pytest.skip("d % zeta")
    A = inputs.gaussian(m, n + pad, seed=2)
    Ad = to_dev(A)[:, :n]                       # lda = n + pad
    ri, v = b.meta(6, m, d, zeta, device=dev())
    ldb = n + pad
    out = torch.full((d, ldb), 7.0, dtype=torch.float16 if precision == "f16acc" else torch.float32,
                     device=dev())
    flags, ws = VARIANTS[variant]
    b.apply(Ad, ri, v, zeta, d, precision=precision, out=out[:, :n], flags=flags, ws=ws)
    sync()
    B = out.cpu().numpy().astype(np.float64)
    assert np.all(B[:, n:] == 7.0)              # padding untouched
    ri_h, v_h = oracle.meta_ref(6, m, d, zeta)
    ref = oracle.sketch_f64(np.ascontiguousarray(A[:, :n]), ri_h, v_h, d, zeta)
    tol = 1e-5 if precision == "f32" else f16_tolerance(m * zeta // d)
    assert oracle.rel_frob(B[:, :n], ref) <= tol


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_empty_input_and_accumulate(precision):
    d, n = 64, 32
    dt = torch.float16 if precision == "f16acc" else torch.float32
    out = torch.full((d, n), 3.0, dtype=dt, device=dev())
    A = torch.empty((0, n), dtype=torch.float32, device=dev())
    b.apply(A, None, None, 4, d, precision=precision, out=out, flags=b.SK_ACCUMULATE)
    sync()
    assert torch.all(out == 3.0)                # B += S*0
    b.apply(A, None, None, 4, d, precision=precision, out=out)
    sync()
    assert torch.all(out == 0.0)                # B = S*0


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_row_chunks_accumulate(precision):
    """Streaming: sketching row chunks with global-row metadata and
    SK_ACCUMULATE gives the same sketch as one call (exact inputs)."""
    m, n, d, zeta = 9000, 32, 64, 4
    A = inputs.integer_matrix(m, n, -1, 1, seed=9)
    Ad = to_dev(A)
    dt = torch.float16 if precision == "f16acc" else torch.float32
    out = torch.zeros((d, n), dtype=dt, device=dev())
    for r0, r1 in [(0, 2500), (2500, 2501), (2501, 9000)]:
        ri, v = b.meta(12, r1 - r0, d, zeta, row_offset=r0, device=dev())
        b.apply(Ad[r0:r1], ri, v, zeta, d, precision=precision, out=out, flags=b.SK_ACCUMULATE)
    sync()
    ri, v = oracle.meta_ref(12, m, d, zeta)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), oracle.sketch_f64(A, ri, v, d, zeta))


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_out_of_range_rows_are_ignored(precision):
    m, n, d, zeta = 256, 32, 64, 4
    A = inputs.integer_matrix(m, n, -1, 1)
    ri_h, v_h = oracle.meta_ref(2, m, d, zeta)
    bad = ri_h.copy()
    bad[::7] = d + 5
    bad[3::11] = -1
    keep = (bad >= 0) & (bad < d)
    ref = oracle.sketch_f64(A, np.where(keep, bad, 0).astype(np.int32), np.where(keep, v_h, 0).astype(np.float32), d, zeta)
    for variant in ALL:
        B, _, _ = run(A, d, zeta, 0, precision, variant, meta=(to_dev(bad), to_dev(v_h)))
        assert np.array_equal(B, ref)


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("variant", ALL)
def test_general_values(precision, variant):
    """Metadata values of differing magnitudes (any FP32 val, not only
    +-1/sqrt(zeta)): every kernel applies val*a per contribution.  Values are
    dyadic, so with integer A every FP32 partial sum is exact; for FP16 the
    products are exact halves/quarters and sums stay below 2^10."""
    say(f"general values {precision} {variant}")
    m, n, d, zeta = 3000, 64, 64, 4
    A = inputs.integer_matrix(m, n, -2, 2, seed=13)
    ri_h, v_h = oracle.meta_ref(9, m, d, zeta)
    g = np.random.default_rng(5)
    v_gen = (v_h * g.choice(np.array([0.25, 0.5, 1.0, 2.0], dtype=np.float32), size=v_h.size)
             ).astype(np.float32)
    v_gen[::97] = v_h[::97]                     # some blocks keep equal magnitudes
    B, _, _ = run(A, d, zeta, 0, precision, variant, meta=(to_dev(ri_h), to_dev(v_gen)))
    ref = oracle.sketch_f64(A, ri_h, v_gen, d, zeta)
    assert np.abs(ref).max() < 1024
    assert np.array_equal(B, ref)


def test_large_d_falls_back_to_flat():
    """d x 8 words exceed LDS: LDS is refused when forced, FLAT serves the default."""
    m, n, d, zeta = 2048, 16, 8192, 4
    A = inputs.integer_matrix(m, n, -2, 2)
    Ad = to_dev(A)
    ri, v = b.meta(3, m, d, zeta, device=dev())
    with pytest.raises(b.SketchError):
        b.apply(Ad, ri, v, zeta, d, precision="f32", flags=b.SK_VARIANT_LDS)
    B = b.apply(Ad, ri, v, zeta, d, precision="f32")
    sync()
    rh, vh = oracle.meta_ref(3, m, d, zeta)
    assert np.array_equal(B.cpu().numpy().astype(np.float64), oracle.sketch_f64(A, rh, vh, d, zeta))


# --------------------------- scale configuration (A 2^20 x 256, d = 512)

@pytest.fixture(scope="module")
def scale_case():
    """A 2^20 x 256 N(0,1) drawn on the device (seeded); zeta = 4, d = 512."""
    m, n, d, zeta, seed = 1 << 20, 256, 512, 4, 1
    say("scale case: drawing A and the fp64 oracle sketch")
    Ad = inputs.gaussian_torch(m, n, seed=0)
    A = Ad.cpu().numpy()
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    return Ad, A, d, zeta, seed, oracle.sketch_f64(A, ri, v, d, zeta)


@pytest.mark.parametrize("variant", ALL)
def test_scale_f32(scale_case, variant):
    Ad, A, d, zeta, seed, ref = scale_case
    say(f"scale f32 {variant}")
    B, _, _ = run(Ad, d, zeta, seed, "f32", variant)
    assert oracle.rel_frob(B, ref) <= 1e-5


@pytest.mark.parametrize("variant", ["lds", "lds_atomic"])
def test_scale_f16acc(scale_case, variant):
    """The LDS two-level FP16 sketch meets the 4e-3 bar."""
    Ad, A, d, zeta, seed, ref = scale_case
    say(f"scale f16acc {variant}")
    B, _, _ = run(Ad, d, zeta, seed, "f16acc", variant)
    err = oracle.rel_frob(B, ref)
    say(f"  rel err {err:.3e}")
    assert err <= 4e-3


def test_scale_f16acc_flat_error_model(scale_case):
    """The page's flat design accumulates K = m*zeta/d = 8192 contributions
    per entry in one FP16 running sum; its error follows the random-walk
    estimate u*sqrt(K/12) (u = 2^-11) and so misses the 4e-3 bar here."""
    Ad, A, d, zeta, seed, ref = scale_case
    B, _, _ = run(Ad, d, zeta, seed, "f16acc", "flat")
    err = oracle.rel_frob(B, ref)
    pred = 2.0**-11 * math.sqrt((A.shape[0] * zeta / d) / 12)
    say(f"  flat rel err {err:.3e} (model {pred:.3e})")
    assert 0.25 * pred < err < 4 * pred


# ---------------------------------------- distortion at d = 2n (coherence)

_DISTORTION = {}


def _distortion_case(m, zeta):
    """U = orth(coherent m x 128) on the device, its metadata and the RN
    emulation oracle's E_OSE (computed once per shape)."""
    key = (m, zeta)
    if key not in _DISTORTION:
        n = 128
        d = 2 * n
        Ud = inputs.orth_torch(inputs.coherent_torch(m, n, seed=0))
        U = Ud.cpu().numpy()
        ri, v = oracle.meta_ref(5, m, d, zeta)
        emu = oracle.sketch_f16_rn_emul(U, ri, v, d, zeta, chunk_rows=4096)
        _DISTORTION.clear()
        _DISTORTION[key] = (Ud, oracle.ose_error(emu.astype(np.float64)))
    return _DISTORTION[key]


@pytest.mark.parametrize("path", ["lds", "reg", "fused"])
@pytest.mark.parametrize("m,zeta", [(1 << 20, 4), (1 << 18, 1), (1 << 18, 8)])
def test_distortion_matches_rn_emulation(m, zeta, path):
    """U = orth(A) of the coherent workload (n = 128), d = 2n: the GPU FP16
    sketch's E_OSE = ||(SU)^T SU - I||_2 is within 1e-2 of the RN-emulation
    oracle's, and its sigma_min/sigma_max stays close to FP32's, on the LDS
    and register applies and the fused sketch (the benchmarked path)."""
    n = 128
    d = 2 * n
    say(f"distortion m={m} zeta={zeta} {path}")
    Ud, e_emu = _distortion_case(m, zeta)
    if path == "fused":
        B16 = b.sketch_fused(Ud, d, zeta, 5, "f16acc")
        B32 = b.sketch_fused(Ud, d, zeta, 5, "f32")
        sync()
        B16 = B16.cpu().numpy().astype(np.float64)
        B32 = B32.cpu().numpy().astype(np.float64)
    else:
        B16, _, _ = run(Ud, d, zeta, 5, "f16acc", path)
        B32, _, _ = run(Ud, d, zeta, 5, "f32", path)
    e_gpu = oracle.ose_error(B16)
    say(f"  E_OSE gpu16 {e_gpu:.5f} emu16 {e_emu:.5f} gpu32 {oracle.ose_error(B32):.5f}")
    assert abs(e_gpu - e_emu) <= 1e-2
    assert abs(oracle.sv_ratio(B16) - oracle.sv_ratio(B32)) <= 1e-2
