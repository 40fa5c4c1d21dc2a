"""GPU parity of the register apply (sk_apply_f32 / sk_apply_f16acc with
SK_VARIANT_REG) against the CPU oracle (FP16 sketching page §III-A, §III-B,
§III-C).

Bars as for the other apply variants: exact-sum inputs (integers, {-1,0,1},
dyadic values, coordinate inputs) bit for bit against fp64; N(0,1) inputs
within 1e-5 (FP32) and 4e-3 (FP16) relative Frobenius error; and, since
the order of additions is fixed, two calls give the same bits."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu

MI355X = dict(num_cu=256, max_lds=160 * 1024)
PREC = {"f32": b.SK_PRECISION_F32, "f16acc": b.SK_PRECISION_F16ACC}


def reg_plan(precision, m, n, d, zeta, lda=None):
    return b.sk_fused_plan_describe(PREC[precision], m, n, lda or n, 16, d, zeta, **MI355X)


def run_reg(A, ri, v, zeta, d, precision, flags=b.SK_VARIANT_REG, out=None):
    Ad = A if isinstance(A, torch.Tensor) else to_dev(A)
    B = b.apply(Ad, ri, v, zeta, d, precision=precision, flags=flags, ws=True, out=out)
    sync()
    return B


# (m, n, d, zeta, plan16, plan32): plan = (words per lane, R, G) for FP16
# (one word per lane at most 128 columns) and FP32 (four words per lane
# wider than 128 columns)
@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("m,n,d,zeta,plan16,plan32", [
    (4096, 256, 64, 4, (2, 4, 1), (2, 4, 1)),         # R = 4 (too few rows for four words)
    (3000, 128, 128, 4, (1, 8, 1), (2, 8, 1)),        # R = 8, a short last stage
    (5000, 260, 256, 8, (2, 16, 1), (4, 16, 1)),      # R = 16, zeta = 8, ragged second slice
    (4096, 128, 512, 8, (1, 32, 1), (2, 32, 1)),      # R = 32 (FP16 one word per lane)
    (3001, 128, 1024, 4, (1, 32, 2), (2, 32, 2)),     # FP16 one word, d = 1024 in two groups
    (2500, 136, 1024, 1, (2, 32, 2), (4, 16, 4)),     # row groups (A read 2 / 4 times)
    (3001, 256, 512, 4, (2, 32, 1), (4, 16, 2)),      # FP32 four words, ragged 64-row stage
    (777, 512, 128, 2, (2, 8, 1), (4, 8, 1)),         # FP32 four words, R = 8, two slices
])
def test_register_apply_vs_oracle(precision, m, n, d, zeta, plan16, plan32):
    say(f"register apply {precision} m={m} n={n} d={d} zeta={zeta}")
    p = reg_plan(precision, m, n, d, zeta)
    assert p["fused"] == 1
    assert (p["words"], p["rows_per_wave"], p["groups"]) == (plan32 if precision == "f32"
                                                             else plan16)
    A = inputs.gaussian(m, n, seed=3)
    ri, v = b.meta(5, m, d, zeta, device=dev())
    B = run_reg(A, ri, v, zeta, d, precision).float().cpu().numpy().astype(np.float64)
    ri_h, v_h = oracle.meta_ref(5, m, d, zeta)
    err = oracle.rel_frob(B, oracle.sketch_f64(A, ri_h, v_h, d, zeta))
    assert err <= (1e-5 if precision == "f32" else 4e-3), err


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("n", [128, 256])
def test_register_exact_inputs_and_general_values(precision, n):
    """Integer A (FP32) / {-1,0,1} A (FP16) with stored values scaled by
    dyadic factors: every product and partial sum is exact, so B equals
    fp64 bit for bit; values differ from entry to entry (every chunk takes
    the kernel's per-hit-product redo), or a single entry differs (one
    workgroup's chunk does).  FP32 at 256 columns runs four words per
    lane."""
    m, d, zeta = 3000, 128, 4
    say(f"register exact/general {precision} n={n}")
    lo, hi = (-8, 8) if precision == "f32" else (-1, 1)
    A = inputs.integer_matrix(m, n, lo, hi, seed=13)
    ri_h, v_h = oracle.meta_ref(9, m, d, zeta)
    g = np.random.default_rng(5)
    v_gen = (v_h * g.choice(np.array([0.25, 0.5, 1.0, 2.0], dtype=np.float32), size=v_h.size)
             ).astype(np.float32)
    v_one = v_h.copy()
    v_one[1234 * zeta + 2] *= 2
    for vals in (v_h, v_gen, v_one):
        B = run_reg(A, to_dev(ri_h), to_dev(vals), zeta, d, precision)
        ref = oracle.sketch_f64(A, ri_h, vals, d, zeta)
        assert np.abs(ref).max() < 1024
        assert np.array_equal(B.float().cpu().numpy().astype(np.float64), ref)


def test_register_f16_conversion_ties_subnormals_overflow():
    """Coordinate input times special values: one contribution per output
    entry, so B is RN_f16 of that contribution (ties to even, subnormals
    kept, overflow to infinity), signs of zero included."""
    n, d, zeta = 128, 64, 4
    specials = np.array([2.0**-24, 2.0**-23, 3 * 2.0**-24, 2.0**-20 * 3, 2.0**16, 65504 * 2,
                         65520 * 2, 2.0**-26 * 2, -(2.0**-23), 1 + 2.0**-10, 1 + 3 * 2.0**-11,
                         2.0**-14, 2.0**-15 * 3, 1e-9, -7.0e4 * 2, 12345.678], dtype=np.float32)
    A = inputs.coordinate(4096, n) * np.resize(specials, n)[None, :]
    ri, v = b.meta(3, 4096, d, zeta, device=dev())
    B = run_reg(A, ri, v, zeta, d, "f16acc").float().cpu().numpy()
    ri_h, v_h = oracle.meta_ref(3, 4096, d, zeta)
    expect = oracle.sketch_f16_rn_emul(A, ri_h, v_h, d, zeta)
    assert np.isinf(expect).sum() >= 2 and (expect == 0).sum() > 0
    assert np.array_equal(B.astype(np.float64), expect.astype(np.float64), equal_nan=True)
    assert np.array_equal(np.signbit(B), np.signbit(expect))


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_register_out_of_range_entries_ignored(precision):
    m, n, d, zeta = 700, 128, 64, 4
    A = inputs.integer_matrix(m, n, -1, 1)
    ri_h, v_h = oracle.meta_ref(2, m, d, zeta)
    bad = ri_h.copy()
    bad[::7] = d + 5
    bad[3::11] = -1
    bad[5::13] = (bad[5::13] + d // zeta) % d     # inside [0, d) but in another block
    t = np.arange(bad.size) % zeta
    keep = (bad >= t * (d // zeta)) & (bad < (t + 1) * (d // zeta))
    ref = oracle.sketch_f64(A, np.where(keep, bad, 0).astype(np.int32),
                            np.where(keep, v_h, 0).astype(np.float32), d, zeta)
    B = run_reg(A, to_dev(bad), to_dev(v_h), zeta, d, precision)
    assert np.array_equal(B.float().cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_register_general_values_gaussian(precision, tol):
    """N(0,1) input with values of random magnitude in a few rows spread
    over the chunks, zeta = 8: the chunks holding them are redone with
    per-hit products; the sketch meets the bars against fp64."""
    m, n, d, zeta = 40000, 256, 256, 8
    A = inputs.gaussian(m, n, seed=21)
    ri_h, v_h = oracle.meta_ref(4, m, d, zeta)
    vals = v_h.copy()
    g = np.random.default_rng(8)
    rows = g.choice(m, 40, replace=False)
    vals.reshape(m, zeta)[rows] *= g.uniform(0.1, 3.0, size=(40, zeta)).astype(np.float32)
    B = run_reg(A, to_dev(ri_h), to_dev(vals), zeta, d, precision)
    err = oracle.rel_frob(B.float().cpu().numpy().astype(np.float64),
                          oracle.sketch_f64(A, ri_h, vals, d, zeta))
    assert err <= tol, err


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_register_reproducible(precision):
    """N(0,1) input: two calls agree bit for bit (fixed order of additions)
    and match the fused sketch of the same S to the FP32/FP16 bars."""
    m, n, d, zeta = 20000, 256, 512, 4
    Ad = to_dev(inputs.gaussian(m, n, seed=7))
    ri, v = b.meta(11, m, d, zeta, device=dev())
    B1 = run_reg(Ad, ri, v, zeta, d, precision)
    B2 = run_reg(Ad, ri, v, zeta, d, precision)
    assert torch.equal(B1, B2)
    Bf = b.sketch_fused(Ad, d, zeta, 11, precision)
    sync()
    err = float((B1.double() - Bf.double()).norm() / Bf.double().norm())
    assert err <= (1e-6 if precision == "f32" else 4e-3)


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_register_row_chunks_and_padded_strides(precision):
    """Row chunks with global-row metadata and SK_ACCUMULATE over lda = n + 4
    and a padded B: the padding is untouched and the sum equals one call
    (exact inputs)."""
    m, n, d, zeta = 9000, 128, 64, 4
    A = inputs.integer_matrix(m, n + 4, -1, 1, seed=9)
    Ad = to_dev(A)[:, :n]
    dt = torch.float16 if precision == "f16acc" else torch.float32
    out = torch.full((d, n + 8), 5.0, dtype=dt, device=dev())
    out[:, :n] = 0
    for r0, r1 in [(0, 2500), (2500, 2501), (2501, 9000)]:
        ri, v = b.meta(12, r1 - r0, d, zeta, row_offset=r0, device=dev())
        b.apply(Ad[r0:r1], ri, v, zeta, d, precision=precision, out=out[:, :n],
                flags=b.SK_ACCUMULATE | b.SK_VARIANT_REG)
    sync()
    Bh = out.float().cpu().numpy().astype(np.float64)
    assert np.all(Bh[:, n:] == 5.0)
    ri_h, v_h = oracle.meta_ref(12, m, d, zeta)
    assert np.array_equal(Bh[:, :n], oracle.sketch_f64(np.ascontiguousarray(A[:, :n]), ri_h,
                                                       v_h, d, zeta))


def test_register_forced_errors():
    """SK_VARIANT_REG on a shape it does not cover (d = 40, not a multiple
    of 16), without a workspace, with a misaligned one, or together with
    another variant."""
    d, zeta = 64, 4
    A = to_dev(inputs.gaussian(4096, 128))
    ri, v = b.meta(1, 4096, d, zeta, device=dev())
    ri40, v40 = b.meta(1, 4096, 40, zeta, device=dev())
    B = torch.empty((40, 128), dtype=torch.float32, device=dev())
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev())
    A2 = to_dev(inputs.gaussian(4096, 128))
    B2 = torch.empty((d, 128), dtype=torch.float32, device=dev())
    need = b.sk_apply_workspace_size(b.SK_PRECISION_F32, 4096, 128, d, zeta, b.SK_VARIANT_REG)
    ws2 = torch.empty(need + 64, dtype=torch.uint8, device=dev())
    with pytest.raises(b.SketchError) as e:
        b.sk_apply_f32_ws(A, 4096, 128, 128, ri40, v40, zeta, B, 40, 128, b.SK_VARIANT_REG, ws, 0)
    assert e.value.status == b.SK_ERR_UNSUPPORTED
    for Ax, Bx, w, nbytes, flags, expect in [
            (A2, B2, None, 0, b.SK_VARIANT_REG, b.SK_ERR_NULL),
            (A2, B2, ws2[4:], need, b.SK_VARIANT_REG, b.SK_ERR_ALIGN),
            (A2, B2, ws2, need - 4, b.SK_VARIANT_REG, b.SK_ERR_ARG),
            (A2, B2, ws2, need, b.SK_VARIANT_REG | b.SK_VARIANT_LDS, b.SK_ERR_ARG)]:
        with pytest.raises(b.SketchError) as e:
            b.sk_apply_f32_ws(Ax, 4096, Ax.shape[1], Ax.shape[1], ri, v, zeta, Bx, d,
                              Bx.shape[1], flags, w, nbytes)
        assert e.value.status == expect
    # zeta = 16: a wavefront's 8 rows of a stage hold more than 64 entries
    ri16, v16 = b.meta(1, 4096, d, 16, device=dev())
    assert b.sk_apply_workspace_size(b.SK_PRECISION_F32, 4096, 128, d, 16, b.SK_VARIANT_REG) == 0
    with pytest.raises(b.SketchError) as e:
        b.sk_apply_f32_ws(A2, 4096, 128, 128, ri16, v16, 16, B2, d, 128, b.SK_VARIANT_REG, ws2, need)
    assert e.value.status == b.SK_ERR_UNSUPPORTED


# --------------------------- scale configuration (A 2^20 x 256, d = 512)

@pytest.fixture(scope="module")
def scale_case():
    """A 2^20 x 256 N(0,1) drawn on the device (seeded); zeta = 4, d = 512."""
    m, n, d, zeta, seed = 1 << 20, 256, 512, 4, 1
    Ad = inputs.gaussian_torch(m, n, seed=0)
    A = Ad.cpu().numpy()
    ri_h, v_h = oracle.meta_ref(seed, m, d, zeta)
    return Ad, d, zeta, seed, oracle.sketch_f64(A, ri_h, v_h, d, zeta)


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_register_scale(scale_case, precision, tol):
    """The bench's configuration through sk_meta_generate + the register
    apply, as the bench's stored-metadata leg runs it."""
    Ad, d, zeta, seed, ref = scale_case
    assert reg_plan(precision, Ad.shape[0], Ad.shape[1], d, zeta)["fused"] == 1
    ri, v = b.meta(seed, Ad.shape[0], d, zeta, device=dev())
    B = run_reg(Ad, ri, v, zeta, d, precision)
    err = oracle.rel_frob(B.float().cpu().numpy().astype(np.float64), ref)
    say(f"  register apply scale {precision} rel err {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_register_scale_general_values(scale_case, precision, tol):
    """The scale configuration with values of another magnitude in 64 rows
    (so about 64 of the 256 workgroups redo their chunk with per-hit
    products) against fp64 of the same values."""
    Ad, d, zeta, seed, _ = scale_case
    m = Ad.shape[0]
    ri_h, v_h = oracle.meta_ref(seed, m, d, zeta)
    g = np.random.default_rng(17)
    rows = g.choice(m, 64, replace=False)
    vals = v_h.copy()
    vals.reshape(m, zeta)[rows] *= g.uniform(0.1, 3.0, size=(64, zeta)).astype(np.float32)
    B = run_reg(Ad, to_dev(ri_h), to_dev(vals), zeta, d, precision)
    ref = oracle.sketch_f64(Ad.cpu().numpy(), ri_h, vals, d, zeta)
    err = oracle.rel_frob(B.float().cpu().numpy().astype(np.float64), ref)
    say(f"  register apply scale, general values, {precision} rel err {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_default_variant_choice(precision):
    """flags = 0: the register apply where it covers the shape and the
    workspace holds its partials (bit-identical to forcing it), else the
    LDS apply (zeta = 16; or a workspace only large enough for LDS).  Exact
    inputs, so every path equals fp64 bit for bit."""
    m, n, d = 6000, 128, 256
    A = inputs.integer_matrix(m, n, -1, 1, seed=23)
    Ad = to_dev(A)
    prec = PREC[precision]
    for zeta in (4, 16):
        ri, v = b.meta(6, m, d, zeta, device=dev())
        ri_h, v_h = oracle.meta_ref(6, m, d, zeta)
        ref = oracle.sketch_f64(A, ri_h, v_h, d, zeta)
        need_def = b.sk_apply_workspace_size(prec, m, n, d, zeta, 0)
        need_reg = b.sk_apply_workspace_size(prec, m, n, d, zeta, b.SK_VARIANT_REG)
        need_lds = b.sk_apply_workspace_size(prec, m, n, d, zeta, b.SK_VARIANT_LDS)
        assert need_def == max(need_reg, need_lds)
        assert (need_reg > 0) == (zeta <= 8)
        B0 = b.apply(Ad, ri, v, zeta, d, precision=precision, flags=0, ws=True)
        sync()
        assert np.array_equal(B0.float().cpu().numpy().astype(np.float64), ref)
        if zeta <= 8:
            Br = run_reg(Ad, ri, v, zeta, d, precision)
            assert torch.equal(B0, Br)
            # a workspace the LDS plan fits but the register plan does not
            assert 0 < need_lds < need_reg
            ws = torch.empty(need_lds, dtype=torch.uint8, device=dev())
            B1 = b.apply(Ad, ri, v, zeta, d, precision=precision, flags=0, ws=ws)
            sync()
            assert np.array_equal(B1.float().cpu().numpy().astype(np.float64), ref)
