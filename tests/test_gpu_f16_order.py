"""GPU checks that the FP16-accumulate paths accumulate in FP16 from the
first contribution on (FP16 sketching page §III-B, §III-D: each FP32
product is rounded to FP16 nearest-even and added with FP16 nearest-even
additions; §IV-E, §V-E: nearest-even conversion erases every contribution
of magnitude at most h/2, h = 2^-24).

An implementation that summed the products in FP32 and rounded the total
once would pass a relative-error bar; these tests it fails:

* order-free inputs with hundreds of contributions per output entry:
  (a) every contribution at most h/2 in magnitude: each converts to zero,
      so the sketch is exactly +0 everywhere (in FP32 the sums are several
      h); (b) every contribution just above h/2: each converts to +-h, so
      every entry is h times a signed count, exactly, in any order (in FP32
      the sums are about 0.51 h times the count);
* the register paths' fixed order: a sketch accumulated in 64-row calls
  (one row chunk per call) equals the oracle's RN emulation with the same
  64-row chunks bit for bit, for Gaussian inputs whose every addition rounds.
Run on every FP16 path: the fused sketch, the register, LDS and flat
applies and the boundary call without a workspace."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu

H = 2.0**-24


def sketch16(path, Ad, d, zeta, seed, ri, v):
    """The FP16 sketch of Ad by one path (fp64 host copy)."""
    if path == "fused":
        B = b.sketch_fused(Ad, d, zeta, seed, "f16acc")
    elif path == "fused_combine_f32":
        B = b.sketch_fused(Ad, d, zeta, seed, "f16acc", flags=b.SK_COMBINE_F32)
    elif path == "reg":
        B = b.apply(Ad, ri, v, zeta, d, "f16acc", flags=b.SK_VARIANT_REG, ws=True)
    elif path == "lds":
        B = b.apply(Ad, ri, v, zeta, d, "f16acc", flags=b.SK_VARIANT_LDS, ws=True)
    elif path == "lds_atomic":
        B = b.apply(Ad, ri, v, zeta, d, "f16acc", flags=b.SK_VARIANT_LDS, ws=None)
    elif path == "flat":
        B = b.apply(Ad, ri, v, zeta, d, "f16acc", flags=b.SK_VARIANT_FLAT, ws=None)
    elif path == "boundary":             # sk_apply_f16acc, no workspace, default variant
        B = b.apply(Ad, ri, v, zeta, d, "f16acc", flags=0, ws=None)
    else:
        raise ValueError(path)
    sync()
    return B.cpu().numpy().astype(np.float64)


PATHS = ["fused", "fused_combine_f32", "reg", "lds", "lds_atomic", "flat", "boundary"]
# (m, n, d, zeta): mean load m*zeta/d = 1024 contributions per output entry,
# many row chunks; 256 columns (two words per lane in the fused kernel),
# 128 and 64 (one word per lane)
SHAPES = [(1 << 17, 256, 512, 4), (1 << 17, 128, 512, 4), (1 << 16, 64, 256, 4)]


def _magnitudes(m, n, lo, hi, seed):
    """Magnitudes uniform in (lo, hi) (exclusive) with random signs, FP32."""
    g = np.random.default_rng(seed)
    u = g.uniform(0.0, 1.0, (m, n))
    u = np.clip(u, 1e-6, 1 - 1e-6)
    a = (lo + (hi - lo) * u).astype(np.float32)
    a = np.clip(a, np.nextafter(np.float32(lo), np.float32(np.inf)),
                np.nextafter(np.float32(hi), np.float32(0)))
    return np.where(g.integers(0, 2, (m, n)) == 1, -a, a).astype(np.float32)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("m,n,d,zeta", SHAPES)
def test_contributions_below_half_h_vanish(path, m, n, d, zeta):
    """|a| <= 2^-24, scale 1/2: every contribution is at most h/2 and
    converts to zero (the tie h/2 included), so B is +0 everywhere."""
    say(f"erasure {path} {m}x{n} d={d} zeta={zeta}")
    A = _magnitudes(m, n, 0.0, 2.0**-24, seed=11)
    A[0, :] = np.float32(2.0**-24)                  # the tie itself: q = h/2 exactly
    seed = 7
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    B64 = oracle.sketch_f64(A, ri, v, d, zeta)
    # the test can fail: summed first, most entries would round to nonzero
    assert (np.abs(B64) > H).mean() > 0.5
    B = sketch16(path, to_dev(A), d, zeta, seed, *b.meta(seed, m, d, zeta, device=dev()))
    assert np.count_nonzero(B) == 0
    assert not np.signbit(B).any()                  # +0: sums start from +0


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("m,n,d,zeta", SHAPES)
def test_contributions_above_half_h_count_exactly(path, m, n, d, zeta):
    """2^-24 < |a| < 3 * 2^-24, scale 1/2: every contribution q has
    h/2 < |q| < 3h/2 and converts to +-h, so each entry is h times the
    signed count of its contributions, exact while every partial sum stays
    below 2048 h (the load bound below), in any order."""
    say(f"exact h counts {path} {m}x{n} d={d} zeta={zeta}")
    A = _magnitudes(m, n, 2.0**-24, 3 * 2.0**-24, seed=12)
    seed = 8
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    assert np.bincount(ri, minlength=d).max() < 2048
    # each contribution is sign(a) sign(val) h, and sign(val) = 2 val at zeta = 4
    expect = 2 * H * oracle.sketch_f64(np.sign(A).astype(np.float32), ri, v, d, zeta)
    B64 = oracle.sketch_f64(A, ri, v, d, zeta)
    summed = B64.astype(np.float32).astype(np.float16).astype(np.float64)
    assert (summed != expect).mean() > 0.5          # a sum-then-round kernel fails here
    B = sketch16(path, to_dev(A), d, zeta, seed, *b.meta(seed, m, d, zeta, device=dev()))
    assert np.array_equal(B, expect)
    # the same entries by the oracle's own RN emulation, on a sample of columns
    cols = np.arange(0, n, max(1, n // 8))
    emu = oracle.sketch_f16_rn_emul(np.ascontiguousarray(A[:, cols]), ri, v, d, zeta)
    assert np.array_equal(B[:, cols], emu.astype(np.float64))


# ------------------------------------------ fixed order of the register paths

# (n, d, zeta, paths): 64-row calls; contributions per entry per call
# 64*zeta/d = 8-16, calls chained with SK_ACCUMULATE
ORDER_SHAPES = [(256, 64, 16, ("fused",)), (256, 64, 8, ("fused", "reg")),
                (128, 128, 8, ("fused", "reg")), (64, 128, 16, ("fused",)),
                (96, 128, 4, ("fused", "reg"))]


@pytest.mark.parametrize("combine", [0, b.SK_COMBINE_F32])
@pytest.mark.parametrize("n,d,zeta,paths", ORDER_SHAPES)
def test_register_paths_follow_rn_emulation_order(n, d, zeta, paths, combine):
    """A call of at most 64 rows is one row chunk, accumulated from +0 in
    ascending row order; chained calls add each chunk's FP16 partial to B
    with one addition (FP16 nearest-even; FP32 then one rounding gives the
    same for a single addition of two binary16 values).  So 48 chained
    calls equal the oracle's two-level RN emulation with 64-row chunks bit
    for bit.  The inputs (N(0,1) x 37) make nearly every addition round."""
    rows, calls, seed = 64, 48, 21
    m = rows * calls
    A = (inputs.gaussian(m, n, seed=13) * np.float32(37.0)).astype(np.float32)
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    expect = oracle.sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=rows).astype(np.float64)
    B64 = oracle.sketch_f64(A, ri, v, d, zeta)
    summed = B64.astype(np.float32).astype(np.float16).astype(np.float64)
    assert (summed != expect).mean() > 0.3          # the order is visible in the result
    Ad = to_dev(A)
    rid, vd = b.meta(seed, m, d, zeta, device=dev())
    for path in paths:
        say(f"order {path} n={n} d={d} zeta={zeta} combine={combine}")
        out = torch.empty((d, n), dtype=torch.float16, device=dev())
        for c in range(calls):
            r0 = c * rows
            flags = combine | (b.SK_ACCUMULATE if c else 0)
            if path == "fused":
                b.sketch_fused(Ad[r0:r0 + rows], d, zeta, seed, "f16acc", row_offset=r0,
                               out=out, flags=flags)
            else:
                b.apply(Ad[r0:r0 + rows], rid[r0 * zeta:(r0 + rows) * zeta],
                        vd[r0 * zeta:(r0 + rows) * zeta], zeta, d, "f16acc", out=out,
                        flags=flags | b.SK_VARIANT_REG, ws=True)
        sync()
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, expect), path


# ------------------------------------------- the two combines at scale

@pytest.fixture(scope="module")
def scale_sketch():
    """A 2^20 x 256 N(0,1) (device-drawn, seeded), zeta = 4, d = 512."""
    m, n, d, zeta, seed = 1 << 20, 256, 512, 4, 1
    say("scale case: drawing A and the fp64 oracle sketch")
    Ad = inputs.gaussian_torch(m, n, seed=0)
    A = Ad.cpu().numpy()
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    return Ad, d, zeta, seed, oracle.sketch_f64(A, ri, v, d, zeta)


def test_combines_at_scale(scale_sketch):
    """Both combines of the fused FP16 sketch meet the 4e-3 bar; the FP16
    combine's extra additions show as a larger error than the FP32
    combine's, and the two results differ."""
    Ad, d, zeta, seed, ref = scale_sketch
    B16 = b.sketch_fused(Ad, d, zeta, seed, "f16acc")
    B32c = b.sketch_fused(Ad, d, zeta, seed, "f16acc", flags=b.SK_COMBINE_F32)
    sync()
    e16 = oracle.rel_frob(B16.cpu().numpy().astype(np.float64), ref)
    e32c = oracle.rel_frob(B32c.cpu().numpy().astype(np.float64), ref)
    say(f"  rel err FP16 combine {e16:.3e}, FP32 combine {e32c:.3e}")
    assert e16 <= 4e-3 and e32c <= 4e-3
    assert e32c < e16
    assert not torch.equal(B16, B32c)
