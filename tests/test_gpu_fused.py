"""GPU parity of the fused SparseStack sketch (sk_sketch_f32 /
sk_sketch_f16acc: metadata drawn inside the apply kernel) against the CPU
oracle, whose metadata comes from its own Philox (FP16 sketching page
§III-C; FlashSketch page §5.2).

Bars as for the stored-metadata apply: exact inputs bit for bit, FP32
within relative Frobenius 1e-5 of fp64, FP16 within 4e-3 (or the error
model's bar for degenerate shapes), and FP16 sketches of Gaussian inputs
bit for bit equal to the oracle's RN emulation of the library's order (at
multi-chunk sizes, and on sampled columns at the bench's full size).  Shapes cover the fused kernel's own
plans (each rows-per-wave size, row groups, several slices, ragged chunks,
row offsets) and the shapes it hands to the metadata + LDS fallback."""
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


def fused_used(precision, m, n, lda, d, zeta):
    return b.sk_fused_plan_describe(PREC[precision], m, n, lda, 16, d, zeta, **MI355X)["fused"]


def run_fused(A, d, zeta, seed, precision, row_offset=0, out=None, flags=0):
    Ad = A if isinstance(A, torch.Tensor) else to_dev(A)
    B = b.sketch_fused(Ad, d, zeta, seed, precision, row_offset=row_offset, out=out, flags=flags)
    sync()
    return B.cpu().numpy().astype(np.float64)


# (m, n, d, zeta): rows per wave 4, 8, 16, 32; row groups 1 and 2; one and
# several column slices; ragged row counts and single partial stages.  FP32
# wider than 128 columns takes four words per lane (64-row stages): the
# 256-, 384-, 260- and 512-column shapes cover R = 8 and 16, one to four row
# groups and ragged slices there; FP16 of at most 128 columns takes one word
# per lane (the 128-, 96-, 66- and 64-column shapes; two workgroups per CU up
# to R = 32).  zeta is 1, 4 or 16 (scale a power of two)
# so that integer inputs keep every product exact.
FUSED_SHAPES = [
    (4096, 128, 64, 4),         # R = 4
    (4096, 128, 64, 1),         # CountSketch
    (3001, 256, 128, 4),        # R = 8, ragged last stage
    (1000, 128, 256, 16),       # R = 16, zeta = 16 (four Philox blocks per row)
    (2500, 384, 512, 4),        # R = 32 (FP32: 16, two groups), two slices, ragged slice
    (5000, 128, 1024, 4),       # two row groups (FP16: one word per lane, R = 32, two per CU)
    (129, 256, 512, 1),         # one stage plus one row
    (1, 128, 64, 4),            # a single row
    (4096, 64, 128, 4),         # 64 columns at d = 128: the owner kernel (FP16 and FP32)
    (3000, 68, 64, 4),          # 68 columns, lanes past the row clamped
    (6000, 512, 1024, 4),       # FP32 four words: R = 16, four row groups, two slices
    (2049, 260, 256, 16),       # FP32 four words: a 4-column second slice, zeta = 16
    (65, 256, 256, 4),          # FP32 four words: one 64-row stage plus one row
    (2000, 96, 512, 4),         # FP16 one word, R = 32 two per CU, lanes past 96 columns clamped
    (777, 66, 256, 16),         # FP16 one word, R = 16 two per CU, zeta = 16, 66 columns
    (5000, 2, 512, 4),          # a right-hand side: 2 columns, all other lanes clamped
    (3001, 8, 256, 16),         # 8 columns, zeta = 16, ragged last stage
    (4096, 32, 64, 4),          # 32 columns, R = 4 two per CU
]


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("m,n,d,zeta", FUSED_SHAPES)
def test_fused_exact_inputs_bit_exact(precision, m, n, d, zeta):
    """Integer inputs: every partial sum is exact (FP32 |A| <= 8; FP16
    {-1,0,1} with sums far below 2^11), so the fused sketch must equal the
    fp64 oracle bit for bit: a wrong hash, sign, lost or doubled hit changes
    it."""
    say(f"fused exact {precision} m={m} n={n} d={d} zeta={zeta}")
    assert fused_used(precision, m, n, n, d, zeta)
    lo, hi = (-8, 8) if precision == "f32" else (-1, 1)
    A = inputs.integer_matrix(m, n, lo, hi, seed=21)
    B = run_fused(A, d, zeta, 17, precision)
    ri, v = oracle.meta_ref(17, m, d, zeta)
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    if precision == "f16acc":
        assert np.abs(ref).max() < 1024
    assert np.array_equal(B, ref)


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("zeta", [2, 8])
def test_fused_inexact_scales(precision, zeta):
    """zeta = 2, 8: the scale 1/sqrt(zeta) is not a power of two, so the
    products round; tolerance bars against fp64."""
    m, n, d = 20000, 128, 256
    A = inputs.gaussian(m, n, seed=6)
    assert fused_used(precision, m, n, n, d, zeta)
    B = run_fused(A, d, zeta, 3, precision)
    ri, v = oracle.meta_ref(3, m, d, zeta)
    tol = 1e-5 if precision == "f32" else 4e-3
    assert oracle.rel_frob(B, oracle.sketch_f64(A, ri, v, d, zeta)) <= tol


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_fused_general_values_and_padding(precision):
    """N(0,1) input with padded strides (lda > n, ldb > n): tolerance bars,
    and B's padding columns are left untouched."""
    m, n, d, zeta, pad = 7000, 256, 512, 4, 8
    A = inputs.gaussian(m, n + pad, seed=4)
    Ad = to_dev(A)[:, :n]
    assert fused_used(precision, m, n, n + pad, d, zeta)
    dt = torch.float16 if precision == "f16acc" else torch.float32
    out = torch.full((d, n + pad), 7.0, dtype=dt, device=dev())
    b.sketch_fused(Ad, d, zeta, 5, precision, out=out[:, :n])
    sync()
    B = out.cpu().numpy().astype(np.float64)
    assert np.all(B[:, n:] == 7.0)
    ri, v = oracle.meta_ref(5, m, d, zeta)
    ref = oracle.sketch_f64(np.ascontiguousarray(A[:, :n]), ri, v, d, zeta)
    tol = 1e-5 if precision == "f32" else 4e-3
    assert oracle.rel_frob(B[:, :n], ref) <= tol


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_fused_row_offset_chunks_accumulate(precision):
    """Row chunks sketched with their global row offsets and SK_ACCUMULATE
    give the sketch of the whole matrix (exact inputs)."""
    m, n, d, zeta = 9000, 128, 256, 4
    A = inputs.integer_matrix(m, n, -1, 1, seed=9)
    Ad = to_dev(A)
    dt = torch.float16 if precision == "f16acc" else torch.float32
    out = torch.zeros((d, n), dtype=dt, device=dev())
    for r0, r1 in [(0, 2500), (2500, 2501), (2501, 9000)]:
        b.sketch_fused(Ad[r0:r1], d, zeta, 12, precision, row_offset=r0, out=out,
                       flags=b.SK_ACCUMULATE)
    sync()
    ri, v = oracle.meta_ref(12, m, d, zeta)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), oracle.sketch_f64(A, ri, v, d, zeta))


def test_fused_large_row_offset():
    """Global rows past 2^32 use both counter words of the Philox block."""
    m, n, d, zeta, off = 3000, 128, 64, 4, (1 << 32) + 12345
    A = inputs.integer_matrix(m, n, -4, 4, seed=2)
    B = run_fused(A, d, zeta, 99, "f32", row_offset=off)
    ri, v = oracle.meta_ref(99, m, d, zeta, row_offset=off)
    assert np.array_equal(B, oracle.sketch_f64(A, ri, v, d, zeta))


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("m,n,d,zeta,lda", [
    (4096, 32, 40, 4, 32),      # narrow rows and d not a multiple of 16
    (2048, 128, 128, 64, 128),  # zeta above the fused metadata stage
    (3001, 128, 40, 4, 128),    # d not a multiple of 16
    (2048, 128, 64, 4, 130),    # rows not 16-byte aligned (FP16) / fine for FP32
    (5, 2, 16, 16, 2),          # tiny, zeta = d
])
def test_fused_fallback_shapes(precision, m, n, d, zeta, lda):
    """Shapes the fused kernel does not cover run metadata + LDS apply from
    the same call and give the same sketch (scales 1/sqrt(zeta) that are
    powers of two and {-1,0,1} inputs keep every sum exact)."""
    say(f"fused fallback {precision} m={m} n={n} d={d} zeta={zeta} lda={lda}")
    A = inputs.integer_matrix(m, lda, -1, 1, seed=3)
    Ad = to_dev(A)[:, :n]
    B = run_fused(Ad, d, zeta, 8, precision)
    ri, v = oracle.meta_ref(8, m, d, zeta)
    ref = oracle.sketch_f64(np.ascontiguousarray(A[:, :n]), ri, v, d, zeta)
    assert np.array_equal(B, ref)


@pytest.mark.parametrize("offset,lda", [(0, 256), (2, 258), (2, 256), (1, 257)])
def test_fused_f32_word_width_by_alignment(offset, lda):
    """FP32 rows of 256 columns: a 16-byte base with lda % 4 == 0 takes four
    words per lane, an 8-byte base or lda % 4 == 2 two words, a 4-byte base
    the fallback; every plan gives the same exact sketch, and the workspace
    the size query reports suffices for each."""
    m, n, d, zeta = 3000, 256, 512, 4
    say(f"fused f32 alignment offset={offset} lda={lda}")
    A = inputs.integer_matrix(m + 1, lda, -8, 8, seed=12)
    flat = to_dev(A).reshape(-1)
    Ad = flat[offset:offset + m * lda].reshape(m, lda)[:, :n]
    align = 16 if offset == 0 else 8 if offset == 2 else 4
    assert Ad.data_ptr() % 16 == (0 if offset == 0 else offset * 4)
    p = b.sk_fused_plan_describe(b.SK_PRECISION_F32, m, n, lda, align, d, zeta, **MI355X)
    want = (1, 4) if (align == 16 and lda % 4 == 0) else (1, 2) if align >= 8 and lda % 2 == 0 \
        else (0, 0)
    assert (p["fused"], p["words"]) == want
    B = run_fused(Ad, d, zeta, 21, "f32")
    A_host = np.ascontiguousarray(A.reshape(-1)[offset:offset + m * lda].reshape(m, lda)[:, :n])
    ri, v = oracle.meta_ref(21, m, d, zeta)
    assert np.array_equal(B, oracle.sketch_f64(A_host, ri, v, d, zeta))


@pytest.mark.parametrize("m,n,lda,offset,d,zeta", [
    (5000, 1, 1, 0, 512, 4),        # a vector
    (3001, 31, 33, 1, 256, 16),     # odd width and stride, 4-byte aligned base
    (4096, 63, 64, 3, 128, 1),      # 63 columns, CountSketch
    (2000, 64, 67, 0, 1024, 4),     # 64 columns, d = 1024 in two row groups
])
def test_fused_f32_one_word_lanes(m, n, lda, offset, d, zeta):
    """FP32 of at most 64 columns runs one word per lane with 4-byte loads:
    any width, stride and base.  Integer inputs keep every sum exact, so the
    sketch equals the fp64 oracle bit for bit."""
    say(f"fused f32 one word m={m} n={n} lda={lda} offset={offset} d={d} zeta={zeta}")
    A = inputs.integer_matrix(m + 1, lda, -8, 8, seed=31)
    flat = to_dev(A).reshape(-1)
    Ad = flat[offset:offset + m * lda].reshape(m, lda)[:, :n]
    p = b.sk_fused_plan_describe(b.SK_PRECISION_F32, m, n, lda, 16 if offset == 0 else 4, d,
                                 zeta, **MI355X)
    assert (p["fused"], p["words"]) == (1, 1)
    B = run_fused(Ad, d, zeta, 5, "f32")
    A_host = np.ascontiguousarray(A.reshape(-1)[offset:offset + m * lda].reshape(m, lda)[:, :n])
    ri, v = oracle.meta_ref(5, m, d, zeta)
    assert np.array_equal(B, oracle.sketch_f64(A_host, ri, v, d, zeta))


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_fused_empty_input(precision):
    d, n = 64, 128
    dt = torch.float16 if precision == "f16acc" else torch.float32
    out = torch.full((d, n), 3.0, dtype=dt, device=dev())
    A = torch.empty((0, n), dtype=torch.float32, device=dev())
    b.sketch_fused(A, d, 4, 1, precision, out=out, flags=b.SK_ACCUMULATE)
    sync()
    assert torch.all(out == 3.0)
    b.sketch_fused(A, d, 4, 1, precision, out=out)
    sync()
    assert torch.all(out == 0.0)


def test_fused_workspace_too_small_is_refused():
    m, n, d, zeta = 4096, 256, 512, 4
    Ad = to_dev(inputs.gaussian(m, n))
    need = b.sk_sketch_workspace_size(b.SK_PRECISION_F16ACC, m, n, d, zeta)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=dev())
    with pytest.raises(b.SketchError):
        b.sketch_fused(Ad, d, zeta, 1, "f16acc", ws=ws)


def test_fused_equals_meta_plus_apply_f32_exact():
    """Same seed: the fused call and sk_meta_generate + sk_apply_f32 give the
    same sketch (exact inputs, so the order of additions cannot matter)."""
    m, n, d, zeta = 20000, 256, 512, 4
    A = inputs.integer_matrix(m, n, -8, 8, seed=31)
    Ad = to_dev(A)
    Bf = b.sketch_fused(Ad, d, zeta, 77, "f32")
    Bm = b.sketch(Ad, d, zeta, 77, "f32")
    sync()
    assert torch.equal(Bf, Bm)


# --------------------------- scale configuration (A 2^20 x 256, d = 512)

@pytest.fixture(scope="module")
def scale_case():
    """A 2^20 x 256 N(0,1) drawn on the device (seeded); zeta = 4, d = 512."""
    m, n, d, zeta, seed = 1 << 20, 256, 512, 4, 1
    say("fused scale case: drawing A and the fp64 oracle sketch")
    Ad = inputs.gaussian_torch(m, n, seed=0)
    A = Ad.cpu().numpy()
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    return Ad, A, d, zeta, seed, oracle.sketch_f64(A, ri, v, d, zeta)


@pytest.mark.parametrize("precision,tol", [("f32", 1e-5), ("f16acc", 4e-3)])
def test_fused_scale(scale_case, precision, tol):
    """The bench's configuration, in the launch configuration bench.py times."""
    Ad, A, d, zeta, seed, ref = scale_case
    assert fused_used(precision, *Ad.shape, Ad.shape[1], d, zeta)
    B = run_fused(Ad, d, zeta, seed, precision)
    err = oracle.rel_frob(B, ref)
    say(f"  fused scale {precision} rel err {err:.3e}")
    assert err <= tol


def test_fused_scale_sampled_rows_exact(scale_case):
    """At full size, sampled output rows recomputed one by one: with the
    input rounded to multiples of 1/4 in [-4, 4] every FP32 partial sum is
    exact, so each sampled row must match the oracle's bit for bit."""
    Ad, A, d, zeta, seed, _ = scale_case
    Aq = torch.clamp(torch.round(Ad * 4) / 4, -4, 4)
    B = run_fused(Aq, d, zeta, seed + 1, "f32")
    Aq_h = Aq.cpu().numpy().astype(np.float64)
    ri, v = oracle.meta_ref(seed + 1, Aq_h.shape[0], d, zeta)
    for r in (0, 1, 127, 128, 255, 300, 511):
        hit = np.nonzero(ri == r)[0]
        row = (v[hit].astype(np.float64)[:, None] * Aq_h[hit // zeta]).sum(axis=0)
        assert np.array_equal(B[r], row), r


def test_fused_f16_scale_sampled_columns_library_order(scale_case):
    """At full size, sampled columns: the FP16 sketch (register kernel) is
    the oracle's RN emulation of the library's order bit for bit: each
    output entry adds its contributions per row chunk of the plan in
    ascending row order from +0, and the chunk partials in the reduce's
    four contiguous groups (FP16 sketching page §III-B, §III-D).  The
    columns of the FP16 sum are independent, so a few columns of A emulate
    those columns of the sketch."""
    Ad, A, d, zeta, seed, _ = scale_case
    m, n = A.shape
    p = b.sk_sketch_plan_describe(b.SK_PRECISION_F16ACC, m, n, n, 16, d, zeta, **MI355X)
    assert p["kernel"] == 1 and p["chunks"] > 4
    B = run_fused(Ad, d, zeta, seed, "f16acc")
    cols = [0, 1, 127, 128, 254, 255]
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    exp = oracle.sketch_f16_rn_emul(np.ascontiguousarray(A[:, cols]), ri, v, d, zeta,
                                    chunk_rows=p["rows_per_chunk"], groups=4)
    assert np.array_equal(B[:, cols], exp.astype(np.float64))


def test_fused_f16_coherence_scale_sampled_rows_library_order():
    """The coherence sweep's heaviest point at full size (A 2^20 x 128,
    zeta = 8, d = 1024: one word per lane in two row groups, two workgroups
    per CU), sampled output rows in both row groups and several blocks: bit
    for bit the oracle's RN emulation with the plan's row chunks and the
    reduce's four groups.  An output row's sum involves only its own
    contributions, so the emulation keeps the metadata entries of the
    sampled rows and drops the rest (an entry outside its block adds
    nothing)."""
    m, n, d, zeta, seed = 1 << 20, 128, 1024, 8, 3
    p = b.sk_sketch_plan_describe(b.SK_PRECISION_F16ACC, m, n, n, 16, d, zeta, **MI355X)
    q = b.sk_fused_plan_describe(b.SK_PRECISION_F16ACC, m, n, n, 16, d, zeta, **MI355X)
    assert p["kernel"] == 1 and p["chunks"] > 4 and q["groups"] == 2 and q["per_cu"] == 2
    say("fused coherence-scale case: 2^20 x 128, zeta = 8, d = 1024")
    Ad = inputs.gaussian_torch(m, n, seed=5)
    B = run_fused(Ad, d, zeta, seed, "f16acc")
    A = Ad.cpu().numpy()
    del Ad
    rows = np.array([0, 1, 127, 128, 511, 512, 640, 1023])
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    ri_s = np.where(np.isin(ri, rows), ri, -1).astype(np.int32)
    exp = oracle.sketch_f16_rn_emul(A, ri_s, v, d, zeta, chunk_rows=p["rows_per_chunk"],
                                    groups=4)
    assert np.array_equal(B[rows], exp[rows].astype(np.float64))


# (m, n, d, zeta): register-kernel plans with many row chunks (one and two
# words per lane, one and two workgroups per CU, 128- and 64-row stages)
ORDER_SHAPES = [(20000, 256, 512, 4), (30000, 128, 1024, 8), (20000, 384, 512, 4),
                (9000, 128, 256, 1), (3001, 256, 128, 4), (50000, 96, 512, 2),
                (12000, 128, 2048, 4)]     # one word per lane, four row groups


@pytest.mark.parametrize("m,n,d,zeta", ORDER_SHAPES)
def test_fused_f16_library_order(m, n, d, zeta):
    """The whole FP16 sketch at multi-chunk sizes equals the oracle's RN
    emulation with the plan's row chunks and the reduce's four groups, bit
    for bit, on Gaussian inputs whose additions round."""
    p = b.sk_sketch_plan_describe(b.SK_PRECISION_F16ACC, m, n, n, 16, d, zeta, **MI355X)
    assert p["kernel"] == 1 and p["chunks"] > 1
    say(f"library order {m}x{n} d={d} zeta={zeta} chunks={p['chunks']}")
    A = (inputs.gaussian(m, n, seed=41) * np.float32(3.0)).astype(np.float32)
    ri, v = oracle.meta_ref(17, m, d, zeta)
    exp = oracle.sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=p["rows_per_chunk"], groups=4)
    assert np.array_equal(run_fused(A, d, zeta, 17, "f16acc"), exp.astype(np.float64))
