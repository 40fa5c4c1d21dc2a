"""GPU parity of the fused sketch on narrow rows, where the owner kernel runs
(lanes own output rows; each stage's hits are counting-sorted into per-row
lists and walked in ascending row order).

Its order of additions is the register kernel's: each output entry adds the
FP16 RN contributions of its workgroup's row chunk in ascending row order
from +0, and the reduce sums the chunk partials in four contiguous groups
(each from +0 in chunk order, then the group sums in order).  So the FP16
sketch equals the oracle's RN emulation with the plan's chunk rows and
groups=4 bit for bit (FP16 sketching page §III-B, §III-D), on Gaussian
inputs whose additions round.  FP32 sketches are checked against fp64
(relative Frobenius 1e-5) and bit for bit on integer inputs.  Shapes cover
the plan's word widths (1 to 16 words per lane), padded rows (a row's words
not a power of two), strided and 8-byte-aligned A, zeta up to 16, small and
ragged m, row offsets past 2^32, and stages where an output row has more
hits than its list holds (the walk from the mask)."""
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

# (m, n, d, zeta)
OWNER_SHAPES = [
    (50000, 2, 512, 4),         # the m x 2 right-hand side shape (one word per lane)
    (16384, 64, 128, 4),        # the range workload's shape, four words per lane
    (10000, 32, 1024, 1),       # sixteen words per lane, CountSketch
    (3001, 6, 48, 3),           # 3 column pairs padded to 4 words, ragged m
    (20000, 16, 128, 16),       # zeta = 16: four Philox blocks per row
    (777, 2, 64, 4),            # a single wavefront per workgroup
    (65536, 64, 256, 8),        # eight words per lane
    (1, 4, 64, 4),              # a single row
    (130, 8, 96, 2),            # one stage plus two rows
    (40000, 64, 512, 4),        # FP16 sixteen words per lane, four load slots
    (30000, 32, 512, 4),        # FP32 sixteen words per lane, two load slots
    (300000, 32, 1024, 4),      # FP16 two load slots over several stages per chunk
]


def plan(precision, m, n, lda, align, d, zeta):
    return b.sk_sketch_plan_describe(PREC[precision], m, n, lda, align, d, zeta, **MI355X)


def sketch(Ad, d, zeta, seed, precision, row_offset=0, out=None, flags=0):
    B = b.sketch_fused(Ad, d, zeta, seed, precision, row_offset=row_offset, out=out, flags=flags)
    sync()
    return B.cpu().numpy().astype(np.float64)


def f16_expect(A, seed, d, zeta, p, row_offset=0, combine="f16", B0=None):
    ri, v = oracle.meta_ref(seed, A.shape[0], d, zeta, row_offset)
    return oracle.sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=p["rows_per_chunk"],
                                     groups=4, combine=combine, B0=B0).astype(np.float64)


def same(got, exp):
    return np.array_equal(got, exp, equal_nan=True)


@pytest.mark.parametrize("m,n,d,zeta", OWNER_SHAPES)
def test_owner_fp16_matches_rn_emulation(m, n, d, zeta):
    p = plan("f16acc", m, n, n, 16, d, zeta)
    assert p["kernel"] == 2
    say(f"owner f16 {m}x{n} d={d} zeta={zeta} V={p['words']} L={p['lanes_per_row']} "
        f"S={p['stage_rows']} cap={p['cap']} chunks={p['chunks']}")
    A = (inputs.gaussian(m, n, seed=31) * np.float32(3.0)).astype(np.float32)
    got = sketch(to_dev(A), d, zeta, 7, "f16acc")
    assert same(got, f16_expect(A, 7, d, zeta, p))


@pytest.mark.parametrize("m,n,d,zeta", OWNER_SHAPES)
def test_owner_fp32(m, n, d, zeta):
    p = plan("f32", m, n, n, 16, d, zeta)
    say(f"owner f32 {m}x{n} d={d} zeta={zeta} kernel={p['kernel']}")
    seed = 9
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    A = inputs.gaussian(m, n, seed=32)
    got = sketch(to_dev(A), d, zeta, seed, "f32")
    exp = oracle.sketch_f64(A, ri, v, d, zeta)
    assert np.linalg.norm(got - exp) <= 1e-5 * np.linalg.norm(exp)
    # small integers, zeta a power of four: every product and sum is exact
    if zeta in (1, 4, 16):
        Ai = inputs.integer_matrix(m, n, -3, 3, seed=33)
        assert np.array_equal(sketch(to_dev(Ai), d, zeta, seed, "f32"),
                              oracle.sketch_f64(Ai, ri, v, d, zeta))


def _stage_counts_exceed_cap(m, d, zeta, seed, p):
    """Does some output row get more hits in some stage than its list holds
    (counted from the oracle's metadata on the plan's chunks and stages)?"""
    ri, _ = oracle.meta_ref(seed, m, d, zeta)
    rows = np.repeat(np.arange(m, dtype=np.int64), zeta)
    rpc, S = p["rows_per_chunk"], p["stage_rows"]
    stage_id = (rows // rpc) * (rpc // S) + (rows % rpc) // S
    key = stage_id * d + ri.astype(np.int64)
    return int(np.bincount(key).max()) > p["cap"]


# (m, n, d, zeta, barriers per stage in the FP16 plan, in the FP32 plan)
ONE_BARRIER_SHAPES = [
    (5 * 256 * 512 - 77, 2, 256, 4, 1, 1),     # lists overflow; five stages per chunk
    (3 * 256 * 256 + 100, 32, 256, 8, 1, 2),   # four words per lane, ragged last chunk
    ((1 << 20) - 3, 8, 128, 4, 1, 1),          # FP16: two workgroups per CU
    ((1 << 20) - 3, 4, 128, 4, 2, 1),          # FP32: two workgroups per CU
    (300001, 24, 192, 16, 1, 1),               # zeta = 16, 4 and 8 words per lane
    (400000, 6, 192, 8, 1, 1),                 # 3 column pairs padded to 4 words, one-word loads
]


@pytest.mark.parametrize("m,n,d,zeta,bar16,bar32", ONE_BARRIER_SHAPES)
def test_owner_one_barrier_pipeline_over_several_stages(m, n, d, zeta, bar16, bar32):
    """Shapes the one-barrier pipeline serves, with several stages per chunk
    (the three stage buffers rotate more than once) and a ragged last chunk,
    next to the two-barrier pipeline where the plan keeps it."""
    seed = 13
    A = (inputs.gaussian(m, n, seed=35) * np.float32(3.0)).astype(np.float32)
    Ad = to_dev(A)
    for prec, bar in (("f16acc", bar16), ("f32", bar32)):
        p = plan(prec, m, n, n, 16, d, zeta)
        say(f"owner one-barrier {prec} {m}x{n} d={d} zeta={zeta} V={p['words']} S={p['stage_rows']} "
            f"barriers={p['barriers']} per_cu={p['per_cu']} chunks={p['chunks']}")
        assert p["kernel"] == 2 and p["barriers"] == bar
        assert p["rows_per_chunk"] // p["stage_rows"] >= 4
        if prec == "f16acc":
            assert same(sketch(Ad, d, zeta, seed, prec), f16_expect(A, seed, d, zeta, p))
        else:
            ri, v = oracle.meta_ref(seed, m, d, zeta)
            exp = oracle.sketch_f64(A, ri, v, d, zeta)
            got = sketch(Ad, d, zeta, seed, prec)
            assert np.linalg.norm(got - exp) <= 1e-5 * np.linalg.norm(exp)
    if n == 2:
        assert _stage_counts_exceed_cap(m, d, zeta, seed, plan("f16acc", m, n, n, 16, d, zeta))


def test_owner_list_overflow_walks_the_mask():
    """Enough stages that some output row has more hits in a stage than its
    list holds (checked on the host from the oracle's metadata): those hits
    are walked from the row's mask, in the same order."""
    m, n, d, zeta, seed = 1 << 18, 2, 512, 4, 5
    p = plan("f16acc", m, n, n, 16, d, zeta)
    assert p["kernel"] == 2
    assert _stage_counts_exceed_cap(m, d, zeta, seed, p)
    A = (inputs.gaussian(m, n, seed=34) * np.float32(5.0)).astype(np.float32)
    Ad = to_dev(A)
    assert same(sketch(Ad, d, zeta, seed, "f16acc"), f16_expect(A, seed, d, zeta, p))
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    got = sketch(Ad, d, zeta, seed, "f32")
    exp = oracle.sketch_f64(A, ri, v, d, zeta)
    assert np.linalg.norm(got - exp) <= 1e-5 * np.linalg.norm(exp)


@pytest.mark.parametrize("lda_extra,offset", [(2, 0), (4, 0), (0, 2), (6, 2)])
def test_owner_strided_and_unaligned(lda_extra, offset):
    """A as a view: rows lda = n + lda_extra floats apart, base offset floats
    past a 256-byte boundary (8-byte aligned: one-word loads)."""
    m, n, d, zeta, seed = 9000, 16, 128, 4, 3
    lda = n + lda_extra
    A = inputs.gaussian(m, n, seed=35)
    big = torch.zeros(m * lda + offset + 8, dtype=torch.float32, device=dev())
    view = big[offset:offset + m * lda].view(m, lda)[:, :n]
    view.copy_(to_dev(A))
    align = 16 if offset == 0 else 8
    p = plan("f16acc", m, n, lda, align, d, zeta)
    assert p["kernel"] == 2 and p["load_words"] == (2 if align == 16 and lda % 4 == 0 else 1)
    say(f"owner strided lda={lda} offset={offset} load_words={p['load_words']}")
    assert same(sketch(view, d, zeta, seed, "f16acc"), f16_expect(A, seed, d, zeta, p))


def test_owner_row_offset_past_2_32():
    m, n, d, zeta, seed, off = 5000, 8, 64, 4, 11, (1 << 32) + 12345
    A = inputs.gaussian(m, n, seed=36)
    p = plan("f16acc", m, n, n, 16, d, zeta)
    assert p["kernel"] == 2
    got = sketch(to_dev(A), d, zeta, seed, "f16acc", row_offset=off)
    assert same(got, f16_expect(A, seed, d, zeta, p, row_offset=off))


@pytest.mark.parametrize("combine", ["f16", "f32"])
def test_owner_accumulate(combine):
    """B += S A onto an existing FP16 sketch, with the FP16 or the FP32
    combine: the reduce starts from B's words."""
    m, n, d, zeta, seed = 20000, 32, 256, 4, 13
    A = (inputs.gaussian(m, n, seed=37) * np.float32(7.0)).astype(np.float32)
    B0 = (inputs.gaussian(d, n, seed=38) * np.float32(50.0)).astype(np.float16)
    p = plan("f16acc", m, n, n, 16, d, zeta)
    assert p["kernel"] == 2
    out = torch.from_numpy(B0.copy()).to(dev())
    flags = b.SK_ACCUMULATE | (b.SK_COMBINE_F32 if combine == "f32" else 0)
    got = sketch(to_dev(A), d, zeta, seed, "f16acc", out=out, flags=flags)
    assert same(got, f16_expect(A, seed, d, zeta, p, combine=combine, B0=B0))


def test_owner_range_shape_full_size_sampled_rows():
    """The range workload's shape at full size (4,194,304 x 64 FP16, zeta =
    4, d = 128: the owner kernel at four words per lane), sampled output
    rows from every block: bit for bit the oracle's RN emulation with the
    plan's chunks and the reduce's groups.  An output row's sum involves
    only its own contributions, so the emulation keeps the metadata entries
    of the sampled rows and drops the rest (an entry outside its block adds
    nothing)."""
    m, n, d, zeta, seed = 4194304, 64, 128, 4, 2
    p = plan("f16acc", m, n, n, 16, d, zeta)
    assert p["kernel"] == 2 and p["words"] == 4 and p["chunks"] > 4
    say(f"owner range shape full size: chunks={p['chunks']} rows_per_chunk={p['rows_per_chunk']}")
    Ad = inputs.gaussian_torch(m, n, seed=6)
    got = sketch(Ad, d, zeta, seed, "f16acc")
    A = Ad.cpu().numpy()
    del Ad
    rows = np.array([0, 1, 31, 32, 63, 64, 100, 127])
    ri, v = oracle.meta_ref(seed, m, d, zeta)
    ri_s = np.where(np.isin(ri, rows), ri, -1).astype(np.int32)
    exp = oracle.sketch_f16_rn_emul(A, ri_s, v, d, zeta, chunk_rows=p["rows_per_chunk"], groups=4)
    assert same(got[rows], exp[rows].astype(np.float64))


def test_owner_right_hand_side_full_size():
    """Sketch-and-solve's right-hand side at full size (2^20 x 2 FP16, zeta
    = 4, d = 512: one word per lane): every output entry bit for bit the
    oracle's RN emulation of the library order."""
    m, n, d, zeta, seed = 1 << 20, 2, 512, 4, 4
    p = plan("f16acc", m, n, n, 16, d, zeta)
    assert p["kernel"] == 2 and p["words"] == 1 and p["chunks"] > 4
    A = (inputs.gaussian(m, n, seed=7) * np.float32(3.0)).astype(np.float32)
    assert same(sketch(to_dev(A), d, zeta, seed, "f16acc"), f16_expect(A, seed, d, zeta, p))
