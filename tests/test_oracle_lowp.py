"""Pins of the conversion-variant oracle (oracle/lowp.py) against things
other than itself: the scalar Philox, a brute-force table of every finite
FP16 value, closed-form stochastic-rounding counts, torch's own BFloat16
conversion and addition on the CPU, and the RN oracle as a special case
(FP16 sketching page §III-D, §V-E)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta_ref, sketch_f16_rn_emul, sketch_f64, sketch_lowp_emul
from oracle.philox import philox_scalar
from sparse_sketching_amd import inputs


def f16_table():
    """Every finite binary16 value, ascending (brute force over all bit patterns)."""
    v = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    return np.unique(v[np.isfinite(v)])


def test_sr_words_match_scalar_philox():
    g = np.array([0, 7, (1 << 32) + 3, 12345678901], dtype=np.uint64)
    t = np.array([0, 1, 2, 15])
    c = np.array([0, 5, 11, 255])
    seed = 0xDEADBEEF12345
    w = oracle.sr_words(seed, g, t, c)
    for k in range(4):
        gi, ti, ci = int(g[k]), int(t[k]), int(c[k])
        ref = philox_scalar((gi & 0xFFFFFFFF, gi >> 32, ci >> 2, 3 + 4 * ti),
                            (seed & 0xFFFFFFFF, seed >> 32))[ci & 3]
        assert int(w[k]) == ref


def test_sr_words_differ_from_metadata_words():
    """Same seed, row and column group: the SR stream is not the metadata stream."""
    w = oracle.sr_words(1, np.arange(64), 0, 0)
    meta = oracle.philox4x32_10(np.arange(64), 0, 0, 0, 1, 0)[0]
    assert not np.array_equal(w, meta)


def test_f16_neighbours_brute_force():
    table = f16_table()
    pos = table[table >= 0]
    rng = np.random.default_rng(3)
    z = np.concatenate([np.abs(rng.standard_normal(4000)) * 2.0 ** rng.integers(-30, 17, 4000),
                        pos[::97], [0.0, 2.0**-25, 2.0**-24, 65504.0, 65505.0, 65519.9, 65520.0,
                                    65536.0, 1e6]]).astype(np.float32).astype(np.float64)
    l, v = oracle.f16_neighbours(z)
    k = np.searchsorted(pos, z, side="right") - 1          # largest value <= z
    assert np.array_equal(l, pos[k])
    nxt = np.where(k + 1 < pos.size, pos[np.minimum(k + 1, pos.size - 1)], 65536.0)
    assert np.array_equal(v, nxt)


def test_sr_representable_unchanged_and_neighbours_only():
    table = f16_table()
    rng = np.random.default_rng(4)
    rep = table[rng.integers(0, table.size, 2000)].astype(np.float32)
    r = rng.integers(0, 1 << 32, rep.size, dtype=np.uint64)
    assert np.array_equal(oracle.sr_f16(rep, r).astype(np.float64), rep.astype(np.float64))
    q = (rng.standard_normal(5000) * 2.0 ** rng.integers(-28, 14, 5000)).astype(np.float32)
    r = rng.integers(0, 1 << 32, q.size, dtype=np.uint64)
    out = oracle.sr_f16(q, r).astype(np.float64)
    l, v = oracle.f16_neighbours(np.abs(q).astype(np.float64))
    assert np.all((np.abs(out) == l) | (np.abs(out) == v))
    assert np.all(np.signbit(out) == np.signbit(q))


def test_sr_closed_form_counts():
    """Over the 2^16 evenly spaced draws r = k * 2^16 the number of round-ups
    is ceil(frac * 2^16): the empirical mean is q to within one 2^-16 step of
    the neighbour gap (finite-bit unbiasedness)."""
    q = np.array([1 + 2.0**-12, 1 + 3 * 2.0**-13, 2.0**-26, 3 * 2.0**-27, 0.1, 1000.3, 2.0**-20 / 3],
                 dtype=np.float32)
    r = (np.arange(1 << 16, dtype=np.uint64) << np.uint64(16))
    for x in q:
        out = oracle.sr_f16(np.full(r.size, x, np.float32), r).astype(np.float64)
        l, v = oracle.f16_neighbours(np.array([float(x)]))
        frac = (float(x) - l[0]) / (v[0] - l[0])
        ups = int(np.sum(out == v[0]))
        assert ups == int(np.ceil(frac * 65536))
        assert abs(out.mean() - float(x)) <= (v[0] - l[0]) / 65536


def test_sr_special_cases():
    h = 2.0**-24
    # half the smallest subnormal: RN erases it, SR keeps it with probability 1/2
    x = np.float32(h / 2)
    assert float(np.float16(x)) == 0.0
    assert float(oracle.sr_f16(np.array([x]), np.array([2**31 - 1]))[0]) == h
    assert float(oracle.sr_f16(np.array([x]), np.array([2**31]))[0]) == 0.0
    # past the largest finite value: 2^16 is the overflow neighbour
    y = np.array([65520.0, -65520.0, 65504.0], np.float32)
    assert np.isinf(oracle.sr_f16(y, np.array([0, 0, 0]))[:2]).all()
    assert float(oracle.sr_f16(y, np.array([2**31, 2**31, 0]))[0]) == 65504.0
    assert float(oracle.sr_f16(y, np.array([0, 0, 0]))[2]) == 65504.0
    # signed zeros stay
    z = oracle.sr_f16(np.array([0.0, -0.0], np.float32), np.array([0, 0]))
    assert np.array_equal(np.signbit(z), [False, True])


def _bf16_cases():
    rng = np.random.default_rng(7)
    with np.errstate(over="ignore"):
        x = (rng.standard_normal(20000) * 2.0 ** rng.integers(-140, 128, 20000)).astype(np.float32)
    # ties: an odd number of 2^-8 ulps above a BF16 value, both parities
    base = np.float32(1.0) + np.arange(64, dtype=np.float32) * np.float32(2.0**-7)
    ties = base + np.float32(2.0**-8)
    sub = np.array([1e-40, -3e-39, 1.2e-38, 2.0**-133], np.float32)
    big = np.array([3.38e38, 3.39e38, 3.4e38, -3.4e38, np.finfo(np.float32).max], np.float32)
    return np.concatenate([x, ties, sub, big, np.array([0.0, -0.0], np.float32)])


def test_rn_bf16_matches_torch():
    x = _bf16_cases()
    ours = oracle.rn_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref, equal_nan=True)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
    assert np.isnan(oracle.rn_bf16(np.array([np.nan], np.float32))[0])


def test_rn_bf16_add_matches_torch():
    rng = np.random.default_rng(8)
    a = oracle.rn_bf16((rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 30, 20000)).astype(np.float32))
    b = oracle.rn_bf16((rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 30, 20000)).astype(np.float32))
    ours = oracle.rn_bf16_add(a, b)
    ref = (torch.from_numpy(a).to(torch.bfloat16) + torch.from_numpy(b).to(torch.bfloat16)).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_lowp_rn_f16_reduces_to_rn_oracle():
    m, n, d, zeta = 600, 12, 32, 4
    A = inputs.gaussian(m, n, seed=1)
    ri, v = oracle.meta_ref(3, m, d, zeta)
    assert np.array_equal(oracle.sketch_lowp_emul(A, ri, v, d, zeta, "f16", "rn"),
                          oracle.sketch_f16_rn_emul(A, ri, v, d, zeta))


def test_lowp_bf16_exact_inputs_equal_fp64():
    m, n, d, zeta = 800, 10, 32, 4
    A = inputs.integer_matrix(m, n, -3, 3, seed=2)
    ri, v = oracle.meta_ref(5, m, d, zeta)
    B = oracle.sketch_lowp_emul(A, ri, v, d, zeta, "bf16", "rn")
    assert np.array_equal(B.astype(np.float64), oracle.sketch_f64(A, ri, v, d, zeta))


def test_lowp_sr_coordinate_input_is_one_conversion_per_entry():
    """A = [I_n 0]^T * x: output entry (row_idx(i,t), i) receives exactly one
    contribution q = x_i * val, so it equals SR(q) with that entry's draw."""
    m, n, d, zeta, seed, off = 256, 24, 64, 4, 9, 1000
    x = (np.random.default_rng(2).standard_normal(n) * 2.0**-18).astype(np.float32)
    A = inputs.coordinate(m, n) * x[None, :]
    ri, v = oracle.meta_ref(4, m, d, zeta, row_offset=off)
    B = oracle.sketch_lowp_emul(A, ri, v, d, zeta, "f16", "sr", sr_seed=seed, row_offset=off)
    for i in range(n):
        for t in range(zeta):
            q = np.float32(x[i]) * v[i * zeta + t]
            r = oracle.sr_words(seed, off + i, t, i)
            assert B[ri[i * zeta + t], i] == oracle.sr_f16(np.array([q]), np.array([r]))[0]


def test_lowp_sr_mean_over_draws_is_unbiased():
    """Tiny contributions that RN erases (|q| < h/2) survive SR in
    expectation: the error of the mean over N independent SR draws falls
    like 1/sqrt(N) (a biased rule would level off), and 16x more draws cut
    it about 4x."""
    m, n, d, zeta = 200, 8, 16, 4
    A = (inputs.gaussian(m, n, seed=3) * np.float32(2.0**-26)).astype(np.float32)
    ri, v = oracle.meta_ref(2, m, d, zeta)
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    rn = oracle.sketch_lowp_emul(A, ri, v, d, zeta, "f16", "rn").astype(np.float64)

    def mean_err(seeds):
        mean = np.mean([oracle.sketch_lowp_emul(A, ri, v, d, zeta, "f16", "sr", sr_seed=s)
                        .astype(np.float64) for s in seeds], axis=0)
        return oracle.rel_frob(mean, ref)

    e12, e192 = mean_err(range(12)), mean_err(range(100, 292))
    assert oracle.rel_frob(rn, ref) > 0.9                  # RN loses nearly everything
    assert e192 < 0.3 and e12 / e192 > 2.5, (e12, e192)


@pytest.mark.parametrize("fmt,conv", [("f16", "rn"), ("f16", "sr"), ("bf16", "rn")])
def test_lowp_chunked_orders(fmt, conv):
    """Chunks of one row: each partial holds at most one contribution per
    output entry, so the chunked order equals the flat one; the whole matrix
    as one chunk equals it too; FP16 RN chunks equal the RN oracle's own
    chunked order (an independent implementation)."""
    m, n, d, zeta = 300, 6, 16, 4
    A = (inputs.gaussian(m, n, seed=2) * np.float32(29.0)).astype(np.float32)
    ri, v = meta_ref(3, m, d, zeta)
    flat = sketch_lowp_emul(A, ri, v, d, zeta, fmt, conv, sr_seed=5, row_offset=7)
    one = sketch_lowp_emul(A, ri, v, d, zeta, fmt, conv, sr_seed=5, row_offset=7, chunk_rows=1)
    whole = sketch_lowp_emul(A, ri, v, d, zeta, fmt, conv, sr_seed=5, row_offset=7,
                             chunk_rows=m)
    assert np.array_equal(one, flat) and np.array_equal(whole, flat)
    if fmt == "f16" and conv == "rn":
        for ch in (7, 64):
            assert np.array_equal(sketch_lowp_emul(A, ri, v, d, zeta, chunk_rows=ch),
                                  sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=ch))
            assert np.array_equal(
                sketch_lowp_emul(A, ri, v, d, zeta, chunk_rows=ch, combine="f32"),
                sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=ch, combine="f32"))


def test_lowp_bf16_chunked_exact_sums():
    """Integer inputs whose every partial sum is exact in BF16: any chunking
    and either combine equal fp64."""
    m, n, d, zeta = 2048, 8, 64, 4
    A = inputs.integer_matrix(m, n, -3, 3, seed=8)
    ri, v = meta_ref(2, m, d, zeta)
    ref = sketch_f64(A, ri, v, d, zeta)
    assert np.abs(ref).max() <= 256
    for ch, comb in ((64, "fmt"), (100, "f32"), (None, "fmt")):
        got = sketch_lowp_emul(A, ri, v, d, zeta, "bf16", "rn", chunk_rows=ch, combine=comb)
        assert np.array_equal(got.astype(np.float64), ref)
