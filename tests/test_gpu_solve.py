"""GPU sketch-and-solve, ridge regression and sketch-quality metrics
against the CPU oracle (FP16 sketching page §V-A, §V-C, §V-D; FlashSketch
page App. F.1).

The oracle forms its own fp64 sketch from its own metadata and solves it;
the GPU pipeline sketches with the fused kernels and solves with FP32 QR.
Bars: FP32-sketch residuals within 1e-4 (relative) of the oracle's; FP16
residuals (every addition in FP16, the page's arithmetic), with the FP16 or
the FP32 combine of the chunk partials (SK_COMBINE_F32), within 1e-4 of the
residual of the oracle's RN emulation of the library's own order (each
sketch's plan chunks, the reduce's four groups: the sketches agree bit for
bit, the QR is FP32 against the oracle's fp64), and no worse than the
page's flat (single running sum) order.  The FP16 residual increase is the FP16 accumulation
of b's sketch itself: the noise (0.1) is small next to ||Ax0||, so the
accumulation error of Sb is large next to the residual (the oracle's flat
emulation gives +18% on the low-coherence system and +131% on the coherent
one, whose 1e3-scaled head rows dominate the entries they land in);
metric functions equal to the oracle's on the same arrays."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from sparse_sketching_amd import solve
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu


def system(m, n, seed, coherent=False, noise=0.1):
    A = inputs.coherent(m, n, seed=seed) if coherent else inputs.gaussian(m, n, seed=seed)
    g = np.random.default_rng(seed + 100)
    x0 = g.standard_normal(n).astype(np.float32)
    rhs = (A.astype(np.float64) @ x0 + noise * g.standard_normal(m)).astype(np.float32)
    return A, rhs


def oracle_residual(A, rhs, d, zeta, seed):
    ri, v = oracle.meta_ref(seed, A.shape[0], d, zeta)
    SA = oracle.sketch_f64(A, ri, v, d, zeta)
    Sb = oracle.sketch_f64(rhs[:, None], ri, v, d, zeta)[:, 0]
    x = oracle.sketch_solve(SA, Sb)
    return oracle.residual(A, x, rhs), x


def oracle_f16_residual(A, rhs, d, zeta, seed, chunk_rows, chunk_rows_b=None, groups=None,
                        combine="f16"):
    """Residual of the solve on the oracle's RN-emulated FP16 sketches of A
    and [b 0], for the flat order (chunk_rows=None) or row chunks (of
    chunk_rows rows for A, chunk_rows_b for [b 0]) combined with FP16
    additions, one after another or in `groups` groups (or, combine="f32",
    in FP32 rounded once)."""
    ri, v = oracle.meta_ref(seed, A.shape[0], d, zeta)
    B2 = np.zeros((A.shape[0], 2), dtype=np.float32)
    B2[:, 0] = rhs
    cb = chunk_rows if chunk_rows_b is None else chunk_rows_b
    SA = oracle.sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=chunk_rows, groups=groups,
                                   combine=combine).astype(np.float64)
    Sb = oracle.sketch_f16_rn_emul(B2, ri, v, d, zeta, chunk_rows=cb, groups=groups,
                                   combine=combine)[:, 0]
    return oracle.residual(A, oracle.sketch_solve(SA, Sb.astype(np.float64)), rhs)


def sketch_chunk_rows(m, n, d, zeta):
    """Rows per chunk of the fused FP16 sketch's plan (MI355X)."""
    return b.sk_sketch_plan_describe(b.SK_PRECISION_F16ACC, m, n, n, 16, d, zeta,
                                     num_cu=256, max_lds=160 * 1024)["rows_per_chunk"]


@pytest.mark.parametrize("coherent", [False, True])
def test_sketch_and_solve_matches_oracle(coherent):
    m, n, zeta, seed = 1 << 16, 128, 4, 7
    d = 2 * n
    A, rhs = system(m, n, 3, coherent)
    Ad, bd = to_dev(A), to_dev(rhs)
    x32, r32 = solve.sketch_and_solve(Ad, bd, d, zeta, seed, "f32")
    x16, r16 = solve.sketch_and_solve(Ad, bd, d, zeta, seed, "f16acc")
    x16c, r16c = solve.sketch_and_solve(Ad, bd, d, zeta, seed, "f16acc", combine="f32")
    sync()
    r_ref, _ = oracle_residual(A, rhs, d, zeta, seed)
    r_opt = oracle.residual(A, oracle.reference_solution(A, rhs), rhs)
    r_flat = oracle_f16_residual(A, rhs, d, zeta, seed, None)
    # the emulation of the library's own order: the fused sketches' chunks
    # (the register kernel's for A, the owner kernel's for the two-column
    # [b 0]) and the reduce's four groups
    ca, cb = sketch_chunk_rows(m, n, d, zeta), sketch_chunk_rows(m, 2, d, zeta)
    r_emu = oracle_f16_residual(A, rhs, d, zeta, seed, ca, cb, groups=4)
    r_emu_c = oracle_f16_residual(A, rhs, d, zeta, seed, ca, cb, groups=4, combine="f32")
    say(f"  coherent={coherent}: residual fp32 {r32:.6f} fp16 {r16:.6f} "
        f"fp16+fp32-combine {r16c:.6f} oracle fp64 {r_ref:.6f} oracle fp16 flat {r_flat:.6f} "
        f"oracle fp16 library order {r_emu:.6f} / {r_emu_c:.6f} unsketched {r_opt:.6f}")
    assert abs(r32 - r_ref) <= 1e-4 * r_ref
    assert r32 >= r_opt * (1 - 1e-6)
    # the FP16 sketches are the emulation's bit for bit; what is left is the
    # FP32 QR against the oracle's fp64 solve
    assert abs(r16 - r_emu) <= 1e-4 * r_emu
    assert abs(r16c - r_emu_c) <= 1e-4 * r_emu_c
    # FP16 accumulation costs residual, but no more than the page's flat
    # order
    assert r_ref * (1 - 1e-2) <= r16 <= r_flat * (1 + 1e-2)


def test_consistent_system_recovered():
    m, n, d, zeta = 1 << 15, 128, 256, 4
    A = inputs.gaussian(m, n, seed=5)
    x0 = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    rhs = (A @ x0).astype(np.float32)
    x, r = solve.sketch_and_solve(to_dev(A), to_dev(rhs), d, zeta, 2, "f32")
    sync()
    assert r < 1e-4
    assert np.linalg.norm(x.cpu().numpy() - x0) / np.linalg.norm(x0) < 1e-3


def test_ridge_on_gpu_sketch_matches_oracle():
    m, n, d, zeta = 1 << 15, 128, 256, 4
    A, rhs = system(m, n, 8)
    SA, Sb = solve.sketch_pair(to_dev(A), to_dev(rhs), d, zeta, 9, "f16acc")
    sync()
    SA_h, Sb_h = SA.cpu().numpy().astype(np.float64), Sb.cpu().numpy().astype(np.float64)
    for lam in (1e-3, 10.0, 1e4):
        x = solve.ridge_sketched(SA, Sb, lam)
        x_ref = oracle.ridge_solve(SA_h, Sb_h, lam)
        assert np.linalg.norm(x.cpu().numpy() - x_ref) <= 1e-4 * np.linalg.norm(x_ref)
        assert abs(solve.residual(to_dev(A), x, to_dev(rhs)) - oracle.residual(A, x_ref, rhs)) < 1e-4


def test_metrics_equal_oracle_on_same_arrays():
    m, n, d, zeta = 1 << 14, 64, 128, 4
    U = inputs.orth(inputs.coherent(m, n, seed=2))
    Ud = to_dev(U)
    SU = torch.from_numpy(np.ascontiguousarray(
        oracle.sketch_f64(U, *oracle.meta_ref(4, m, d, zeta), d, zeta))).to(dev())
    SU_h = SU.cpu().numpy()
    assert abs(solve.ose_error(SU) - oracle.ose_error(SU_h)) < 1e-10
    assert abs(solve.sv_ratio(SU) - oracle.sv_ratio(SU_h)) < 1e-10
    assert abs(solve.gram_rel_error(Ud, SU) - oracle.gram_rel_error(U, SU_h)) < 1e-10


def test_sparsestack_beats_countsketch_on_coherent_system():
    """Spreading each row over zeta targets helps coherent inputs (§V-C,
    §V-D): at d/n = 8 the zeta = 4 sketch-and-solve residual is no worse
    than CountSketch's in FP32.  In FP16 (FP16 row-chunk sums combined in
    FP32), at noise 1e-3, both residuals sit on the FP16 rounding floor of
    the sketched right-hand side (about ten times the FP32 residuals here),
    where the zeta effect is below the floor's seed-to-seed spread: they
    must stay within 10% of each other."""
    m, n = 1 << 16, 64
    d = 8 * n
    A, rhs = system(m, n, 4, coherent=True, noise=1e-3)
    Ad, bd = to_dev(A), to_dev(rhs)
    res = {}
    for zeta in (1, 4):
        for prec in ("f32", "f16acc"):
            res[(zeta, prec)] = min(solve.sketch_and_solve(Ad, bd, d, zeta, s, prec,
                                                           combine="f32")[1]
                                    for s in (1, 2, 3))
    sync()
    say(f"  coherent d/n=8 residuals {res}")
    assert res[(4, "f32")] <= res[(1, "f32")] * 1.0001
    assert res[(4, "f16acc")] <= res[(1, "f16acc")] * 1.1
    assert res[(1, "f16acc")] <= res[(4, "f16acc")] * 1.1


# ------------------------------------------- the library's FP32 QR solver

@pytest.mark.parametrize("d,n", [
    (512, 256),         # the sketch-and-solve size (d = 2n): eight 32-column panels
    (768, 256),         # the ridge system [SA; sqrt(lam) I]
    (100, 37),          # a 32-column panel, then 4- and 1-column panels
    (64, 64),           # square
    (33, 1),            # one column
    (1000, 777),        # 16-column panels, then 8, 1
    (2048, 1024),       # the largest: 8-column panels
])
def test_lstsq_qr_vs_oracle(d, n):
    """sk_lstsq_qr_f32 on N(0,1) systems: x within 5e-5 (relative) of the
    oracle's fp64 QR solution (an FP32 Householder solve of a matrix with
    condition number below ~10 on these shapes), and its residual within
    1e-5 (relative, plus 1e-5 absolute for FP32 rounding on consistent
    square systems) of the fp64 minimum."""
    from sparse_sketching_amd import binding as b
    say(f"lstsq qr d={d} n={n}")
    g = np.random.default_rng(d * 7 + n)
    M = g.standard_normal((d, n)).astype(np.float32)
    y = g.standard_normal(d).astype(np.float32)
    x = b.lstsq_qr(to_dev(M), to_dev(y))
    sync()
    x = x.cpu().numpy().astype(np.float64)
    ref = oracle.lstsq_qr(M, y)
    assert np.linalg.norm(x - ref) <= 5e-5 * np.linalg.norm(ref)
    assert oracle.residual(M, x, y) <= oracle.residual(M, ref, y) * (1 + 1e-5) + 1e-5


@pytest.mark.parametrize("d,n", [(512, 256), (100, 37), (40, 40)])
def test_lstsq_qr_exact_triangular(d, n):
    """SA = [U; 0] with U upper triangular (power-of-two diagonal, small
    integer entries) and Sb = [U x0; 0] for integer x0: every reflector is
    the identity (tau = 0, nothing below the diagonal), so R = U and
    Q^T Sb = Sb exactly, and the blocked back substitution must return x0
    bit for bit (all partial sums are integers below 2^24)."""
    from sparse_sketching_amd import binding as b
    say(f"lstsq exact d={d} n={n}")
    g = np.random.default_rng(n)
    U = np.triu(g.integers(-2, 3, size=(n, n))).astype(np.float64)
    np.fill_diagonal(U, g.choice([-2.0, -1.0, 1.0, 2.0], size=n))
    # z = U x0 is integer; the back substitution's running value at row i
    # is z_i - sum_{j>i} U_ij x0_j = U_ii x0_i, an integer below 2^24 at
    # every step, and dividing it by U_ii (a power of two) gives x0_i
    x0 = g.integers(-3, 4, size=n).astype(np.float64)
    z = U @ x0
    assert np.abs(z).max() < 2 ** 20
    SA = np.zeros((d, n), dtype=np.float32)
    SA[:n] = U
    Sb = np.zeros(d, dtype=np.float32)
    Sb[:n] = z
    x = b.lstsq_qr(to_dev(SA), to_dev(Sb))
    sync()
    assert np.array_equal(x.cpu().numpy().astype(np.float64), x0)


@pytest.mark.parametrize("d,n", [(512, 256), (100, 37)])
def test_lstsq_qr_power_of_two_scaling(d, n):
    """The solver scales every column of [SA | Sb] by a power of two before
    the QR and x back after it, and Householder QR commutes exactly with such
    scalings: with SA's columns scaled by 2^k_j and Sb by 2^kb, x_j comes out
    as x0_j 2^(kb - k_j) bit for bit (x0: the unscaled system's solution);
    with everything scaled by 2^90 or 2^-90, where the squared entries
    overflow or underflow in FP32, x0 itself, bit for bit, and x0 is within
    the oracle's bar."""
    from sparse_sketching_amd import binding as b
    say(f"lstsq power-of-two scaling d={d} n={n}")
    g = np.random.default_rng(d + 5 * n)
    M = g.standard_normal((d, n)).astype(np.float32)
    y = g.standard_normal(d).astype(np.float32)
    assert np.abs(M).min() > 2.0**-30 and np.abs(y).min() > 2.0**-30   # scaled copies stay normal
    x0 = b.lstsq_qr(to_dev(M), to_dev(y))
    sync()
    x0 = x0.cpu().numpy()
    ref = oracle.lstsq_qr(M, y)
    assert np.linalg.norm(x0 - ref) <= 5e-5 * np.linalg.norm(ref)
    k = g.integers(-40, 41, size=n)
    kb = 17
    Mk = np.ldexp(M, k[None, :]).astype(np.float32)
    xk = b.lstsq_qr(to_dev(Mk), to_dev(np.ldexp(y, kb).astype(np.float32)))
    sync()
    assert np.array_equal(xk.cpu().numpy(), np.ldexp(x0, kb - k).astype(np.float32))
    for e in (90, -90):
        Me = np.ldexp(M, e).astype(np.float32)
        sq = Me.astype(np.float32) * Me.astype(np.float32)
        # the test can fail: unscaled, the column norms overflow (underflow)
        assert np.isinf(sq).any() if e > 0 else (sq == 0).all()
        xe = b.lstsq_qr(to_dev(Me), to_dev(np.ldexp(y, e).astype(np.float32)))
        sync()
        assert np.array_equal(xe.cpu().numpy(), x0), e


def test_lstsq_qr_matches_sketch_solve_route():
    """The library's solver on a real sketch (the FP32 fused sketch of a 2^16
    x 128 system, d = 256): same residual as the oracle's FP32 QR of the same
    sketch, within 1e-5 relative."""
    from sparse_sketching_amd import binding as b
    m, n, d, zeta, seed = 1 << 16, 128, 256, 4, 3
    A, rhs = system(m, n, seed=21)
    SA, Sb = solve.sketch_pair(to_dev(A), to_dev(rhs), d, zeta, seed, "f32")
    x = b.lstsq_qr(SA, Sb)
    sync()
    x_or = oracle.sketch_solve(SA.cpu().numpy(), Sb.cpu().numpy())
    r_gpu = oracle.residual(A, x.cpu().numpy(), rhs)
    r_or = oracle.residual(A, x_or, rhs)
    assert abs(r_gpu - r_or) <= 1e-5 * r_or


def test_lstsq_qr_padded_stride():
    """SA as a column slice of a wider matrix (row stride ld = n + 13): the
    same solution as the contiguous copy, bit for bit (the solver reads SA
    once, into its own column-major workspace)."""
    from sparse_sketching_amd import binding as b
    d, n, pad = 300, 97, 13
    g = np.random.default_rng(4)
    M = g.standard_normal((d, n + pad)).astype(np.float32)
    y = g.standard_normal(d).astype(np.float32)
    Md = to_dev(M)
    x_view = b.lstsq_qr(Md[:, :n], to_dev(y))
    x_copy = b.lstsq_qr(Md[:, :n].contiguous(), to_dev(y))
    sync()
    assert torch.equal(x_view, x_copy)
    ref = oracle.lstsq_qr(M[:, :n], y)
    assert np.linalg.norm(x_view.cpu().numpy() - ref) <= 5e-5 * np.linalg.norm(ref)
