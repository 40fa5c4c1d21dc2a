"""GPU sweep over seeded random shapes (tests/sweep_shapes.py): the complete
sketch through the boundary call, against the oracle, for whichever kernel
the plan picks.  FP16 from the register and owner kernels must equal the
oracle's RN emulation in the library's order (per row chunk ascending from
+0, chunk partials combined in four groups) bit for bit; FP32 must be
within the recursive-summation bound of the FP64 sketch; the metadata + LDS
fallback's FP16 additions have no fixed order, so it is held to a relative
bar only where few contributions meet in an entry.  BlockPerm-SJLT shapes
run through both boundary calls (with a workspace where the plan takes
one, and the component kernel without) against the FP64 oracle, and the
FP32 QR solve runs over random (d, n) against the oracle's FP64 QR."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev
from tests.sweep_shapes import BP_SWEEP, QR_SWEEP, SWEEP

pytestmark = pytest.mark.gpu

MI355X = dict(num_cu=256, max_lds=160 * 1024)
PREC = {"f32": b.SK_PRECISION_F32, "f16acc": b.SK_PRECISION_F16ACC}


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_sweep_case_matches_oracle(case):
    c = SWEEP[case]
    prec, m, n, d, zeta, pad = c["precision"], c["m"], c["n"], c["d"], c["zeta"], c["pad"]
    off, seed = c["row_offset"], c["seed"]
    p = b.sk_sketch_plan_describe(PREC[prec], m, n, n + pad, 16, d, zeta, **MI355X)
    say(f"sweep {case}: {prec} m={m} n={n} lda={n + pad} d={d} zeta={zeta} offset={off} "
        f"kernel={p['kernel']} barriers={p['barriers']} chunks={p['chunks']}")
    A = (inputs.gaussian(m, n + pad, seed=case) * np.float32(3.0)).astype(np.float32)
    Ad = to_dev(A)[:, :n]
    dt = torch.float16 if prec == "f16acc" else torch.float32
    out = torch.full((d, n + 2), 7.0, dtype=dt, device=dev())
    b.sketch_fused(Ad, d, zeta, seed, prec, row_offset=off, out=out[:, :n])
    sync()
    B = out.cpu().numpy().astype(np.float64)
    assert np.all(B[:, n:] == 7.0)                  # ldb padding untouched
    B = B[:, :n]
    A = np.ascontiguousarray(A[:, :n])
    ri, v = oracle.meta_ref(seed, m, d, zeta, row_offset=off)
    per_entry = m * zeta / d                        # contributions an entry gets on average
    if prec == "f16acc" and p["kernel"] in (1, 2):
        exp = oracle.sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=p["rows_per_chunk"],
                                        groups=4)
        assert np.array_equal(B, exp.astype(np.float64))
        return
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    assert np.all(np.isfinite(B))
    if prec == "f32":
        # FP32 sums of k terms: error below k u sum|c| deterministically;
        # 4 sqrt(k) u relative is the bar here (random signs)
        tol = max(1e-5, 4.0 * np.sqrt(max(per_entry, 1.0)) * 2.0 ** -24)
        assert oracle.rel_frob(B, ref) <= tol
    elif per_entry <= 2048:
        assert oracle.rel_frob(B, ref) <= 1e-2


@pytest.mark.parametrize("case", range(len(BP_SWEEP)))
def test_blockperm_sweep_case_matches_oracle(case):
    c = BP_SWEEP[case]
    m, n, lda, d, M, kappa, s = c["m"], c["n"], c["lda"], c["d"], c["M"], c["kappa"], c["s"]
    wiring, seed = c["wiring"], c["seed"]
    say(f"blockperm sweep {case}: m={m} n={n} lda={lda} d={d} M={M} kappa={kappa} s={s} "
        f"wiring={wiring}")
    A = inputs.gaussian(m, lda, seed=1000 + case)
    Ad = to_dev(A)[:, :n]
    A = np.ascontiguousarray(A[:, :n])
    ref = oracle.blockperm_f64(A, d, M, kappa, s, seed, kind=wiring)
    # each output row sums about kappa * s * B_c / B_r terms (B_c = m / M)
    terms = max(kappa * s * (m // M) / (d // M), 1.0)
    tol = max(1e-5, 4.0 * np.sqrt(terms) * 2.0 ** -24)
    out = torch.full((d, n + 1), 7.0, dtype=torch.float32, device=dev())
    b.blockperm(Ad, d, M, kappa, seed, s=s, out=out[:, :n], wiring=wiring)
    sync()
    Y = out.cpu().numpy().astype(np.float64)
    assert np.all(Y[:, n:] == 7.0)
    assert oracle.rel_frob(Y[:, :n], ref) <= tol
    if wiring == "shift":
        Yd = torch.full((d, n), 7.0, dtype=torch.float32, device=dev())
        b.sk_apply_blockperm(Ad, m, n, lda, d, M, kappa, s, seed, Yd, n)
        sync()
        assert oracle.rel_frob(Yd.cpu().numpy().astype(np.float64), ref) <= tol


@pytest.mark.parametrize("case", range(len(QR_SWEEP)))
def test_qr_sweep_case_matches_oracle(case):
    """Consistent systems y = M x0 (N(0,1) M): a backward-stable FP32 solve
    is within a small multiple of cond(M) u of x0's FP64 solution, and its
    residual within FP32 rounding of the FP64 minimum."""
    c = QR_SWEEP[case]
    d, n, pad = c["d"], c["n"], c["pad"]
    say(f"qr sweep {case}: d={d} n={n} ld={n + pad}")
    g = np.random.default_rng(5000 + case)
    M = g.standard_normal((d, n + pad)).astype(np.float32)
    x0 = g.standard_normal(n)
    y = (M[:, :n].astype(np.float64) @ x0).astype(np.float32)
    x = b.lstsq_qr(to_dev(M)[:, :n], to_dev(y))
    sync()
    x = x.cpu().numpy().astype(np.float64)
    Mn = np.ascontiguousarray(M[:, :n])
    ref = oracle.lstsq_qr(Mn, y)
    cond = np.linalg.cond(Mn.astype(np.float64))
    assert np.linalg.norm(x - ref) <= (2e-5 + 1e-6 * cond) * np.linalg.norm(ref)
    r_ref = oracle.residual(Mn, ref, y)
    assert oracle.residual(Mn, x, y) <= r_ref * (1 + 1e-5) + 1e-5 * (1 + cond / 100)


APPLY_VARIANTS = (0, b.SK_VARIANT_FLAT, b.SK_VARIANT_LDS, b.SK_VARIANT_REG)


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_apply_sweep_case_matches_oracle(case):
    """The stored-metadata applies on the sweep's shapes, one seeded pick
    of variant (default, flat, LDS, register) and workspace per case: FP16
    through the register kernel bit for bit in the library's order, the
    order-free variants (flat and LDS atomics) to a relative bar where few
    contributions meet, FP32 to the summation bound; the register variant
    forced without a workspace or on a shape it does not cover is
    refused."""
    c = SWEEP[case]
    prec, m, n, d, zeta, pad = c["precision"], c["m"], c["n"], c["d"], c["zeta"], c["pad"]
    pick = np.random.default_rng(8000 + case)
    flags = APPLY_VARIANTS[int(pick.integers(4))]
    use_ws = bool(pick.random() < 0.6)
    say(f"apply sweep {case}: {prec} m={m} n={n} lda={n + pad} d={d} zeta={zeta} "
        f"flags={flags} workspace={use_ws}")
    A = (inputs.gaussian(m, n + pad, seed=2000 + case) * np.float32(3.0)).astype(np.float32)
    Ad = to_dev(A)[:, :n]
    A = np.ascontiguousarray(A[:, :n])
    ri, v = oracle.meta_ref(c["seed"], m, d, zeta)
    fused = b.sk_fused_plan_describe(PREC[prec], m, n, n + pad, 16, d, zeta, **MI355X)
    reg = bool(fused["fused"]) and zeta <= 8        # the shapes the register variant covers
    if flags == b.SK_VARIANT_REG and not (use_ws and reg):
        # forced without its workspace, or on a shape it does not cover
        with pytest.raises(b.SketchError):
            b.apply(Ad, to_dev(ri), to_dev(v), zeta, d, prec, flags=flags,
                    ws=True if use_ws else None)
        sync()
        return
    out = b.apply(Ad, to_dev(ri), to_dev(v), zeta, d, prec, flags=flags,
                  ws=True if use_ws else None)
    sync()
    B = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(B))
    per_entry = m * zeta / d
    if prec == "f16acc" and use_ws and reg and flags in (0, b.SK_VARIANT_REG):
        exp = oracle.sketch_f16_rn_emul(A, ri, v, d, zeta, chunk_rows=fused["rows_per_chunk"],
                                        groups=4)
        assert np.array_equal(B, exp.astype(np.float64))
        return
    ref = oracle.sketch_f64(A, ri, v, d, zeta)
    if prec == "f32":
        tol = max(1e-5, 4.0 * np.sqrt(max(per_entry, 1.0)) * 2.0 ** -24)
        assert oracle.rel_frob(B, ref) <= tol
    elif per_entry <= 2048:
        assert oracle.rel_frob(B, ref) <= 1e-2
