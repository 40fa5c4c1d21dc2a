"""GPU parity for sk_apply_blockperm against the BlockPerm-SJLT oracle
(FlashSketch page §4, §5, App. D): dense brute force on tiny instances,
exact integer inputs, and the full 2^21 x 512 configuration on sampled
columns."""
import numpy as np
import pytest
import torch

import oracle
from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,d,M,kappa,seed", [
    (256, 5, 32, 4, 2, 9),          # B_c = 64, B_r = 8, ragged column tile
    (512, 33, 64, 8, 4, 1),         # two column tiles
    (512, 32, 64, 8, 1, 2),         # kappa = 1: localized block-diagonal
    (1024, 40, 128, 16, 8, 3),      # kappa = 8
    (6 * 100, 7, 6 * 3, 6, 2, 4),   # B_c = 100 (partial row batch), B_r = 3
])
def test_small_vs_dense(m, n, d, M, kappa, seed):
    say(f"blockperm m={m} n={n} d={d} M={M} kappa={kappa}")
    A = inputs.gaussian(m, n, seed=seed)
    Y = b.blockperm(to_dev(A), d, M, kappa, seed)
    sync()
    ref = oracle.blockperm_dense_S(m, d, M, kappa, 1, seed) @ A.astype(np.float64)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


def test_integer_exact_and_accumulate():
    m, n, d, M, kappa = 4096, 64, 256, 16, 4
    A = inputs.integer_matrix(m, n, -8, 8, seed=1)
    Ad = to_dev(A)
    ref = oracle.blockperm_f64(A, d, M, kappa, 1, 77)
    Y = b.blockperm(Ad, d, M, kappa, 77)
    sync()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)
    b.blockperm(Ad, d, M, kappa, 77, out=Y, flags=b.SK_ACCUMULATE)
    sync()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), 2 * ref)


def test_padded_strides():
    m, n, d, M, kappa = 2048, 45, 128, 8, 2
    A = inputs.gaussian(m, 64, seed=3)
    Ad = to_dev(A)[:, :n]
    out = torch.full((d, 50), 5.0, device=dev())
    b.blockperm(Ad, d, M, kappa, 5, out=out[:, :n])
    sync()
    Y = out.cpu().numpy()
    assert np.all(Y[:, n:] == 5.0)
    ref = oracle.blockperm_f64(np.ascontiguousarray(A[:, :n]), d, M, kappa, 1, 5)
    assert oracle.rel_frob(Y[:, :n], ref) <= 1e-5


@pytest.mark.parametrize("path", ["ex", "component"])
def test_full_configuration_sampled_columns(path):
    """A 2^21 x 512 N(0,1) (drawn on the device, seeded), d = 1024, M = 64,
    kappa = 4, s = 1, through sk_apply_blockperm_ex (the register kernel,
    as the benchmark runs it) and sk_apply_blockperm (the component
    kernel).  Every output row is checked on 24 columns spread over all
    column slices and tiles, against the fp64 oracle on those columns."""
    m, n, d, M, kappa, seed = 1 << 21, 512, 1024, 64, 4, 1
    say(f"blockperm full configuration, {path}")
    Ad = inputs.gaussian_torch(m, n, seed=0)
    if path == "ex":
        assert _plan(m, n, d, M, kappa, 1, "shift", seed)["kernel"] == \
            b.SK_BLOCKPERM_KERNEL_REGISTER
        Y = b.blockperm(Ad, d, M, kappa, seed)
    else:
        Y = torch.empty((d, n), dtype=torch.float32, device=Ad.device)
        b.sk_apply_blockperm(Ad, m, n, n, d, M, kappa, 1, seed, Y, n)
    sync()
    cols = np.unique(np.concatenate([np.arange(0, n, 23), [1, 31, 32, 255, 256, 480, 511]]))
    A_cols = Ad[:, torch.from_numpy(cols).to(Ad.device)].cpu().numpy()
    ref = oracle.blockperm_f64(A_cols, d, M, kappa, 1, seed)
    got = Y.cpu().numpy()[:, cols]
    err = oracle.rel_frob(got, ref)
    say(f"  rel err {err:.3e} on {len(cols)} columns")
    assert err <= 1e-5
    # unbiased norm: E||Sx||^2 = ||x||^2 holds for the whole output
    assert abs(float((Y.double() ** 2).sum() / (Ad.double() ** 2).sum()) - 1) < 0.05


# ------------------------------------------------------- general BlockPerm

MI355X = dict(num_cu=256, max_lds=160 * 1024)


@pytest.mark.parametrize("kind,m,n,d,M,kappa,s,seed", [
    ("affine", 512, 33, 64, 8, 3, 1, 5),      # kappa not dividing M
    ("affine", 1024, 40, 128, 16, 4, 2, 6),   # s = 2
    ("affine", 768, 7, 96, 12, 5, 1, 7),      # M = 12 (Hull-Dobell with 4 | M)
    ("affine", 640, 64, 320, 5, 2, 4, 8),     # M prime: a = 1; s = 4 of B_r = 64
    ("shift", 1024, 36, 128, 8, 4, 2, 9),     # shift wiring with s = 2
    ("shift", 6 * 100, 7, 6 * 3, 6, 2, 1, 4), # B_c = 100, B_r = 3
])
def test_general_vs_dense(kind, m, n, d, M, kappa, s, seed):
    say(f"blockperm general {kind} m={m} n={n} d={d} M={M} kappa={kappa} s={s}")
    A = inputs.gaussian(m, n, seed=seed)
    Y = b.blockperm(to_dev(A), d, M, kappa, seed, s=s, wiring=kind)
    sync()
    ref = oracle.blockperm_dense_S(m, d, M, kappa, s, seed, kind) @ A.astype(np.float64)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("kind,kappa,s", [("affine", 4, 1), ("affine", 2, 2), ("shift", 4, 4),
                                          ("affine", 16, 1)])
def test_general_integer_exact(kind, kappa, s):
    """kappa*s a power of 4: the scale is an exact power of two and integer
    inputs give exact sums in any order, so Y must equal fp64 bit for bit."""
    m, n, d, M = 8192, 64, 512, 16
    A = inputs.integer_matrix(m, n, -8, 8, seed=3)
    ref = oracle.blockperm_f64(A, d, M, kappa, s, 21, kind)
    Y = b.blockperm(to_dev(A), d, M, kappa, 21, s=s, wiring=kind)
    sync()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)


def test_split_slices_and_accumulate():
    """Few components x tiles: the plan splits input blocks into row slices
    (the page's split-B_c) and the fixed-order reduce sums them; with
    SK_ACCUMULATE the result adds onto Y."""
    m, n, d, M, kappa = 1 << 16, 64, 1024, 64, 4
    p = b.sk_blockperm_plan_describe(m, n, d, M, kappa, 1, b.SK_WIRING_SHIFT, 5, **MI355X)
    assert p["kernel"] != b.SK_BLOCKPERM_KERNEL_COMPONENT and p["Q"] > 1
    A = inputs.integer_matrix(m, n, -4, 4, seed=6)
    Ad = to_dev(A)
    ref = oracle.blockperm_f64(A, d, M, kappa, 1, 5)
    Y = torch.full((d, n), 2.0, dtype=torch.float32, device=dev())
    b.blockperm(Ad, d, M, kappa, 5, out=Y, flags=b.SK_ACCUMULATE)
    sync()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref + 2.0)


def test_component_kernel_direct_small():
    """sk_apply_blockperm always takes the component kernel; on a small
    shape it must agree with the general kernel and the oracle exactly."""
    m, n, d, M, kappa = 4096, 64, 256, 16, 4
    A = inputs.integer_matrix(m, n, -8, 8, seed=2)
    Ad = to_dev(A)
    Y1 = torch.empty((d, n), dtype=torch.float32, device=dev())
    b.sk_apply_blockperm(Ad, m, n, n, d, M, kappa, 1, 31, Y1, n)
    Y2 = b.blockperm(Ad, d, M, kappa, 31)
    sync()
    ref = oracle.blockperm_f64(A, d, M, kappa, 1, 31)
    assert np.array_equal(Y1.cpu().numpy().astype(np.float64), ref)
    assert torch.equal(Y1, Y2)


# ------------------------------------------------------- register kernel

def _plan(m, n, d, M, kappa, s, kind, seed):
    w = b.SK_WIRING_SHIFT if kind == "shift" else b.SK_WIRING_AFFINE
    return b.sk_blockperm_plan_describe(m, n, d, M, kappa, s, w, seed, **MI355X)


@pytest.mark.parametrize("kind,m,n,d,M,kappa,s,R,G", [
    ("shift", 8 * 1000, 8, 64, 8, 2, 1, 1, 1),       # R = 1; B_c = 1000: a short last stage
    ("affine", 8 * 640, 36, 64, 8, 4, 1, 2, 1),      # R = 2; 36 of 256 columns
    ("shift", 16 * 512, 300, 256, 16, 4, 1, 4, 1),   # R = 4; two column slices, ragged
    ("affine", 16 * 512, 64, 256, 16, 8, 2, 8, 1),   # R = 8; s = 2
    ("shift", 16 * 256, 520, 256, 16, 16, 1, 16, 1), # R = 16; three column slices
    ("affine", 32 * 256, 32, 512, 32, 32, 4, 16, 2), # two row groups; s = 4
    ("affine", 32 * 128, 16, 2048, 32, 32, 1, 16, 8),# eight row groups (B_r = 64)
    ("shift", 64 * 461, 512, 1024, 64, 4, 1, 4, 1),  # row slices of 4 stages, the last 13 rows short
])
def test_register_kernel_vs_oracle(kind, m, n, d, M, kappa, s, R, G):
    """Every built rows-per-wavefront R, row groups, s > 1, both wirings,
    ragged column slices and short last stages, against the fp64 oracle;
    the plan must pick the register kernel with the expected R and G."""
    seed = 11
    p = _plan(m, n, d, M, kappa, s, kind, seed)
    say(f"blockperm register {kind} m={m} n={n} d={d} M={M} kappa={kappa} s={s} plan={p}")
    assert p["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
    assert (p["rows_per_wave"], p["groups"]) == (R, G)
    A = inputs.gaussian(m, n, seed=4)
    Y = b.blockperm(to_dev(A), d, M, kappa, seed, s=s, wiring=kind)
    sync()
    ref = oracle.blockperm_f64(A, d, M, kappa, s, seed, kind)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


def test_register_kernel_dense_brute_force():
    """A tiny register-kernel case against the dense S the oracle builds
    entry by entry (not the block-wise apply)."""
    m, n, d, M, kappa, s, seed = 16 * 100, 12, 256, 16, 4, 2, 3
    assert _plan(m, n, d, M, kappa, s, "affine", seed)["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
    A = inputs.gaussian(m, n, seed=8)
    Y = b.blockperm(to_dev(A), d, M, kappa, seed, s=s, wiring="affine")
    sync()
    ref = oracle.blockperm_dense_S(m, d, M, kappa, s, seed, "affine") @ A.astype(np.float64)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


def test_register_kernel_deterministic_and_accumulate():
    """Fixed summation order: two runs agree bit for bit; integer inputs
    with kappa*s = 4 (scale 1/2) are exact, and SK_ACCUMULATE adds."""
    m, n, d, M, kappa = 16 * 2048, 264, 512, 16, 4
    A = inputs.integer_matrix(m, n, -8, 8, seed=5)
    Ad = to_dev(A)
    assert _plan(m, n, d, M, kappa, 1, "shift", 9)["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
    Y1 = b.blockperm(Ad, d, M, kappa, 9)
    Y2 = b.blockperm(Ad, d, M, kappa, 9)
    sync()
    assert torch.equal(Y1, Y2)
    ref = oracle.blockperm_f64(A, d, M, kappa, 1, 9)
    assert np.array_equal(Y1.cpu().numpy().astype(np.float64), ref)
    b.blockperm(Ad, d, M, kappa, 9, out=Y1, flags=b.SK_ACCUMULATE)
    sync()
    assert np.array_equal(Y1.cpu().numpy().astype(np.float64), 2 * ref)


@pytest.mark.parametrize("how", ["lda", "base"])
def test_register_shape_with_unaligned_A_uses_slice_kernel(how):
    """A shape the register kernel takes, but A's row stride (lda % 4 != 0)
    or base address (4 bytes past a 16-byte boundary) rules out its float4
    loads: the call falls back to the slice kernel, same result."""
    m, n, d, M, kappa, seed = 4096, 64, 256, 16, 4, 6
    assert _plan(m, n, d, M, kappa, 1, "affine", seed)["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
    A = inputs.gaussian(m, n, seed=7)
    if how == "lda":
        buf = torch.zeros((m, n + 2), dtype=torch.float32, device=dev())
        buf[:, :n] = to_dev(A)
        Ad = buf[:, :n]
    else:
        flat = torch.zeros(m * n + 1, dtype=torch.float32, device=dev())
        flat[1:] = to_dev(A).reshape(-1)
        Ad = flat[1:].view(m, n)
        assert Ad.data_ptr() % 16 == 4
    Y = b.blockperm(Ad, d, M, kappa, seed, wiring="affine")
    sync()
    ref = oracle.blockperm_f64(A, d, M, kappa, 1, seed, "affine")
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("kind,m,n,d,M,kappa,s,R,G", [
    ("shift", 1024 * 32, 20, 1024, 1024, 32, 1, 1, 2),        # M = 1024 (largest), kappa = 32, B_r = 1
    ("affine", 16 * 256, 24, 16 * 32, 16, 2, 32, 4, 1),       # s = 32 of B_r = 32
])
def test_register_kernel_limits(kind, m, n, d, M, kappa, s, R, G):
    seed = 13
    p = _plan(m, n, d, M, kappa, s, kind, seed)
    say(f"blockperm register limits {kind} M={M} kappa={kappa} s={s} plan={p}")
    assert p["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
    assert (p["rows_per_wave"], p["groups"]) == (R, G)
    A = inputs.gaussian(m, n, seed=6)
    Y = b.blockperm(to_dev(A), d, M, kappa, seed, s=s, wiring=kind)
    sync()
    # the oracle's sparse S over all blocks at once (its per-block apply
    # rebuilds the wiring for every block: slow at M = 1024)
    ref = oracle.blockperm_matrix(m, d, M, kappa, s, seed, kind=kind) @ A.astype(np.float64)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


def test_register_kernel_padded_strides_accumulate():
    """lda = 68 and ldy = 72 around n = 64 (lda % 4 == 0 keeps the register
    kernel): Y's padding is untouched and SK_ACCUMULATE adds onto it."""
    m, n, d, M, kappa, seed = 16 * 640, 64, 256, 16, 4, 17
    A = inputs.gaussian(m, 68, seed=9)
    Ad = to_dev(A)[:, :n]
    out = torch.full((d, 72), 3.0, device=dev())
    b.blockperm(Ad, d, M, kappa, seed, out=out[:, :n], flags=b.SK_ACCUMULATE)
    sync()
    Y = out.cpu().numpy()
    assert np.all(Y[:, n:] == 3.0)
    ref = oracle.blockperm_f64(np.ascontiguousarray(A[:, :n]), d, M, kappa, 1, seed) + 3.0
    assert oracle.rel_frob(Y[:, :n], ref) <= 1e-5


def test_ex_workspace_errors():
    """sk_apply_blockperm_ex rejects a workspace that is too small
    (SK_ERR_ARG) or not 16-byte aligned (SK_ERR_ALIGN), before any launch,
    and a NULL workspace where the component kernel does not apply
    (affine wiring) with SK_ERR_NULL."""
    m, n, d, M, kappa = 4096, 64, 256, 16, 4
    Ad = to_dev(inputs.gaussian(m, n, seed=1))
    Y = torch.full((d, n), 7.0, device=dev())
    nb = b.sk_blockperm_workspace_size(m, n, d, M, kappa, 1, b.SK_WIRING_AFFINE)
    ws = torch.empty(nb + 64, dtype=torch.uint8, device=dev())
    cases = [(ws, nb - 4, b.SK_ERR_ARG), (ws[4:], nb, b.SK_ERR_ALIGN), (None, 0, b.SK_ERR_NULL)]
    for w, nbytes, expect in cases:
        with pytest.raises(b.SketchError) as e:
            b.sk_apply_blockperm_ex(Ad, m, n, n, d, M, kappa, 1, b.SK_WIRING_AFFINE, 3, Y, n, 0,
                                    w, nbytes)
        assert e.value.status == expect
    sync()
    assert torch.all(Y == 7.0)


# --------------------------- sk_apply_blockperm: no workspace, every shape

def direct(A, d, M, kappa, s, seed, out=None, flags=0, n=None, lda=None):
    """sk_apply_blockperm through the C ABI (shift wiring, no workspace)."""
    m = A.shape[0]
    n = A.shape[1] if n is None else n
    lda = A.stride(0) if lda is None else lda
    Y = torch.empty((d, n), dtype=torch.float32, device=A.device) if out is None else out
    b.sk_apply_blockperm(A, m, n, lda, d, M, kappa, s, seed, Y, Y.stride(0), flags)
    sync()
    return Y


@pytest.mark.parametrize("m,n,d,M,kappa,s,seed", [
    (256, 5, 32, 4, 2, 1, 9),           # B_r = 8, 5 columns (scalar loads)
    (512, 33, 64, 8, 4, 1, 1),          # two column tiles, the second ragged
    (512, 32, 64, 8, 1, 1, 2),          # kappa = 1: block-diagonal
    (1024, 40, 128, 16, 8, 1, 3),       # kappa = 8, 16-byte loads, ragged tile
    (600, 7, 18, 6, 2, 1, 4),           # B_c = 100 (partial stage), B_r = 3
    (1024, 36, 128, 8, 4, 2, 5),        # s = 2
    (2048, 64, 512, 16, 16, 1, 6),      # kappa = M = 16: one component, 512 rows in 8 groups
    (2048, 48, 256, 32, 32, 4, 7),      # kappa = M = 32, s = 4
    (4096, 64, 1024, 16, 4, 8, 8),      # B_r = 64, s = 8: 256 rows in 4 groups
    (64 * 129, 32, 64, 64, 64, 1, 10),  # kappa = 64 (beyond the workspace kernels), B_r = 1
    (128 * 8, 8, 128, 128, 128, 1, 11), # kappa = M = 128
    (2048, 64, 1024, 16, 4, 2, 12),     # FlashSketch Figure 2 (M=16, B_r=64, B_c=128, s=2)
])
def test_direct_vs_oracle(m, n, d, M, kappa, s, seed):
    """Against the fp64 oracle (itself pinned to the dense S brute force):
    the no-workspace kernel over the boundary's domain (any kappa | M,
    s <= B_r)."""
    say(f"blockperm direct m={m} n={n} d={d} M={M} kappa={kappa} s={s}")
    A = inputs.gaussian(m, n, seed=seed)
    Y = direct(to_dev(A), d, M, kappa, s, seed)
    ref = oracle.blockperm_f64(A, d, M, kappa, s, seed)
    assert oracle.rel_frob(Y.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("kappa,s", [(4, 1), (16, 1), (4, 4), (1, 16)])
def test_direct_integer_exact_accumulate_and_repeat(kappa, s):
    """kappa*s a power of 4: integer inputs give exact sums in any order, so
    Y equals fp64 bit for bit (a lost or doubled hit changes it);
    SK_ACCUMULATE adds a second copy.  Within a stage the hits of an output
    row are added in the order the LDS counter handed out their slots, so
    two calls on Gaussian inputs agree to FP32 rounding, not bit for bit."""
    m, n, d, M = 8192, 64, 512, 16
    A = inputs.integer_matrix(m, n, -8, 8, seed=3)
    Ad = to_dev(A)
    ref = oracle.blockperm_f64(A, d, M, kappa, s, 21)
    Y = direct(Ad, d, M, kappa, s, 21)
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)
    direct(Ad, d, M, kappa, s, 21, out=Y, flags=b.SK_ACCUMULATE)
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), 2 * ref)
    G = inputs.gaussian_torch(m, n, seed=4)
    Y1, Y2 = direct(G, d, M, kappa, s, 5), direct(G, d, M, kappa, s, 5)
    assert float(torch.linalg.norm(Y1 - Y2) / torch.linalg.norm(Y1)) <= 1e-6


def test_direct_unaligned_and_padded():
    """A starting one float past a 16-byte boundary with a padded leading
    dimension (scalar loads), and a padded output: columns past n untouched."""
    m, n, d, M, kappa = 4096, 60, 256, 16, 4
    A = inputs.gaussian(m, 72, seed=6)
    Ad = to_dev(A)[:, 1:1 + n]
    out = torch.full((d, 70), 7.0, device=dev())
    Y = direct(Ad, d, M, kappa, 1, 13, out=out[:, :n], n=n, lda=72)
    Yh = out.cpu().numpy()
    assert np.all(Yh[:, n:] == 7.0)
    ref = oracle.blockperm_f64(np.ascontiguousarray(A[:, 1:1 + n]), d, M, kappa, 1, 13)
    assert oracle.rel_frob(Yh[:, :n], ref) <= 1e-5
    del Y


def test_direct_unsupported_stride_rule():
    """s > 1 needs B_r a power of two (the odd stride alpha then gives s
    distinct rows): B_r = 6 with s = 2 is refused before any launch."""
    A = torch.zeros((600, 8), device=dev())
    Y = torch.zeros((36, 8), device=dev())
    with pytest.raises(b.SketchError) as e:
        b.sk_apply_blockperm(A, 600, 8, 8, 36, 6, 2, 2, 1, Y, 8, 0)
    assert e.value.status == b.SK_ERR_UNSUPPORTED
