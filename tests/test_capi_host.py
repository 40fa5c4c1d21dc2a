"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/sk.h declares, and rejects invalid arguments before it
makes any HIP call."""
import ctypes

import pytest

from sparse_sketching_amd import binding as b
from tests.sweep_shapes import BP_SWEEP, SWEEP

FAKE = 1 << 40          # never dereferenced: validation fails before any use


@pytest.fixture(scope="module")
def lib():
    return b.load()


def test_exports_every_declared_symbol(lib):
    names = b.header_symbols()
    assert set(names) == {"sk_meta_generate", "sk_apply_f32", "sk_apply_f16acc",
                          "sk_apply_f32_ws", "sk_apply_f16acc_ws", "sk_apply_workspace_size", "sk_lds_plan_describe",
                          "sk_sketch_f32", "sk_sketch_f16acc", "sk_sketch_workspace_size",
                          "sk_sketch_f16acc_noalloc",
                          "sk_fused_plan_describe", "sk_sketch_plan_describe", "sk_apply_lowp",
                          "sk_apply_blockperm",
                          "sk_apply_blockperm_ex", "sk_blockperm_workspace_size",
                          "sk_blockperm_plan_describe", "sk_lstsq_qr_f32",
                          "sk_lstsq_workspace_size", "sk_status_string"}
    for name in names:
        assert hasattr(lib, name), name


def test_plan_field_lists_match_the_header():
    """Each describe call's field count in include/sk.h equals the length
    of the binding's field-name tuple (the binding sizes its output array
    from the tuple, so a field added on one side only would be lost or
    overrun)."""
    import re
    text = open(b.HEADER).read()
    counts = {k: int(v) for k, v in re.findall(r"#define (SK_\w*PLAN_FIELDS) (\d+)", text)}
    assert counts == {"SK_FUSED_PLAN_FIELDS": len(b.FUSED_PLAN_FIELDS),
                      "SK_SKETCH_PLAN_FIELDS": len(b.SKETCH_PLAN_FIELDS),
                      "SK_BLOCKPERM_PLAN_FIELDS": len(b.BLOCKPERM_PLAN_FIELDS),
                      "SK_PLAN_FIELDS": len(b.PLAN_FIELDS)}


def test_status_strings(lib):
    for s in range(7):
        assert lib.sk_status_string(s)
    assert b.status_string(b.SK_ERR_ALIGN) == "misaligned buffer or stride"


@pytest.mark.parametrize("args,expect", [
    ((1, 0, -1, 64, 4, FAKE, FAKE + 4096), b.SK_ERR_SHAPE),      # m < 0
    ((1, -5, 10, 64, 4, FAKE, FAKE + 4096), b.SK_ERR_SHAPE),     # row_offset < 0
    ((1, 0, 10, 64, 3, FAKE, FAKE + 4096), b.SK_ERR_SHAPE),      # d % zeta
    ((1, 0, 10, 4, 8, FAKE, FAKE + 4096), b.SK_ERR_SHAPE),       # zeta > d
    ((1, 0, 10, 64, 0, FAKE, FAKE + 4096), b.SK_ERR_SHAPE),      # zeta < 1
    ((1, 0, 10, 64, 4, None, FAKE), b.SK_ERR_NULL),
    ((1, 0, 10, 64, 4, FAKE, None), b.SK_ERR_NULL),
    ((1, 0, 10, 64, 4, FAKE, FAKE + 8), b.SK_ERR_ARG),            # outputs overlap
    ((1, 0, 0, 64, 4, None, None), b.SK_OK),                     # empty: nothing to do
])
def test_meta_validation(lib, args, expect):
    assert lib.sk_meta_generate(*args, None) == expect


A, RI, V, B = FAKE, FAKE + (1 << 34), FAKE + (1 << 35), FAKE + (1 << 36)


@pytest.mark.parametrize("fn", ["sk_apply_f32", "sk_apply_f16acc", "sk_apply_f32_ws",
                                "sk_apply_f16acc_ws"])
@pytest.mark.parametrize("args,expect", [
    ((A, 100, 0, 64, RI, V, 4, B, 64, 64, 0), b.SK_ERR_SHAPE),      # n < 1
    ((A, 100, 64, 32, RI, V, 4, B, 64, 64, 0), b.SK_ERR_SHAPE),     # lda < n
    ((A, 100, 64, 64, RI, V, 4, B, 64, 32, 0), b.SK_ERR_SHAPE),     # ldb < n
    ((A, 100, 64, 64, RI, V, 3, B, 64, 64, 0), b.SK_ERR_SHAPE),     # d % zeta
    ((A, -1, 64, 64, RI, V, 4, B, 64, 64, 0), b.SK_ERR_SHAPE),
    ((A, 100, 64, 64, RI, V, 4, B, 0, 64, 0), b.SK_ERR_SHAPE),      # d < 1
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 6), b.SK_ERR_ARG),       # FLAT|LDS
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 10), b.SK_ERR_ARG),      # FLAT|REG
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 12), b.SK_ERR_ARG),      # LDS|REG
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 32), b.SK_ERR_ARG),      # unknown flag
    ((None, 100, 64, 64, RI, V, 4, B, 64, 64, 0), b.SK_ERR_NULL),
    ((A, 100, 64, 64, None, V, 4, B, 64, 64, 0), b.SK_ERR_NULL),
    ((A, 100, 64, 64, RI, None, 4, B, 64, 64, 0), b.SK_ERR_NULL),
    ((A, 100, 64, 64, RI, V, 4, None, 64, 64, 0), b.SK_ERR_NULL),
    ((A, 100, 64, 64, RI, V, 4, A + 256, 64, 64, 0), b.SK_ERR_ARG),  # B inside A
    ((A, 100, 64, 64, RI, V, 4, RI + 64, 64, 64, 0), b.SK_ERR_ARG),  # B inside metadata
])
def test_apply_validation(lib, fn, args, expect):
    tail = (None, 0, None) if fn.endswith("_ws") else (None,)
    assert getattr(lib, fn)(*args, *tail) == expect


@pytest.mark.parametrize("fn,expect", [
    ("sk_apply_f32", b.SK_ERR_ARG),         # FP32 output has no FP16 combine
    ("sk_apply_f32_ws", b.SK_ERR_ARG),
    ("sk_apply_f16acc", b.SK_ERR_ARG),      # no workspace: no reduce to combine in
])
def test_combine_flag_rules(lib, fn, expect):
    args = (A, 100, 64, 64, RI, V, 4, B, 64, 64, b.SK_COMBINE_F32)
    tail = (None, 0, None) if fn.endswith("_ws") else (None,)
    assert getattr(lib, fn)(*args, *tail) == expect


WS = FAKE + (1 << 37)


@pytest.mark.parametrize("fn", ["sk_apply_f32_ws", "sk_apply_f16acc_ws"])
@pytest.mark.parametrize("ws,nbytes,expect", [
    (WS + 2, 1 << 20, b.SK_ERR_ALIGN),            # workspace not 4-byte aligned
    (A + 64, 1 << 20, b.SK_ERR_ARG),              # workspace overlaps A
    (B - 16, 64, b.SK_ERR_ARG),                   # workspace overlaps B
    (RI + 4, 64, b.SK_ERR_ARG),                   # workspace overlaps the metadata
])
def test_workspace_validation(lib, fn, ws, nbytes, expect):
    args = (A, 100, 64, 64, RI, V, 4, B, 64, 64, 0)
    assert getattr(lib, fn)(*args, ws, nbytes, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((3, 100, 64, 64, 4, 0), b.SK_ERR_ARG),        # unknown precision
    ((2, 100, 64, 64, 4, 16), b.SK_OK),            # the reduced-precision sketch: no REG, none
    ((0, 100, 0, 64, 4, 0), b.SK_ERR_SHAPE),       # n < 1
    ((1, 100, 63, 64, 4, 0), b.SK_ERR_SHAPE),      # odd n for FP16
    ((0, 100, 64, 64, 3, 0), b.SK_ERR_SHAPE),      # d % zeta
    ((0, 100, 64, 64, 4, 6), b.SK_ERR_ARG),        # FLAT|LDS
    ((0, 100, 64, 64, 4, 12), b.SK_ERR_ARG),       # LDS|REG
    ((0, 100, 64, 64, 4, 16), b.SK_ERR_ARG),       # FP16 combine on FP32
    ((0, 100, 64, 64, 4, 32), b.SK_ERR_ARG),       # unknown flag
    ((0, 0, 64, 64, 4, 0), b.SK_OK),               # m = 0: no workspace
    ((1, 100, 64, 64, 4, 2), b.SK_OK),             # FLAT: no workspace
])
def test_workspace_size_validation(lib, args, expect):
    out = ctypes.c_size_t(123)
    assert lib.sk_apply_workspace_size(*args, ctypes.byref(out)) == expect
    if expect == b.SK_OK:
        assert out.value == 0
    assert lib.sk_apply_workspace_size(*args, None) == b.SK_ERR_NULL


@pytest.mark.parametrize("args,expect", [
    ((A, 100, 63, 64, RI, V, 4, B, 64, 64, 0), b.SK_ERR_SHAPE),     # odd n
    ((A, 100, 64, 64, RI, V, 4, B, 64, 65, 0), b.SK_ERR_ALIGN),     # odd ldb
    ((A, 100, 64, 64, RI, V, 4, B + 2, 64, 64, 0), b.SK_ERR_ALIGN), # B not 4-byte aligned
    ((A, 100, 64, 65, RI, V, 4, B, 64, 64, 0), b.SK_ERR_ALIGN),     # odd lda
    ((A + 4, 100, 64, 64, RI, V, 4, B, 64, 64, 0), b.SK_ERR_ALIGN), # A not 8-byte aligned
])
def test_f16acc_pair_rules(lib, args, expect):
    assert lib.sk_apply_f16acc(*args, None) == expect
    assert lib.sk_apply_f16acc_ws(*args, None, 0, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, 1000, 64, 64, 64, 64, 4, 1, 7, B, 64, 0), b.SK_ERR_SHAPE),    # m % M
    ((A, 1024, 64, 64, 60, 64, 4, 1, 7, B, 64, 0), b.SK_ERR_SHAPE),    # d % M
    ((A, 1024, 64, 64, 64, 64, 3, 1, 7, B, 64, 0), b.SK_ERR_SHAPE),    # kappa does not divide M
    ((A, 1024, 64, 32, 64, 64, 4, 1, 7, B, 64, 0), b.SK_ERR_SHAPE),    # lda < n
    ((A, 1024, 64, 64, 64, 64, 4, 1, 7, B, 32, 0), b.SK_ERR_SHAPE),    # ldy < n
    ((A, 1024, 64, 64, 64, 64, 4, 2, 7, B, 64, 0), b.SK_ERR_SHAPE),    # s > B_r = 1
    ((A, 1024, 64, 64, 192, 64, 4, 2, 7, B, 64, 0), b.SK_ERR_UNSUPPORTED),  # s = 2, B_r = 3
    ((A, 2048, 64, 64, 2048, 2048, 4, 1, 7, B, 64, 0), b.SK_ERR_UNSUPPORTED),  # M too large
    ((A, 1024, 64, 64, 64, 64, 4, 1, 7, B, 64, 2), b.SK_ERR_ARG),      # variant flag
    ((None, 1024, 64, 64, 64, 64, 4, 1, 7, B, 64, 0), b.SK_ERR_NULL),
    ((A, 1024, 64, 64, 64, 64, 4, 1, 7, None, 64, 0), b.SK_ERR_NULL),
    ((A, 1024, 64, 64, 64, 64, 4, 1, 7, A + 64, 64, 0), b.SK_ERR_ARG),
    ((A, 0, 64, 64, 64, 64, 4, 1, 7, B, 64, 0), b.SK_ERR_SHAPE),
])
def test_blockperm_validation(lib, args, expect):
    assert lib.sk_apply_blockperm(*args, None) == expect


def test_figure2_shape_is_planned(lib):
    # FlashSketch Figure 2: M=16, B_r=64, B_c=128, kappa=4, s=2 (d_in=2048,
    # k=1024): a valid request of the shift wiring; without a workspace the
    # component kernel takes it, kappa*B_r = 256 output rows in 4 row groups
    p = b.sk_blockperm_plan_describe(2048, 64, 1024, 16, 4, 2, b.SK_WIRING_SHIFT, 7,
                                     num_cu=256, max_lds=160 * 1024)
    assert p["ws_bytes"] > 0 or p["kernel"] == b.SK_BLOCKPERM_KERNEL_COMPONENT


@pytest.mark.parametrize("m,n,d,M,kappa,s", [
    (1 << 21, 510, 1024, 64, 4, 1),       # the BlockPerm workload (ragged width)
    (2048, 63, 1024, 16, 4, 2),           # Figure 2 with s = 2
    (256 * 8, 8, 256, 256, 256, 1),       # kappa = M: one component
    (600, 7, 18, 6, 2, 1),                # B_r = 3
    (64 * 129, 37, 64, 64, 64, 1),        # kappa = 64, ragged tiles
    (4096, 65, 1024, 16, 4, 8),           # kappa * B_r = 256, s = 8
])
def test_blockperm_component_grid_covers_every_output_once(m, n, d, M, kappa, s):
    """The component kernel's workgroups (component, row group, column
    tile) own disjoint sets of output elements whose union is all of Y:
    each element is written once, by one workgroup, with no atomics.  The
    index arithmetic is the kernel's: tile = wg % tiles, group = (wg /
    tiles) % groups, component = wg / (tiles * groups); a group holds the
    component's tile rows [64 group, 64 group + 64) of its kappa*B_r.
    Where sk_apply_blockperm_ex plans the component kernel (odd widths rule
    out the register kernel; one CU makes any grid fill the device) its
    groups and tiles are the ones used here."""
    import numpy as np
    Br, C = d // M, M // kappa
    T = kappa * Br
    G, tiles = -(-T // 64), -(-n // 32)
    if kappa <= 32:
        p = b.sk_blockperm_plan_describe(m, n, d, M, kappa, s, b.SK_WIRING_SHIFT, 3, num_cu=1,
                                         max_lds=160 * 1024)
        assert p["kernel"] == b.SK_BLOCKPERM_KERNEL_COMPONENT
        assert (p["groups"], p["slices"]) == (G, tiles)
    seen = np.zeros((C, T, tiles), dtype=np.int64)
    for wg in range(C * G * tiles):
        tile, cg = wg % tiles, wg // tiles
        grp, rho = cg % G, cg // G
        r0 = grp * 64
        seen[rho, r0:min(T, r0 + 64), tile] += 1
    assert (seen == 1).all()
    assert tiles * 32 >= n > (tiles - 1) * 32


# ------------------------------------------------ LDS plan vs kernel bounds

MI355X = dict(num_cu=256, max_lds=160 * 1024)
# the GPU sweep's shapes (m, n, d, zeta), each once
SWEEP_SHAPES = sorted({(c["m"], c["n"], c["d"], c["zeta"]) for c in SWEEP})

PLAN_SHAPES = [
    # (m, n, d, zeta): the scale, coherence, range and tiny workloads, ragged
    # and degenerate test shapes, and wide/narrow extremes
    (1 << 20, 256, 512, 4), (4096, 32, 64, 4), (4096, 32, 64, 1), (1 << 20, 128, 256, 1),
    (1 << 20, 128, 512, 2), (1 << 20, 128, 1024, 8), (1 << 18, 128, 256, 8),
    (4194304, 64, 128, 4), (1000, 38, 96, 3), (777, 130, 40, 8), (5, 2, 16, 16),
    (3001, 64, 5, 5), (2048, 66, 88, 11), (2048, 16, 8192, 4), (9000, 32, 64, 4),
    (1 << 16, 1024, 512, 4), (1 << 16, 512, 640, 4), (1 << 12, 4096, 64, 64), (300, 2, 64, 64),
]


@pytest.mark.parametrize("precision", [b.SK_PRECISION_F32, b.SK_PRECISION_F16ACC])
@pytest.mark.parametrize("wide_ok", [True, False])
@pytest.mark.parametrize("m,n,d,zeta", PLAN_SHAPES)
def test_lds_plan_fits_kernel(lib, precision, wide_ok, m, n, d, zeta):
    """Replays the apply kernel's workgroup mapping and LDS/workspace index
    arithmetic on the plan: every (slice, chunk, block group) is covered
    once, the partial and the wavefronts' dummy rows fit the LDS the plan
    reserves, each workgroup's flush stays inside the workspace, and
    two-word lanes only come with full 64-lane slices (the kernels that
    exist)."""
    f16 = precision == b.SK_PRECISION_F16ACC
    if f16 and n % 2:
        pytest.skip("odd n")
    p = b.sk_lds_plan_describe(precision, m, n, n, d, zeta, wide_ok, **MI355X)
    if not p["lds"]:
        # flat fallback only when the partial cannot fit or zeta > 64
        assert zeta > 64 or (d // zeta) * zeta * 8 * 4 + 16 * 64 * 4 > MI355X["max_lds"]
        return
    w, sp, g, zg = p["words"], p["slice"], p["groups"], p["zg"]
    assert w in (1, 2) and sp in (8, 16, 32, 64) and g * zg == zeta
    if w == 2:
        assert sp == 64 and wide_ok
    units = n // 2 if f16 else n
    assert p["slices"] * sp * w >= units
    assert p["threads"] in (512, 1024)
    nw = p["threads"] // 64
    db = d // zeta
    dl = zg * db
    assert (dl * sp + nw * 64) * w * 4 <= p["lds_bytes"] <= MI355X["max_lds"]
    assert p["chunks"] * p["rows_per_chunk"] >= m > (p["chunks"] - 1) * p["rows_per_chunk"]
    seen = set()
    for wg in range(p["grid"]):
        q = wg >> 3
        grp, uid = q % g, (q // g) * 8 + (wg & 7)
        if uid >= p["slices"] * p["chunks"]:
            continue
        sl, ch = uid % p["slices"], uid // p["slices"]
        assert (sl, ch, grp) not in seen
        seen.add((sl, ch, grp))
        row0 = grp * zg * db
        base = (sl * p["chunks"] + ch) * d * sp * w + row0 * sp * w
        assert (base + dl * sp * w) * 4 <= p["ws_bytes"]
    assert len(seen) == p["slices"] * p["chunks"] * g


def test_plan_describe_validation(lib):
    out = (ctypes.c_int64 * b.PLAN_FIELDS.__len__())()
    assert lib.sk_lds_plan_describe(0, 10, 0, 8, 8, 1, 1, 256, 163840, out) == b.SK_ERR_SHAPE
    assert lib.sk_lds_plan_describe(3, 10, 8, 8, 8, 1, 1, 256, 163840, out) == b.SK_ERR_ARG
    assert lib.sk_lds_plan_describe(1, 10, 7, 8, 8, 1, 1, 256, 163840, out) == b.SK_ERR_SHAPE
    assert lib.sk_lds_plan_describe(0, 10, 8, 8, 8, 1, 1, 0, 163840, out) == b.SK_ERR_ARG
    assert lib.sk_lds_plan_describe(0, 10, 8, 8, 8, 1, 1, 256, 163840, None) == b.SK_ERR_NULL


# ------------------------------------------------------ fused sketch calls

WSF = FAKE + (1 << 38)


@pytest.mark.parametrize("fn", ["sk_sketch_f32", "sk_sketch_f16acc"])
@pytest.mark.parametrize("args,expect", [
    ((1, 0, A, 100, 0, 64, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),     # n < 1
    ((1, -1, A, 100, 64, 64, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),   # row_offset < 0
    ((1, 0, A, -1, 64, 64, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),     # m < 0
    ((1, 0, A, 100, 64, 32, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),    # lda < n
    ((1, 0, A, 100, 64, 64, 64, 3, B, 64, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),    # d % zeta
    ((1, 0, A, 100, 64, 64, 64, 4, B, 32, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),    # ldb < n
    ((1, 0, A, 100, 64, 64, 64, 4, B, 64, 2, WSF, 1 << 30), b.SK_ERR_ARG),      # variant flag
    ((1, 0, A, 100, 64, 64, 64, 4, None, 64, 0, WSF, 1 << 30), b.SK_ERR_NULL),
    ((1, 0, None, 100, 64, 64, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_NULL),
    ((1, 0, A, 100, 64, 64, 64, 4, B, 64, 0, None, 0), b.SK_ERR_NULL),          # no workspace
    ((1, 0, A, 100, 64, 64, 64, 4, B, 64, 0, WSF + 4, 1 << 30), b.SK_ERR_ALIGN),  # 16-byte rule
    ((1, 0, A, 100, 64, 64, 64, 4, A + 64, 64, 0, WSF, 1 << 30), b.SK_ERR_ARG),   # B inside A
    ((1, 0, A, 100, 64, 64, 64, 4, B, 64, 0, A + 16, 1 << 20), b.SK_ERR_ARG),     # ws overlaps A
    ((1, 0, A, 100, 64, 64, 64, 4, B, 64, 0, B - 64, 1 << 20), b.SK_ERR_ARG),     # ws overlaps B
])
def test_sketch_validation(lib, fn, args, expect):
    assert getattr(lib, fn)(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((1, 0, A, 100, 63, 64, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),    # odd n
    ((1, 0, A, 100, 64, 64, 64, 4, B, 63, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),    # ldb < n (odd)
    ((1, 0, A, 100, 64, 64, 64, 4, B, 65, 0, WSF, 1 << 30), b.SK_ERR_ALIGN),    # odd ldb
    ((1, 0, A, 100, 64, 64, 64, 4, B + 2, 64, 0, WSF, 1 << 30), b.SK_ERR_ALIGN),  # B % 4
    ((1, 0, A, 100, 64, 65, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_ALIGN),    # odd lda
    ((1, 0, A + 4, 100, 64, 64, 64, 4, B, 64, 0, WSF, 1 << 30), b.SK_ERR_ALIGN),  # A % 8
])
def test_sketch_f16acc_pair_rules(lib, args, expect):
    assert lib.sk_sketch_f16acc(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((2, 100, 64, 64, 4), b.SK_ERR_ARG),        # unknown precision
    ((0, 100, 0, 64, 4), b.SK_ERR_SHAPE),       # n < 1
    ((1, 100, 63, 64, 4), b.SK_ERR_SHAPE),      # odd n for FP16
    ((0, 100, 64, 64, 3), b.SK_ERR_SHAPE),      # d % zeta
    ((0, -1, 64, 64, 4), b.SK_ERR_SHAPE),
])
def test_sketch_workspace_size_validation(lib, args, expect):
    out = ctypes.c_size_t(123)
    assert lib.sk_sketch_workspace_size(*args, ctypes.byref(out)) == expect
    assert out.value == 0
    assert lib.sk_sketch_workspace_size(0, 100, 64, 64, 4, None) == b.SK_ERR_NULL


FUSED_SHAPES = PLAN_SHAPES + [
    (1 << 20, 256, 1024, 4), (1 << 20, 256, 256, 16), (1 << 20, 512, 512, 1), (130, 128, 512, 4),
    (1, 128, 64, 4), (129, 256, 2048, 2), (1 << 21, 512, 1024, 4), (10_000, 384, 96, 3),
    (5000, 256, 512, 32), (5000, 256, 64, 16),
] + SWEEP_SHAPES


@pytest.mark.parametrize("precision", [b.SK_PRECISION_F32, b.SK_PRECISION_F16ACC])
@pytest.mark.parametrize("m,n,d,zeta", FUSED_SHAPES)
def test_fused_plan_fits_kernel(lib, precision, m, n, d, zeta):
    """Replays the fused kernel's workgroup and wavefront mapping on its
    plan: every (slice, chunk, row group) is covered once, 16 wavefronts x R
    rows x groups tile the d output rows exactly, each wavefront's R rows
    lie inside one stack block (the block whose metadata it scans), chunks
    are whole 128-row stages covering the m rows, the lanes' column loads
    stay inside the row, and every partial store stays inside the
    workspace."""
    f16 = precision == b.SK_PRECISION_F16ACC
    if f16 and n % 2:
        pytest.skip("odd n")
    K2 = 4 if f16 else 2                # floats per lane at two words per lane
    p = b.sk_fused_plan_describe(precision, m, n, n, 16, d, zeta, **MI355X)
    if not p["fused"]:
        assert (zeta > 16 or (n % 2 and (f16 or n > 64)) or d % 16
                or all((d // (16 * g)) not in (4, 8, 16, 32) or (d // zeta) % (d // (16 * g))
                       for g in (1, 2, 4, 8, 16, 32) if d % (16 * g) == 0))
        return
    W, S, per_cu = p["words"], p["stage_rows"], p["per_cu"]
    # four words per lane only for FP32 wider than 128 columns; one word only
    # for FP16 of at most 128 columns; two per CU (64-row stages) for few
    # partial words per lane; 128-row stages only at two words, one per CU
    assert (W, S, per_cu) in ((2, 128, 1), (4, 64, 1), (2, 64, 2), (1, 64, 2))
    assert W != 4 or (not f16 and n > 128 and n % 4 == 0)
    assert W != 1 or (f16 and n <= 128) or (not f16 and n <= 64)
    K = W * (2 if f16 else 1)
    R, g = p["rows_per_wave"], p["groups"]
    assert R in {1: (8, 16, 32, 64), 2: (4, 8, 16, 32), 4: (8, 16)}[W] and 16 * R * g == d
    # the built two-per-CU instances
    assert per_cu == 1 or (W, R) in ((2, 4), (2, 8), (1, 8), (1, 16), (1, 32)) \
        or (not f16 and (W, R) == (2, 16))
    assert (per_cu == 2) == (W <= 2 and W * R + 4 * K <= 40)
    db = d // zeta
    assert db % R == 0
    assert p["rows_per_chunk"] % S == 0
    assert p["chunks"] * p["rows_per_chunk"] >= m > (p["chunks"] - 1) * p["rows_per_chunk"]
    assert p["slices"] * 64 * K >= n > (p["slices"] - 1) * 64 * K
    for lane in (0, 31, 32, 63):
        for sl in range(p["slices"]):
            col = sl * 64 * K + lane * K
            assert 0 <= min(col, n - K) and min(col, n - K) + K <= n
    seen = set()
    for wg in range(p["grid"]):
        q = wg >> 3
        grp, uid = q % g, (q // g) * 8 + (wg & 7)
        if uid >= p["slices"] * p["chunks"]:
            continue
        sl, ch = uid % p["slices"], uid // p["slices"]
        assert (sl, ch, grp) not in seen
        seen.add((sl, ch, grp))
        for wave in (0, 15):
            lo = (grp * 16 + wave) * R
            t = lo // db
            assert t < zeta and t * db <= lo and lo + R <= (t + 1) * db
            for lane in (0, 31, 32, 63):
                # a lane's W words: word sl*64*W + lane*W of the row, stored
                # in the workspace's 128-word slices
                wcol = sl * 64 * W + lane * W
                first = (((wcol >> 7) * p["chunks"] + ch) * d + lo) * 128 + (wcol & 127)
                last = first + (R - 1) * 128 + W - 1
                assert (wcol & 127) + W <= 128
                assert first >= 0 and (last + 1) * 4 <= p["ws_bytes"]
    assert len(seen) == p["slices"] * p["chunks"] * g
    # the fused kernel's metadata stage holds at most 16 blocks
    assert zeta <= 16


OWNER_SHAPES = FUSED_SHAPES + [
    (1 << 20, 2, 512, 4), (1 << 20, 2, 256, 8), (4194304, 64, 128, 4), (1 << 20, 32, 1024, 1),
    (1 << 20, 64, 256, 16), (1 << 16, 4, 64, 1), (777, 6, 48, 3), (5000, 62, 40, 8),
    (64, 64, 128, 4), (1, 2, 64, 4), (1 << 20, 16, 4096, 4), (3000, 2, 16, 16),
    (1 << 20, 64, 512, 4), (1 << 20, 32, 512, 4),
] + SWEEP_SHAPES


@pytest.mark.parametrize("precision", [b.SK_PRECISION_F32, b.SK_PRECISION_F16ACC])
@pytest.mark.parametrize("m,n,d,zeta", OWNER_SHAPES)
@pytest.mark.parametrize("lda_extra,align", [(0, 16), (1, 4), (2, 8)])
def test_sketch_plan_fits_owner_kernel(lib, precision, m, n, d, zeta, lda_extra, align):
    """Replays the owner kernel's indexing on its plan: the workgroup's
    threads are whole wavefronts and cover d output rows x L lanes, each
    lane's V words of a padded row lie inside it, every stage load reads
    inside its row with the load's alignment, the LDS carve (two or three
    stage buffers, mask sets and entry sets, one or two list sets) fits, list reads of 4
    entries stay inside an output row's list, a stage row index fits the
    list entry's 15 bits, and every partial store stays inside the
    workspace.  Shapes the owner kernel does not take report the register
    kernel or the fallback."""
    f16 = precision == b.SK_PRECISION_F16ACC
    if f16 and n % 2:
        pytest.skip("odd n")
    lda = n + lda_extra * (2 if f16 else 1)
    p = b.sk_sketch_plan_describe(precision, m, n, lda, align, d, zeta, **MI355X)
    kc = 2 if f16 else 1
    nw = n // kc
    U = 1 << (nw - 1).bit_length()
    if p["kernel"] != 2:
        # rows the owner kernel leaves: 64 words at more than 8 per lane,
        # wider than its 16 words per lane allow at this d, a d its
        # workgroup cannot tile, or zeta > 16
        if U <= 64 and p["kernel"] != 0:
            kmax = 2 if f16 else 4
            kw = kmax if (nw % kmax == 0 and U % kmax == 0 and lda % (kmax * kc) == 0
                          and align >= kmax * kc * 4) else 1
            V = 1
            while V < U and d * (U // V) > 1024:
                V *= 2
            # (a 128-row stage needs more than four loads per thread)
            assert (U == 64 and d * U > 1024 * 8) or d * U > 1024 * 16 or zeta > 16 or \
                d % zeta or (d * U) % 64 or (lda % kc) or align < 4 * kc or \
                128 * U > 4 * kw * d * (U // V)
        return
    assert U <= 32 or d * U <= 1024 * 8
    V, L, NT, U = p["words"], p["lanes_per_row"], p["threads"], p["row_words"]
    S, cap, kw = p["stage_rows"], p["cap"], p["load_words"]
    assert U >= nw and U & (U - 1) == 0 and U <= 64 and V * L == U and V <= 16
    assert NT == d * L and NT % 64 == 0 and NT <= 1024
    assert S % 128 == 0 and S <= 512 and cap % 4 == 0 and 4 <= cap <= S
    # list entries hold a row's word offset in 15 bits (the -0 row's included)
    assert S * U < 1 << 15
    # loads: kw words = kw * kc floats, at most four per thread and stage
    assert kw in (1, 2, 4) and U % kw == 0 and nw % kw == 0
    fl = kw * kc
    assert lda % fl == 0 and align >= 4 * fl
    nload = -(-(S * U // kw) // NT)
    # load slots: two at 16 words per lane where the stage needs no more
    assert p["load_slots"] == (2 if V == 16 and nload <= 2 else 4)
    assert nload <= p["load_slots"]
    lpr = U // kw
    for tid in (0, 1, NT // 2, NT - 1):
        for i in range(nload):
            q = tid + i * NT
            row, w0 = q // lpr, (q % lpr) * kw
            if row < S and w0 < nw:
                assert w0 * kc + fl <= n                 # inside the row
                assert (w0 * kc) % fl == 0                # aligned
    # LDS carve in words: nb stage buffers of S + 1 rows (row S: the -0
    # row), padding to 16 bytes, 4 trash words, nb mask sets (per output
    # row MW mask words and 4 count words: a byte per 64 stage rows, at most
    # 8), nb entry sets, nb - 1 list sets; nb = 3 with one barrier per stage
    MW = S // 32
    assert S // 64 <= 8

    # row strides: w + 4 words, or (where the LDS allows) the next odd number
    # of 16-byte units
    MS, CS = p["mask_stride"], p["list_stride"]
    spread = MS != MW + 4 or CS != cap + 4 or ((MW // 4) % 2 == 0 and (cap // 4) % 2 == 0)
    for w, st in ((MW, MS), (cap, CS)):
        assert st == (w + 8 if spread and (w // 4) % 2 else w + 4)
    def carve(nb):
        bufs = nb * (S + 1) * U
        trash = -(-bufs // 4) * 4
        masks = trash + 4
        ents = masks + nb * d * MS
        lists = ents + nb * zeta * S
        return trash, masks, ents, lists, lists + (nb - 1) * d * CS

    assert p["barriers"] in (1, 2)
    nb = 3 if p["barriers"] == 1 else 2
    trash, masks, ents, lists, words = carve(nb)
    assert 4 * words == p["lds_bytes"] <= MI355X["max_lds"]
    assert p["per_cu"] in (1, 2) and p["per_cu"] * p["lds_bytes"] <= MI355X["max_lds"]
    # one barrier wherever the three sets fit at the same stage rows and
    # workgroups per CU, with 512 threads or more and 8 hits per output row
    # and stage on average
    w3 = carve(3)[-1]
    fits3 = p["per_cu"] * 4 * w3 <= MI355X["max_lds"]
    assert (nb == 3) == (fits3 and NT >= 512 and S * zeta >= 8 * d)
    assert trash % 4 == 0 and masks % 4 == 0 and ents % 4 == 0 and lists % 4 == 0
    assert MW % 4 == 0 and (S + 1) * U % kw == 0      # the second buffer's stores stay aligned
    # chunks of whole stages cover m; one workgroup per chunk
    rpc = p["rows_per_chunk"]
    assert rpc % S == 0 and p["chunks"] * rpc >= m > (p["chunks"] - 1) * rpc
    assert p["grid"] == p["chunks"] <= 65535
    # partial stores: lane (o, g) writes words [g*V, g*V + V) of row o
    for tid in (0, NT - 1):
        o, g = tid // L, tid % L
        last = ((p["chunks"] - 1) * d + o) * U + g * V + V
        assert o < d and last * 4 <= p["ws_bytes"]
    assert p["ws_bytes"] == p["chunks"] * d * U * 4


def test_sketch_plan_kernel_choice(lib):
    """Narrow rows take the owner kernel (the m x 2 right-hand side of
    sketch-and-solve, the 64-column range workload), wider ones the
    register kernel."""
    P16, P32 = b.SK_PRECISION_F16ACC, b.SK_PRECISION_F32
    q = b.sk_sketch_plan_describe(P16, 1 << 20, 2, 2, 16, 512, 4, **MI355X)
    assert (q["kernel"], q["words"], q["lanes_per_row"], q["threads"]) == (2, 1, 1, 512)
    q = b.sk_sketch_plan_describe(P16, 4194304, 64, 64, 16, 128, 4, **MI355X)
    assert (q["kernel"], q["words"], q["lanes_per_row"], q["threads"], q["row_words"]) == \
        (2, 4, 8, 1024, 32)
    assert b.sk_sketch_plan_describe(P16, 1 << 20, 256, 256, 16, 512, 4, **MI355X)["kernel"] == 1
    assert b.sk_sketch_plan_describe(P32, 1 << 20, 256, 256, 16, 512, 4, **MI355X)["kernel"] == 1
    # 64-word rows: the owner kernel at d = 128 (8 words per lane), the
    # register kernel from d = 256
    q = b.sk_sketch_plan_describe(P32, 4194304, 64, 64, 16, 128, 4, **MI355X)
    assert (q["kernel"], q["words"], q["lanes_per_row"]) == (2, 8, 8)
    for prec, n in ((P32, 64), (P16, 128)):
        assert b.sk_sketch_plan_describe(prec, 1 << 20, n, n, 16, 256, 8, **MI355X)["kernel"] == 1


def test_fused_plan_word_width(lib):
    """FP32 matrices wider than 128 columns with 16-byte rows take four
    words per lane (256 columns per workgroup, two row groups at d = 512);
    an 8-byte-aligned base, lda % 4 != 0, 128 columns or FP16 keep two."""
    P16, P32 = b.SK_PRECISION_F16ACC, b.SK_PRECISION_F32
    p = b.sk_fused_plan_describe(P32, 1 << 20, 256, 256, 16, 512, 4, **MI355X)
    assert (p["fused"], p["words"], p["stage_rows"], p["rows_per_wave"], p["groups"],
            p["slices"]) == (1, 4, 64, 16, 2, 1)
    assert p["grid"] == 256 and p["chunks"] == 128
    for args in ((256, 256, 8), (256, 258, 16), (128, 128, 16)):
        q = b.sk_fused_plan_describe(P32, 1 << 20, args[0], args[1], args[2], 512, 4, **MI355X)
        assert (q["fused"], q["words"], q["stage_rows"]) == (1, 2, 128)
    q = b.sk_fused_plan_describe(P16, 1 << 20, 512, 512, 16, 512, 4, **MI355X)
    assert (q["fused"], q["words"]) == (1, 2)
    # FP16 rows of at most 128 columns: one word per lane (8-byte loads);
    # R <= 32 two per CU, d = 1024 and 2048 in two and four row groups
    for d, R, G in ((256, 16, 1), (512, 32, 1), (1024, 32, 2), (2048, 32, 4)):
        q = b.sk_fused_plan_describe(P16, 1 << 20, 128, 128, 8, d, 4, **MI355X)
        assert (q["fused"], q["words"], q["rows_per_wave"], q["groups"], q["per_cu"],
                q["slices"]) == (1, 1, R, G, 2, 1)
        assert q["grid"] == 512
    # FP32 of at most 64 columns: one word per lane, any width or stride;
    # R = 8 two per CU, 64-row stages, chunks for 512 workgroups
    q = b.sk_fused_plan_describe(P32, 1 << 22, 64, 64, 16, 128, 4, **MI355X)
    assert (q["words"], q["rows_per_wave"], q["per_cu"], q["stage_rows"], q["grid"]) == \
        (1, 8, 2, 64, 512)
    for n, lda, align in ((1, 1, 4), (31, 33, 4), (64, 65, 4)):
        q = b.sk_fused_plan_describe(P32, 1 << 20, n, lda, align, 512, 4, **MI355X)
        assert (q["fused"], q["words"], q["rows_per_wave"], q["per_cu"]) == (1, 1, 32, 2)
    # two words per lane and R <= 8 (FP32 between 65 and 128 columns)
    q = b.sk_fused_plan_describe(P32, 1 << 22, 128, 128, 16, 128, 4, **MI355X)
    assert (q["words"], q["rows_per_wave"], q["per_cu"], q["stage_rows"]) == (2, 8, 2, 64)


def test_fused_plan_alignment_and_validation(lib):
    P16, P32 = b.SK_PRECISION_F16ACC, b.SK_PRECISION_F32
    assert b.sk_fused_plan_describe(P16, 1 << 20, 256, 256, 16, 512, 4, **MI355X)["fused"] == 1
    # wide FP16 rows with an 8-byte base or lda % 4 != 0, an odd FP32 lda
    # above 64 columns: the fallback
    assert b.sk_fused_plan_describe(P16, 1 << 20, 256, 256, 8, 512, 4, **MI355X)["fused"] == 0
    assert b.sk_fused_plan_describe(P16, 1 << 20, 256, 258, 16, 512, 4, **MI355X)["fused"] == 0
    assert b.sk_fused_plan_describe(P32, 1 << 20, 256, 257, 16, 512, 4, **MI355X)["fused"] == 0
    assert b.sk_fused_plan_describe(P16, 1 << 20, 64, 64, 16, 128, 4, **MI355X)["fused"] == 1
    # narrow rows are covered (one word per lane, any FP32 width up to 64);
    # an odd FP32 width or lda above 64 columns is not
    assert b.sk_fused_plan_describe(P16, 1 << 20, 60, 60, 16, 128, 4, **MI355X)["fused"] == 1
    assert b.sk_fused_plan_describe(P32, 1 << 20, 62, 62, 16, 128, 4, **MI355X)["fused"] == 1
    assert b.sk_fused_plan_describe(P16, 1 << 20, 2, 2, 8, 512, 4, **MI355X)["fused"] == 1
    assert b.sk_fused_plan_describe(P32, 1 << 20, 2, 2, 8, 512, 4, **MI355X)["fused"] == 1
    assert b.sk_fused_plan_describe(P32, 1 << 20, 31, 31, 16, 128, 4, **MI355X)["fused"] == 1
    assert b.sk_fused_plan_describe(P32, 1 << 20, 1, 1, 16, 128, 4, **MI355X)["fused"] == 1
    assert b.sk_fused_plan_describe(P32, 1 << 20, 65, 65, 16, 128, 4, **MI355X)["fused"] == 0
    # LDS smaller than the kernel's stages
    assert b.sk_fused_plan_describe(P16, 1 << 20, 256, 256, 16, 512, 4, num_cu=256,
                                    max_lds=64 * 1024)["fused"] == 0
    out = (ctypes.c_int64 * len(b.FUSED_PLAN_FIELDS))()
    assert lib.sk_fused_plan_describe(0, 10, 0, 8, 1, 8, 1, 256, 163840, out) == b.SK_ERR_SHAPE
    assert lib.sk_fused_plan_describe(3, 10, 8, 8, 1, 8, 1, 256, 163840, out) == b.SK_ERR_ARG
    assert lib.sk_fused_plan_describe(1, 10, 7, 8, 1, 8, 1, 256, 163840, out) == b.SK_ERR_SHAPE
    assert lib.sk_fused_plan_describe(0, 10, 8, 8, 1, 8, 1, 0, 163840, out) == b.SK_ERR_ARG
    assert lib.sk_fused_plan_describe(0, 10, 8, 8, 1, 8, 1, 256, 163840, None) == b.SK_ERR_NULL


# ------------------------------------------------- conversion variants

@pytest.mark.parametrize("args,expect", [
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 2, 0, 0, 0, 0), b.SK_ERR_ARG),      # unknown format
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 0, 2, 0, 0, 0), b.SK_ERR_ARG),      # unknown conversion
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 0, 0, 0, 0, 4), b.SK_ERR_ARG),      # LDS variant
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 0, 0, 0, 0, 10), b.SK_ERR_ARG),     # FLAT|REG
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 0, 0, 0, 0, 16), b.SK_ERR_ARG),     # combine, no REG
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 0, 1, 0, 0, 8), b.SK_ERR_NULL),     # REG, no workspace
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 0, 1, 0, -1, 0), b.SK_ERR_SHAPE),   # row_offset < 0
    ((A, 100, 63, 64, RI, V, 4, B, 64, 64, 0, 0, 0, 0, 0), b.SK_ERR_SHAPE),    # odd n
    ((A, 100, 64, 64, RI, V, 3, B, 64, 64, 0, 0, 0, 0, 0), b.SK_ERR_SHAPE),    # d % zeta
    ((A, 100, 64, 64, RI, V, 4, B + 2, 64, 64, 0, 0, 0, 0, 0), b.SK_ERR_ALIGN),  # B % 4
    ((A, 100, 64, 65, RI, V, 4, B, 64, 64, 1, 0, 0, 0, 0), b.SK_ERR_ALIGN),    # odd lda
    ((A, 100, 64, 64, RI, V, 4, B, 64, 64, 1, 1, 0, 0, 0), b.SK_ERR_UNSUPPORTED),  # BF16 + SR
    ((A, 100, 64, 64, None, V, 4, B, 64, 64, 0, 0, 0, 0, 0), b.SK_ERR_NULL),
    ((A, 100, 64, 64, RI, V, 4, A + 256, 64, 64, 0, 0, 0, 0, 0), b.SK_ERR_ARG),  # B inside A
])
def test_lowp_validation(lib, args, expect):
    assert lib.sk_apply_lowp(*args, None, 0, None) == expect


# ------------------------------------------------------- general BlockPerm

@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 12, 60, 64, 97, 100, 128, 1024])
@pytest.mark.parametrize("seed", [0, 1, 12345678901])
def test_blockperm_affine_params_match_oracle(M, seed):
    """The host's affine wiring parameters are the oracle's (independent
    implementations of the same drawing rule), and a^-1 inverts a."""
    import oracle
    p = b.sk_blockperm_plan_describe(M * 64, 32, M * 4, M, 1, 1, b.SK_WIRING_AFFINE, seed,
                                     num_cu=256, max_lds=160 * 1024)
    a, bb = oracle.affine_params(seed, M)
    assert p["kernel"] == b.SK_BLOCKPERM_KERNEL_SLICE
    assert (p["a"], p["b"]) == (a % max(M, 1) if M > 1 else 1, bb)
    if M > 1:
        assert (p["a"] * p["ainv"]) % M == 1


@pytest.mark.parametrize("m,n,d,M,kappa,s,wiring,kernel,R,G", [
    (1 << 21, 512, 1024, 64, 4, 1, 0, 2, 4, 1),     # the bench workload
    (1 << 21, 512, 1024, 64, 4, 2, 0, 2, 4, 1),     # s > 1
    (1 << 21, 512, 1024, 64, 4, 1, 1, 2, 4, 1),     # affine wiring
    (1 << 16, 64, 1024, 64, 4, 1, 0, 2, 4, 1),      # few workgroups: row slices
    (1 << 16, 300, 1024, 64, 32, 1, 1, 2, 16, 2),   # kappa*B_r = 512: two row groups
    (1 << 16, 300, 4096, 64, 32, 1, 1, 2, 16, 8),   # kappa*B_r = 2048: eight
    (1 << 12, 8, 64, 8, 2, 1, 0, 2, 1, 1),          # kappa*B_r = 16: R = 1
    (4096, 32, 256, 16, 5, 3, 1, 1, 0, 0),          # B_r = 16, kappa*B_r = 80: slice kernel
    (4096, 30, 256, 16, 4, 1, 1, 1, 0, 0),          # n % 4 != 0: slice kernel
    (1 << 16, 1022, 1024, 64, 4, 1, 0, 0, 0, 0),    # shift, n % 4 != 0, 32 tiles x 16: component
])
def test_blockperm_plan_bounds(m, n, d, M, kappa, s, wiring, kernel, R, G):
    p = b.sk_blockperm_plan_describe(m, n, d, M, kappa, s, wiring, 7, num_cu=256,
                                     max_lds=160 * 1024)
    Bc, Br = m // M, d // M
    assert p["kernel"] == kernel
    if kernel == b.SK_BLOCKPERM_KERNEL_COMPONENT:
        assert wiring == 0 and s == 1 and p["ws_bytes"] == 0
        return
    Q, rps = p["Q"], p["rows_per_slice"]
    assert Q >= 1 and rps * Q >= Bc > rps * (Q - 1)
    assert p["ws_bytes"] >= Q * kappa * d * n * 4
    # the largest partial index either kernel writes stays inside it
    last = ((((M - 1) * Q + Q - 1) * kappa + kappa - 1) * Br + Br - 1) * n + n - 1
    assert (last + 1) * 4 <= p["ws_bytes"]
    if kernel == b.SK_BLOCKPERM_KERNEL_SLICE:
        assert Q * M <= 65535 and p["rows_per_wave"] == 0
        return
    # register kernel: 16 wavefronts x R rows x G groups cover kappa*B_r,
    # a wavefront's rows inside one reader's block, whole stages per slice
    assert (p["rows_per_wave"], p["groups"]) == (R, G)
    assert 16 * R * G == kappa * Br and Br % R == 0 and rps % 64 == 0
    assert p["slices"] * 256 >= n > (p["slices"] - 1) * 256


@pytest.mark.parametrize("case", range(len(BP_SWEEP)))
def test_blockperm_sweep_plans_fit_kernels(case):
    """The GPU sweep's BlockPerm shapes: whichever kernel the plan picks,
    the component kernel's workgroups own every output element once, and
    the general kernels' partial indices stay inside the workspace, with
    the register kernel's wavefronts tiling kappa*B_r inside one block."""
    import numpy as np
    c = BP_SWEEP[case]
    m, n, d, M, kappa, s = c["m"], c["n"], c["d"], c["M"], c["kappa"], c["s"]
    w = b.SK_WIRING_SHIFT if c["wiring"] == "shift" else b.SK_WIRING_AFFINE
    p = b.sk_blockperm_plan_describe(m, n, d, M, kappa, s, w, 7, num_cu=256, max_lds=160 * 1024)
    Bc, Br = m // M, d // M
    T = kappa * Br
    if w == b.SK_WIRING_SHIFT:
        # sk_apply_blockperm's component grid (and _ex's where it plans it)
        G, tiles, C = -(-T // 64), -(-n // 32), M // kappa
        seen = np.zeros((C, T, tiles), dtype=np.int64)
        for wg in range(C * G * tiles):
            tile, cg = wg % tiles, wg // tiles
            r0 = (cg % G) * 64
            seen[cg // G, r0:min(T, r0 + 64), tile] += 1
        assert (seen == 1).all()
    if p["kernel"] == b.SK_BLOCKPERM_KERNEL_COMPONENT:
        assert w == b.SK_WIRING_SHIFT and p["ws_bytes"] == 0
        return
    Q, rps = p["Q"], p["rows_per_slice"]
    assert Q >= 1 and rps * Q >= Bc
    last = ((((M - 1) * Q + Q - 1) * kappa + kappa - 1) * Br + Br - 1) * n + n - 1
    assert (last + 1) * 4 <= p["ws_bytes"]
    if p["kernel"] == b.SK_BLOCKPERM_KERNEL_SLICE:
        # (trailing slices past the block may be empty: their workgroups
        # find no rows and store zero partials)
        assert Q * M <= 65535
        return
    assert Bc > rps * (Q - 1)
    R, G = p["rows_per_wave"], p["groups"]
    assert 16 * R * G == T and Br % R == 0 and rps % 64 == 0
    assert p["slices"] * 256 >= n > (p["slices"] - 1) * 256


def test_blockperm_register_grid_covers_every_unit_once():
    """Replays the kernel's workgroup -> (unit, row group) mapping on the
    host: every (input block, row slice, column slice, group) is owned by
    exactly one workgroup and the rest of the grid exits."""
    for (m, n, d, M, kappa) in [(1 << 21, 512, 1024, 64, 4), (1 << 16, 300, 4096, 64, 32),
                                (1 << 12, 8, 64, 8, 2), (3 * 1000, 520, 3 * 16, 3, 2)]:
        p = b.sk_blockperm_plan_describe(m, n, d, M, kappa, 1, 1, 7, num_cu=256,
                                         max_lds=160 * 1024)
        assert p["kernel"] == b.SK_BLOCKPERM_KERNEL_REGISTER
        G, Q, slices = p["groups"], p["Q"], p["slices"]
        units = M * Q * slices
        grid = (units + 7) // 8 * 8 * G
        seen = set()
        for wg in range(grid):
            qq = wg >> 3
            unit = (qq // G) * 8 + (wg & 7)
            if unit >= units:
                continue
            key = (unit, qq % G)
            assert key not in seen
            seen.add(key)
        assert len(seen) == units * G


@pytest.mark.parametrize("args,expect", [
    ((A, 4096, 32, 32, 256, 16, 4, 1, 2, 1, B, 32, 0, WSF, 1 << 30), b.SK_ERR_ARG),    # wiring
    ((A, 4096, 32, 32, 256, 16, 3, 1, 0, 1, B, 32, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),  # kappa !| M (shift)
    ((A, 4096, 32, 32, 256, 16, 17, 1, 1, 1, B, 32, 0, WSF, 1 << 30), b.SK_ERR_SHAPE), # kappa > M
    ((A, 4096, 32, 32, 192, 16, 4, 2, 1, 1, B, 32, 0, WSF, 1 << 30), b.SK_ERR_UNSUPPORTED),  # B_r = 12, s > 1
    ((A, 4096, 32, 32, 256, 16, 4, 17, 1, 1, B, 32, 0, WSF, 1 << 30), b.SK_ERR_SHAPE),  # s > B_r
    ((A, 4096, 32, 32, 256, 16, 4, 1, 1, 1, B, 32, 2, WSF, 1 << 30), b.SK_ERR_ARG),     # flag
    ((None, 4096, 32, 32, 256, 16, 4, 1, 1, 1, B, 32, 0, WSF, 1 << 30), b.SK_ERR_NULL),
    ((A, 4096, 32, 32, 256, 16, 4, 1, 1, 1, A + 64, 32, 0, WSF, 1 << 30), b.SK_ERR_ARG),  # Y in A
])
def test_blockperm_ex_validation(lib, args, expect):
    assert lib.sk_apply_blockperm_ex(*args, None) == expect


def test_lstsq_validation(lib):
    """sk_lstsq_qr_f32 rejects bad arguments before any HIP call (host
    buffers stand in for device pointers; every call here fails validation,
    so nothing is launched), and the workspace size is (n + 1)(d + 1) + 1024
    floats (the columns, the panel's T, the column exponents)."""
    d, n = 64, 32
    SA = (ctypes.c_float * (d * n))()
    Sb = (ctypes.c_float * d)()
    x = (ctypes.c_float * n)()
    ws = (ctypes.c_float * ((n + 1) * (d + 1) + 1025))()
    nb = ((n + 1) * (d + 1) + 1024) * 4
    f = lib.sk_lstsq_qr_f32
    A, B, X, Wp = (ctypes.addressof(t) for t in (SA, Sb, x, ws))
    assert f(A, d, d + 1, d + 1, B, X, Wp, nb, None) == b.SK_ERR_SHAPE      # n > d
    assert f(A, d, 0, n, B, X, Wp, nb, None) == b.SK_ERR_SHAPE              # n < 1
    assert f(A, 2049, n, n, B, X, Wp, nb, None) == b.SK_ERR_SHAPE           # d above 2048
    assert f(A, d, n, n - 1, B, X, Wp, nb, None) == b.SK_ERR_SHAPE          # ld < n
    assert f(None, d, n, n, B, X, Wp, nb, None) == b.SK_ERR_NULL
    assert f(A, d, n, n, None, X, Wp, nb, None) == b.SK_ERR_NULL
    assert f(A, d, n, n, B, None, Wp, nb, None) == b.SK_ERR_NULL
    assert f(A, d, n, n, B, X, None, nb, None) == b.SK_ERR_NULL
    assert f(A, d, n, n, B, X, Wp + 2, nb, None) == b.SK_ERR_ALIGN         # 4-byte rule
    assert f(A, d, n, n, B, X, Wp, nb - 4, None) == b.SK_ERR_ARG           # too small
    assert f(A, d, n, n, B, X, A, nb, None) == b.SK_ERR_ARG                # workspace = SA
    assert f(A, d, n, n, B, A, Wp, nb, None) == b.SK_ERR_ARG               # x inside SA
    out = ctypes.c_size_t(0)
    assert lib.sk_lstsq_workspace_size(d, n, ctypes.byref(out)) == b.SK_OK and out.value == nb
    assert lib.sk_lstsq_workspace_size(d, d + 1, ctypes.byref(out)) == b.SK_ERR_SHAPE
    assert lib.sk_lstsq_workspace_size(d, n, None) == b.SK_ERR_NULL


# The four entry points of the sketching boundary, with their parameter
# lists: (type, name) pairs.  The stream is a hipStream_t passed as void*
# (the header includes no HIP header).
BOUNDARY = {
    "sk_meta_generate": [("uint64_t", "seed"), ("int64_t", "row_offset"), ("int64_t", "m"),
                         ("int32_t", "d"), ("int32_t", "zeta"), ("int32_t *", "row_idx"),
                         ("float *", "val"), ("void *", "stream")],
    "sk_apply_f32": [("const float *", "A"), ("int64_t", "m"), ("int32_t", "n"),
                     ("int64_t", "lda"), ("const int32_t *", "row_idx"), ("const float *", "val"),
                     ("int32_t", "zeta"), ("float *", "B"), ("int32_t", "d"), ("int64_t", "ldb"),
                     ("uint32_t", "flags"), ("void *", "stream")],
    "sk_apply_f16acc": [("const float *", "A"), ("int64_t", "m"), ("int32_t", "n"),
                        ("int64_t", "lda"), ("const int32_t *", "row_idx"),
                        ("const float *", "val"), ("int32_t", "zeta"), ("uint16_t *", "B"),
                        ("int32_t", "d"), ("int64_t", "ldb"), ("uint32_t", "flags"),
                        ("void *", "stream")],
    "sk_apply_blockperm": [("const float *", "A"), ("int64_t", "m"), ("int32_t", "n"),
                           ("int64_t", "lda"), ("int32_t", "d"), ("int32_t", "M"),
                           ("int32_t", "kappa"), ("int32_t", "s"), ("uint64_t", "seed"),
                           ("float *", "Y"), ("int64_t", "ldy"), ("uint32_t", "flags"),
                           ("void *", "stream")],
}


def _declaration(name):
    import re
    with open(b.HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    m = re.search(r"sk_status\s+" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = []
    for p in m.group(1).split(","):
        p = " ".join(p.split())
        pm = re.match(r"(.*?)\s*(\w+)$", p)
        params.append((pm.group(1).replace(" *", " *").strip(), pm.group(2)))
    return params


@pytest.mark.parametrize("name", sorted(BOUNDARY))
def test_boundary_signatures(lib, name):
    """The boundary calls take exactly their documented parameter lists
    (no workspace), and the binding declares the same arity."""
    assert _declaration(name) == BOUNDARY[name]
    assert len(b._SIGNATURES[name][1]) == len(BOUNDARY[name])
