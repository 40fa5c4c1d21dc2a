"""GPU checks of sk_sketch_f16acc_noalloc, the allocation-free form of the
fused FP16 sketch (static device scratch instead of a workspace): through
the C ABI it gives sk_sketch_f16acc's result bit for bit (same kernels,
same fixed order of additions), on consecutive calls of decreasing size
that share the scratch, and refuses shapes whose partials do not fit."""
import numpy as np
import pytest
import torch

from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync

pytestmark = pytest.mark.gpu


def _pair(A, d, zeta, seed, flags=0, B0=None, row_offset=0):
    """(noalloc result, workspace result) of the same call."""
    m, n = A.shape
    outs = []
    for use_ws in (False, True):
        B = torch.empty((d, n), dtype=torch.float16, device=dev()) if B0 is None else B0.clone()
        if use_ws:
            ws = b.sketch_workspace(A, d, zeta, "f16acc")
            b.sk_sketch_f16acc(seed, row_offset, A, m, n, A.stride(0), d, zeta, B, B.stride(0),
                               flags, ws, 0)
        else:
            b.sk_sketch_f16acc_noalloc(seed, row_offset, A, m, n, A.stride(0), d, zeta, B,
                                       B.stride(0), flags)
        outs.append(B)
    sync()
    return outs


def test_noalloc_equals_workspace_call_twice_shrinking():
    """Calls in a row, each on a smaller input (the last a right-hand side
    of two columns, which the owner kernel sketches): each equals the
    workspace call bit for bit (a call's reduce reads only what it wrote,
    whatever the one before left in the scratch)."""
    for (m, n, d, zeta, seed) in ((1 << 20, 256, 512, 4, 1), (70001, 128, 256, 8, 2),
                                  (50000, 2, 512, 4, 3)):
        say(f"noalloc {m}x{n} d={d} zeta={zeta}")
        A = inputs.gaussian_torch(m, n, seed=seed)
        got, want = _pair(A, d, zeta, seed)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert torch.isfinite(got.float()).all() and float(got.float().abs().max()) > 0


def test_noalloc_flags_and_offsets():
    """SK_COMBINE_F32 and SK_ACCUMULATE (onto a given B) with a row offset,
    then a shape of two row groups and narrow rows."""
    m, n, d, zeta = 30000, 64, 128, 4
    A = inputs.gaussian_torch(m, n, seed=4)
    B0 = inputs.gaussian_torch(d, n, seed=5).half()
    for flags in (b.SK_COMBINE_F32, b.SK_ACCUMULATE, b.SK_ACCUMULATE | b.SK_COMBINE_F32):
        say(f"noalloc flags={flags}")
        got, want = _pair(A, d, zeta, 9, flags=flags, B0=B0, row_offset=12345)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    A2 = inputs.gaussian_torch(5000, 384, seed=6)
    got, want = _pair(A2, 1024, 4, 3)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_noalloc_refuses_what_it_does_not_cover():
    """Partials beyond the 128 MiB scratch (262144 FP16 columns, d = 512:
    1024 column slices of 256 KiB) and shapes neither fused kernel covers
    (256 columns, wider than the owner kernel's rows, with d not a multiple
    of 16) return SK_ERR_UNSUPPORTED; m = 0 zeroes B."""
    A = torch.zeros((64, 1 << 18), dtype=torch.float32, device=dev())
    B = torch.empty((512, 1 << 18), dtype=torch.float16, device=dev())
    with pytest.raises(b.SketchError) as e:
        b.sk_sketch_f16acc_noalloc(1, 0, A, 64, 1 << 18, 1 << 18, 512, 4, B, 1 << 18, 0)
    assert e.value.status == b.SK_ERR_UNSUPPORTED
    del A, B
    A = inputs.gaussian_torch(1000, 256, seed=1)
    B = torch.empty((40, 256), dtype=torch.float16, device=dev())
    with pytest.raises(b.SketchError) as e:
        b.sk_sketch_f16acc_noalloc(1, 0, A, 1000, 256, 256, 40, 4, B, 256, 0)
    assert e.value.status == b.SK_ERR_UNSUPPORTED
    B = torch.full((64, 64), 3.0, dtype=torch.float16, device=dev())
    b.sk_sketch_f16acc_noalloc(1, 0, None, 0, 64, 64, 64, 4, B, 64, 0)
    sync()
    assert int(torch.count_nonzero(B)) == 0
