"""The binding's helpers launched on a stream that is not the current one.

The helpers allocate outputs and workspaces with torch on the current
stream and enqueue the library's kernels on the caller's stream; they mark
those tensors as in use on the launch stream, so the caching allocator does
not hand the memory to other work while the kernels may still touch it.
Here the side stream is held busy (a bounded spin kernel) while the current
stream allocates blocks of the same sizes and fills them: without that
marking the fills would land in the pending calls' workspaces.  Every result
must equal the same call made on the current stream, bit for bit (integer
inputs keep the unordered paths exact)."""
import numpy as np
import pytest
import torch

from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000            # about 10 ms of one spinning wavefront


def churn(tensors):
    """Allocate and fill blocks of the helpers' sizes on the current stream."""
    junk = [torch.empty_like(t).fill_(3) if t.dtype != torch.uint8 else
            torch.full_like(t, 0xAB) for t in tensors]
    return junk


def run_on_side(call):
    """call(stream) on a busy side stream while the current stream churns;
    returns call's result after both streams finish."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN_CYCLES)          # the side stream's work is still pending
    out = call(side)
    keep = churn([o for o in (out if isinstance(out, tuple) else (out,))] + [
        torch.empty(64 << 20, dtype=torch.uint8, device=dev())])
    side.synchronize()
    sync()
    del keep
    return out


def test_sketch_fused_on_side_stream():
    m, n, d, zeta, seed = 40000, 256, 512, 4, 3
    A = to_dev(inputs.integer_matrix(m, n, -2, 2, seed=4))
    for precision in ("f16acc", "f32"):
        say(f"side stream: sketch_fused {precision}")
        ref = b.sketch_fused(A, d, zeta, seed, precision)
        sync()
        got = run_on_side(lambda s: b.sketch_fused(A, d, zeta, seed, precision, stream=s))
        assert torch.equal(got, ref), precision


def test_apply_on_side_stream():
    m, n, d, zeta, seed = 30000, 128, 256, 4, 5
    A = to_dev(inputs.integer_matrix(m, n, -1, 1, seed=6))
    ri, v = b.meta(seed, m, d, zeta, device=dev())
    for precision in ("f16acc", "f32"):
        for flags in (b.SK_VARIANT_REG, b.SK_VARIANT_LDS):
            say(f"side stream: apply {precision} flags={flags}")
            ref = b.apply(A, ri, v, zeta, d, precision, flags=flags, ws=True)
            sync()
            got = run_on_side(lambda s: b.apply(A, ri, v, zeta, d, precision, flags=flags,
                                                ws=True, stream=s))
            assert torch.equal(got, ref), (precision, flags)


def test_blockperm_and_qr_on_side_stream():
    m, n, d, M, kappa, seed = 1 << 15, 64, 256, 16, 4, 7
    A = to_dev(inputs.integer_matrix(m, n, -1, 1, seed=8))
    say("side stream: blockperm (register kernel, workspace)")
    ref = b.blockperm(A, d, M, kappa, seed)
    sync()
    got = run_on_side(lambda s: b.blockperm(A, d, M, kappa, seed, stream=s))
    assert torch.equal(got, ref)
    say("side stream: lstsq_qr")
    g = np.random.default_rng(9)
    SA = to_dev(g.standard_normal((512, 256)).astype(np.float32))
    Sb = to_dev(g.standard_normal(512).astype(np.float32))
    ref = b.lstsq_qr(SA, Sb)
    sync()
    got = run_on_side(lambda s: b.lstsq_qr(SA, Sb, stream=s))
    assert torch.equal(got, ref)
