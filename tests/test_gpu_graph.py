"""The entry points under HIP graph capture: the library allocates nothing,
synchronizes nothing and records no memset (B is initialized by kernels),
so a captured call replays to the eager result.  Each path is captured once
and replayed three times with eager work on the same buffers in between;
every replay must equal the eager result bit for bit (integer inputs keep
even the unordered LDS path exact)."""
import numpy as np
import pytest
import torch

from sparse_sketching_amd import binding as b
from sparse_sketching_amd import inputs
from tests.gpuutil import dev, say, sync, to_dev

pytestmark = pytest.mark.gpu


def replay_matches_eager(call, out):
    """call() writes out on the current stream; capture it, then replay."""
    call()
    sync()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                  # warm-up on a side stream, as capture needs
    torch.cuda.current_stream().wait_stream(side)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    sync()
    for i in range(3):
        out.fill_(7.0)                          # eager work between replays
        if i == 1:
            call()                              # and an eager call of the same path
        sync()
        g.replay()
        sync()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
def test_fused_sketch_in_graph(precision):
    m, n, d, zeta = 20000, 256, 512, 4
    A = to_dev(inputs.integer_matrix(m, n, -1, 1, seed=1))
    dt = torch.float16 if precision == "f16acc" else torch.float32
    B = torch.empty((d, n), dtype=dt, device=dev())
    ws = b.sketch_workspace(A, d, zeta, precision)
    fn = b.sk_sketch_f16acc if precision == "f16acc" else b.sk_sketch_f32
    say(f"graph fused {precision}")
    replay_matches_eager(lambda: fn(5, 0, A, m, n, n, d, zeta, B, n, 0, ws, 0,
                                    torch.cuda.current_stream().cuda_stream), B)


@pytest.mark.parametrize("precision", ["f32", "f16acc"])
@pytest.mark.parametrize("flags,with_ws", [(b.SK_VARIANT_LDS, True), (b.SK_VARIANT_LDS, False),
                                           (b.SK_VARIANT_REG, True)])
def test_apply_in_graph(precision, flags, with_ws):
    m, n, d, zeta = 9000, 128, 256, 4
    A = to_dev(inputs.integer_matrix(m, n, -1, 1, seed=2))
    ri, v = b.meta(3, m, d, zeta, device=dev())
    dt = torch.float16 if precision == "f16acc" else torch.float32
    B = torch.empty((d, n), dtype=dt, device=dev())
    ws = b.workspace(A, d, zeta, precision, flags) if with_ws else None
    fn = b.sk_apply_f16acc_ws if precision == "f16acc" else b.sk_apply_f32_ws
    say(f"graph apply {precision} flags={flags} ws={with_ws}")
    replay_matches_eager(lambda: fn(A, m, n, n, ri, v, zeta, B, d, n, flags, ws, 0,
                                    torch.cuda.current_stream().cuda_stream), B)


@pytest.mark.parametrize("wiring", [b.SK_WIRING_SHIFT, b.SK_WIRING_AFFINE])
def test_blockperm_in_graph(wiring):
    m, n, d, M, kappa = 16 * 2048, 264, 512, 16, 4
    A = to_dev(inputs.integer_matrix(m, n, -4, 4, seed=3))
    Y = torch.empty((d, n), dtype=torch.float32, device=dev())
    nb = b.sk_blockperm_workspace_size(m, n, d, M, kappa, 1, wiring)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev())
    say(f"graph blockperm wiring={wiring}")
    replay_matches_eager(lambda: b.sk_apply_blockperm_ex(
        A, m, n, n, d, M, kappa, 1, wiring, 7, Y, n, 0, ws, nb,
        torch.cuda.current_stream().cuda_stream), Y)
    assert np.isfinite(Y.cpu().numpy()).all()
