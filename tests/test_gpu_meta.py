"""GPU parity: sk_meta_generate against the oracle's metadata, bit-exact
(FP16 sketching page §III-C)."""
import numpy as np
import pytest
import torch

from oracle import meta_ref
from sparse_sketching_amd import binding as b
from tests.gpuutil import dev, say, sync

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,d,zeta,seed,offset", [
    (4096, 64, 4, 1, 0),            # tiny configuration
    (4096, 64, 1, 1, 0),            # CountSketch
    (1 << 20, 512, 4, 3, 0),        # scale configuration
    (4097, 96, 3, 7, 0),            # ragged m, zeta not a power of two
    (1000, 64, 8, 2**40 + 5, 123),  # two key words, zeta = 8
    (777, 160, 5, 11, 2**32 - 3),   # row counter crosses 2^32
    (1, 16, 16, 0, 0),              # one row, zeta = d
    (333, 1024, 2, 9, 0),
])
def test_meta_bit_exact(m, d, zeta, seed, offset):
    say(f"meta m={m} d={d} zeta={zeta} seed={seed} offset={offset}")
    ri, v = b.meta(seed, m, d, zeta, row_offset=offset, device=dev())
    sync()
    ri_ref, v_ref = meta_ref(seed, m, d, zeta, row_offset=offset)
    assert np.array_equal(ri.cpu().numpy(), ri_ref)
    assert np.array_equal(v.cpu().numpy().view(np.uint32), v_ref.view(np.uint32))


def test_meta_unaligned_outputs():
    """Outputs not 16-byte aligned take the scalar-store path."""
    m, d, zeta = 1000, 64, 4
    d0 = dev()
    ri = torch.zeros(m * zeta + 1, dtype=torch.int32, device=d0)
    v = torch.zeros(m * zeta + 1, dtype=torch.float32, device=d0)
    b.sk_meta_generate(5, 0, m, d, zeta, ri.data_ptr() + 4, v.data_ptr() + 4)
    sync()
    ri_ref, v_ref = meta_ref(5, m, d, zeta)
    assert np.array_equal(ri.cpu().numpy()[1:], ri_ref) and ri[0].item() == 0
    assert np.array_equal(v.cpu().numpy()[1:], v_ref)


def test_meta_chunks_equal_whole():
    m, d, zeta = 50_000, 256, 4
    whole = b.meta(21, m, d, zeta, device=dev())[0]
    parts = [b.meta(21, n, d, zeta, row_offset=o, device=dev())[0]
             for o, n in [(0, 12_345), (12_345, 20_000), (32_345, m - 32_345)]]
    assert torch.equal(torch.cat(parts), whole)
