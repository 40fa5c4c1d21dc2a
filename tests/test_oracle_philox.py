"""Pins for the oracle's Philox (Salmon et al., SC'11) against two library
implementations it shares no code with: NumPy's Philox-4x64-10 bit
generator (pins the round structure, key schedule and round count) and
rocRAND's public host-callable Philox-4x32-10 engine (pins the 32-bit
constants and the counter/key word order)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle.philox import PHILOX4x32, PHILOX4x64, philox4x32_10, philox_scalar

ROCRAND_HDR = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.mark.parametrize("key,ctr", [((0, 0), (0, 0, 0, 0)),
                                     ((1, 2), (5, 0, 0, 0)),
                                     ((2**64 - 1, 12345), (2**64 - 2, 7, 2**63, 99)),
                                     ((0xDEADBEEF, 0xCAFEF00D), (1, 2, 3, 4))])
def test_philox4x64_matches_numpy(key, ctr):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(ctr, dtype=np.uint64))
    raw = bg.random_raw(8)
    # NumPy increments the 256-bit counter before each block.
    c = sum(int(x) << (64 * i) for i, x in enumerate(ctr))
    for blk in range(2):
        cc = (c + 1 + blk) % (1 << 256)
        words = [(cc >> (64 * i)) & (2**64 - 1) for i in range(4)]
        out = philox_scalar(words, key, PHILOX4x64)
        assert [int(x) for x in raw[4 * blk:4 * blk + 4]] == list(out)


def test_vectorised_matches_scalar():
    g = np.random.default_rng(7)
    c = g.integers(0, 2**32, size=(4, 200), dtype=np.uint64)
    for k0, k1 in [(0, 0), (0xFFFFFFFF, 1), (123456789, 987654321)]:
        out = philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
        for j in range(200):
            ref = philox_scalar([c[0, j], c[1, j], c[2, j], c[3, j]], (k0, k1), PHILOX4x32)
            assert tuple(int(o[j]) for o in out) == ref


def _rocrand_tool(tmp):
    src = os.path.join(tmp, "rr.cpp")
    exe = os.path.join(tmp, "rr")
    with open(src, "w") as f:
        f.write(r'''
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  unsigned long long seed, sub, g;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &g) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ULL * g);
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
''')
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    src, "-o", exe], check=True, capture_output=True)
    return exe


@pytest.mark.skipif(not (os.path.exists(ROCRAND_HDR) and shutil.which("g++")),
                    reason="rocRAND header or g++ not available")
def test_philox4x32_matches_rocrand():
    # rocRAND's engine(seed, subsequence, offset=4g) evaluates the block with
    # counter (g lo, g hi, subsequence lo, subsequence hi) and key (seed lo, seed hi).
    g = np.random.default_rng(3)
    cases = [(0, 0, 0), (1, 0, 5), (2**64 - 1, 3, 2**40 + 17)]
    cases += [(int(a), int(b), int(c)) for a, b, c in zip(
        g.integers(0, 2**63, 60, dtype=np.uint64), g.integers(0, 2**31, 60),
        g.integers(0, 2**50, 60, dtype=np.uint64))]
    with tempfile.TemporaryDirectory() as tmp:
        exe = _rocrand_tool(tmp)
        inp = "".join(f"{s} {t} {r}\n" for s, t, r in cases)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    lines = out.strip().split("\n")
    assert len(lines) == len(cases)
    for (seed, sub, gg), line in zip(cases, lines):
        ref = tuple(int(x) for x in line.split())
        mine = philox4x32_10(gg & 0xFFFFFFFF, gg >> 32, sub & 0xFFFFFFFF, sub >> 32,
                             seed & 0xFFFFFFFF, seed >> 32)
        assert tuple(int(x) for x in mine) == ref


def test_philox_output_statistics():
    # Uniform bytes over a counter sweep: chi-square on the 256 byte values.
    w = philox4x32_10(np.arange(1 << 16), 0, 0, 0, 42, 0)
    b = np.concatenate([x.view(np.uint8) for x in w])
    cnt = np.bincount(b, minlength=256)
    exp = b.size / 256
    chi2 = float(((cnt - exp) ** 2 / exp).sum())
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)
