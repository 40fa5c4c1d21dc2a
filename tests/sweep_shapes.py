"""Seeded random sketch shapes shared by the host plan replays and the GPU
sweep: sizes, column counts, stack sizes, padded strides and row offsets
drawn across the plans' branches (register kernel, owner kernel with one
or two barriers, the metadata + LDS fallback), each small enough for the
oracle's FP16 emulation to finish in about a second."""
import numpy as np

_D = (16, 32, 40, 48, 64, 96, 128, 128, 192, 256, 256, 384, 512, 512, 768, 1024, 1024, 2048)
_N32 = (1, 2, 3, 4, 6, 8, 12, 16, 24, 31, 32, 48, 64, 96, 128, 200, 256)
_N16 = (2, 4, 6, 8, 12, 16, 24, 32, 48, 62, 64, 96, 128, 130, 256)
_ZETA = (1, 2, 3, 4, 5, 8, 16)


def _draw(count=80, seed=20261203):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        f16 = len(out) % 2 == 0
        zeta = int(g.choice(_ZETA))
        ds = [d for d in _D if d % zeta == 0 and d >= zeta]
        d = int(g.choice(ds))
        n = int(g.choice(_N16 if f16 else _N32))
        # (FP16 rows are read as column pairs: lda even)
        pad = int(g.choice((0, 0, 0, 0, 0, 2, 4, 8) if f16 else (0, 0, 0, 0, 0, 1, 2, 4, 8)))
        top = min(300000.0, 2e7 / (n * zeta))
        lo = 0.0 if g.random() < 0.3 else np.log(min(2000.0, top))
        m = int(np.exp(g.uniform(lo, np.log(top))))
        row_offset = 0 if g.random() < 0.5 else int(g.integers(0, 1 << 40))
        out.append(dict(precision="f16acc" if f16 else "f32", m=max(m, 1), n=n, d=d, zeta=zeta,
                        pad=pad, row_offset=row_offset, seed=int(g.integers(0, 1 << 62))))
    return out


SWEEP = _draw()
