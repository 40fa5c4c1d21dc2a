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


def _draw_blockperm(count=40, seed=20261204):
    """(m, n, lda, d, M, kappa, s, wiring, seed) for BlockPerm-SJLT: shift
    wiring (kappa dividing M) and affine wiring, B_r = d / M from 1 to 32,
    s up to B_r (B_r a power of two when s > 1), ragged widths."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        shift = len(out) % 2 == 0
        M = int(g.choice((1, 2, 3, 4, 5, 6, 8, 12, 16, 32, 64, 128)))
        kappas = [k for k in range(1, min(M, 32) + 1) if (M % k == 0 or not shift)]
        kappa = int(g.choice(kappas))
        Br = int(g.choice((1, 2, 3, 4, 8, 16, 32)))
        d = M * Br
        if d > 4096:
            continue
        s = 1
        if Br > 1 and Br & (Br - 1) == 0 and g.random() < 0.4:
            s = int(g.choice([v for v in (2, 4, 8, Br) if v <= min(Br, 32)]))
        n = int(g.choice((1, 2, 3, 7, 16, 31, 32, 33, 64, 100, 128, 255, 256, 300, 512)))
        pad = int(g.choice((0, 0, 0, 1, 3)))
        top = max(1.0, min(65536.0, 2e7 / (n * kappa * s * M)))
        Bc = int(np.exp(g.uniform(0.0, np.log(top)))) if top > 1 else 1
        out.append(dict(m=M * max(Bc, 1), n=n, lda=n + pad, d=d, M=M, kappa=kappa, s=s,
                        wiring="shift" if shift else "affine", seed=int(g.integers(0, 1 << 62))))
    return out


BP_SWEEP = _draw_blockperm()


def _draw_qr(count=24, seed=20261205):
    """(d, n, pad) for the FP32 QR solve: n from 1 to 1024 and d from n to
    2048 (panel widths 32, 16 and 8 with every power-of-two tail), some
    with a padded row stride."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(count):
        n = int(np.exp(g.uniform(0.0, np.log(1024.0)))) if i % 2 else int(g.integers(256, 1025))
        extra = int(np.exp(g.uniform(0.0, np.log(2049.0 - n)))) - 1
        d = n + extra if i % 3 else int(g.integers(max(n, 1506), 2049))   # 8-column panels
        out.append(dict(d=d, n=n, pad=int(g.choice((0, 0, 0, 5, 16)))))
    return out


QR_SWEEP = _draw_qr()
