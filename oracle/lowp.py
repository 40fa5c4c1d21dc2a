"""Conversion variants of the reduced-precision sketch.  TEST INFRASTRUCTURE ONLY.

Follows "On the Robustness of Sparse Randomized Sketching to FP16 Rounding
on GPUs":

* §III-D: the contribution (the FP32 product a*val) is converted to the
  accumulation format by one of several rules and then fed to the same
  packed nearest-even accumulation.  Stochastic rounding (SR) picks one of
  the two neighbouring FP16 values l <= q <= v, the upper one with
  probability about (q - l)/(v - l), and leaves a representable q
  unchanged; the page's implementation draws finitely many random bits, so
  it calls it stochastic conversion.
* §V-E: a BF16 variant (8-bit exponent, 8-bit significand) stays finite
  over the whole rescaling range.

Readings where the page is silent (each listed in the design notes):
* SR draws one 32-bit word r per (global row g, stack block t, column c):
  word c mod 4 of Philox-4x32-10 with counter (g mod 2^32, g >> 32,
  c div 4, 3 + 4t) and key (sr_seed mod 2^32, sr_seed >> 32).  The fourth
  counter word keeps these draws apart from the metadata (0 mod 4) and
  BlockPerm (1, 2) streams.
* SR works on magnitudes: with l <= |q| < v the FP16 neighbours of |q|,
  frac = (|q| - l)/(v - l), the magnitude rounds up to v exactly when
  r < frac * 2^32, and the sign of q is kept.  This is the page's rule with
  probability ceil(frac * 2^32) / 2^32.
* Above the largest finite FP16 value 65504 the next value is taken as
  2^16 and means overflow: |q| in (65504, 65536) becomes +-inf with
  probability frac, larger |q| always.
* BF16 conversion and addition are nearest-even on the 8-bit significand
  (the format's IEEE-style rounding), with subnormals kept.
"""
import numpy as np

from .philox import philox4x32_10
from .sparsestack import rn_f16_add

F16_MAX = 65504.0
F16_NEXT_PAST_MAX = 65536.0


def sr_words(sr_seed, g, t, c):
    """The 32-bit SR draw for global row g, stack block t, column c
    (broadcastable integer arrays); uint32 array."""
    g, t, c = np.broadcast_arrays(np.asarray(g, dtype=np.uint64), np.asarray(t, dtype=np.uint64),
                                  np.asarray(c, dtype=np.uint64))
    w = philox4x32_10(g & np.uint64(0xFFFFFFFF), g >> np.uint64(32), c >> np.uint64(2),
                      np.uint64(3) + np.uint64(4) * t, int(sr_seed) & 0xFFFFFFFF,
                      (int(sr_seed) >> 32) & 0xFFFFFFFF)
    j = (c & np.uint64(3)).astype(np.int64)
    return np.choose(j, w).astype(np.uint32)


def f16_neighbours(z):
    """For magnitudes z >= 0 (float64 array of FP32 values): (l, v), the
    largest FP16 value <= z and the smallest FP16 value > l (2^16 past the
    largest finite value).  Where z is representable l == z."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        x = z.astype(np.float16)                    # nearest-even, may be inf
    xf = x.astype(np.float64)
    below = xf <= z                                 # x is the lower neighbour
    l16 = np.where(below, x, np.nextafter(x, np.float16(0)))
    l16 = np.where(np.isinf(x), np.float16(F16_MAX), l16)
    lf = l16.astype(np.float64)
    with np.errstate(over="ignore"):
        v16 = np.nextafter(l16, np.float16(np.inf))
    vf = np.where(lf == F16_MAX, F16_NEXT_PAST_MAX, v16.astype(np.float64))
    return lf, vf


def sr_f16(q, r):
    """Stochastic conversion of FP32 values q to FP16 with the 32-bit draws
    r (same shape); float16 array."""
    q = np.asarray(q, dtype=np.float32)
    z = np.abs(q).astype(np.float64)
    l, v = f16_neighbours(z)
    frac = np.where(v > l, (z - l) / np.where(v > l, v - l, 1.0), 0.0)
    up = np.asarray(r, dtype=np.float64) < frac * 4294967296.0
    mag = np.where(z == l, z, np.where(up, v, l))
    with np.errstate(over="ignore"):
        mag16 = np.where(mag >= F16_NEXT_PAST_MAX, np.inf, mag).astype(np.float16)
    return np.where(np.signbit(q), -mag16, mag16).astype(np.float16)


def rn_bf16(x):
    """Nearest-even conversion of FP32 values to BF16, returned as float32
    values whose low 16 bits are zero.  NaN stays NaN; values past the
    largest finite BF16 round to +-inf."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    rounded = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), np.float32(np.nan), out).astype(np.float32)


def rn_bf16_add(a, b):
    """BF16 addition with nearest-even rounding: the FP32 sum rounded once
    to BF16.  FP32 (p' = 24) satisfies p' >= 2p + 2 for BF16's p = 8, so the
    double rounding gives the correctly rounded sum (Figueroa, 1995)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return rn_bf16(np.asarray(a, np.float32) + np.asarray(b, np.float32))


def contributions(A, row_idx, val, zeta, e, fmt, conv, sr_seed=0, row_offset=0):
    """Converted contributions of metadata entries e (rows x n): the FP32
    product a*val (§III-A), then RN to FP16, SR to FP16, or RN to BF16."""
    e = np.asarray(e, dtype=np.int64)
    i = e // zeta
    q = A[i].astype(np.float32, copy=False) * val[e].astype(np.float32)[:, None]
    if fmt == "bf16":
        if conv != "rn":
            raise ValueError("BF16 takes nearest-even conversion only")
        return rn_bf16(q)
    if conv == "rn":
        with np.errstate(over="ignore"):
            return q.astype(np.float16)
    cols = np.arange(A.shape[1], dtype=np.int64)[None, :]
    g = (np.int64(row_offset) + i)[:, None]
    r = sr_words(sr_seed, g, (e % zeta)[:, None], cols)
    return sr_f16(q, r)


def _lowp_flat(A, row_idx, val, d, zeta, fmt, conv, sr_seed, row_offset, e0, e1):
    """Entries [e0, e1) accumulated from +0 in the format, each output entry
    adding its contributions one at a time in ascending entry order."""
    m, n = A.shape
    db = d // zeta
    e_all = np.arange(e0, e1, dtype=np.int64)
    r_all = row_idx[e0:e1].astype(np.int64)
    t_all = e_all % zeta
    keep = (r_all >= t_all * db) & (r_all < (t_all + 1) * db)
    e_all, r_all = e_all[keep], r_all[keep]
    out_t = np.float16 if fmt == "f16" else np.float32
    B = np.zeros((d, n), dtype=out_t)
    if e_all.size == 0:
        return B
    order = np.argsort(r_all, kind="stable")
    counts = np.bincount(r_all, minlength=d)
    starts = np.concatenate(([0], np.cumsum(counts)[:-1]))
    buckets = np.arange(d)
    for k in range(int(counts.max())):
        act = buckets[counts > k]
        sel = e_all[order[starts[act] + k]]
        c = contributions(A, row_idx, val, zeta, sel, fmt, conv, sr_seed, row_offset)
        B[act] = rn_f16_add(B[act], c) if fmt == "f16" else rn_bf16_add(B[act], c)
    return B


def sketch_lowp_emul(A, row_idx, val, d, zeta, fmt="f16", conv="rn", sr_seed=0, row_offset=0,
                     chunk_rows=None, combine="fmt", B0=None):
    """Reduced-precision sketch with per-contribution conversion and
    nearest-even accumulation in the same format.  Entries outside their own
    stack block contribute nothing.  Returns float16 (fmt "f16") or float32
    holding BF16 values (fmt "bf16").

    chunk_rows=None: every output entry adds its contributions one at a time
    in ascending (i, t) order starting from +0 (the order of one atomic per
    contribution applied row by row).
    chunk_rows=R: each run of R input rows is accumulated that way into its
    own partial starting from +0, and the partials are added in chunk order:
    with nearest-even additions in the format (combine="fmt", every
    addition in the format), or (combine="f32") summed in FP32 and the total
    rounded to the format once.  B0 (float16, or float32 holding BF16
    values): the sum starts from B0 instead of +0."""
    m = A.shape[0]
    if combine not in ("fmt", "f32"):
        raise ValueError("combine is 'fmt' or 'f32'")
    add = rn_f16_add if fmt == "f16" else rn_bf16_add
    out_t = np.float16 if fmt == "f16" else np.float32
    if chunk_rows is None:
        B = _lowp_flat(A, row_idx, val, d, zeta, fmt, conv, sr_seed, row_offset, 0, m * zeta)
        return B if B0 is None else add(np.asarray(B0, out_t), B).astype(out_t)
    parts = [_lowp_flat(A, row_idx, val, d, zeta, fmt, conv, sr_seed, row_offset, r0 * zeta,
                        min(m, r0 + chunk_rows) * zeta) for r0 in range(0, m, chunk_rows)]
    start = np.zeros((d, A.shape[1]), out_t) if B0 is None else np.asarray(B0, out_t)
    if combine == "fmt":
        B = start
        for P in parts:
            B = add(B, P).astype(out_t)
        return B
    acc = start.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        for P in parts:
            acc = acc + P.astype(np.float32)
        return acc.astype(np.float16) if fmt == "f16" else rn_bf16(acc)
