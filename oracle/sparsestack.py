"""SparseStack / CountSketch oracle.  TEST INFRASTRUCTURE ONLY.

Follows "On the Robustness of Sparse Randomized Sketching to FP16 Rounding
on GPUs":

* §I and §II-A: CountSketch sends each input row to one random output row
  with a random sign; SparseStack spreads each row over zeta independent
  CountSketch blocks.  S is d x m, A is m x n (m >> n), B = SA is d x n.
* §IV-A/§IV-B: the scale is 1/sqrt(zeta) (zeta=4 gives exactly 1/2; each
  entry of A appears zeta times with squared scale 1/zeta).
* §III-C: the routing row index and signed value of every (row, block)
  pair come from a coupled Philox kernel and are stored as contiguous
  int32 and FP32 arrays of length m*zeta.
* §III-B and §III-D: the mixed-precision variant forms the signed product
  in FP32, converts each contribution to FP16 with round-to-nearest-even,
  and accumulates it with FP16 RN additions.

Readings where the page is silent (each listed in the design notes):
* block t occupies output rows [t*d/zeta, (t+1)*d/zeta) ("stacked");
* metadata entry (i, t) sits at index i*zeta + t;
* one Philox-4x32-10 block per (global row, group of four stack blocks):
  counter = (g mod 2^32, g >> 32, t div 4, 0), key = (seed mod 2^32,
  seed >> 32); stack block t takes output word w = w_{t mod 4}; the bucket
  is the multiply-high floor(w * (d/zeta) / 2^32) and the sign is negative
  when bit 0 of w is set ("coupled": one word routes and signs);
* the stored value is sign * float32(1/sqrt(zeta)), the scale rounded once
  from fp64 on the host;
* entry i*zeta + t belongs to stack block t, a CountSketch of the block's
  d/zeta rows: an entry whose row lies outside [t*d/zeta, (t+1)*d/zeta)
  is not an entry of a SparseStack S and contributes nothing, in every
  function here (the metadata this oracle generates never holds one).
"""
import numpy as np
import scipy.sparse as sp

from .philox import philox4x32_10


def scale_f32(zeta):
    """float32(1/sqrt(zeta)) rounded once from fp64 (§IV-A scale)."""
    return np.float32(1.0 / np.sqrt(np.float64(zeta)))


def meta_ref(seed, m, d, zeta, row_offset=0):
    """Metadata (row_idx int32[m*zeta], val float32[m*zeta]) for rows
    row_offset .. row_offset+m-1 of S's column space (§III-C).

    The counter is the global row index, so the metadata of a row chunk
    equals the matching slice of the whole matrix's metadata.
    """
    if d % zeta:
        raise ValueError("d must be a multiple of zeta")
    db = d // zeta
    g = np.arange(m, dtype=np.uint64) + np.uint64(row_offset)
    seed = int(seed)
    k0, k1 = seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF
    row_idx = np.empty((m, zeta), dtype=np.int32)
    val = np.empty((m, zeta), dtype=np.float32)
    c = scale_f32(zeta)
    for grp in range((zeta + 3) // 4):
        words = philox4x32_10(g & np.uint64(0xFFFFFFFF), g >> np.uint64(32),
                              np.uint64(grp), np.uint64(0), k0, k1)
        for j in range(4):
            t = 4 * grp + j
            if t >= zeta:
                break
            w = words[j].astype(np.uint64)
            bucket = (w * np.uint64(db)) >> np.uint64(32)
            row_idx[:, t] = (t * db + bucket).astype(np.int32)
            neg = (w & np.uint64(1)).astype(bool)
            val[:, t] = np.where(neg, -c, c)
    return row_idx.reshape(-1), val.reshape(-1)


def in_block(row_idx, d, zeta):
    """Mask of metadata entries whose row lies in their own stack block
    (entry i*zeta + t in rows [t*d/zeta, (t+1)*d/zeta))."""
    db = d // zeta
    r = np.asarray(row_idx, dtype=np.int64)
    t = np.arange(r.size, dtype=np.int64) % zeta
    return (r >= t * db) & (r < (t + 1) * db)


def sketch_matrix(row_idx, val, m, d, zeta):
    """S as a d x m sparse matrix (fp64 entries equal to the stored fp32);
    entries outside their block are left out."""
    cols = np.repeat(np.arange(m, dtype=np.int64), zeta)
    keep = in_block(row_idx, d, zeta)
    return sp.csr_matrix((val.astype(np.float64)[keep],
                          (row_idx.astype(np.int64)[keep], cols[keep])), shape=(d, m))


def dense_S(row_idx, val, m, d, zeta):
    """Dense S built entry by entry (tiny inputs only)."""
    db = d // zeta
    S = np.zeros((d, m), dtype=np.float64)
    for i in range(m):
        for t in range(zeta):
            e = i * zeta + t
            if t * db <= row_idx[e] < (t + 1) * db:
                S[row_idx[e], i] += float(val[e])
    return S


def sketch_f64(A, row_idx, val, d, zeta, chunk_rows=1 << 17):
    """B = S A in fp64, summing row chunks of A (S is a fixed linear map)."""
    m, n = A.shape
    B = np.zeros((d, n), dtype=np.float64)
    for r0 in range(0, m, chunk_rows):
        r1 = min(m, r0 + chunk_rows)
        e0, e1 = r0 * zeta, r1 * zeta
        S = sketch_matrix(row_idx[e0:e1], val[e0:e1], r1 - r0, d, zeta)
        B += S @ np.asarray(A[r0:r1], dtype=np.float64)
    return B


def countsketch_f64(A, bucket, sign, d):
    """CountSketch (§I): row i of A is added, times sign[i], to row bucket[i]."""
    B = np.zeros((d, A.shape[1]), dtype=np.float64)
    for i in range(A.shape[0]):
        B[bucket[i]] += float(sign[i]) * np.asarray(A[i], dtype=np.float64)
    return B


def rn_f16_add(a16, b16):
    """FP16 addition with round-to-nearest-even.

    The sum of two binary16 values is formed in binary32 and rounded once
    to binary16.  binary32 has p'=24 >= 2p+2 = 24 for binary16's p=11, so
    this double rounding gives the correctly rounded sum (Figueroa, 1995).
    """
    with np.errstate(over="ignore", invalid="ignore"):
        return (a16.astype(np.float32) + b16.astype(np.float32)).astype(np.float16)


def _f16_contrib(A, val, zeta, e):
    """RN-to-FP16 of the FP32 signed products for metadata entries e
    (§III-B: FP32 product, nearest-even conversion)."""
    i = e // zeta
    q = A[i].astype(np.float32, copy=False) * val[e].astype(np.float32)[:, None]
    with np.errstate(over="ignore"):
        return q.astype(np.float16)


def _accumulate_flat(A, row_idx, val, d, zeta, e0, e1):
    """FP16 sketch of entries [e0, e1), each output entry accumulating its
    contributions in ascending entry order starting from +0."""
    n = A.shape[1]
    B = np.zeros((d, n), dtype=np.float16)
    if e1 <= e0:
        return B
    e = np.arange(e0, e1, dtype=np.int64)
    # (entry i*zeta + t: a range starting at a whole row has the same block
    # index t at each position as the full array)
    assert e0 % zeta == 0
    keep = in_block(row_idx[e0:e1], d, zeta)
    e = e[keep]
    if e.size == 0:
        return B
    r = row_idx[e].astype(np.int64)
    order = np.argsort(r, kind="stable")          # by bucket, then entry
    counts = np.bincount(r, minlength=d)
    starts = np.concatenate(([0], np.cumsum(counts)[:-1]))
    buckets = np.arange(d)
    for k in range(int(counts.max())):
        act = buckets[counts > k]
        sel = e[order[starts[act] + k]]
        B[act] = rn_f16_add(B[act], _f16_contrib(A, val, zeta, sel))
    return B


def sketch_f16_rn_emul(A, row_idx, val, d, zeta, chunk_rows=None, combine="f16", B0=None,
                       groups=None):
    """FP16-accumulated sketch with per-contribution RN conversion.

    chunk_rows=None: every output entry adds its contributions one at a
    time in ascending (i, t) order, the order of one atomic per
    contribution applied row by row.
    chunk_rows=R: each run of R input rows is accumulated that way into its
    own FP16 partial starting from +0, and the partials are then added in
    chunk order.  combine="f16" adds them with FP16 RN additions: both
    orders are then valid instances of "accumulate the RN contributions with
    FP16 RN additions" (atomics fix no order).  combine="f32" instead sums
    the FP16 partials in FP32 in chunk order and rounds the total to FP16
    once: not the page's arithmetic, but a combine step a two-level
    implementation may take (it is more accurate than FP16 additions).
    B0 (float16 d x n): the sum starts from B0 instead of +0 (a sketch
    accumulated onto an existing one); with combine="f32" B0 is the first
    term of the FP32 sum.
    groups=G (with chunk_rows): the P chunk partials are combined in G
    contiguous groups, group w holding chunks [w*P//G, (w+1)*P//G); each
    group is summed from +0 in chunk order, and the non-empty group sums are
    added in group order onto B0 or +0 (FP16 RN additions throughout, or,
    with combine="f32", FP32 additions and one rounding of the total).
    This is one more fixed order of the same FP16 RN additions; groups=None
    adds the chunk partials one after another.
    """
    m = A.shape[0]
    if combine not in ("f16", "f32"):
        raise ValueError("combine is 'f16' or 'f32'")
    if chunk_rows is None:
        B = _accumulate_flat(A, row_idx, val, d, zeta, 0, m * zeta)
        return B if B0 is None else rn_f16_add(np.asarray(B0, np.float16), B)
    parts = [_accumulate_flat(A, row_idx, val, d, zeta, r0 * zeta, min(m, r0 + chunk_rows) * zeta)
             for r0 in range(0, m, chunk_rows)]
    start = np.zeros((d, A.shape[1]), dtype=np.float16) if B0 is None else \
        np.asarray(B0, dtype=np.float16)
    if groups is not None:
        P = len(parts)
        spans = [(w * P // groups, (w + 1) * P // groups) for w in range(groups)]
        if combine == "f16":
            B = start
            for lo, hi in spans:
                if hi > lo:
                    q = np.zeros_like(start)
                    for part in parts[lo:hi]:
                        q = rn_f16_add(q, part)
                    B = rn_f16_add(B, q)
            return B
        acc = start.astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            for lo, hi in spans:
                if hi > lo:
                    q = np.zeros(start.shape, dtype=np.float32)
                    for part in parts[lo:hi]:
                        q = q + part.astype(np.float32)
                    acc = acc + q
            return acc.astype(np.float16)
    if combine == "f16":
        B = start
        for P in parts:
            B = rn_f16_add(B, P)
        return B
    acc = start.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        for P in parts:
            acc = acc + P.astype(np.float32)
        return acc.astype(np.float16)


def f16_zero_subnormal_counts(q):
    """For FP32 magnitudes q >= 0: (how many nonzero q convert to 0, how
    many to a nonzero subnormal, how many are nonzero) under nearest-even
    conversion to binary16.  With h = 2^-24 the subnormal spacing: (0, h/2]
    goes to 0 (the tie h/2 to the even 0), (h/2, 2^-14 - h/2) to the
    subnormals, and from 2^-14 - h/2 up (the tie there to the even 2^-14)
    the result is normal."""
    q = np.asarray(q, dtype=np.float32)
    half_h = np.float32(2.0**-25)
    top = np.float32(2.0**-14 - 2.0**-25)
    nz = int(np.count_nonzero(q))
    zero = int(np.count_nonzero((q > 0) & (q <= half_h)))
    sub = int(np.count_nonzero((q > half_h) & (q < top)))
    return zero, sub, nz


def f16_erasures(A, row_idx, val, d, zeta):
    """Counts of the FP16 conversion's losses at the bottom of the range
    (FP16 page §IV-E, §V-E: nearest-even conversion sends every contribution
    of magnitude at most h/2 = 2^-25 to zero, and keeps subnormals above it).

    Returns (erased, subnormal, total): contributions q = fl32(a*val) with
    q != 0 whose RN-to-FP16 conversion is zero, those that convert to a
    nonzero subnormal (0 < |RN(q)| < 2^-14), and the nonzero contributions,
    over the in-block metadata entries."""
    mask = in_block(row_idx, d, zeta)
    mag = np.abs(np.asarray(val, dtype=np.float32))
    if mask.all() and mag.size and (mag == mag[0]).all():
        # every entry of a row scales the row by the same magnitude c, and
        # the sign does not change whether a product converts to zero or to
        # a subnormal: count the row's products once and take zeta of them
        c = mag[0]
        m = A.shape[0]
        erased = sub = total = 0
        for r0 in range(0, m, 1 << 18):
            q = np.abs(A[r0:r0 + (1 << 18)].astype(np.float32, copy=False)) * c
            z, s_, t = f16_zero_subnormal_counts(q)
            erased, sub, total = erased + z, sub + s_, total + t
        return zeta * erased, zeta * sub, zeta * total
    keep = np.nonzero(mask)[0]
    erased = sub = total = 0
    for e0 in range(0, keep.size, 1 << 16):
        e = keep[e0:e0 + (1 << 16)]
        q = A[e // zeta].astype(np.float32, copy=False) * val[e].astype(np.float32)[:, None]
        with np.errstate(over="ignore"):
            c = q.astype(np.float16)
        nz = q != 0
        total += int(nz.sum())
        erased += int((nz & (c == 0)).sum())
        ac = np.abs(c.astype(np.float64))
        sub += int(((ac > 0) & (ac < 2.0**-14)).sum())
    return erased, sub, total
