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
  from fp64 on the host.
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


def sketch_matrix(row_idx, val, m, d, zeta):
    """S as a d x m sparse matrix (fp64 entries equal to the stored fp32)."""
    cols = np.repeat(np.arange(m, dtype=np.int64), zeta)
    return sp.csr_matrix((val.astype(np.float64), (row_idx.astype(np.int64), cols)),
                         shape=(d, m))


def dense_S(row_idx, val, m, d, zeta):
    """Dense S built entry by entry (tiny inputs only)."""
    S = np.zeros((d, m), dtype=np.float64)
    for i in range(m):
        for t in range(zeta):
            e = i * zeta + t
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
    r = row_idx[e0:e1].astype(np.int64)
    order = np.argsort(r, kind="stable")          # by bucket, then entry
    counts = np.bincount(r, minlength=d)
    starts = np.concatenate(([0], np.cumsum(counts)[:-1]))
    buckets = np.arange(d)
    for k in range(int(counts.max())):
        act = buckets[counts > k]
        sel = e[order[starts[act] + k]]
        B[act] = rn_f16_add(B[act], _f16_contrib(A, val, zeta, sel))
    return B


def sketch_f16_rn_emul(A, row_idx, val, d, zeta, chunk_rows=None):
    """FP16-accumulated sketch with per-contribution RN conversion.

    chunk_rows=None: every output entry adds its contributions one at a
    time in ascending (i, t) order, the order of one atomic per
    contribution applied row by row.
    chunk_rows=R: each run of R input rows is accumulated that way into its
    own FP16 partial starting from +0, and the partials are then added in
    FP16 in chunk order.  Both orders are valid instances of "accumulate
    the RN contributions with FP16 RN additions"; atomics fix no order.
    """
    m = A.shape[0]
    if chunk_rows is None or chunk_rows >= m:
        return _accumulate_flat(A, row_idx, val, d, zeta, 0, m * zeta)
    B = np.zeros((d, A.shape[1]), dtype=np.float16)
    for r0 in range(0, m, chunk_rows):
        r1 = min(m, r0 + chunk_rows)
        P = _accumulate_flat(A, row_idx, val, d, zeta, r0 * zeta, r1 * zeta)
        B = rn_f16_add(B, P)
    return B
