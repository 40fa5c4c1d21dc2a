"""Philox counter-based generator (oracle side).  TEST INFRASTRUCTURE ONLY.

The FP16 sketching page (§III-C) says the routing and sign metadata come
from "a coupled Philox kernel".  The page does not print Philox itself; it
is the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11).  It is written here from that
published definition:

* a Philox-4xW block maps a counter of four W-bit words and a key of two
  W-bit words to four W-bit words;
* one round multiplies counter words 0 and 2 by the round multipliers
  M0 and M1, keeping both halves of each 2W-bit product, and outputs
  (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
* between rounds the key is bumped by the Weyl constants (W0, W1);
* ten rounds are applied (Philox-4xW-10).

Two implementations live here, written independently of each other:
``philox_scalar`` works on Python integers for any word size (used to pin
the round structure against NumPy's own Philox-4x64-10), and
``philox4x32_10`` is a vectorised NumPy version for W=32, pinned against
``philox_scalar`` and against rocRAND's public host-callable engine.
"""
import numpy as np

# (M0, M1, W0, W1, word bits) as published with the algorithm.
PHILOX4x32 = (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85, 32)
PHILOX4x64 = (0xD2E7470EE14C6C93, 0xCA5A826395121157,
              0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B, 64)


def philox_scalar(counter, key, params=PHILOX4x32, rounds=10):
    """One Philox-4xW block on Python ints.  counter: 4 words, key: 2 words."""
    m0, m1, w0, w1, bits = params
    mask = (1 << bits) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in counter)
    k0, k1 = (int(x) & mask for x in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * c0
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> bits) ^ c1 ^ k0, p1 & mask,
                          (p0 >> bits) ^ c3 ^ k1, p0 & mask)
    return (c0, c1, c2, c3)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox-4x32-10.

    All arguments are broadcastable integer arrays (or scalars) holding
    32-bit values; the result is four uint32 arrays.  Products are formed
    exactly in uint64 (both factors are below 2**32).
    """
    m0, m1, w0, w1, _ = PHILOX4x32
    lo32 = np.uint64(0xFFFFFFFF)
    sh = np.uint64(32)
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & lo32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + w0) & 0xFFFFFFFF)
            k1 = np.uint64((int(k1) + w1) & 0xFFFFFFFF)
        p0 = np.uint64(m0) * c0
        p1 = np.uint64(m1) * c2
        c0, c1, c2, c3 = ((p1 >> sh) ^ c1 ^ k0, p1 & lo32,
                          (p0 >> sh) ^ c3 ^ k1, p0 & lo32)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))
