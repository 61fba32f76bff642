"""Philox counter-based random numbers, written from the published definition.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this module; it shares no code with the
HIP library.

The pages name dropout as one of the elementwise steps a training forward
pass applies to the probabilities before the product with V (zerotofrontier
"Efficient attention: memory-bound", section "Real code moves even more") and
give no random-number contract. The one taken here is Philox-4x32-10 from
Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11), section 3.2 (the Philox S-P network) and Table 2 (its constants):

  * state: a counter of four W-bit words (c0, c1, c2, c3) and a key of two
    (k0, k1);
  * one round: multiply c0 by M0 and c2 by M1, each giving a 2W-bit product
    split into (hi, lo); the new counter is
        (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0));
  * the key is bumped by the Weyl constants (k0 + W0, k1 + W1) mod 2^W
    between rounds, so round r (from 0) uses k + r (W0, W1);
  * the output is the counter after R rounds.

`philox_ref` is the scalar version in Python integers for any word size (the
W = 64 instance is checked against numpy's Philox bit generator, W = 32
against the published known-answer vectors); `philox4x32_10` is the
vectorised 32-bit version the dropout mask uses (checked against the scalar
one).
"""
from __future__ import annotations

import numpy as np

# Multipliers and Weyl key increments (the paper's Table 2 for W = 32 and 64).
CONSTANTS = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def philox_ref(counter, key, width: int = 32, rounds: int = 10):
    """Philox-4xW-R of one counter: four Python ints in [0, 2^W)."""
    cst = CONSTANTS[width]
    mask = (1 << width) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in counter)
    k0, k1 = (int(x) & mask for x in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + cst["W0"]) & mask
            k1 = (k1 + cst["W1"]) & mask
        p0 = cst["M0"] * c0
        p1 = cst["M1"] * c2
        hi0, lo0 = p0 >> width, p0 & mask
        hi1, lo1 = p1 >> width, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox-4x32-10 on arrays of counters (broadcast together), one key.

    Returns four uint32 arrays. Products of two 32-bit words are exact in
    uint64."""
    cst = CONSTANTS[32]
    m32 = np.uint64(0xFFFFFFFF)
    shp = np.broadcast(np.asarray(c0), np.asarray(c1), np.asarray(c2), np.asarray(c3)).shape
    x0, x1, x2, x3 = (np.broadcast_to(np.asarray(c, dtype=np.uint64) & m32, shp).copy()
                      for c in (c0, c1, c2, c3))
    key0, key1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    M0, M1 = np.uint64(cst["M0"]), np.uint64(cst["M1"])
    for r in range(10):
        if r > 0:
            key0 = (key0 + cst["W0"]) & 0xFFFFFFFF
            key1 = (key1 + cst["W1"]) & 0xFFFFFFFF
        p0 = M0 * x0
        p1 = M1 * x2
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ np.uint64(key0), p1 & m32,
                          (p0 >> np.uint64(32)) ^ x3 ^ np.uint64(key1), p0 & m32)
    return tuple(x.astype(np.uint32) for x in (x0, x1, x2, x3))
