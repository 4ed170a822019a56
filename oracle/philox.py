"""Philox counter-based random numbers, the oracle's copy.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
CPU baseline of the benchmark, never by the library.

Philox-4xW-R (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
easy as 1, 2, 3", SC'11): a keyed bijection of a 4-word counter.  One round
multiplies words 0 and 2 by the constants M0 and M1, takes the high and low
halves of the double-width products, and returns
``(hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0))``; between
rounds the two key words grow by the Weyl constants W0 and W1 (modulo 2^W).
Ten rounds are the published default.  The pages of the operator fix no
generator; dropout masks here are defined with Philox4x32-10 (the word size
the GPU multiplies natively).

Pinned in ``tests/test_oracle_dropout.py``: the published known-answer
vectors, and the 4x64 instance against numpy's ``Philox`` bit generator.
"""

from __future__ import annotations

import numpy as np

# (M0, M1, W0, W1) per word size
CONSTANTS = {
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}


def philox4(counter, key, bits=32, rounds=10):
    """Philox-4x``bits``-``rounds`` of one counter, in Python integers.

    ``counter``: 4 words, ``key``: 2 words, each in ``[0, 2**bits)``.
    Returns the 4 output words."""
    m0, m1, w0, w1 = CONSTANTS[bits]
    mask = (1 << bits) - 1
    x = [int(v) & mask for v in counter]
    k0, k1 = (int(v) & mask for v in key)
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + w0) & mask, (k1 + w1) & mask
        p0, p1 = m0 * x[0], m1 * x[2]
        x = [(p1 >> bits) ^ x[1] ^ k0, p1 & mask, (p0 >> bits) ^ x[3] ^ k1, p0 & mask]
    return x


def philox4x32_array(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32 of many counters at once: ``c0..c3`` equal-shaped integer
    arrays (values below 2**32), ``k0, k1`` scalars.  Products are formed in
    uint64, which holds a 32x32-bit product exactly.  Returns 4 uint32
    arrays."""
    m0, m1, w0, w1 = CONSTANTS[32]
    u64 = np.uint64
    lo32 = u64(0xFFFFFFFF)
    x = [np.asarray(c, dtype=np.uint64) & lo32 for c in (c0, c1, c2, c3)]
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + w0) & 0xFFFFFFFF, (k1 + w1) & 0xFFFFFFFF
        p0 = x[0] * u64(m0)
        p1 = x[2] * u64(m1)
        x = [(p1 >> u64(32)) ^ x[1] ^ u64(k0), p1 & lo32,
             (p0 >> u64(32)) ^ x[3] ^ u64(k1), p0 & lo32]
    return [v.astype(np.uint32) for v in x]
