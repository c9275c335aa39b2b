"""Philox counter-based generator (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The GPU library has
its own implementation of the same published definition; the two share no
code.

Definition (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3", SC 2011, the Philox-4xW-R family): a 4-word counter is passed
through R rounds keyed by a 2-word key.  One round maps (x0, x1, x2, x3) with
round key (k0, k1) to

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))

where hi/lo are the upper/lower W bits of the 2W-bit product, and the key
advances by the Weyl constants (W0, W1) (modulo 2^W) between rounds.  The
4x32 and 4x64 constants are the paper's; the default is R = 10.

`philox_block` is a plain Python-integer version of any width (used by the
pins); `philox4x32` is the vectorised numpy version of the 4x32-10 instance
used to draw dropout masks.
"""
from __future__ import annotations

import numpy as np

CONSTANTS = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def philox_block(ctr, key, width: int = 32, rounds: int = 10):
    """Philox-4x`width`-`rounds` of one counter (4 ints) under one key (2
    ints); returns the 4 output words as Python ints."""
    c = CONSTANTS[width]
    mask = (1 << width) - 1
    x = [int(w) & mask for w in ctr]
    k0, k1 = (int(w) & mask for w in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + c["W0"]) & mask
            k1 = (k1 + c["W1"]) & mask
        p0 = c["M0"] * x[0]
        p1 = c["M1"] * x[2]
        x = [(p1 >> width) ^ x[1] ^ k0, p1 & mask, (p0 >> width) ^ x[3] ^ k1, p0 & mask]
    return x


def philox4x32(c0, c1, c2, c3, k0: int, k1: int, rounds: int = 10):
    """Philox-4x32-`rounds` over arrays of counter words (broadcast together),
    one key.  Returns four uint32 arrays."""
    c = CONSTANTS[32]
    m32 = np.uint64(0xFFFFFFFF)
    x0, x1, x2, x3 = (np.asarray(w, dtype=np.uint64) & m32 for w in np.broadcast_arrays(c0, c1, c2, c3))
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    M0, M1 = np.uint64(c["M0"]), np.uint64(c["M1"])
    for r in range(rounds):
        if r:
            k0 = (k0 + c["W0"]) & 0xFFFFFFFF
            k1 = (k1 + c["W1"]) & 0xFFFFFFFF
        p0 = M0 * x0  # exact: both factors < 2^32
        p1 = M1 * x2
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ np.uint64(k0), p1 & m32,
                          (p0 >> np.uint64(32)) ^ x3 ^ np.uint64(k1), p0 & m32)
    return tuple(w.astype(np.uint32) for w in (x0, x1, x2, x3))
