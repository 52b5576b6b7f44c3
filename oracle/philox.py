"""Philox counter-based generators, written from their published definition.

TEST INFRASTRUCTURE ONLY (part of the oracle): see ``oracle/__init__.py``.

Philox-4xW-R (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11, Section 5): a 4-word counter (c0, c1, c2, c3) and a 2-word key
(k0, k1) go through R rounds of

    (hi0, lo0) = mulhilo(M0, c0);  (hi1, lo1) = mulhilo(M1, c2)
    (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)

with the key bumped by the Weyl constants (W0, W1) between rounds.  The
random-sentinel sampler of the routing oracle uses Philox4x32-10; the 4x64
variant is kept only so its round structure can be checked against numpy's
``numpy.random.Philox`` (which implements Philox4x64-10).
"""
from __future__ import annotations

M32 = 0xFFFFFFFF
M64 = 0xFFFFFFFFFFFFFFFF

_P32 = dict(mul=(0xD2511F53, 0xCD9E8D57), weyl=(0x9E3779B9, 0xBB67AE85), bits=32, mask=M32)
_P64 = dict(mul=(0xD2E7470EE14C6C93, 0xCA5A826395121157),
            weyl=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B), bits=64, mask=M64)


def _philox(params, ctr, key, rounds):
    m0, m1 = params["mul"]
    w0, w1 = params["weyl"]
    bits, mask = params["bits"], params["mask"]
    c0, c1, c2, c3 = (int(v) & mask for v in ctr)
    k0, k1 = (int(v) & mask for v in key)
    for rnd in range(rounds):
        if rnd:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> bits, p0 & mask
        hi1, lo1 = p1 >> bits, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0, c1, c2, c3)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds: four 32-bit counter words, two 32-bit key words
    -> four 32-bit output words."""
    return _philox(_P32, ctr, key, 10)


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds (64-bit words)."""
    return _philox(_P64, ctr, key, 10)
