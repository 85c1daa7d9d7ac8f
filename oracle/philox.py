"""Philox4x64-10 counter-based generator, written from its published definition.

Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11): a Philox-4x64 round multiplies counter words 0 and 2 by two fixed
odd 64-bit constants, takes the high and low halves of the 128-bit products,
and permutes/xors them with words 1 and 3 and the round key; the key is bumped
by two Weyl constants between rounds; ten rounds.

The random draws of the sampling verifier come from this block function keyed
(seed, 0) with counter (1, request_id, position, 0); see ``verify.uniforms``.
Plain Python integers, no vectorisation: this is the checkable statement.
"""

MASK64 = (1 << 64) - 1

# Multipliers and Weyl increments of Philox-4x64 as printed in the SC'11 paper.
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1


def _round(ctr, key):
    c0, c1, c2, c3 = ctr
    p0 = PHILOX_M0 * c0
    p1 = PHILOX_M1 * c2
    hi0, lo0 = p0 >> 64, p0 & MASK64
    hi1, lo1 = p1 >> 64, p1 & MASK64
    return (hi1 ^ c1 ^ key[0], lo1, hi0 ^ c3 ^ key[1], lo0)


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for one 256-bit counter block."""
    ctr = tuple(int(c) & MASK64 for c in counter)
    k = [int(key[0]) & MASK64, int(key[1]) & MASK64]
    for r in range(10):
        if r > 0:
            k = [(k[0] + PHILOX_W0) & MASK64, (k[1] + PHILOX_W1) & MASK64]
        ctr = _round(ctr, k)
    return ctr
