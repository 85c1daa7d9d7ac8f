"""Pins for the oracle's Philox4x64-10 and the uniforms built on it.

Independent references: numpy's own Philox bit generator (a separate
implementation; numpy increments counter word 0, with carry, before each block,
so a numpy counter of c - 1 yields block c), and the published known-answer
vectors of the Random123 distribution that accompanies the SC'11 paper
(tests/golden/philox4x64_10_kat.txt).
"""

import os

import numpy as np
import pytest

from oracle.philox import philox4x64_10
from oracle.verify import uniforms

M64 = (1 << 64) - 1
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x64_10_kat.txt")


def numpy_block(ctr, key):
    v = (ctr[0] | ctr[1] << 64 | ctr[2] << 128 | ctr[3] << 192) - 1
    v &= (1 << 256) - 1
    words = np.array([(v >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


def test_known_answer_vectors():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(t, 16) for t in line.split()]
            ctr, key, expect = w[0:4], w[4:6], tuple(w[6:10])
            assert philox4x64_10(ctr, key) == expect
            n += 1
    assert n >= 3


@pytest.mark.parametrize("seed", [0, 1, 12345, M64, 0xDEADBEEFCAFEF00D])
def test_matches_numpy_philox(seed):
    rng = np.random.default_rng(seed & 0xFFFFFFFF)
    for _ in range(40):
        ctr = [int(x) for x in rng.integers(0, 2**63, 4, dtype=np.uint64)]
        ctr[0] |= 1  # keep word 0 non-zero so c - 1 does not borrow
        assert philox4x64_10(ctr, (seed, 0)) == numpy_block(ctr, (seed, 0))


def test_carry_into_word1():
    # counter word 0 == 0 needs a borrow on the numpy side: exercises carry
    ctr = (0, 7, 9, 0)
    assert philox4x64_10(ctr, (3, 0)) == numpy_block(ctr, (3, 0))


def test_uniforms_from_words():
    for rid, pos in [(0, 0), (5, 4097), (2**40 + 3, 2**33)]:
        w = numpy_block((1, rid, pos, 0), (77, 0))
        ua, ur = uniforms(77, rid, pos)
        assert ua == (w[0] >> 11) / 2.0**53
        assert ur == (w[1] >> 11) / 2.0**53
        assert 0.0 <= ua < 1.0 and 0.0 <= ur < 1.0


def test_uniforms_are_uniform():
    # Kolmogorov-Smirnov style bound on 4096 draws of each stream
    ua = np.array([uniforms(5, r, 100)[0] for r in range(4096)])
    ur = np.array([uniforms(5, r, 100)[1] for r in range(4096)])
    for u in (ua, ur):
        s = np.sort(u)
        ks = np.max(np.abs(s - (np.arange(1, s.size + 1) - 0.5) / s.size))
        assert ks < 1.95 / np.sqrt(s.size)  # ~0.1 % false-alarm level
    assert abs(np.corrcoef(ua, ur)[0, 1]) < 0.06
