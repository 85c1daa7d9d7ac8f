"""The sampler's float64 exponential (csrc/exp64.hpp), checked on the CPU.

The kernels' weights exp((l - m) / tau) come from exp64, a range-reduced
polynomial rather than the library exponential.  Its constants are read out of
the header and its operation sequence is replayed with every step rounded to
double as the GPU rounds it (fused multiply-adds rounded once), against a
200-bit exponential: relative error at most 4e-16 (2 ulp) over the weights'
range, exactly 0 at -inf, and the subnormal range handled.  A slip in a
coefficient, in the Cody-Waite split of ln 2 or in the order of the Horner
steps moves the error far above that bound.
"""

import os
import re

import numpy as np
import pytest

mp = pytest.importorskip("mpmath")

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "block_draft_verification_amd", "csrc", "exp64.hpp")


def _constants():
    text = open(HDR).read()
    vals = dict(re.findall(r"constexpr double (\w+) = ([0-9.eE+-]+);", text))
    coef = [float(vals[f"c{i}"]) for i in range(11)]
    return float(vals["kLog2e"]), float(vals["kLn2Hi"]), float(vals["kLn2Lo"]), coef


def _exp64(x, consts):
    """exp64's steps, each rounded to double (fma: one rounding)."""
    log2e, hi, lo, c = consts
    mp.mp.prec = 200
    rnd = lambda v: mp.mpf(float(v))
    fma = lambda a, b, d: rnd(mp.mpf(a) * mp.mpf(b) + mp.mpf(d))
    x = max(x, -746.0)
    k = float(np.rint(float(rnd(mp.mpf(x) * log2e))))
    r = fma(-k, hi, x)
    r = fma(-k, lo, r)
    p = mp.mpf(c[10])
    for i in range(9, -1, -1):
        p = fma(p, r, c[i])
    return float(np.ldexp(float(p), int(k)))


def test_split_of_ln2_is_exact_for_the_exponent_range():
    _, hi, lo, _ = _constants()
    mp.mp.prec = 200
    # the high part has 32 significant bits, so k * hi is exact for |k| < 2^21
    m, e = np.frexp(hi)
    assert float(m * 2.0 ** 32) == int(m * 2.0 ** 32)
    assert abs(mp.mpf(hi) + mp.mpf(lo) - mp.log(2)) < mp.mpf(2) ** -80


def test_relative_error_within_two_ulp():
    consts = _constants()
    rng = np.random.default_rng(7)
    xs = np.concatenate([-rng.exponential(4.0, 1500), -rng.uniform(0.0, 708.0, 400),
                         rng.uniform(0.0, 1.0, 100), [0.0, -1e-300, -0.5 * np.log(2), 0.5 * np.log(2)]])
    worst = 0.0
    mp.mp.prec = 200
    for x in xs:
        got = _exp64(float(x), consts)
        ref = mp.exp(mp.mpf(float(x)))
        worst = max(worst, float(abs(mp.mpf(got) / ref - 1)))
    assert worst <= 4e-16, worst


def test_limits():
    consts = _constants()
    assert _exp64(float("-inf"), consts) == 0.0
    assert _exp64(-746.0, consts) == 0.0
    assert _exp64(0.0, consts) == 1.0
    # subnormal results: within one unit of the last place of exp
    for x in (-709.5, -720.0, -740.0):
        got = _exp64(x, consts)
        ref = float(mp.exp(mp.mpf(x)))
        assert 0.0 < got and abs(got - ref) <= np.spacing(ref), (x, got, ref)
