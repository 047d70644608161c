"""The quantizers divide x by the scale s with three binary32 operations
instead of an IEEE division (q0 = x*r, e' = fma(q0, s, -x),
q = fma(-e', r, q0), r = fl32(1/s)). This CPU test replays those operations
exactly (each rounded once to binary32) over every pair (significand of the
block maximum, significand of an element) of bf16 and checks that the result
is the IEEE quotient, bit for bit, including the sign of zero. The kernels'
GPU parity tests repeat the same grid through the hardware."""
from fractions import Fraction

import numpy as np

import synth


def fl32_exact(r: Fraction) -> np.float32:
    if r == 0:
        return np.float32(0.0)
    neg = r < 0
    r = -r if neg else r
    e = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    e = max(e, -126)
    qu = Fraction(2) ** (e - 23)
    n = r / qu
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = np.float32(float(fl * qu))
    return -v if neg else v


def fast_quotient(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The kernels' quotient, each binary32 operation emulated exactly."""
    r = (np.float32(1.0) / s).astype(np.float32)                     # IEEE reciprocal
    x64, s64, r64 = x.astype(np.float64), s.astype(np.float64), r.astype(np.float64)
    q0 = (x64 * r64).astype(np.float32)                                 # 48-bit product, one rounding
    t = q0.astype(np.float64) * s64                                    # exact
    en64 = t - x64                                                     # exact (Sterbenz)
    assert np.all((en64 + x64 == t) | (x64 == 0))
    en = en64.astype(np.float32)
    u = -(en.astype(np.float64) * r64)                                 # exact
    tot = q0.astype(np.float64) + u
    exact = (tot - q0.astype(np.float64)) == u
    q = tot.astype(np.float32)
    for idx in zip(*np.nonzero(~exact)):                               # rare: exact rounding by hand
        q[idx] = fl32_exact(Fraction(float(q0[idx])) + Fraction(float(u[idx])))
    return q   # numpy's float64 sums follow IEEE signed-zero rules: -0 + -0 = -0


def test_fast_quotient_equals_ieee_on_significand_grid():
    g = synth.quotient_grid(amax_exponents=(0,))
    g[::7, 5] = 0x8000                                                  # some -0
    g[::11, 9] = 0x0000                                                 # some +0
    x = (g.astype(np.uint32) << 16).view(np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    xs = x
    ss = np.broadcast_to(s[:, None], x.shape)
    want = (xs.astype(np.float64) / ss.astype(np.float64)).astype(np.float32)
    got = fast_quotient(xs, ss)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_plain_remainder_loses_the_sign_of_zero():
    # the unnegated form q0 + fma(x - q0*s)*r turns -0 into +0: the reason the
    # kernels negate the remainder
    x, s = np.float32(-0.0), np.float32(0.5)
    r = np.float32(1.0) / s
    q0 = x * r
    e = np.float32(np.float64(x) - np.float64(q0) * np.float64(s))
    q_plain = np.float32(np.float64(e) * np.float64(r) + np.float64(q0))
    assert not np.signbit(q_plain)
    assert np.signbit(fast_quotient(np.array([x]), np.array([s]))[0])
