"""The quantiser's quotient on the GPU, checked on the CPU.

rotate_quant_kernel does not divide every element by the token's scale: it
computes inv = RN(1/div) once, then q0 = RN(v * inv) and
q = RN(q0 + RN(v - q0 * div) * inv) with two fused multiply-adds.  By
Markstein's theorem this is the correctly rounded quotient RN(v / div)
whenever nothing underflows or overflows, so the int8 codes equal those of the
oracle's IEEE division (the quantiser of [P1] section 4, ties to even).  These
tests evaluate that formula here with exact rational arithmetic for the fused
operations and compare it with IEEE float32 division, on random quotients and
on quotients placed next to the rounding boundaries k + 1/2 that decide a
code.  The GPU parity tests check the kernel's codes themselves.
"""
from fractions import Fraction

import numpy as np

F32 = np.float32


def rn32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32 (ties to even)."""
    f = F32(float(x))  # float(x) is the correctly rounded double
    # correct a possible double rounding: pick the nearest of the float32
    # neighbours of f by exact comparison
    best = None
    for c in (np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))):
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.frombuffer(c.tobytes(), dtype=np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def fma32(a, b, c) -> np.float32:
    return rn32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def markstein_quotient(v: np.float32, div: np.float32) -> np.float32:
    inv = F32(1.0) / div                      # IEEE division, once per token
    q0 = F32(v * inv)
    return fma32(fma32(-q0, div, v), inv, q0)


def _check(vs, divs):
    for v, d in zip(vs, divs):
        q = markstein_quotient(F32(v), F32(d))
        ref = F32(v) / F32(d)
        assert q.tobytes() == ref.tobytes(), (v, d, q, ref)
        # and therefore the same int8 code
        assert np.rint(q) == np.rint(ref)


def test_rn32_rounds_ties_to_even():
    one = Fraction(1)
    ulp = Fraction(2) ** -23
    assert rn32(one + ulp / 2) == F32(1.0)                 # tie -> even (1.0)
    assert rn32(one + ulp + ulp / 2) == F32(1.0) + F32(2.0 ** -22)  # tie -> even
    assert rn32(one + ulp / 2 + ulp / 1024) == np.nextafter(F32(1.0), F32(2.0))


def test_markstein_equals_ieee_division_random():
    rng = np.random.default_rng(11)
    n = 4000
    # activations like the rotated ones: |v| <= absmax, scales absmax / 127
    absmax = np.exp(rng.uniform(-6, 6, n)).astype(F32)
    div = (absmax / F32(127.0)).astype(F32)
    v = (absmax * rng.uniform(-1, 1, n).astype(F32)).astype(F32)
    _check(v, div)


def test_markstein_equals_ieee_division_near_half_integers():
    # quotients within a few ulp of k + 1/2, where the rounded quotient decides
    # the code, including exact ties
    rng = np.random.default_rng(12)
    vs, ds = [], []
    for _ in range(3000):
        d = F32(np.exp(rng.uniform(-8, 4)) / 127.0)
        k = int(rng.integers(-127, 127))
        target = F32(k + 0.5)
        v = F32(target * d)
        for step in range(-3, 4):
            vv = v
            for _ in range(abs(step)):
                vv = np.nextafter(vv, F32(np.inf) if step > 0 else F32(-np.inf))
            vs.append(vv)
            ds.append(d)
    _check(vs, ds)


def test_markstein_equals_ieee_division_exact_ties():
    # v = (k + 1/2) * div exactly representable: the quotient is the tie itself
    vs, ds = [], []
    for e in range(-20, 10):
        d = F32(2.0 ** e)
        for k in range(-127, 127):
            vs.append(F32((k + 0.5) * 2.0 ** e))
            ds.append(d)
    _check(vs, ds)
