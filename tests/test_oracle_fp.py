"""Pins for the exact FP32/FP16 rounding helpers of the oracle (brute force with Fractions)."""
from fractions import Fraction as Fr

import numpy as np

from oracle import fp

F32 = np.float32


def rn_fraction_to_f32(x):
    """Reference: nearest float32 to an exact rational, ties to even (finite range)."""
    f = F32(float(x))
    cands = [np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))]
    best = None
    for c in cands:
        dist = abs(Fr(float(c)) - x)
        key = (dist, int(np.asarray(c, dtype=F32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def rn_fraction_to_f16(x):
    """Reference: nearest float16 to an exact rational, ties to even (finite range)."""
    f = np.float16(float(x))
    cands = [np.nextafter(f, np.float16(-np.inf)), f, np.nextafter(f, np.float16(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        dist = abs(Fr(float(c)) - x)
        key = (dist, int(np.asarray(c, dtype=np.float16).view(np.uint16)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def random_f32(rng, n, emin=-30, emax=30):
    m = rng.integers(1 << 23, 1 << 24, size=n)
    e = rng.integers(emin, emax, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return (s * m * np.exp2(e - 23.0)).astype(F32)


def test_fma32_random_matches_fraction():
    rng = np.random.default_rng(1)
    a = random_f32(rng, 3000)
    b = random_f32(rng, 3000)
    c = random_f32(rng, 3000, -60, 60)
    # cancellation-heavy cases: c close to -a*b
    c[:1000] = (-(a[:1000].astype(np.float64) * b[:1000])).astype(F32)
    got = fp.fma32(a, b, c)
    for i in range(len(a)):
        ex = Fr(float(a[i])) * Fr(float(b[i])) + Fr(float(c[i]))
        assert got[i] == rn_fraction_to_f32(ex), (a[i], b[i], c[i])


def test_fma32_double_rounding_midpoints():
    # (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24 lies exactly halfway between two float32 values
    a = F32(1 + 2.0 ** -12)
    tiny = F32(2.0 ** -60)
    up = fp.fma32(a, a, tiny)
    down = fp.fma32(a, a, -tiny)
    tie = fp.fma32(a, a, F32(0))
    lo = F32(1 + 2.0 ** -11)
    hi = np.nextafter(lo, F32(2))
    assert up == hi and down == lo and tie == lo  # tie goes to the even mantissa (lo)


def test_rn32_sum_matches_fraction():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(4000) * np.exp2(rng.integers(-40, 40, 4000))
    b = rng.standard_normal(4000) * np.exp2(rng.integers(-40, 40, 4000))
    got = fp.rn32_sum(a, b)
    for i in range(len(a)):
        assert got[i] == rn_fraction_to_f32(Fr(float(a[i])) + Fr(float(b[i])))


def test_rn16_exhaustive_midpoints():
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)  # every finite non-negative float16 below the largest
    v = bits.view(np.float16).astype(np.float64)
    nxt = (bits + 1).view(np.float16).astype(np.float64)
    mid = (v + nxt) / 2  # exact in float64
    even = np.where(bits % 2 == 0, v, nxt)
    assert np.array_equal(fp.rn16(mid).astype(np.float64), even)
    above = mid + (nxt - v) * 2.0 ** -20
    below = mid - (nxt - v) * 2.0 ** -20
    assert np.array_equal(fp.rn16(above).astype(np.float64), nxt)
    assert np.array_equal(fp.rn16(below).astype(np.float64), v)
    assert np.array_equal(fp.rn16(-mid).astype(np.float64), -even)


def test_fract32_floor_ldexp():
    w = np.array([1.5, -1.5, -1e-10, -0.0, 3.0, -2.0, 2.75], dtype=F32)
    f = fp.fract32(w)
    assert f[0] == F32(0.5) and f[1] == F32(0.5)
    assert f[2] == np.nextafter(F32(1), F32(0))  # 1 - 1e-10 rounds to 1.0, clamped below 1
    assert f[4] == 0 and f[5] == 0 and f[6] == F32(0.75)
    assert list(fp.floor_i32(w)) == [1, -2, -1, 0, 3, -2, 2]
    assert fp.ldexp32(F32(1.5), -149) == F32(2.0 ** -148)  # 1.5 * 2^-149 rounds to even: 2^-148
    assert fp.ldexp32(F32(1.0), -150) == 0
    assert fp.ldexp32(F32(1.0), -149) == F32(2.0 ** -149)


def random_f16(rng, n):
    """Random float16 values below 128 in magnitude (normal and subnormal), both signs."""
    bits = rng.integers(0, 0x5800, size=n).astype(np.uint16)
    sign = (rng.integers(0, 2, size=n) << 15).astype(np.uint16)
    return (bits | sign).view(np.float16)


def test_fma16_random_matches_fraction():
    rng = np.random.default_rng(21)
    n = 4000
    a = random_f16(rng, n)
    b = random_f16(rng, n)
    c = random_f16(rng, n)
    # a power of two (the rescale factor) with c of similar size to a*b: the kernel's case
    a[:1500] = np.exp2(-rng.integers(0, 30, 1500).astype(np.float64)).astype(np.float16)
    c[:1500] = (b[:1500].astype(np.float64) * rng.uniform(-2, 2, 1500)).astype(np.float16)
    # cancellation-heavy cases
    c[1500:2000] = (-(a[1500:2000].astype(np.float64) * b[1500:2000])).astype(np.float16)
    got = fp.fma16(a, b, c)
    for i in range(n):
        ex = Fr(float(a[i])) * Fr(float(b[i])) + Fr(float(c[i]))
        want = rn_fraction_to_f16(ex)
        assert got[i] == want, (a[i], b[i], c[i], got[i], want)


def test_fma16_midpoint_ties():
    # 1 + 2^-11 is the midpoint between 1 and 1 + 2^-10: ties go to even (1), a nudge decides otherwise
    one = np.float16(1.0)
    half_ulp = np.float16(2.0 ** -11)
    tiny = np.float16(2.0 ** -24)
    assert fp.fma16(one, one, half_ulp) == np.float16(1.0)
    # 1 * (1 + 2^-10) + 2^-11: midpoint between 1 + 2^-10 (odd) and 1 + 2^-9 (even) -> up
    assert fp.fma16(one, np.float16(1 + 2.0 ** -10), half_ulp) == np.float16(1 + 2.0 ** -9)
    # exact value 1 + 2^-11 + 2^-24 (just above the midpoint) rounds up; one below rounds down
    b = np.float16(2.0 ** -11)
    assert fp.fma16(np.float16(1 + 2.0 ** -10), b, one) == np.float16(1 + 2.0 ** -10)  # 1 + 2^-11 + 2^-21
    assert fp.fma16(np.float16(1 - 2.0 ** -11), b, one) == one  # 1 + 2^-11 - 2^-22
    assert fp.fma16(tiny, one, np.float16(1 + 2.0 ** -10)) == np.float16(1 + 2.0 ** -10)
    assert fp.fma16(np.float16(-2.0 ** -11), one, one) == np.float16(1 - 2.0 ** -11)
