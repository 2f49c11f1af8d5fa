"""Exact IEEE-754 rounding helpers (oracle; test infrastructure only).

The kernel computes some quantities in FP32 that later decide integers (4-bit
codes, block-scale exponents, the integer running max).  To take those
decisions in the same precision, the oracle emulates each FP32 operation with a
single, correct round-to-nearest-even step:

* products of two FP32 values are exact in FP64 (24 + 24 < 53 bits);
* sums use an error-free two-sum in FP64 and fix the rare FP64 -> FP32 double
  rounding (when the FP64 sum lands exactly on an FP32 midpoint, the sign of
  the two-sum error decides the side);
* FP16 rounding uses NumPy's correctly rounded float16 conversion; the FP16
  fused multiply-add uses the same two-sum route with FP16 as the target.

Every helper is pinned against ``fractions.Fraction`` brute force in
``tests/test_oracle_fp.py``.
"""

import numpy as np

F32 = np.float32
F64 = np.float64

# largest float32 below 1.0: the hardware fract result is clamped to it
ONE_MINUS_ULP32 = np.nextafter(F32(1.0), F32(0.0))


def _rn_sum(a, b, dtype):
    """Round the exact sum a + b (FP64 inputs) once to ``dtype`` (float32 or float16), ties to even."""
    a = np.asarray(a, dtype=F64)
    b = np.asarray(b, dtype=F64)
    s = a + b
    bb = s - a
    err = (a - (s - bb)) + (b - bb)  # exact: a + b == s + err (two-sum)
    with np.errstate(over="ignore", invalid="ignore"):
        r = s.astype(dtype)
        r64 = r.astype(F64)
        diff = s - r64
        toward = np.where(diff > 0, dtype(np.inf), dtype(-np.inf)).astype(dtype)
        o = np.nextafter(r, toward)
        o64 = o.astype(F64)
        at_mid = (diff != 0) & np.isfinite(s) & (np.abs(diff) == np.abs(o64 - s))
        # the true value s + err lies on the side of err; move to o when err points at o
        go_o = at_mid & (err != 0) & (np.sign(err) == np.sign(o64 - s))
    return np.where(go_o, o, r).astype(dtype)


def rn32_sum(a, b):
    """Round the exact sum a + b (FP64 inputs) once to the nearest FP32 (ties to even)."""
    return _rn_sum(a, b, F32)


def fma16(a, b, c):
    """FP16 fused multiply-add: RN16(a*b + c) with a single rounding (a, b, c are FP16 values).

    The FP64 product of two FP16 values is exact (11 + 11 < 53 bits); the sum is rounded
    once to FP16 through the two-sum route above.
    """
    a = np.asarray(a, dtype=np.float16).astype(F64)
    b = np.asarray(b, dtype=np.float16).astype(F64)
    c = np.asarray(c, dtype=np.float16).astype(F64)
    return _rn_sum(a * b, c, np.float16)


def fma32(a, b, c):
    """FP32 fused multiply-add: RN32(a*b + c) with a single rounding (a, b, c are FP32)."""
    a = np.asarray(a, dtype=F32).astype(F64)
    b = np.asarray(b, dtype=F32).astype(F64)
    c = np.asarray(c, dtype=F32).astype(F64)
    return rn32_sum(a * b, c)  # the FP64 product is exact


def mul32(a, b):
    """FP32 multiply with one rounding."""
    return (np.asarray(a, dtype=F32).astype(F64) * np.asarray(b, dtype=F32).astype(F64)).astype(F32)


def add32(a, b):
    """FP32 add with one rounding."""
    return rn32_sum(np.asarray(a, dtype=F32).astype(F64), np.asarray(b, dtype=F32).astype(F64))


def div32(a, b):
    """IEEE FP32 division (NumPy float32 division is correctly rounded)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return (np.asarray(a, dtype=F32) / np.asarray(b, dtype=F32)).astype(F32)


def fract32(w):
    """Fractional part as the GPU's fract computes it: RN32(w - floor(w)), clamped below 1."""
    w = np.asarray(w, dtype=F32)
    f = (w.astype(F64) - np.floor(w.astype(F64))).astype(F32)  # exact difference, one rounding
    return np.minimum(f, ONE_MINUS_ULP32).astype(F32)


def floor_i32(w):
    """floor(w) converted to int32 with saturation (as a float->int conversion does)."""
    w = np.asarray(w, dtype=F64)
    fl = np.floor(w)
    fl = np.clip(fl, -2.0 ** 31, 2.0 ** 31 - 1)
    return fl.astype(np.int64)


def ldexp32(x, n):
    """x * 2**n in FP32 with IEEE rounding (gradual underflow), n an integer array."""
    x = np.asarray(x, dtype=F32)
    n = np.clip(np.asarray(n, dtype=np.int64), -1000, 1000).astype(np.int32)
    with np.errstate(over="ignore", under="ignore"):
        return np.ldexp(x, n).astype(F32)


def rn16(x):
    """Round FP64/FP32 values once to FP16 (ties to even)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=F64).astype(np.float16)
