"""4-bit block format: E2M1 codes with a power-of-two scale per 32-element block.

[HiFA4] Abstract: Q, K, V and the attention weights P-hat are quantized to a
4-bit format (HIF4).  The visible pages do not give its bit layout; this
package uses E2M1 elements (sign, 2 exponent bits, 1 mantissa bit: magnitudes
0, 0.5, 1, 1.5, 2, 3, 4, 6) with one power-of-two (E8M0) scale per block of 32
elements, the layout gfx950's scaled FP4 matrix instructions consume.

Readings where the pages are silent:
* scale rule: the smallest exponent e with 6 * 2**e >= amax (no element is
  clipped): with amax = M * 2**E, M in [1, 2): e = E - 2 if M <= 1.5 else E - 1;
  clamped to [-127, 127]; an all-zero block gets e = -127 (scale byte 0);
* element rounding: round to nearest, ties to the even code, saturating at 6;
* the sign bit is copied from the input (so -0.0 and tiny negatives give 0x8);
* packing: byte = code[2i] | code[2i+1] << 4; scale byte = e + 127.

Accuracy variant (rule "floor"): the shared-exponent rule of the OCP microscaling format,
e = floor(log2 amax) - 2 (2 = the largest E2M1 exponent), clamped the same way; magnitudes in
(6, 8) * 2**e then saturate to 6.  It is not the method's rule: it clips up to a quarter of the
block maximum, and it serves the comparison of the two rules.
"""

import numpy as np

F64 = np.float64

MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=F64)
HALF_UNITS = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)  # 2 * MAG, exact integers
BLOCK = 32


def scale_exponent(amax):
    """Block exponent e from the block's largest magnitude (see module docstring)."""
    amax = np.asarray(amax, dtype=F64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    m, E = np.frexp(amax[nz])  # amax = m * 2**E, m in [0.5, 1)
    M = 2.0 * m
    E = E.astype(np.int64) - 1
    e_nz = np.where(M <= 1.5, E - 2, E - 1)
    e[nz] = np.clip(e_nz, -127, 127)
    return e


def scale_exponent_floor(amax):
    """OCP microscaling shared exponent: floor(log2 amax) - 2, clamped; -127 for a zero block."""
    amax = np.asarray(amax, dtype=F64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    _, E = np.frexp(amax[nz])  # amax = m * 2**E, m in [0.5, 1): floor(log2 amax) = E - 1
    e[nz] = np.clip(E.astype(np.int64) - 1 - 2, -127, 127)
    return e


SCALE_RULES = {"no_clip": scale_exponent, "floor": scale_exponent_floor}


def rne_code(y):
    """4-bit code of y (already divided by the block scale): RNE onto the E2M1 grid, saturating.

    A magnitude moves up one code each time it passes a midpoint of the grid;
    at an exact midpoint it goes to the even code (the code with mantissa bit 0).
    """
    y = np.asarray(y, dtype=F64)
    a = np.abs(y)
    code = ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    sign = np.signbit(y).astype(np.int64)
    return (code | (sign << 3)).astype(np.uint8)


def code_value(code):
    """Value of a 4-bit code (without the block scale)."""
    code = np.asarray(code).astype(np.int64)
    v = MAG[code & 7]
    return np.where(code & 8, -v, v)


def code_half_units(code):
    """Signed value * 2 as an exact integer (0, +-1, +-2, +-3, +-4, +-6, +-8, +-12)."""
    code = np.asarray(code).astype(np.int64)
    v = HALF_UNITS[code & 7]
    return np.where(code & 8, -v, v)


def quantize_blocks(x, rule="no_clip"):
    """Quantize along the last axis (length a multiple of 32) with a scale rule of SCALE_RULES.

    Returns (codes uint8 [..., n], exponents int64 [..., n // 32]).
    """
    x = np.asarray(x, dtype=F64)
    n = x.shape[-1]
    assert n % BLOCK == 0, "block axis must be a multiple of 32"
    xb = x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.abs(xb).max(axis=-1)
    e = SCALE_RULES[rule](amax)
    y = xb * np.exp2(-e.astype(F64))[..., None]  # exact power-of-two scaling
    codes = rne_code(y).reshape(x.shape)
    return codes, e


def dequantize_blocks(codes, e):
    """Inverse of quantize_blocks (exact)."""
    codes = np.asarray(codes)
    n = codes.shape[-1]
    v = code_value(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    return (v * np.exp2(np.asarray(e, dtype=F64))[..., None]).reshape(codes.shape)


def pack_codes(codes):
    """Two codes per byte, the lower-index element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


def scale_bytes(e):
    return (np.asarray(e) + 127).astype(np.uint8)


def scale_from_bytes(b):
    return np.asarray(b).astype(np.int64) - 127
