"""Pins for the oracle's 4-bit block quantizer: brute force, the scale rule, invariants, a worked example."""
import numpy as np

from oracle import mx

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def brute_code(y):
    """Nearest of the 8 magnitudes by explicit distance search; a tie goes to the even code index."""
    a = np.abs(y)[:, None]
    dist = np.abs(a - GRID[None, :])
    dmin = dist.min(axis=1, keepdims=True)
    cand = dist == dmin
    even_ok = cand & (np.arange(8)[None, :] % 2 == 0)
    idx = np.where(even_ok.any(axis=1), even_ok.argmax(axis=1), cand.argmax(axis=1))
    return (idx | (np.signbit(y).astype(int) << 3)).astype(np.uint8)


def test_rne_code_exhaustive_fp16_times_scales():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float64)
    x = x[np.isfinite(x)]
    for e in range(-30, 21):
        y = x * 2.0 ** (-e)
        assert np.array_equal(mx.rne_code(y), brute_code(y)), e


def test_rne_code_midpoints_and_saturation():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(mx.rne_code(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(mx.rne_code(np.nextafter(mids, 10))) == [1, 2, 3, 4, 5, 6, 7]
    assert list(mx.rne_code(np.array([6.0, 7.0, 1e30, -7.0, -0.0, -1e-30]))) == [7, 7, 7, 15, 8, 8]


def brute_scale(amax):
    """Smallest e with 6 * 2**e >= amax, clamped to [-127, 127]; zero blocks get -127."""
    out = []
    for a in amax:
        if a == 0:
            out.append(-127)
            continue
        e = -200
        while 6.0 * 2.0 ** e < a:
            e += 1
        out.append(int(np.clip(e, -127, 127)))
    return np.array(out)


def test_scale_rule_matches_search():
    rng = np.random.default_rng(3)
    amax = np.concatenate([
        np.exp2(rng.uniform(-140, 120, 3000)),
        np.array([6.0, 6.0000001, 5.9999, 1.5, 1.5000001, 3.0, 3.0000001, 2.0 ** -130, 2.0 ** -149, 0.0, 1e38]),
        6.0 * np.exp2(np.arange(-20, 20)), 3.0 * np.exp2(np.arange(-20, 20)),
    ])
    assert np.array_equal(mx.scale_exponent(amax), brute_scale(amax))


def test_block_max_never_clips_and_invariants():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((500, 64)) * np.exp2(rng.integers(-20, 20, (500, 1)))
    codes, e = mx.quantize_blocks(x)
    deq = mx.dequantize_blocks(codes, e)
    # no clipping: the block max is represented within half a grid step, never saturated from above
    amax = np.abs(x.reshape(500, 2, 32)).max(axis=2)
    assert np.all(amax <= 6.0 * np.exp2(e))
    # idempotence on values: the grid points of a block are reproduced exactly
    c2, e2 = mx.quantize_blocks(deq)
    assert np.array_equal(mx.dequantize_blocks(c2, e2), deq)
    # quantization error is at most half a grid step of the block (a quarter of 2**e at the bottom)
    assert np.all(np.abs(deq - x) <= np.repeat(np.exp2(e), 32, axis=1))
    # power-of-two equivariance
    c3, e3 = mx.quantize_blocks(x * 2.0 ** 7)
    assert np.array_equal(c3, codes) and np.array_equal(e3, np.clip(e + 7, -127, 127))


def test_worked_example():
    # constructed from the rules above: amax 6.5 = 1.625 * 2^2 -> e = 1; y = x / 2
    blk = np.zeros(32)
    blk[:8] = [1.0, 0.3, -5.0, 6.5, 0.24, -0.26, 2.9, -0.0]
    blk[7] = -0.0
    codes, e = mx.quantize_blocks(blk[None, :])
    assert e[0, 0] == 1 and mx.scale_bytes(e)[0, 0] == 0x80
    assert list(codes[0, :8]) == [0x1, 0x0, 0xC, 0x5, 0x0, 0x8, 0x3, 0x8]
    assert list(mx.pack_codes(codes)[0, :4]) == [0x01, 0x5C, 0x80, 0x83]
    deq = mx.dequantize_blocks(codes, e)[0, :8]
    assert list(deq) == [1.0, 0.0, -4.0, 6.0, 0.0, -0.0, 3.0, -0.0]
    assert np.signbit(deq[5]) and np.signbit(deq[7])


def test_pack_roundtrip_and_zero_block():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    assert np.array_equal(mx.unpack_codes(mx.pack_codes(codes)), codes)
    c, e = mx.quantize_blocks(np.zeros((1, 32)))
    assert e[0, 0] == -127 and mx.scale_bytes(e)[0, 0] == 0 and not c.any()


def brute_scale_floor(amax):
    """Search: the e with 4 * 2**e <= amax < 8 * 2**e (E2M1's top binade holds the maximum), clamped."""
    out = []
    for a in np.asarray(amax, dtype=np.float64):
        if a == 0:
            out.append(-127)
            continue
        e = -200
        while not (a < 8.0 * 2.0 ** e):
            e += 1
        assert 4.0 * 2.0 ** e <= a or e == -200
        out.append(min(max(e, -127), 127))
    return np.array(out)


def test_floor_rule_matches_search_and_ocp_examples():
    rng = np.random.default_rng(31)
    amax = np.concatenate([np.exp2(rng.uniform(-120, 120, 2000)),
                           np.array([6.0, 7.0, 7.9999, 8.0, 4.0, 3.9999, 1.0, 0.0])])
    assert np.array_equal(mx.scale_exponent_floor(amax), brute_scale_floor(amax))
    # OCP examples: 6 -> e = 0 (6 kept); 7 -> e = 0 and 7 saturates to 6; 8 -> e = 1 (4 kept)
    codes, e = mx.quantize_blocks(np.array([[6.0] + [0.0] * 31, [7.0] + [0.0] * 31, [8.0] + [0.0] * 31]), "floor")
    assert list(e[:, 0]) == [0, 0, 1]
    assert list(codes[:, 0]) == [7, 7, 6]  # 6, 6 (saturated), 4


def test_floor_rule_clips_where_the_method_rule_does_not():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((400, 32)) * np.exp2(rng.integers(-10, 10, (400, 1)))
    c_f, e_f = mx.quantize_blocks(x, "floor")
    c_n, e_n = mx.quantize_blocks(x, "no_clip")
    amax = np.abs(x).max(axis=1)
    # floor never exceeds the method's exponent, and is one below it exactly when amax / 2^floor > 6
    assert np.all(e_f[:, 0] <= e_n[:, 0]) and np.all(e_n[:, 0] - e_f[:, 0] <= 1)
    clip = amax > 6.0 * np.exp2(e_f[:, 0])
    assert np.array_equal(clip, e_n[:, 0] == e_f[:, 0] + 1)
    # clipped blocks saturate their maximum at 6 * 2^e
    deq = mx.dequantize_blocks(c_f, e_f)
    assert np.all(np.abs(deq).max(axis=1) <= 6.0 * np.exp2(e_f[:, 0]))
