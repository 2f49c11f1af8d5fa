"""Pins for the FP32 RoPE of the fused prologue (oracle/rope.py) and its RoPE tables (synth).

Each pin fails for a plausible mistake: a swapped sign or half (the quarter-turn and inverse
rotations), a fused or reordered rounding (Fraction brute force), a wrong angle or position
convention (FP64 closed form, relative-position invariance, identity at position 0), and a
broken hand-off to the quantizer (identity tables reduce to the pinned path).
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import synth
from oracle import attention as A
from oracle import rope
from test_oracle_fp import rn_fraction_to_f32

F32 = np.float32
F64 = np.float64


def _x16(rng, shape, scale=3.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def test_table_matches_fp64_angles():
    cos32, sin32 = synth.rope_table(1e6, 300, 128)
    assert cos32.dtype == F32 and cos32.shape == (300, 64)
    for p in (0, 1, 17, 299):
        for i in (0, 1, 31, 63):
            ang = p * 1e6 ** (-2.0 * i / 128)
            assert cos32[p, i] == F32(np.cos(ang)) and sin32[p, i] == F32(np.sin(ang))
    assert np.all(cos32[0] == 1) and np.all(sin32[0] == 0)


def test_position_zero_is_identity():
    rng = np.random.default_rng(11)
    x = _x16(rng, (2, 3, 1, 64))
    cos32, sin32 = synth.rope_table(1e4, 4, 64)
    y = rope.apply_rope32(x, cos32, sin32, [0])
    assert np.array_equal(y, x.astype(F32))


def test_quarter_turn_and_half_turn_are_exact():
    rng = np.random.default_rng(12)
    x = _x16(rng, (1, 2, 5, 32))
    h = 16
    c = np.zeros((1, h), F32)
    s = np.ones((1, h), F32)
    y = rope.apply_rope32(x, c, s, [0] * 5)
    xf = x.astype(F32)
    assert np.array_equal(y[..., :h], -xf[..., h:]) and np.array_equal(y[..., h:], xf[..., :h])
    y2 = rope.apply_rope32(x, -np.ones((1, h), F32), np.zeros((1, h), F32), [0] * 5)
    assert np.array_equal(y2, -xf)


def test_each_step_rounds_once_fraction_brute_force():
    rng = np.random.default_rng(13)
    x = _x16(rng, (1, 1, 40, 8), scale=50.0)
    cos32, sin32 = synth.rope_table(10.0, 40, 8)
    y = rope.apply_rope32(x, cos32, sin32, np.arange(40))
    for t in range(40):
        for i in range(4):
            a, b = Fr(float(x[0, 0, t, i])), Fr(float(x[0, 0, t, i + 4]))
            c, s = Fr(float(cos32[t, i])), Fr(float(sin32[t, i]))
            ac, bs = rn_fraction_to_f32(a * c), rn_fraction_to_f32(b * s)
            bc, as_ = rn_fraction_to_f32(b * c), rn_fraction_to_f32(a * s)
            lo = rn_fraction_to_f32(Fr(float(ac)) - Fr(float(bs)))
            hi = rn_fraction_to_f32(Fr(float(bc)) + Fr(float(as_)))
            assert y[0, 0, t, i] == lo and y[0, 0, t, i + 4] == hi, (t, i)


def test_close_to_fp64_rotation_and_inverse():
    rng = np.random.default_rng(14)
    d, n = 128, 257
    x = _x16(rng, (1, 2, n, d))
    cos32, sin32 = synth.rope_table(1e6, n, d)
    y = rope.apply_rope32(x, cos32, sin32, np.arange(n)).astype(F64)
    a, b = x[..., :64].astype(F64), x[..., 64:].astype(F64)
    c, s = cos32.astype(F64), sin32.astype(F64)
    ref = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    bound = 3 * 2.0 ** -24 * np.concatenate([np.abs(a) + np.abs(b)] * 2, axis=-1)
    assert np.all(np.abs(y - ref) <= bound + 1e-30)
    # rotating back by the transpose recovers the input (a sign error in either half would not)
    yl, yh = y[..., :64], y[..., 64:]
    back = np.concatenate([yl * c + yh * s, yh * c - yl * s], axis=-1)
    assert np.max(np.abs(back - x.astype(F64))) < 1e-5 * np.max(np.abs(x.astype(F64)))


def test_relative_position_invariance():
    """q at m and k at n: the rotated dot product depends on m - n only (up to FP32 rounding)."""
    rng = np.random.default_rng(15)
    d = 64
    q = _x16(rng, (1, 1, 1, d))
    k = _x16(rng, (1, 1, 1, d))
    cos32, sin32 = synth.rope_table(1e4, 600, d)
    dots = []
    for m, n in [(7, 3), (107, 103), (507, 503)]:
        qm = rope.apply_rope32(q, cos32, sin32, [m]).astype(F64)
        kn = rope.apply_rope32(k, cos32, sin32, [n]).astype(F64)
        dots.append(float(np.sum(qm * kn)))
    scale = float(np.sum(np.abs(q.astype(F64)) * np.abs(k.astype(F64))))
    assert max(dots) - min(dots) < 2e-4 * scale


def test_identity_tables_reduce_to_the_pinned_quantizer():
    cfg = synth.config(1, B=1, Hq=4, Hkv=2, Lq=40, Lk=70)
    q, k, v = synth.make_qkv(cfg)
    qc, kc = synth.make_calibration(cfg)
    from oracle import smooth
    s32, inv32, gate = smooth.calibrate(qc, kc, 0.5, 4.0)
    ones = np.ones((70, 64), F32)
    zeros = np.zeros((70, 64), F32)
    a = rope.quantize_qkv_rope(q, k, v, s32, inv32, ones, zeros)
    b = A.quantize_qkv(q, k, v, s32, inv32)
    for x, y in zip(a.packed(), b.packed()):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("cfg_id", [0, 1, 3])
def test_prologue_matches_rotation_then_quantization(cfg_id):
    """quantize_qkv_rope = apply_rope32 at the stated positions, then RN32 smoothing, then MX."""
    over = dict(B=1, Hq=4, Hkv=2, Lq=9, Lk=33) if cfg_id else {}
    cfg = synth.config(cfg_id, **over)
    theta = cfg["rope_theta"] or 1e4
    q, k, v = synth.make_qkv(cfg, pre_rope=True)
    qc, kc = synth.make_calibration(cfg)
    from oracle import mx, smooth
    s32, inv32, _ = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
    lq, lk, d = cfg["Lq"], cfg["Lk"], cfg["d"]
    cos32, sin32 = synth.rope_table(theta, lk, d)
    got = rope.quantize_qkv_rope(q, k, v, s32, inv32, cos32, sin32)
    group = cfg["Hq"] // cfg["Hkv"]
    qr = rope.apply_rope32(q, cos32, sin32, np.arange(lk - lq, lk))
    kr = rope.apply_rope32(k, cos32, sin32, np.arange(lk))
    qs = (qr.astype(F64) * np.asarray(s32)[np.arange(cfg["Hq"]) // group][None, :, None, :]).astype(F32)
    ks = (kr.astype(F64) * np.asarray(inv32)[None, :, None, :]).astype(F32)
    qcode, qe = mx.quantize_blocks(qs.astype(F64))
    kcode, ke = mx.quantize_blocks(ks.astype(F64))
    assert np.array_equal(got.qc, qcode) and np.array_equal(got.qe, qe)
    assert np.array_equal(got.kc, kcode) and np.array_equal(got.ke, ke)
    assert np.array_equal(got.vc, A.quantize_qkv(q, k, v).vc)
