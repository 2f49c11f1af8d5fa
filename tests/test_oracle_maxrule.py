"""Pins for the round-to-nearest running max (accuracy variant MAX_NEAREST16 of the oracle).

The method's reading keeps m = max over tiles of ceil(fp32(max S * C)), an integer; the variant
keeps the FP16 value nearest to fp32(max S * C) and rescales by the FP16 exp2 of the difference.
Each pin compares with something other than the recurrence itself:
* uniform tiles: every score of a tile equal, so P-hat is known in closed form and the output
  must match true softmax attention (a wrong sign or operand in alpha, or m rounded up, fails);
  the same input under the integer rule gives a value worked out by hand from the E2M1 grid;
* shift equivariance: adding a constant that keeps every quantity exact leaves the variant's
  output bit-identical (softmax is shift-invariant and m follows the true maximum), while the
  integer rule, whose grid is tied to integers, changes;
* the identity quantizer without state rounding reduces to textbook softmax attention.
"""
import math

import numpy as np

from oracle import attention as A
from oracle import fp

F32 = np.float32
F64 = np.float64


def _run(scores, v_vals, bc, rule):
    """Level-P recurrence over crafted FP32 log2-domain scores (C = 1) and V-hat values.

    scores [R, N] (N a multiple of bc), v_vals [N] in {0.5, 1, 2, ...}: every channel of key c holds
    v_vals[c] as code 2 (value 1) times 2^(log2 v), i.e. half units 2 and block exponent log2 v.
    """
    r_n, n = scores.shape
    d = 32
    vh = np.full((d, n), 2, dtype=np.int64)
    exps = np.log2(np.asarray(v_vals, dtype=F64)).astype(np.int64)
    assert np.all(2.0 ** exps == np.asarray(v_vals)) and np.all(exps.reshape(-1, 32) == exps.reshape(-1, 32)[:, :1])
    ve = np.repeat(exps.reshape(-1, 32)[:, 0][None, :], d, axis=0)
    vis = np.ones((r_n, n), dtype=bool)
    st = A.recurrence_p(scores.astype(F32), vis, vh, ve, F32(1.0), bc, A.P_REORDERED, 0, n // bc, max_rule=rule)
    return st, A.finish(st, "P")


def test_uniform_tiles_two_steps_worked_example():
    # tile 1: 32 keys with log2-score 0 and V = 1; tile 2: 32 keys with log2-score 0.7 and V = 2
    scores = np.concatenate([np.zeros(32), np.full(32, 0.7)])[None, :].astype(F32)
    v_vals = [1.0] * 32 + [2.0] * 32
    true = (1.0 + 2.0 * 2 ** 0.7) / (1.0 + 2 ** 0.7)  # softmax attention of these scores
    st, out = _run(scores, v_vals, 32, A.MAX_NEAREST16)
    assert st.m[0] == F32(np.float16(F32(0.7)))  # the FP16 value nearest to fp32(0.7)
    # P-hat of each tile is exactly its code 4 at scale 2^-2, so only the FP16 state rounds
    assert abs(float(out[0, 0]) - true) <= 1e-3 * true
    assert np.all(out == out[0, 0])
    # integer rule: m = 1, alpha = 1/2, tile 2's probability 2^(0.7 - 1 + 2) = 3.25 (FP16) lies
    # below the E2M1 midpoint 3.5 and becomes 3: O = 32/2 + 32 * (3/4) * 2 = 64, l = 16 + 24 = 40
    st_c, out_c = _run(scores, v_vals, 32, A.MAX_CEIL)
    assert st_c.m[0] == 1.0 and float(st_c.l[0]) == 40.0 and float(st_c.o[0, 0]) == 64.0
    assert float(out_c[0, 0]) == float(np.float16(1.6))


def test_uniform_tiles_three_steps_against_softmax():
    # three rising, non-integer tile maxima: two non-power-of-two rescales of the FP16 state
    lv = [0.0, 0.7, 1.9]
    vv = [1.0, 2.0, 0.5]
    scores = np.concatenate([np.full(32, x) for x in lv])[None, :].astype(F32)
    v_vals = sum(([v] * 32 for v in vv), [])
    w = [2.0 ** x for x in lv]
    true = sum(wi * vi for wi, vi in zip(w, vv)) / sum(w)
    _, out = _run(scores, v_vals, 32, A.MAX_NEAREST16)
    assert abs(float(out[0, 0]) - true) <= 2e-3 * true
    # a falling maximum leaves m (and alpha = 1) alone
    scores2 = np.concatenate([np.full(32, x) for x in [1.9, 0.7, 0.0]])[None, :].astype(F32)
    v2 = sum(([v] * 32 for v in vv[::-1]), [])
    st2, out2 = _run(scores2, v2, 32, A.MAX_NEAREST16)
    assert st2.m[0] == F32(np.float16(F32(1.9)))
    true2 = sum(wi * vi for wi, vi in zip(w[::-1], vv[::-1])) / sum(w)
    assert abs(float(out2[0, 0]) - true2) <= 8e-2 * true2  # P-hat quantization error only (~4 %)


def test_shift_equivariance_of_the_nearest_rule():
    rng = np.random.default_rng(71)
    r_n, n, bc = 16, 128, 32
    # log2-domain scores on a 1/64 grid in (-6, 6): exact in FP16, and stay exact after the shift
    scores = (rng.integers(-380, 380, size=(r_n, n)) / 64.0).astype(F32)
    v_vals = np.repeat(2.0 ** rng.integers(-1, 2, size=n // 32), 32)
    _, base = _run(scores, v_vals, bc, A.MAX_NEAREST16)
    _, base_c = _run(scores, v_vals, bc, A.MAX_CEIL)
    changed = 0
    for delta in (0.375, -1.5, 2.0 + 5.0 / 64):
        _, shifted = _run(scores + F32(delta), v_vals, bc, A.MAX_NEAREST16)
        assert np.array_equal(shifted.view(np.uint16), base.view(np.uint16)), delta
        _, shifted_c = _run(scores + F32(delta), v_vals, bc, A.MAX_CEIL)
        changed += int(np.count_nonzero(shifted_c.view(np.uint16) != base_c.view(np.uint16)))
    assert changed > 0  # the integer rule's grid moves with a fractional shift


def test_textbook_reduction_for_any_rule():
    rng = np.random.default_rng(72)
    lq, lk, d = 40, 200, 64
    q = rng.standard_normal((lq, d)) * 2
    k = rng.standard_normal((lk, d)) * 2
    v = rng.standard_normal((lk, d))
    s = q @ k.T / math.sqrt(d)
    mask = np.arange(lk)[None, :] <= np.arange(lq)[:, None] + (lk - lq)
    s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p @ v) / p.sum(axis=1, keepdims=True)
    for rule in (A.MAX_CEIL, A.MAX_NEAREST16):
        for bc in (64, 128):
            got = A.attention_s(q, k, v, True, bc, quantize=False, round_state=False, max_rule=rule)
            assert np.max(np.abs(got - ref)) < 1e-12


def test_nearest_rule_alpha_is_the_fp16_exp2_of_the_fp32_difference():
    # two tiles whose maxima differ by a value that is not a multiple of 2^-10: the FP32
    # difference and its FP16 rounding both matter; alpha must be rn16(2^rn16(m1 - m2))
    s1, s2 = F32(0.123), F32(3.456)
    scores = np.concatenate([np.full(32, s1), np.full(32, s2)])[None, :].astype(F32)
    v_vals = [1.0] * 64
    st, out = _run(scores, v_vals, 32, A.MAX_NEAREST16)
    m1 = F32(np.float16(s1))
    m2 = F32(np.float16(s2))
    assert st.m[0] == m2
    diff = F32(F64(m1) - F64(m2))
    alpha = np.float16(2.0 ** F64(np.float16(diff)))
    # tile 1 alone: O = l = rn16(32 * p1) with p1 = P-hat of the uniform tile; then
    # l = fma16(alpha, l1, rn16(32 * p2)); V = 1 makes O and l identical
    assert float(out[0, 0]) == 1.0
    l1 = np.float16(32 * 1.0)  # code 4 at scale 2^-2: P-hat = 1 for a uniform tile under this rule
    want_l = fp.fma16(alpha, l1, np.float16(32 * 1.0))
    assert st.l[0] == want_l
