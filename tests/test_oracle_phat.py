"""Pins for P-hat (per-32-key block scales, the per-tile variant, Direct-P codes), the epsilon
tile statistics and the split-KV merge of the attention oracle.

[HiFA4] Abstract: P-hat is the 4-bit operand of the PV product; the library's 4-bit format has one
power-of-two scale per 32 elements along the contraction axis, i.e. per (query row, 32-key block).
Each check below compares the oracle with a hand derivation, an independent search, exact rational
arithmetic or plain scalar loops, never with a re-call of the function under test.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import attention as A
from oracle import mx
from test_oracle_attention import nearest_e2m1_code, rand_qkv
from test_oracle_fp import rn_fraction_to_f16, rn_fraction_to_f32

F32 = np.float32
F64 = np.float64
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _run(scores, v_vals, bc, phat_scale, phat_rule=A.PHAT_EXP16):
    """Level-P recurrence over FP32 log2-domain scores (C = 1); key c's V-hat is v_vals[c] in
    every channel, stored as code 2 (value 1) at block exponent log2 v (constant per 32 keys)."""
    r_n, n = scores.shape
    d = 32
    vh = np.full((d, n), 2, dtype=np.int64)
    exps = np.log2(np.asarray(v_vals, dtype=F64)).astype(np.int64)
    ve = np.repeat(exps.reshape(-1, 32)[:, 0][None, :], d, axis=0)
    vis = np.ones((r_n, n), dtype=bool)
    st = A.recurrence_p(scores.astype(F32), vis, vh, ve, F32(1.0), bc, A.P_REORDERED, 0, n // bc,
                        phat_scale=phat_scale, phat_rule=phat_rule)
    return st, A.finish(st, "P")


# ---------------------------------------------------------------- per-block scales: worked example

BLOCK0 = [0.0, -0.5, -1.0, -2.5, -3.0, -10.0] + [-40.0] * 26


def test_block32_worked_example():
    """Two 32-key blocks in one 64-key tile; block 1 is block 0 shifted by -6 in the log2 domain.

    Hand derivation (m = ceil(0) = 0):
    * block 0: e = ceil(0 - log2 6) = -2; 2^(u + 2) = 4, 2.83, 2, 0.707, 0.5, 2^-8 give the FP16
      probabilities 4, 2.828125, 2, 0.70703125, 0.5, 0.00390625 and the E2M1 codes 4, 3, 2, 0.5,
      0.5, 0 (2.83 lies above the midpoint 2.5, 0.707 below 0.75): P-hat = 1, .75, .5, .125, .125,
      0, sum 2.5;
    * block 1 with its own scale: e = ceil(-6 - log2 6) = -8, the same codes, sum 2.5 * 2^-6;
    * block 1 under one scale per tile (e = -2): 2^(u + 2) <= 2^-4 < 0.25, every code 0.
    With V = 1 on block 0 and V = 2 on block 1: per block, l = 2.5 + 0.0390625 = 2.5390625,
    O = 2.5 + 2 * 0.0390625 = 2.578125, out = fp16(2.578125 / 2.5390625) = 1040/1024; per tile
    l = O = 2.5, out = 1.  Softmax attention of these scores is (1 + 2^-5) / (1 + 2^-6).
    """
    scores = np.array([BLOCK0 + [x - 6.0 for x in BLOCK0]], dtype=F32)
    v_vals = [1.0] * 32 + [2.0] * 32
    st, out = _run(scores, v_vals, 64, A.PHAT_BLOCK32)
    assert st.m[0] == 0.0 and float(st.l[0]) == 2.5390625 and np.all(st.o[0].astype(F64) == 2.578125)
    assert np.all(out.astype(F64) == 1040 / 1024)
    st_t, out_t = _run(scores, v_vals, 64, A.PHAT_TILE)
    assert float(st_t.l[0]) == 2.5 and np.all(st_t.o[0].astype(F64) == 2.5) and np.all(out_t == 1.0)
    true = (1 + 2.0 ** -5) / (1 + 2.0 ** -6)
    assert abs(float(out[0, 0]) - true) < 3e-4 and abs(float(out_t[0, 0]) - true) > 0.015


def test_phat_tile_codes_and_exponents_worked_example():
    """The same block 0 plus log2-domain scores -1.7 and -1.2, where the two code rules differ.

    exp16: 2^0.3 -> FP16 1.2314 lies below the midpoint 1.25 (code 2, value 1); 2^0.8 -> 1.7412
    below 1.75 (code 3, value 1.5).  Direct-P: x = w + delta with delta = -0.0425; 2^0 * (1 + 0.2575)
    = 1.2575 rounds up to 1.5 (code 3); 1 + 0.7575 = 1.7575 rounds up to 2 (code 4).  The first six
    keys: x = 1.9575, 1.4575, 0.9575, -0.5425, -1.0425, -8.04 give 3.915, 2.915, 1.9575, 0.7288,
    0.4894, ~0 and the codes 4, 3, 2, 0.5, 0.5, 0 as under exp16.  Both rules: e = -2.
    """
    row = [0.0, -0.5, -1.0, -2.5, -3.0, -10.0, -1.7, -1.2] + [-40.0] * 24
    st = np.array([row], dtype=F32)
    vt = np.ones_like(st, dtype=bool)
    mm = np.zeros(1, dtype=F32)
    codes, eb, p16 = A.phat_tile(st, vt, F32(1.0), mm, 1, A.PHAT_BLOCK32, A.PHAT_EXP16)
    assert eb.tolist() == [[-2]]
    assert codes[0, :8].tolist() == [6, 5, 4, 1, 1, 0, 2, 3] and not codes[0, 8:].any()
    assert [float(x) for x in p16[0, :6]] == [4.0, 2.828125, 2.0, 0.70703125, 0.5, 0.00390625]
    codes_d, eb_d, p_d = A.phat_tile(st, vt, F32(1.0), mm, 1, A.PHAT_BLOCK32, A.PHAT_DIRECT)
    assert eb_d.tolist() == [[-2]] and p_d is None
    assert codes_d[0, :8].tolist() == [6, 5, 4, 1, 1, 0, 3, 4] and not codes_d[0, 8:].any()


# ---------------------------------------------------------------- per-block scales: brute force

def test_block32_codes_against_search_and_exact_exp2():
    """Per (row, 32-key block): the exponent is the smallest e with 6 * 2^e >= the block's largest
    exact probability (found by search) and each code is the nearest E2M1 value of 2^u / 2^e,
    except within 2^-8 (log2) of a midpoint or of an exponent boundary, where FP32/FP16 rounding
    may decide.  Masked keys give code 0 and a block without a visible key the exponent -127."""
    rng = np.random.default_rng(40)
    r_n, bc = 48, 128
    c32 = A.softmax_scale_log2(128)
    st = (rng.standard_normal((r_n, bc)) * rng.choice([2.0, 20.0, 60.0], (r_n, 1))).astype(F32)
    st += (rng.integers(-3, 3, (r_n, bc // 32)) * 30.0).repeat(32, axis=1).astype(F32)  # blocks far apart
    vt = rng.random((r_n, bc)) < 0.9
    vt[0, 32:64] = False  # a fully masked block
    u_max = np.max(np.where(vt, st.astype(F64) * float(c32), -np.inf), axis=1)
    mm = np.ceil(u_max).astype(F32)
    codes, eb, _ = A.phat_tile(st, vt, c32, mm, bc // 32)
    assert eb[0, 1] == -127 and not codes[0, 32:64].any()
    mids = np.log2([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    checked = 0
    for r in range(r_n):
        for j in range(bc // 32):
            sl = slice(32 * j, 32 * j + 32)
            if not vt[r, sl].any():
                assert eb[r, j] == -127
                continue
            u = st[r, sl].astype(F64) * float(c32) - float(mm[r])
            top = np.max(u[vt[r, sl]])
            e = 127
            while e > -127 and 6.0 * 2.0 ** (e - 1) >= 2.0 ** top:
                e -= 1
            if abs((top - math.log2(6.0)) - round(top - math.log2(6.0))) > 2.0 ** -8:
                assert eb[r, j] == e, (r, j)
            for i in range(32):
                c = 32 * j + i
                if not vt[r, c]:
                    assert codes[r, c] == 0
                    continue
                w = u[i] - eb[r, j]
                if np.min(np.abs(w - mids)) > 2.0 ** -8:
                    assert codes[r, c] == nearest_e2m1_code(2.0 ** w), (r, c)
                    checked += 1
    assert checked > 3000


# ---------------------------------------------------------------- Direct-P

def _nearest_f32(ref):
    x = F32(float(ref))
    cands = [np.nextafter(x, F32(-np.inf)), x, np.nextafter(x, F32(np.inf))]
    return min(cands, key=lambda c: abs(Decimal(float(c)) - ref))


def test_direct_constants_are_nearest_fp32():
    getcontext().prec = 60
    log2_15 = Decimal(3) / Decimal(2)
    log2_15 = log2_15.ln() / Decimal(2).ln()
    delta = Decimal(1) / Decimal(4) - log2_15 / 2
    assert A.DIRECT_DELTA == _nearest_f32(delta)
    assert A.DIRECT_TOP == _nearest_f32(delta - Decimal("2.5"))


def test_direct_value_is_the_linear_mantissa_exp2_bit_exactly():
    """z = 2^n (1 + f) with n + f = y / 2^23 - 127, y the single FP32 rounding of the exact
    s C 2^23 + K 2^23 and K = fp32(fp32(127 - big_m) + delta); the mantissa f is truncated to
    23 bits (exact rational arithmetic)."""
    rng = np.random.default_rng(41)
    n = 3000
    s = (rng.standard_normal(n) * 40).astype(F32)
    c32 = F32(rng.choice([A.softmax_scale_log2(64), A.softmax_scale_log2(128), A.softmax_scale_log2(256)]))
    big_m = np.round(s.astype(F64) * float(c32) + rng.uniform(-3, 6, n)).astype(F32)
    _, z = A.direct_codes(s, c32, big_m)
    delta = Fr(float(A.DIRECT_DELTA))
    for i in range(n):
        k = rn_fraction_to_f32(rn_fraction_to_f32(Fr(127) - Fr(float(big_m[i]))) + delta)
        y = rn_fraction_to_f32(Fr(float(s[i])) * Fr(float(c32)) * 2 ** 23 + Fr(float(k)) * 2 ** 23)
        yf = Fr(float(y))
        if yf <= 0:
            assert z[i] == 0.0
            continue
        t = math.floor(yf)
        x = Fr(t, 2 ** 23) - 127
        ex = math.floor(x)
        frac = x - ex
        want = Fr(2) ** ex * (1 + frac)
        assert Fr(float(z[i])) == want, (i, float(z[i]), float(want))


def test_direct_codes_are_log_domain_nearest():
    """For values >= 1 (x >= 0), the Direct-P code is the E2M1 value nearest in the log2 domain
    to 2^w: the boundaries sit at n + log2(1.5)/2 and n + (1 + log2 1.5)/2."""
    w = np.linspace(0.06, 2.49, 400001).astype(F32)
    codes, _ = A.direct_codes(w, F32(1.0), np.zeros_like(w))
    logs = np.log2([1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d = np.abs(w.astype(F64)[:, None] - logs[None, :])
    want = np.argmin(d, axis=1) + 2  # codes 2 .. 7
    srt = np.sort(d, axis=1)
    far = (srt[:, 1] - srt[:, 0]) > 1e-4  # K and y carry x with 2^-17 resolution
    assert far.sum() > 390000
    assert np.array_equal(codes[far], want[far])
    # the code never decreases as the score grows, anywhere in the range
    wide = np.linspace(-12.0, 2.5, 600001).astype(F32)
    cw, _ = A.direct_codes(wide, F32(1.0), np.zeros_like(wide))
    assert np.all(np.diff(cw.astype(int)) >= 0) and cw.max() <= 7


def test_direct_block_max_value_in_three_to_six():
    """The Direct-P block exponent puts every block maximum on code 5, 6 or 7 (value in (3, 6])."""
    rng = np.random.default_rng(42)
    st = (rng.standard_normal((64, 128)) * 30).astype(F32)
    vt = np.ones_like(st, dtype=bool)
    c32 = A.softmax_scale_log2(128)
    mm = np.ceil(np.max(st.astype(F64) * float(c32), axis=1)).astype(F32)
    codes, eb, _ = A.phat_tile(st, vt, c32, mm, 4, A.PHAT_BLOCK32, A.PHAT_DIRECT)
    for r in range(64):
        for j in range(4):
            sl = slice(32 * j, 32 * j + 32)
            top = int(np.argmax(st[r, sl]))
            if eb[r, j] > -127:
                assert codes[r, 32 * j + top] in (5, 6, 7)
                assert codes[r, sl].max() == codes[r, 32 * j + top]


# ---------------------------------------------------------------- epsilon statistics

def test_tile_stats_against_independent_sums():
    """Per (16-row block, key tile): sum of P-hat and of the FP16 probabilities P-tilde over the
    visible entries, recomputed by plain loops (exact rationals for every FP32 rounding, an
    independent E2M1 search, the per-block exponent rule), on a ragged causal case with
    Lq < Lk: three row blocks (the last of 5 rows) and three 64-key tiles (the last of 22 keys)."""
    rng = np.random.default_rng(43)
    lq, lk, d, bc = 37, 150, 64, 64
    q, k, v = rand_qkv(rng, 1, 1, 1, lq, lk, d, outlier=12.0)
    qq = A.quantize_qkv(q, k, v)
    got = {(rb, t): (sph, sp) for rb, t, sph, sp in A.tile_stats_p(qq, True, bc, 0, 0)}
    c = A.softmax_scale_log2(d)
    l6 = F32(math.log2(6.0))
    qv = mx.dequantize_blocks(qq.qc[0, 0], qq.qe[0, 0])
    kv = mx.dequantize_blocks(qq.kc[0, 0], qq.ke[0, 0])
    shift = lk - lq
    want = {}
    for r in range(lq):
        m = -math.inf
        for t in range(-(-lk // bc)):
            keys = [cc for cc in range(t * bc, min(lk, t * bc + bc)) if cc <= r + shift]
            if not keys:
                continue
            srow = {cc: float(np.dot(qv[r], kv[cc])) for cc in keys}
            assert all(F32(x) == x for x in srow.values())  # exact scores
            m = max(m, math.ceil(float(F32(F32(max(srow.values())) * c))))
            sph = sp = 0.0
            for b0 in range(t * bc, t * bc + bc, 32):
                blk = [cc for cc in keys if b0 <= cc < b0 + 32]
                if not blk:
                    continue
                v_top = rn_fraction_to_f32(Fr(max(srow[cc] for cc in blk)) * Fr(float(c)) - m)
                e = max(-127, math.ceil(float(F32(F32(v_top) - l6))))
                for cc in blk:
                    u = rn_fraction_to_f32(Fr(srow[cc]) * Fr(float(c)) - (m + e))
                    p16 = float(np.float16(math.pow(2.0, float(np.float16(u)))))
                    sph += E2M1[nearest_e2m1_code(p16)] * 2.0 ** e
                    sp += p16 * 2.0 ** e
            a = want.setdefault((r // 16, t), [0.0, 0.0])
            a[0] += sph
            a[1] += sp
    assert set(got) == set(want)
    for key, (sph, sp) in want.items():
        assert math.isclose(got[key][0], sph, rel_tol=1e-12) and math.isclose(got[key][1], sp, rel_tol=1e-12), key


def test_single_tile_inconsistent_scales_rows_by_phat_over_p():
    """Theorem 1 at Level P, one tile per row (Bc >= Lk): both normalizers share O, so each
    output row of the inconsistent formulation is the P-Reordered one times l_cons / l_incons,
    up to the FP16 rounding of the two quotients; with 16 rows in one statistics block, the
    block sums give the ratio of the summed normalizers."""
    rng = np.random.default_rng(44)
    q, k, v = rand_qkv(rng, 1, 1, 1, 16, 128, 64, outlier=10.0)
    qq = A.quantize_qkv(q, k, v)
    cons = A.attention_p(qq, False, 128, A.P_REORDERED).astype(F64)[0, 0]
    inc = A.attention_p(qq, False, 128, A.INCONSISTENT).astype(F64)[0, 0]
    (rb, t, sph, sp), = A.tile_stats_p(qq, False, 128, 0, 0)
    assert (rb, t) == (0, 0) and sph < sp  # net probability-mass loss on this tile
    big = np.abs(cons) > 0.05
    ratio = inc[big] / cons[big]
    rows = np.nonzero(big)[0]
    for r in np.unique(rows):
        rr = ratio[rows == r]
        assert np.max(rr) - np.min(rr) < 8e-3  # channel-independent up to FP16 rounding
    assert abs(np.median(ratio) - sph / sp) < 0.02


# ---------------------------------------------------------------- split-KV merge

def _replay_merge(parts):
    """Exact-rational replay of the FP16 merge: m = max; o = rn16(rn32(a1 o + rn32(a2 o_s)))
    with a1 = 2^(m - m_new) (0 while m = -inf), a2 = 2^(m_s - m_new); splits with m_s = -inf
    are skipped; out = rn16(rn32(o / l))."""
    m = -math.inf
    o = [np.float16(0)] * len(parts[0][2])
    l = np.float16(0)
    for ms, ls, os in parts:
        if ms == -math.inf:
            continue
        mn = max(m, ms)
        a1 = Fr(0) if m == -math.inf else Fr(2) ** int(m - mn)
        a2 = Fr(2) ** int(ms - mn)

        def step(old, new):  # rn16(rn32(a1 old + rn32(a2 new)))
            mo = Fr(float(rn_fraction_to_f32(a2 * Fr(float(new)))))
            return rn_fraction_to_f16(Fr(float(rn_fraction_to_f32(a1 * Fr(float(old)) + mo))))
        o = [step(oo, x) for oo, x in zip(o, os)]
        l = step(l, ls)
        m = mn
    return [rn_fraction_to_f16(Fr(float(rn_fraction_to_f32(Fr(float(oo)) / Fr(float(l)))))) for oo in o]


def test_merge_splits_bit_exact_against_rational_replay():
    rng = np.random.default_rng(45)
    d = 16
    cases = [[3, 10, -math.inf, 9], [-math.inf, 0, 0, -5], [7, -math.inf, -math.inf, 7], [2, -30, 1, 40],
             [-12, -11, -10, -9], [5, -140, 5, -math.inf]]
    for ms_list in cases:
        states = []
        for ms in ms_list:
            if ms == -math.inf:
                states.append(A.State(np.array([-np.inf], dtype=F32), np.zeros(1, dtype=np.float16),
                                      np.zeros((1, d), dtype=np.float16)))
            else:
                l = np.float16(rng.uniform(1, 60))
                o = (rng.standard_normal(d) * 20).astype(np.float16)
                states.append(A.State(np.array([ms], dtype=F32), np.array([l]), o[None, :]))
        got = A.finish(A.merge_splits(states), "P")[0]
        parts = [(float(s.m[0]), s.l[0], s.o[0]) for s in states]
        want = _replay_merge(parts)
        assert [float(x) for x in got] == [float(x) for x in want], ms_list
    # a single live split reproduces its own quotient
    st = A.State(np.array([4.0], dtype=F32), np.array([np.float16(3.0)]), np.array([[np.float16(1.5)] * d]))
    assert np.all(A.finish(A.merge_splits([st]), "P") == np.float16(0.5))
