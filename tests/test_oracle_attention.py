"""Pins for the attention oracle: textbook reductions, exact invariants, Theorem 1, brute force.

Every check here compares the oracle with something other than itself: the
textbook softmax formula, closed forms (V = 1 gives exactly 1; a causal first
row returns its own value), the scaling law of Theorem 1, the true exp2, exact
rational arithmetic, or an independent scalar-loop evaluation.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import fp, mx, smooth
import synth

F32 = np.float32


def rand_qkv(rng, b, hq, hkv, lq, lk, d, outlier=8.0):
    q = rng.standard_normal((b, hq, lq, d))
    k = rng.standard_normal((b, hkv, lk, d))
    k[..., 3] *= outlier
    k[..., d // 2 + 3] *= outlier
    v = rng.standard_normal((b, hkv, lk, d))
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


# ---------------------------------------------------------------- exp2 used for P-tilde

def test_exp2_cubic_passes_through_midpoints():
    g = lambda t: fp.fma32(fp.fma32(fp.fma32(A.EXP2_C3, t, A.EXP2_C2), t, A.EXP2_C1), t, F32(1))
    for v in (1.25, 1.5, 1.75):
        got = float(g(F32(math.log2(v))))
        assert abs(got - v) <= 4 * 2.0 ** -23, (v, got)
    n = np.arange(-149, 120)
    assert np.array_equal(A.exp2_x(n.astype(F32)), np.ldexp(F32(1), n.astype(np.int32)).astype(F32))


def test_exp2_close_to_true_exp2_and_monotone():
    w = np.linspace(-30, 3, 400001).astype(F32)
    x = A.exp2_x(w).astype(np.float64)
    rel = np.abs(x / np.exp2(w.astype(np.float64)) - 1)
    assert rel.max() < 5e-4
    inner = np.floor(w[1:]) == np.floor(w[:-1])
    assert np.all(np.diff(x)[inner] >= -1e-7 * x[1:][inner])


def test_p_codes_equal_rne_of_true_exp2_away_from_midpoints():
    w = np.linspace(-4, 2.6, 2_000_001).astype(F32)
    px = A.exp2_x(w).astype(np.float64)
    pt = np.exp2(w.astype(np.float64))
    for e in (-3, -2, -1, 0):
        cx = mx.rne_code(px * 2.0 ** -e)
        ct = mx.rne_code(pt * 2.0 ** -e)
        mids = np.log2(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 2.0 ** e)
        near = np.min(np.abs(w.astype(np.float64)[:, None] - mids[None, :]), axis=1) < 1e-6
        assert np.array_equal(cx[~near], ct[~near])
        assert (cx[near] != ct[near]).sum() <= near.sum()


# ---------------------------------------------------------------- matrix-instruction model

def test_mfma_seq_matches_sequential_fraction_rounding():
    from fractions import Fraction as Fr
    from test_oracle_fp import rn_fraction_to_f32
    rng = np.random.default_rng(8)
    n = 400
    blocks = [rng.integers(-4608, 4609, n) * np.exp2(rng.integers(-40, 40, n).astype(float)) for _ in range(4)]
    got, exact = A.mfma_seq(blocks)
    for i in range(n):
        acc = Fr(0)
        ok = True
        for b in blocks:
            tot = acc + Fr(float(b[i]))
            r = rn_fraction_to_f32(tot)
            ok &= Fr(float(r)) == tot
            acc = Fr(float(r))
        assert got[i] == F32(float(acc)) and exact[i] == ok


def test_scores_exact_for_small_scale_spread():
    from fractions import Fraction as Fr
    rng = np.random.default_rng(9)
    qc = rng.integers(0, 16, (6, 128)).astype(np.uint8)
    kc = rng.integers(0, 16, (9, 128)).astype(np.uint8)
    qe = rng.integers(-3, 3, (6, 4))
    ke = rng.integers(-3, 3, (9, 4))
    s, exact = A.scores_p(qc, qe, kc, ke)
    assert exact.all()
    qv = mx.dequantize_blocks(qc, qe)
    kv = mx.dequantize_blocks(kc, ke)
    for i in range(6):
        for j in range(9):
            ex = sum(Fr(float(a)) * Fr(float(b)) for a, b in zip(qv[i], kv[j]))
            assert Fr(float(s[i, j])) == ex


# ---------------------------------------------------------------- recurrence: textbook and closed forms

def softmax_attention(q, k, v, causal):
    s = q @ k.T / math.sqrt(q.shape[1])
    if causal:
        lq, lk = s.shape
        s = np.where(A.visibility(np.arange(lq), lq, lk, lk, True), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p @ v) / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("lq,lk,causal,bc,splits", [
    (64, 64, False, 64, 1), (100, 300, False, 64, 1), (200, 200, True, 128, 1), (37, 150, True, 64, 1),
    (1, 517, True, 128, 3), (1, 640, False, 64, 4), (96, 96, True, 64, 2)])
def test_identity_quantizer_is_textbook_attention(lq, lk, causal, bc, splits):
    rng = np.random.default_rng(lq * 7 + lk)
    d = 64
    q = rng.standard_normal((lq, d)) * 2
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, d))
    got = A.attention_s(q, k, v, causal, bc, quantize=False, round_state=False, num_splits=splits)
    assert np.allclose(got, softmax_attention(q, k, v, causal), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal,bc,lq,lk,splits", [
    (False, 64, 128, 128, 1), (True, 128, 256, 256, 1), (True, 64, 70, 200, 1), (False, 128, 33, 333, 1),
    (True, 128, 1, 700, 3)])
def test_v_all_ones_gives_exactly_one(causal, bc, lq, lk, splits):
    rng = np.random.default_rng(10)
    q, k, _ = rand_qkv(rng, 1, 2, 1, lq, lk, 64)
    v = np.ones((1, 1, lk, 64), dtype=np.float16)
    qq = A.quantize_qkv(q, k, v)
    out = A.attention_p(qq, causal, bc, A.P_REORDERED, num_splits=splits)
    assert np.all(out == 1.0)
    # the inconsistent normalizer does not give 1: it gives sum(P-hat)/sum(P) per row
    inc = A.attention_p(qq, causal, bc, A.INCONSISTENT, num_splits=splits)
    assert np.all(inc[..., 1:] == inc[..., :1]) and not np.all(inc == 1.0)


def test_causal_first_row_returns_its_value():
    rng = np.random.default_rng(11)
    q, k, v = rand_qkv(rng, 1, 2, 2, 96, 96, 64)
    qq = A.quantize_qkv(q, k, v)
    out = A.attention_p(qq, True, 64)
    vhat = mx.dequantize_blocks(qq.vc, qq.ve)  # [B, H, d, Lk32]
    for h in range(2):
        assert np.array_equal(out[0, h, 0].astype(np.float64), vhat[0, h, :, 0].astype(np.float16).astype(np.float64))


def test_theorem1_coherent_scaling():
    """Inconsistent normalizer: every channel of a row is scaled by the same factor sum(P-hat)/sum(P)."""
    rng = np.random.default_rng(12)
    d, lq, lk = 64, 50, 260
    q = rng.standard_normal((lq, d)) * 2
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, d))
    for bc, causal in ((64, True), (128, False), (512, False)):
        cons = A.attention_s(q, k, v, causal, bc, A.P_REORDERED, quantize=True, round_state=False)
        inc = A.attention_s(q, k, v, causal, bc, A.INCONSISTENT, quantize=True, round_state=False)
        ratio = inc / cons
        assert np.allclose(ratio, ratio[:, :1], rtol=1e-10)
        if bc >= lk:  # one tile: the factor is exactly sum(P-hat) / sum(P) = 1 + epsilon
            ones = A.attention_s(q, k, np.ones((lk, d)), causal, bc, A.INCONSISTENT, quantize=True, round_state=False)
            assert np.allclose(ones, ratio[:, :1], rtol=1e-10)


# ---------------------------------------------------------------- independent scalar evaluation

def scalar_attention_p(qq, b, h, causal, bc, mode):
    """Level P by plain loops over rows, tiles, blocks and elements."""
    from test_oracle_fp import rn_fraction_to_f32  # noqa: F401  (exactness helper is pinned there)
    hq, hkv = qq.qc.shape[1], qq.kc.shape[1]
    g = h // (hq // hkv)
    lq, d = qq.qc.shape[2], qq.qc.shape[3]
    lk = qq.lk
    c = A.softmax_scale_log2(d)
    qv = mx.code_half_units(qq.qc[b, h])
    kv = mx.code_half_units(qq.kc[b, g])
    vv = mx.code_half_units(qq.vc[b, g])
    out = np.zeros((lq, d), dtype=np.float16)
    ntiles = -(-lk // bc)
    for r in range(lq):
        def s_of(col):
            acc = 0.0
            for blk in range(d // 32):
                i = sum(int(qv[r, blk * 32 + t]) * int(kv[col, blk * 32 + t]) for t in range(32))
                val = math.ldexp(i, int(qq.qe[b, h, r, blk] + qq.ke[b, g, col, blk] - 2))
                acc = float(fp.rn32_sum(acc, val))
            return F32(acc)
        m = -math.inf
        l16 = np.float16(0)
        o16 = np.zeros(d, dtype=np.float16)
        for t in range(ntiles):
            keys = [cc for cc in range(t * bc, min(t * bc + bc, lk)) if (not causal or cc <= r + lk - lq)]
            if not keys:
                continue
            svals = {cc: s_of(cc) for cc in keys}
            tm = math.ceil(float(F32(float(max(svals.values())) * float(c))))
            m_new = max(m, tm)
            alpha = 0.0 if m == -math.inf else 2.0 ** (m - m_new)
            ptil = {cc: float(A.exp2_x(fp.fma32(svals[cc], c, F32(-m_new)))) for cc in keys}
            # one P-hat scale for the row in this tile, from the tile's largest score
            top = max(svals.values())
            e = int(mx.scale_exponent(np.array([float(A.exp2_x(fp.fma32(top, c, F32(-m_new))))]))[0])
            escale = {blk0: e for blk0 in range(t * bc, t * bc + bc, 32)}
            phat = {cc: int(mx.code_half_units(mx.rne_code(np.array([ptil[cc] * 2.0 ** -e])))[0]) for cc in keys}
            pv = np.zeros(d, dtype=F32)
            for ch in range(d):
                acc = 0.0
                for blk0 in range(t * bc, t * bc + bc, 32):
                    i = sum(phat.get(cc, 0) * int(vv[ch, cc]) for cc in range(blk0, blk0 + 32) if cc < vv.shape[1])
                    val = math.ldexp(i, escale[blk0] + int(qq.ve[b, g, ch, blk0 // 32]) - 2) if blk0 // 32 < qq.ve.shape[3] else 0.0
                    acc = float(fp.rn32_sum(acc, val))
                pv[ch] = acc
            acc = 0.0
            for blk0 in range(t * bc, t * bc + bc, 32):
                i = sum(2 * phat.get(cc, 0) for cc in range(blk0, blk0 + 32))
                acc = float(fp.rn32_sum(acc, math.ldexp(i, escale[blk0] - 2)))
            lsum = F32(acc)
            if mode == A.INCONSISTENT:
                parts = []
                for blk0 in range(t * bc, t * bc + 128, 32):
                    vals = [F32(ptil.get(cc, 0.0)) for cc in range(blk0, blk0 + 32)]
                    while len(vals) > 1:
                        h2 = len(vals) // 2
                        vals = [F32(vals[j] + vals[j + h2]) for j in range(h2)]
                    parts.append(vals[0] if blk0 < t * bc + bc else F32(0))
                lsum = F32(F32(parts[0] + parts[1]) + F32(parts[2] + parts[3]))
            for ch in range(d):
                o16[ch] = np.float16(fp.fma32(F32(alpha), F32(o16[ch]), pv[ch]))
            l16 = np.float16(fp.fma32(F32(alpha), F32(l16), lsum))
            m = m_new
        out[r] = (o16.astype(F32) / F32(l16)).astype(np.float16)
    return out


@pytest.mark.parametrize("mode", [A.P_REORDERED, A.INCONSISTENT])
def test_scalar_loops_match_vectorized(mode):
    rng = np.random.default_rng(13)
    q, k, v = rand_qkv(rng, 1, 2, 1, 24, 80, 64)
    qq = A.quantize_qkv(q, k, v)
    vec = A.attention_p(qq, True, 64, mode)
    for h in range(2):
        sc = scalar_attention_p(qq, 0, h, True, 64, mode)
        assert np.array_equal(sc, vec[0, h])


# ---------------------------------------------------------------- level P against level S, splits

def test_level_p_tracks_level_s_on_config0():
    cfg = synth.config(0)
    q, k, v = synth.make_qkv(cfg)
    qc, kc = synth.make_calibration(cfg)
    s, inv, gate = smooth.calibrate(qc, kc, cfg["alpha"])
    assert gate
    qq = A.quantize_qkv(q, k, v, s, inv)
    diag = A.Diag()
    outp = A.attention_p(qq, cfg["causal"], cfg["kv_tile"], diag=diag)
    qv = mx.dequantize_blocks(qq.qc, qq.qe)
    kv = mx.dequantize_blocks(qq.kc, qq.ke)
    vv = np.swapaxes(mx.dequantize_blocks(qq.vc, qq.ve), 2, 3)
    for h in range(2):
        outs = A.attention_s(qv[0, h], kv[0, h], vv[0, h], False, 64)
        delta = np.abs(outs.astype(np.float64) - outp[0, h].astype(np.float64))
        rms = np.sqrt(np.mean(outs.astype(np.float64) ** 2))
        assert np.mean(delta > 2e-3 * rms) < 0.01
        assert delta.max() < 0.1 * np.abs(outs).max()
    assert diag.inexact_s == 0


def test_splits_one_live_split_equals_unsplit_and_many_track():
    rng = np.random.default_rng(14)
    q, k, v = rand_qkv(rng, 1, 4, 1, 1, 128, 64)
    qq = A.quantize_qkv(q, k, v)
    base = A.attention_p(qq, True, 128)
    assert np.array_equal(A.attention_p(qq, True, 128, num_splits=4), base)  # one tile: splits 1..3 are empty
    q, k, v = rand_qkv(rng, 1, 4, 1, 1, 1024, 64)
    qq = A.quantize_qkv(q, k, v)
    base = A.attention_p(qq, True, 128).astype(np.float64)
    for s in (2, 3, 8):
        got = A.attention_p(qq, True, 128, num_splits=s).astype(np.float64)
        assert np.max(np.abs(got - base)) <= 4e-3 * np.abs(base).max()


def test_reference_fp32_matches_float64_textbook():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((40, 64))
    k = rng.standard_normal((90, 64))
    v = rng.standard_normal((90, 64))
    got = A.reference_fp32(q, k, v, True)
    assert np.allclose(got, softmax_attention(q, k, v, True), rtol=1e-4, atol=1e-5)
