"""Smooth-QK: calibration-static per-channel rescaling of Q and K after RoPE.

[HiFA4] Abstract: Smooth-QK rescales Q and K channel by channel after RoPE,
leaving QK^T unchanged, so that the hard-to-quantize outliers of K move into
Q; the factors are fixed ahead of time from a little calibration data, so
inference adds only an element-wise multiply that fuses into the quantizer.  The abstract also
names an applicability gate that turns Smooth-QK off for some models and a
"mild smoothing" setting for Gemma2-9B, without giving formulas.

Readings (the pages give no formula):
* per (KV head g, channel j): a_K = max |K_cal| over tokens, a_Q = max |Q_cal|
  over tokens and over the query heads of group g;
* s = a_K**alpha / a_Q**(1 - alpha) (SmoothQuant-style migration strength
  alpha; alpha = 0.5 by default, a smaller alpha is the "mild" setting);
* gate: rho = max(a_K) / median(a_K) over all (g, j); Smooth-QK is on iff
  rho >= tau (tau = 4 by default); when off, or where a maximum is zero, s = 1;
* Q' = RN32(Q * s32), K' = RN32(K * inv32) with s32 = fp32(s) and
  inv32 = fp32(1 / s32) computed in FP64.
"""

import math

import numpy as np

F32 = np.float32
F64 = np.float64


def channel_maxima(q_cal, k_cal):
    """a_Q, a_K of shape [H_kv, d] from q_cal [H_q, N, d] and k_cal [H_kv, N, d]."""
    q = np.abs(np.asarray(q_cal, dtype=F64))
    k = np.abs(np.asarray(k_cal, dtype=F64))
    hq, n, d = q.shape
    hkv = k.shape[0]
    assert hq % hkv == 0
    group = hq // hkv
    a_k = k.max(axis=1)
    a_q = q.reshape(hkv, group, n, d).max(axis=(1, 2))
    return a_q, a_k


def calibrate(q_cal, k_cal, alpha=0.5, tau=4.0):
    """Returns (s32, inv32, gate_on) with s32, inv32 float32 [H_kv, d]."""
    a_q, a_k = channel_maxima(q_cal, k_cal)
    rho = a_k.max() / np.median(a_k) if np.median(a_k) > 0 else np.inf
    gate = bool(rho >= tau)
    s = np.ones_like(a_k)
    if gate:
        ok = (a_k > 0) & (a_q > 0)
        # the C library's pow, element by element
        for idx in zip(*np.nonzero(ok)):
            s[idx] = math.pow(a_k[idx], alpha) / math.pow(a_q[idx], 1.0 - alpha)
    s32 = s.astype(F32)
    inv32 = (1.0 / s32.astype(F64)).astype(F32)
    return s32, inv32, gate


def apply(x, scale32, head_to_group):
    """RN32(x * scale32[group(h), :]) for x [B, H, L, d] (FP16 values), one rounding per element."""
    x = np.asarray(x).astype(F32)
    sc = np.asarray(scale32, dtype=F32)[np.asarray(head_to_group)]  # [H, d]
    return (x.astype(F64) * sc[None, :, None, :].astype(F64)).astype(F32)
