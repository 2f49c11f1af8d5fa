"""Rotary position embedding in FP32 ahead of Smooth-QK and quantization (fused prologue).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[HiFA4] Abstract: Smooth-QK rescales Q and K per channel after RoPE, and at inference only an
element-wise scaling remains, which can be fused into the step before the attention kernel.
The pages do not define RoPE itself; the models they evaluate (Qwen3-8B, Gemma2-9B) use the
rotate-half form, and that is the reading here.

Readings (the pages fix none of this):
* rotate-half pairs (i, i + d/2), i < d/2, at position p with the FP32 table entries
  c = cos_tab[p, i], s = sin_tab[p, i] (the caller's cached tables, FP64 angles rounded once);
* each product and each sum is rounded once to FP32, no fused multiply-add:
      y_i       = RN32(RN32(x_i c)       - RN32(x_{i+d/2} s))
      y_{i+d/2} = RN32(RN32(x_{i+d/2} c) + RN32(x_i s));
* the rotated values stay in FP32 (the fusion removes the FP16 round trip), then
  Q' = RN32(y * s32) and K' = RN32(y * inv32) as in smooth.py, then the block quantization;
* positions: key t is at position t; query r at position r + Lk - Lq (bottom-right aligned,
  the same convention as the causal mask), so a decode query sits at Lk - 1.
"""

import numpy as np

from . import fp
from . import mx
from .attention import Quantized

F32 = np.float32
F64 = np.float64


def apply_rope32(x, cos32, sin32, positions):
    """Rotate-half RoPE of FP16 values x [..., L, d] at the given positions [L], in FP32 steps."""
    x = np.asarray(x)
    d = x.shape[-1]
    half = d // 2
    pos = np.asarray(positions, dtype=np.int64)
    c = np.asarray(cos32, dtype=F32)[pos]  # [L, d/2]
    s = np.asarray(sin32, dtype=F32)[pos]
    a = x[..., :half].astype(F32)  # FP16 -> FP32 is exact
    b = x[..., half:].astype(F32)
    ac = fp.mul32(a, c)
    bs = fp.mul32(b, s)
    bc = fp.mul32(b, c)
    as_ = fp.mul32(a, s)
    lo = fp.add32(ac, -bs)  # negation is exact
    hi = fp.add32(bc, as_)
    return np.concatenate([lo, hi], axis=-1).astype(F32)


def quantize_qkv_rope(q, k, v, s32, inv32, cos32, sin32):
    """RoPE (FP32), Smooth-QK (if scales are given) and 4-bit block quantization of pre-RoPE inputs.

    q [B, Hq, Lq, d], k, v [B, Hkv, Lk, d] hold FP16 values; cos32, sin32 are FP32 [n_pos, d/2]
    with n_pos >= Lk.  V is quantized exactly as in attention.quantize_qkv.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b, hq, lq, d = q.shape
    hkv, lk = k.shape[1], k.shape[2]
    group = hq // hkv
    qr = apply_rope32(q, cos32, sin32, np.arange(lk - lq, lk))
    kr = apply_rope32(k, cos32, sin32, np.arange(lk))
    if s32 is not None:
        sq = np.asarray(s32, dtype=F32)[np.arange(hq) // group]  # [Hq, d]
        qr = fp.mul32(qr, sq[None, :, None, :])
        kr = fp.mul32(kr, np.asarray(inv32, dtype=F32)[None, :, None, :])
    qc, qe = mx.quantize_blocks(qr.astype(F64))
    kc, ke = mx.quantize_blocks(kr.astype(F64))
    lk32 = -(-lk // 32) * 32
    vt = np.zeros((b, hkv, d, lk32), dtype=F64)
    vt[..., :lk] = np.swapaxes(v.astype(F64), 2, 3)
    vc, ve = mx.quantize_blocks(vt)
    return Quantized(qc, qe, kc, ke, vc, ve, lk)
