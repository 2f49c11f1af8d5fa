"""GPU parity of the fused RoPE prologue (hifa4_quantize_qkv_rope) against oracle/rope.py.

Pre-RoPE FP16 inputs and the FP32 RoPE tables go to both sides; every code and scale byte must
match, and the attention computed from the GPU's codes must match the oracle's attention of the
oracle's codes (max |d| <= 2e-3 * RMS).  Full size: the batched prefill workload's K and Q,
compared on sampled (batch, head) slices.
"""
import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
from oracle import attention as A
from oracle import rope
from oracle import smooth
import synth
from gpu_helpers import NAMES, assert_codes_equal, compare_out, to_dev

pytestmark = pytest.mark.gpu


def _case(cfg_id, causal, kv_tile, smooth_qk=True, **over):
    import torch
    cfg = synth.config(cfg_id, **over)
    theta = cfg["rope_theta"] or 1e4
    q, k, v = synth.make_qkv(cfg, pre_rope=True)
    qc, kc = synth.make_calibration(cfg)
    s32, inv32, gate = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
    if not smooth_qk:
        s32 = inv32 = None
    cos32, sin32 = synth.rope_table(theta, cfg["Lk"], cfg["d"])
    print("case rope", cfg_id, over, "smooth" if smooth_qk else "no smooth", flush=True)
    sd = to_dev(s32) if s32 is not None else None
    invd = to_dev(inv32) if inv32 is not None else None
    res = hf.quantize_qkv_rope(to_dev(q), to_dev(k), to_dev(v), sd, invd, to_dev(cos32), to_dev(sin32))
    qq = rope.quantize_qkv_rope(q, k, v, s32, inv32, cos32, sin32)
    assert_codes_equal(res, qq)
    dims = hf.make_dims(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["Lq"], cfg["Lk"])
    splits = hf.decode_num_splits(dims, hf.make_opts(causal, 0, kv_tile, 0))
    out = hf.attention_fwd(res, dims, causal, 0, kv_tile)
    torch.cuda.synchronize()
    want = A.attention_p(qq, causal, kv_tile, 0, num_splits=splits if cfg["Lq"] == 1 else 1)
    compare_out(out.cpu().numpy(), want, "rope-%d" % cfg_id)
    # decode: the fused-Q entry point rotates the pre-RoPE query in its prologue, bit-identically;
    # prefill refuses the tables (the streaming RoPE quantizer is the faster route there)
    kv_only = {n: res[n] for n in NAMES[2:]}
    q16 = (to_dev(q), sd, to_dev(cos32), to_dev(sin32))
    if cfg["Lq"] == 1:
        out16 = hf.attention_fwd(kv_only, dims, causal, 0, kv_tile, q16=q16)
        torch.cuda.synchronize()
        assert torch.equal(out16.view(torch.int16), out.view(torch.int16)), "fused-Q RoPE output differs"
    else:
        with pytest.raises(hf.Hifa4Error):
            hf.attention_fwd(kv_only, dims, causal, 0, kv_tile, q16=q16)


def test_rope_tiny_noncausal_d64():
    _case(0, False, 64)


def test_rope_qwen_shaped_reduced():
    _case(1, True, 128, B=2, Hq=8, Hkv=2, Lq=300, Lk=300)


def test_rope_ragged_more_keys_than_queries():
    _case(1, True, 64, B=1, Hq=4, Hkv=1, Lq=77, Lk=333)


def test_rope_gemma_shaped_d256():
    _case(3, True, 128, B=1, Hq=4, Hkv=2, Lq=200, Lk=200)


def test_rope_decode_query():
    _case(1, True, 128, B=3, Hq=8, Hkv=2, Lq=1, Lk=1000)


def test_rope_decode_d64_and_d256():
    _case(0, True, 64, B=2, Hq=4, Hkv=2, Lq=1, Lk=200)
    _case(3, True, 128, B=2, Hq=8, Hkv=2, Lq=1, Lk=300)


def test_rope_wide_group_d256():
    # 64 query heads share each Smooth-QK row at d = 256; 24 positions, fewer than one
    # work-group's 32
    _case(3, False, 128, B=1, Hq=128, Hkv=2, Lq=24, Lk=24)


def test_rope_without_smooth_qk_one_past_a_work_group():
    # no Smooth-QK tables (rotation and quantization only); 129 positions at d = 128: a
    # work-group takes 128, so the second one has a single live row and pads K's scale planes
    # to 160
    _case(1, True, 128, smooth_qk=False, B=2, Hq=8, Hkv=2, Lq=129, Lk=129)
    _case(0, False, 64, smooth_qk=False, B=1, Hq=2, Hkv=2, Lq=257, Lk=257)


def test_rope_one_launch_equals_separate_calls():
    """Given Q, K and V, the entry point quantizes all three in one launch; given one tensor per
    call, it launches that tensor's quantizer alone.  Both routes must write the same bytes."""
    import torch
    for cfg_id, d in ((0, 64), (1, 128), (3, 256)):
        cfg = synth.config(cfg_id, B=2, Hq=8, Hkv=2, Lq=70, Lk=190, d=d)
        theta = cfg["rope_theta"] or 1e4
        q, k, v = synth.make_qkv(cfg, pre_rope=True)
        qc, kc = synth.make_calibration(cfg)
        s32, inv32, _ = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
        cos32, sin32 = synth.rope_table(theta, cfg["Lk"], d)
        print("case rope one launch vs separate, d", d, flush=True)
        dims = hf.make_dims(2, 8, 2, d, 70, 190)
        t = dict(q=to_dev(q), k=to_dev(k), v=to_dev(v))
        tabs = dict(s=to_dev(s32), inv_s=to_dev(inv32), rope_cos=to_dev(cos32), rope_sin=to_dev(sin32), dims=dims)
        all3 = hf.quantize_qkv_rope(t["q"], t["k"], t["v"], **tabs)
        for src in ("q", "k", "v"):
            one = hf.quantize_qkv_rope(**{n: (t[n] if n == src else None) for n in ("q", "k", "v")}, **tabs)
            torch.cuda.synchronize()
            for name in NAMES:
                if name[0] == src:
                    assert torch.equal(one[name], all3[name]), "%s differs (d = %d)" % (name, d)


def test_rope_full_size_batched_prefill():
    import torch
    cfg = synth.config(2)
    b_n, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    print("case rope full size config 2", flush=True)
    q, k, v = synth.make_qkv_device(cfg, pre_rope=True)
    qc, kc = synth.make_calibration(cfg)
    s32, inv32, gate = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
    cos32, sin32 = synth.rope_table(cfg["rope_theta"], lk, d)
    res = hf.quantize_qkv_rope(q, k, v, to_dev(s32), to_dev(inv32), to_dev(cos32), to_dev(sin32))
    torch.cuda.synchronize()
    group = hq // hkv
    for (b, h) in [(0, 0), (3, 17), (7, 31)]:
        g = h // group
        qh = q[b:b + 1, h:h + 1].cpu().numpy()
        kh = k[b:b + 1, g:g + 1].cpu().numpy()
        vh = v[b:b + 1, g:g + 1].cpu().numpy()
        qq = rope.quantize_qkv_rope(qh, kh, vh, s32[g:g + 1], inv32[g:g + 1], cos32, sin32)
        for name, want, head in zip(NAMES, qq.packed(), [h, h, g, g, g, g]):
            got = res[name][b, head].cpu().numpy()
            bad = np.count_nonzero(got != want[0, 0])
            assert bad == 0, "(b=%d, head %d) %s: %d bytes differ" % (b, head, name, bad)
