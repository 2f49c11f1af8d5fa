"""GPU parity of the 4-bit KV-cache append (hifa4_cache_append) and of attention over a cache.

Keys are appended in uneven chunks (single keys, partial and whole 32-key blocks, several blocks
at once).  After every append the first L keys of the cache must equal the oracle's quantization
of those L keys byte for byte (the V-hat blocks re-quantized from the FP16 stage), and decode and
prefill attention read through the cache's capacity strides must match the oracle on the prefix.
"""
import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
from oracle import attention as A
from oracle import rope
from oracle import smooth
import synth
from gpu_helpers import compare_out, to_dev

pytestmark = pytest.mark.gpu

CHUNKS = [1, 5, 26, 1, 31, 32, 33, 71]  # 200 keys


def _check_prefix(cache, qq, lk):
    import torch
    torch.cuda.synchronize()
    packed = qq.packed()  # q_codes, q_scales, k_codes, k_scales, v_codes, v_scales of the prefix
    lk32 = -(-lk // 32) * 32
    kc = cache["k_codes"][:, :, :lk].cpu().numpy()
    ks = cache["k_scales"][:, :, :, :lk].cpu().numpy()
    vc = cache["v_codes"][:, :, :lk32 // 32].cpu().numpy()
    vs = cache["v_scales"][:, :, :lk32 // 32].cpu().numpy()
    assert np.array_equal(kc, packed[2]), "k_codes differ at L=%d" % lk
    assert np.array_equal(ks, packed[3][..., :lk]), "k_scales differ at L=%d" % lk
    assert np.array_equal(vc, packed[4]), "v_codes differ at L=%d" % lk
    assert np.array_equal(vs, packed[5]), "v_scales differ at L=%d" % lk


@pytest.mark.parametrize("cfg_id,d,use_rope", [(1, 128, False), (1, 128, True), (0, 64, True), (3, 256, False)])
def test_append_in_chunks_matches_whole_sequence(cfg_id, d, use_rope):
    import torch
    total = sum(CHUNKS)
    cfg = synth.config(cfg_id, B=2, Hq=8, Hkv=2, Lq=1, Lk=total, d=d)
    theta = cfg["rope_theta"] or 1e4
    q, k, v = synth.make_qkv(cfg, pre_rope=use_rope)
    qc, kc = synth.make_calibration(cfg)
    s32, inv32, _ = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
    cos32, sin32 = synth.rope_table(theta, total, d)
    print("case cache append cfg", cfg_id, "d", d, "rope", use_rope, flush=True)
    capacity = 250  # not a multiple of 32: the strides round it up
    cache = hf.make_cache(2, 2, d, capacity)
    kd, vd = to_dev(k), to_dev(v)
    invd = to_dev(inv32)
    cosd, sind = (to_dev(cos32), to_dev(sin32)) if use_rope else (None, None)
    lk = 0
    for n in CHUNKS:
        kn = kd[:, :, lk:lk + n].contiguous()
        vn = vd[:, :, lk:lk + n].contiguous()
        lk = hf.cache_append(cache, kn, vn, invd, cosd, sind)
        qpre = q  # one decode query, at position lk - 1
        if use_rope:
            qq = rope.quantize_qkv_rope(qpre, k[:, :, :lk], v[:, :, :lk], s32, inv32, cos32, sin32)
        else:
            qq = A.quantize_qkv(qpre, k[:, :, :lk], v[:, :, :lk], s32, inv32)
        _check_prefix(cache, qq, lk)
    # decode over the cache: the fused-Q path (with the query's RoPE when the keys had it)
    dims = hf.make_dims(2, 8, 2, d, 1, lk)
    q16 = (to_dev(q), to_dev(s32), cosd, sind) if use_rope else (to_dev(q), to_dev(s32))
    out = hf.attention_fwd(cache, dims, True, 0, 128, 3, q16=q16, kv_capacity=capacity)
    torch.cuda.synchronize()
    want = A.attention_p(qq, True, 128, 0, num_splits=3)
    compare_out(out.cpu().numpy(), want, "cache-decode-d%d" % d)


def test_prefill_reads_through_cache_strides():
    """Causal prefill over keys held in a larger cache (capacity strides, ragged length)."""
    import torch
    lk = 333
    cfg = synth.config(1, B=1, Hq=4, Hkv=2, Lq=77, Lk=lk)
    q, k, v = synth.make_qkv(cfg)
    qc, kc = synth.make_calibration(cfg)
    s32, inv32, _ = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
    print("case prefill through cache strides", flush=True)
    cache = hf.make_cache(1, 2, 128, 1000)
    hf.cache_append(cache, to_dev(k), to_dev(v), to_dev(inv32))
    qq = A.quantize_qkv(q, k, v, s32, inv32)
    _check_prefix(cache, qq, lk)
    res = hf.quantize_qkv(to_dev(q), None, None, to_dev(s32), to_dev(inv32),
                          dims=hf.make_dims(1, 4, 2, 128, 77, lk))
    qkv = {"q_codes": res["q_codes"], "q_scales": res["q_scales"]}
    qkv.update({n: cache[n] for n in ("k_codes", "k_scales", "v_codes", "v_scales")})
    for kv_tile in (64, 128):
        out = hf.attention_fwd(qkv, hf.make_dims(1, 4, 2, 128, 77, lk), True, 0, kv_tile, kv_capacity=1000)
        torch.cuda.synchronize()
        want = A.attention_p(qq, True, kv_tile, 0)
        compare_out(out.cpu().numpy(), want, "cache-prefill-%d" % kv_tile)
