"""GPU parity at the full benchmark sizes, in the launch configuration bench.py times.

Each workload is generated on the GPU at full size, calibrated by the library, quantized and
attended by the HIP path in one launch each.  The oracle then quantizes sampled (batch, head)
slices of the same FP16 inputs (codes and scales must match those slices of the GPU output bit
for bit) and computes sampled query rows one by one (max |d| <= 2e-3 * RMS of the oracle rows).
"""
import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
from oracle import attention as A
from oracle import smooth
import synth
from gpu_helpers import compare_out

pytestmark = pytest.mark.gpu


def _sample_rows(rng, lq, kv_tile, n):
    """First and last rows, rows at tile edges, and random rows."""
    rows = {0, lq - 1}
    for t in (1, lq // kv_tile // 2, lq // kv_tile - 1):
        if 0 < t * kv_tile < lq:
            rows.update({t * kv_tile - 1, t * kv_tile})
    rows.update(int(r) for r in rng.choice(lq, size=min(n, lq), replace=False))
    return np.array(sorted(r for r in rows if 0 <= r < lq))


def _slice_bytes(res, name, b, head):
    return res[name][b, head].cpu().numpy()


def run_full(cfg_id, heads, n_rows, normalizer=A.P_REORDERED):
    import torch
    cfg = synth.config(cfg_id)
    b_n, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    group = hq // hkv
    print("case full-size config", cfg_id, cfg["name"], "normalizer", normalizer, flush=True)
    q, k, v = synth.make_qkv_device(cfg)
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    so, invo, gateo = smooth.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    assert gate == gateo and np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(inv.view(np.uint32), invo.view(np.uint32))
    dims = hf.make_dims(b_n, hq, hkv, d, lq, lk)
    res = hf.quantize_qkv(q, k, v, torch.from_numpy(s).cuda(), torch.from_numpy(inv).cuda(), dims=dims)
    splits = hf.decode_num_splits(dims, hf.make_opts(cfg["causal"], normalizer, cfg["kv_tile"], 0))
    out = hf.attention_fwd(res, dims, cfg["causal"], normalizer, cfg["kv_tile"])
    # the launch bench.py times: K-hat, V-hat from the quantizer, Q quantized inside the kernel
    out16 = hf.attention_fwd(res, dims, cfg["causal"], normalizer, cfg["kv_tile"],
                             q16=(q, torch.from_numpy(s).cuda()))
    torch.cuda.synchronize()
    assert torch.equal(out16.view(torch.int16), out.view(torch.int16)), "fused-Q output differs"
    rng = np.random.default_rng(7000 + cfg_id)
    worst = 0.0
    for (b, h) in heads:
        g = h // group
        qh = q[b:b + 1, h:h + 1].cpu().numpy()
        kh = k[b:b + 1, g:g + 1].cpu().numpy()
        vh = v[b:b + 1, g:g + 1].cpu().numpy()
        qq = A.quantize_qkv(qh, kh, vh, so[g:g + 1], invo[g:g + 1])
        want_bytes = qq.packed()
        for name, want, head in zip(["q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"],
                                    want_bytes, [h, h, g, g, g, g]):
            got = _slice_bytes(res, name, b, head)
            bad = np.count_nonzero(got != want[0, 0])
            assert bad == 0, "config %d (b=%d, head %d) %s: %d bytes differ" % (cfg_id, b, head, name, bad)
        rows = _sample_rows(rng, lq, cfg["kv_tile"], n_rows)
        want = A.attention_head_p(qq, 0, 0, rows, cfg["causal"], cfg["kv_tile"], normalizer,
                                  num_splits=splits if lq == 1 else 1)
        got = out[b, h].cpu().numpy()[rows]
        r, _ = compare_out(got, want, "full config %d b%d h%d rows %d" % (cfg_id, b, h, len(rows)))
        worst = max(worst, r)
    return worst


def test_full_qwen_shaped_L2048():
    run_full(1, [(0, 0), (0, 13), (0, 31)], 24)


@pytest.mark.parametrize("normalizer", [A.P_REORDERED, A.INCONSISTENT])
def test_full_batched_B8_L4096(normalizer):
    run_full(2, [(0, 0), (3, 17), (7, 31)], 16, normalizer)


def test_full_gemma_shaped_d256_L8192():
    run_full(3, [(0, 1), (1, 14)], 12)


def test_full_decode_B64_Lk32768():
    run_full(4, [(0, 0), (17, 5), (63, 31)], 1)
