"""Shared helpers for the GPU parity tests: run the HIP path and the oracle on the same inputs."""
import numpy as np

import bit_quantized_flashattention_amd as hf
from oracle import attention as A
from oracle import smooth

TOL = 2e-3  # max |GPU - oracle| <= TOL * RMS(oracle output)

NAMES = ["q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"]


def to_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def gpu_quantize(q, k, v, s, inv):
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sd = to_dev(s) if s is not None else None
    invd = to_dev(inv) if inv is not None else None
    return hf.quantize_qkv(qd, kd, vd, sd, invd)


def assert_codes_equal(res, qq):
    import torch
    torch.cuda.synchronize()
    for name, want in zip(NAMES, qq.packed()):
        got = res[name].cpu().numpy()
        assert got.shape == want.shape, (name, got.shape, want.shape)
        bad = np.count_nonzero(got != want)
        assert bad == 0, "%s: %d of %d bytes differ" % (name, bad, got.size)


def compare_out(got, want, label=""):
    """Tolerance check; returns (max_abs/rms, n_not_identical)."""
    got = np.asarray(got).astype(np.float64)
    want = np.asarray(want).astype(np.float64)
    assert np.all(np.isfinite(got)), label + ": non-finite output"
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.max(np.abs(got - want)))
    ndiff = int(np.count_nonzero(got != want))
    print("%s: max|d|/rms=%.3e  rms=%.4f  non-identical=%d/%d" % (label, err / rms, rms, ndiff, got.size))
    assert err <= TOL * rms, "%s: max|d| = %.3e > %.1e * rms (%.4f); %d elements differ" % (label, err, TOL, rms, ndiff)
    return err / rms, ndiff


def run_case(q, k, v, causal, kv_tile, normalizer=A.P_REORDERED, alpha=0.5, calib=None, num_splits=0,
             stats=False, smooth_on=True, max_rule=A.MAX_CEIL, phat_scale=A.PHAT_BLOCK32, phat_rule=A.PHAT_EXP16):
    """Product path (library calibrate + GPU quantize + GPU attention) and the oracle on the same inputs."""
    import torch
    b, hq, lq, d = q.shape
    hkv, lk = k.shape[1], k.shape[2]
    s = inv = None
    if smooth_on and calib is not None:
        s, inv, gate = hf.calibrate(calib[0], calib[1], alpha, 4.0)
        so, invo, gateo = smooth.calibrate(calib[0], calib[1], alpha, 4.0)
        assert gate == gateo and np.array_equal(s.view(np.uint32), so.view(np.uint32))
        if not gate:
            s = inv = None
    res = gpu_quantize(q, k, v, s, inv)
    qq = A.quantize_qkv(q, k, v, s, inv)
    assert_codes_equal(res, qq)
    dims = hf.make_dims(b, hq, hkv, d, lq, lk)
    splits_used = hf.decode_num_splits(dims, hf.make_opts(causal, normalizer, kv_tile, num_splits))
    r = hf.attention_fwd(res, dims, causal, normalizer, kv_tile, num_splits, tile_stats=True if stats else None,
                         max_rule=max_rule, phat_scale=phat_scale, phat_rule=phat_rule)
    out, st = (r if stats else (r, None))
    # the fused-Q entry point must reproduce the two-call path bit for bit
    kv_only = {n: res[n] for n in NAMES[2:]}
    r16 = hf.attention_fwd(kv_only, dims, causal, normalizer, kv_tile, num_splits, tile_stats=True if stats else None,
                           q16=(to_dev(q), to_dev(s) if s is not None else None), max_rule=max_rule,
                           phat_scale=phat_scale, phat_rule=phat_rule)
    out16, st16 = (r16 if stats else (r16, None))
    torch.cuda.synchronize()
    assert torch.equal(out16.view(torch.int16), out.view(torch.int16)), "fused-Q output differs"
    if stats:
        assert torch.equal(st16, st), "fused-Q tile statistics differ"
    diag = A.Diag()
    want = A.attention_p(qq, causal, kv_tile, normalizer, num_splits=splits_used if lq == 1 else 1, diag=diag,
                         max_rule=max_rule, phat_scale=phat_scale, phat_rule=phat_rule)
    # sums the matrix instructions cannot return exactly: there the accumulation model decides
    print("  inexact sums (oracle): scores %d/%d, PV %d/%d, l %d"
          % (diag.inexact_s, diag.total_s, diag.inexact_pv, diag.total_pv, diag.inexact_l))
    return out.cpu().numpy(), want, qq, diag, (st.cpu().numpy() if st is not None else None)
