"""GPU parity at the full benchmark sizes, in the launch configuration bench.py times.

Each workload is generated on the GPU at full size, calibrated by the library, quantized and
attended by the HIP path in one launch each.  The oracle then quantizes sampled (batch, head)
slices of the same FP16 inputs (codes and scales must match those slices of the GPU output bit
for bit) and computes query rows, which must equal the GPU's bit for bit (the tolerance check
max |d| <= 2e-3 * RMS is reported too):
* every row of one full (batch, head) of each prefill workload, so every tile class the kernel
  has (interior, causal diagonal, ragged) is compared at full size;
* one row from every 128-row query block of further heads;
* for decode, every query head of two batch entries.
Rows are independent in the recurrence, so the oracle's rows are spread over a pool of worker
processes.  Each case prints the oracle's count of sums that are not exactly representable in
FP32 (scores, PV, l): there the matrix instructions' accumulation order decides the result.
"""
import multiprocessing as mp
import os

import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
from oracle import attention as A
from oracle import smooth
import synth
from gpu_helpers import compare_out

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(len(os.sched_getaffinity(0)), 16))


def _oracle_rows(job):
    qq, h, rows, causal, kv_tile, normalizer, splits, phat_rule = job
    diag = A.Diag()
    out = A.attention_head_p(qq, 0, h, rows, causal, kv_tile, normalizer, num_splits=splits, diag=diag,
                             phat_rule=phat_rule)
    return out, (diag.inexact_s, diag.inexact_pv, diag.inexact_l, diag.total_pv)


def _block_rows(rng, lq, block=128):
    """One random row from every block of 128 query rows, plus the first and last rows."""
    rows = {0, lq - 1}
    for b0 in range(0, lq, block):
        rows.add(int(rng.integers(b0, min(lq, b0 + block))))
    return np.array(sorted(rows))


def run_full(cfg_id, heads, normalizer=A.P_REORDERED, causal=None, phat_rule=A.PHAT_EXP16, over=None):
    """heads: list of (batch, query head, all_rows); all_rows False takes a row per 128-row block.
    causal overrides the workload's mask (the bench's non-causal legs); phat_rule selects the
    P-hat code rule (the bench's Direct-P legs); over overrides workload fields (e.g. B)."""
    import torch
    cfg = dict(synth.config(cfg_id, **(over or {})))
    if causal is not None:
        cfg["causal"] = causal
    b_n, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    group = hq // hkv
    print("case full-size config", cfg_id, cfg["name"], "normalizer", normalizer, "causal", cfg["causal"],
          "phat_rule", phat_rule, flush=True)
    q, k, v = synth.make_qkv_device(cfg)
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    so, invo, gateo = smooth.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    assert gate == gateo and np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(inv.view(np.uint32), invo.view(np.uint32))
    dims = hf.make_dims(b_n, hq, hkv, d, lq, lk)
    res = hf.quantize_qkv(q, k, v, torch.from_numpy(s).cuda(), torch.from_numpy(inv).cuda(), dims=dims)
    splits = hf.decode_num_splits(dims, hf.make_opts(cfg["causal"], normalizer, cfg["kv_tile"], 0))
    out = hf.attention_fwd(res, dims, cfg["causal"], normalizer, cfg["kv_tile"], phat_rule=phat_rule)
    # the launch bench.py times: K-hat, V-hat from the quantizer, Q quantized inside the kernel
    out16 = hf.attention_fwd(res, dims, cfg["causal"], normalizer, cfg["kv_tile"],
                             q16=(q, torch.from_numpy(s).cuda()), phat_rule=phat_rule)
    torch.cuda.synchronize()
    assert torch.equal(out16.view(torch.int16), out.view(torch.int16)), "fused-Q output differs"
    rng = np.random.default_rng(7000 + cfg_id)
    # one oracle quantization per (batch, KV head) with the query heads of its group
    by_group = {}
    for b, h, all_rows in heads:
        by_group.setdefault((b, h // group), []).append((h, all_rows))
    jobs, meta = [], []
    for (b, g), hs in by_group.items():
        qh = q[b:b + 1, g * group:(g + 1) * group].cpu().numpy()
        kh = k[b:b + 1, g:g + 1].cpu().numpy()
        vh = v[b:b + 1, g:g + 1].cpu().numpy()
        qq = A.quantize_qkv(qh, kh, vh, so[g:g + 1], invo[g:g + 1])
        packed = qq.packed()
        for h, all_rows in hs:
            hl = h - g * group
            for name, want, head, want_head in zip(["q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"],
                                                   packed, [h, h, g, g, g, g], [hl, hl, 0, 0, 0, 0]):
                got = res[name][b, head].cpu().numpy()
                bad = np.count_nonzero(got != want[0, want_head])
                assert bad == 0, "config %d (b=%d, head %d) %s: %d bytes differ" % (cfg_id, b, head, name, bad)
            rows = np.arange(lq) if all_rows else _block_rows(rng, lq)
            chunks = [c for c in np.array_split(rows, max(1, min(len(rows), 4 * WORKERS))) if len(c)]
            for c in chunks:
                jobs.append((qq, hl, c, cfg["causal"], cfg["kv_tile"], normalizer, splits if lq == 1 else 1, phat_rule))
                meta.append((b, h, all_rows, c))
    with mp.get_context("spawn").Pool(WORKERS) as pool:
        results = pool.map(_oracle_rows, jobs, chunksize=1)
    totals = np.sum([r[1] for r in results], axis=0)
    n_rows = 0
    gots, wants = [], []
    for b, h, all_rows in heads:
        parts = [(m[3], r[0]) for m, r in zip(meta, results) if m[0] == b and m[1] == h and m[2] == all_rows]
        rows = np.concatenate([p[0] for p in parts])
        want = np.concatenate([p[1] for p in parts])
        got = out[b, h].cpu().numpy()[rows]
        n_rows += len(rows)
        if lq > 1:
            _, ndiff = compare_out(got, want, "full config %d b%d h%d %s (%d rows)"
                                   % (cfg_id, b, h, "all rows" if all_rows else "a row per 128-row block", len(rows)))
            assert ndiff == 0, "config %d b%d h%d: %d outputs differ from the oracle" % (cfg_id, b, h, ndiff)
        else:
            gots.append(got)
            wants.append(want)
    if gots:  # decode: one query row per head, compared together
        _, ndiff = compare_out(np.concatenate(gots), np.concatenate(wants), "full config %d, %d query heads" % (cfg_id, len(gots)))
        assert ndiff == 0, "config %d: %d outputs differ from the oracle" % (cfg_id, ndiff)
    print("config %d: %d rows compared; inexact sums (oracle): scores %d, PV %d of %d, l %d"
          % (cfg_id, n_rows, totals[0], totals[1], totals[3], totals[2]), flush=True)


def test_full_qwen_shaped_L2048():
    run_full(1, [(0, 13, True), (0, 0, False), (0, 31, False)])


@pytest.mark.parametrize("normalizer", [A.P_REORDERED, A.INCONSISTENT])
def test_full_batched_B8_L4096(normalizer):
    run_full(2, [(3, 17, True), (0, 0, False), (7, 31, False)], normalizer)


def test_full_batched_B8_L4096_direct_p():
    """The bench's direct_p leg: Direct-P codes at the batched workload."""
    run_full(2, [(5, 9, True), (1, 30, False)], phat_rule=A.PHAT_DIRECT)


@pytest.mark.parametrize("phat_rule", [A.PHAT_EXP16, A.PHAT_DIRECT])
def test_full_batched_B8_L4096_noncausal(phat_rule):
    """The bench's non-causal legs (both code rules): a row per 128-row block of two heads."""
    run_full(2, [(2, 6, False), (6, 27, False)], causal=False, phat_rule=phat_rule)


def test_full_gemma_shaped_d256_L8192():
    run_full(3, [(1, 14, True), (0, 1, False), (1, 0, False)])


def test_full_decode_B64_Lk32768():
    """Decode: every query head of batch entries 0 and 63 (a head's one row is its query)."""
    run_full(4, [(b, h, True) for b in (0, 63) for h in range(32)])


def test_full_length_decode_small_batch():
    """Decode at the full cache length with B = 2: automatic splits give 32 splits x 8 KV heads
    x 2 = 512 single-wave work-groups, at most one per SIMD, so the split kernel keeps three
    tiles in flight per wave; every query head of both batch entries."""
    run_full(4, [(b, h, True) for b in (0, 1) for h in range(32)], over=dict(B=2, name="decode-B2-Lk32768"))
