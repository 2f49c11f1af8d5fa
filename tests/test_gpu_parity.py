"""GPU parity: the HIP path through the C ABI against the oracle, on seeded synthetic inputs.

4-bit codes and scales must match bit for bit; attention outputs within max|d| <= 2e-3 * RMS of
the oracle output.  Sizes span several tiles and ragged tails; edge cases cover GQA groups,
d in {64, 128, 256}, both normalizers, both tile widths, causal with Lq < Lk and split-KV decode.
"""
import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
from oracle import attention as A
from oracle import mx
import synth
from gpu_helpers import compare_out, run_case, gpu_quantize, assert_codes_equal, to_dev

pytestmark = pytest.mark.gpu


def gen(cfg_id, **over):
    cfg = synth.config(cfg_id, **over)
    q, k, v = synth.make_qkv(cfg)
    return cfg, q, k, v, synth.make_calibration(cfg)


def test_library_loads_on_gpu():
    import torch
    assert torch.cuda.is_available()
    hf.lib()


def test_config0_full():
    cfg, q, k, v, cal = gen(0)
    print("case config0", flush=True)
    got, want, qq, diag, _ = run_case(q, k, v, cfg["causal"], cfg["kv_tile"], calib=cal, alpha=cfg["alpha"])
    compare_out(got, want, "config0")
    assert diag.inexact_s == 0


@pytest.mark.parametrize("normalizer", [A.P_REORDERED, A.INCONSISTENT])
def test_qwen_shaped_reduced(normalizer):
    cfg, q, k, v, cal = gen(1, B=1, Hq=8, Hkv=2, Lq=384, Lk=384)
    print("case qwen-reduced norm", normalizer, flush=True)
    got, want, qq, diag, _ = run_case(q, k, v, True, 128, normalizer, calib=cal)
    compare_out(got, want, "qwen-reduced")


@pytest.mark.parametrize("kv_tile", [64, 128])
def test_ragged_noncausal_no_gqa(kv_tile):
    cfg, q, k, v, cal = gen(1, B=2, Hq=2, Hkv=2, Lq=100, Lk=300)
    print("case ragged kv_tile", kv_tile, flush=True)
    got, want, *_ = run_case(q, k, v, False, kv_tile, calib=cal)
    compare_out(got, want, "ragged-%d" % kv_tile)


def test_causal_bottom_right_d64():
    cfg, q, k, v, cal = gen(0, B=1, Hq=4, Hkv=2, Lq=77, Lk=333)
    print("case causal-br d64", flush=True)
    got, want, *_ = run_case(q, k, v, True, 64, calib=cal)
    compare_out(got, want, "causal-br-d64")


@pytest.mark.parametrize("normalizer", [A.P_REORDERED, A.INCONSISTENT])
def test_gemma_shaped_d256(normalizer):
    cfg, q, k, v, cal = gen(3, B=1, Hq=4, Hkv=2, Lq=300, Lk=300)
    print("case gemma-d256 norm", normalizer, flush=True)
    got, want, *_ = run_case(q, k, v, True, 128, normalizer, alpha=0.25, calib=cal)
    compare_out(got, want, "gemma-d256")


def test_wide_gqa_group_of_16():
    cfg, q, k, v, cal = gen(1, B=1, Hq=32, Hkv=2, Lq=64, Lk=200)
    print("case gqa16", flush=True)
    got, want, *_ = run_case(q, k, v, True, 128, calib=cal)
    compare_out(got, want, "gqa16")


def test_v_all_ones_is_exactly_one():
    cfg, q, k, v, cal = gen(1, B=1, Hq=8, Hkv=2, Lq=256, Lk=256)
    v = np.ones_like(v)
    print("case v-ones", flush=True)
    got, want, *_ = run_case(q, k, v, True, 128, calib=cal)
    assert np.all(got == 1.0) and np.all(want == 1.0)


@pytest.mark.parametrize("d,splits,normalizer", [(128, 1, 0), (128, 3, 0), (128, 0, 0), (128, 0, 1), (64, 2, 0),
                                                 (256, 4, 0)])
def test_decode_split_kv(d, splits, normalizer):
    cfg_id = 3 if d == 256 else 1
    over = dict(B=3, Hq=8, Hkv=2, Lq=1, Lk=1000, d=d)
    cfg, q, k, v, cal = gen(cfg_id, **over)
    print("case decode d", d, "splits", splits, "norm", normalizer, flush=True)
    got, want, *_ = run_case(q, k, v, True, 128, normalizer, calib=cal, num_splits=splits)
    compare_out(got, want, "decode-d%d-s%d" % (d, splits))


@pytest.mark.parametrize("d", [64, 128])
def test_decode_grid_beyond_one_wave_per_simd(d):
    """16 x 8 (batch, KV head) units x 12 splits = 1536 single-wave work-groups, more than the
    1024 SIMDs of the chip: the split kernel then keeps one tile in flight (two operand sets)
    instead of three, the small-grid choice the other decode cases take.  17 tiles of 128 keys
    (the last ragged) over 12 splits of 2 leave three splits empty."""
    cfg, q, k, v, cal = gen(1, B=16, Hq=8, Hkv=8, Lq=1, Lk=2100, d=d)
    print("case decode large grid d", d, flush=True)
    got, want, *_ = run_case(q, k, v, True, 128, calib=cal, num_splits=12)
    compare_out(got, want, "decode-grid-d%d" % d)


def test_decode_workspace_reuse_and_head_chunks():
    """GQA group of 32 (two 16-head chunks per KV head, two split waves per (batch, KV head,
    split)); repeated calls on one workspace give identical outputs."""
    import torch
    cfg, q, k, v, cal = gen(1, B=2, Hq=32, Hkv=1, Lq=1, Lk=777, d=128)
    print("case decode group 32, workspace reuse", flush=True)
    got, want, *_ = run_case(q, k, v, True, 128, calib=cal, num_splits=3)
    compare_out(got, want, "decode-g32-s3")
    res = gpu_quantize(q, k, v, None, None)
    dims = hf.make_dims(2, 32, 1, 128, 1, 777)
    opts = hf.make_opts(True, 0, 128, 3)
    n = hf.attention_workspace_bytes(dims, opts)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    outs = [hf.attention_fwd(res, dims, True, 0, 128, 3, workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("b,hq,hkv,lq,lk,d,causal,kv_tile", [
    (1, 4, 1, 1, 1, 128, True, 128),     # decode over a single key
    (2, 2, 2, 1, 31, 64, False, 64),     # decode, non-causal flag, less than one scale block
    (1, 2, 1, 3, 3, 64, True, 64),       # three-row causal prefill
    (1, 2, 2, 2, 40, 256, False, 64),    # two rows, one partial tile pair, d = 256
    (1, 1, 1, 33, 31, 128, False, 128),  # more queries than keys (non-causal)
    (3, 6, 3, 17, 129, 128, True, 128),  # one key past a tile, rows past a 16-row block
])
def test_tiny_and_ragged_shapes(b, hq, hkv, lq, lk, d, causal, kv_tile):
    cfg, q, k, v, cal = gen(1 if d != 256 else 3, B=b, Hq=hq, Hkv=hkv, Lq=lq, Lk=lk, d=d)
    print("case tiny", b, hq, hkv, lq, lk, d, causal, kv_tile, flush=True)
    got, want, *_ = run_case(q, k, v, causal, kv_tile, calib=cal)
    compare_out(got, want, "tiny-%d-%d-%d" % (lq, lk, d))


@pytest.mark.parametrize("b,hq,hkv,lq,lk,d,causal,kv_tile", [
    (1, 4, 1, 200, 200, 128, True, 128),   # GQA 4: one head group per work-group, ragged rows
    (2, 2, 2, 150, 150, 128, True, 64),    # MHA: 128 or 64 rows of one head per work-group
    (1, 16, 1, 70, 70, 128, False, 128),   # GQA 16: 8 or 4 heads per work-group
    (2, 8, 2, 100, 260, 64, True, 64),     # d = 64, fewer queries than keys (bottom-right causal)
    (1, 4, 2, 150, 150, 256, True, 128),   # d = 256, GQA 2
])
def test_prefill_work_group_shapes(b, hq, hkv, lq, lk, d, causal, kv_tile):
    """4- and 8-wave prefill work-groups (opts.prefill_waves) give the same bits as the automatic
    choice, which matches the oracle bit for bit."""
    import torch
    cfg, q, k, v, cal = gen(1, B=b, Hq=hq, Hkv=hkv, Lq=lq, Lk=lk, d=d)
    print("case work-group shapes", b, hq, hkv, lq, lk, d, causal, kv_tile, flush=True)
    got, want, *_ = run_case(q, k, v, causal, kv_tile, calib=cal)
    _, ndiff = compare_out(got, want, "wg-auto")
    assert ndiff == 0
    res = gpu_quantize(q, k, v, None, None)
    dims = hf.make_dims(b, hq, hkv, d, lq, lk)
    auto = hf.attention_fwd(res, dims, causal, 0, kv_tile)
    q16 = (to_dev(q), None)
    kv_only = {n: res[n] for n in ["k_codes", "k_scales", "v_codes", "v_scales"]}
    for w in (4, 8):
        o = hf.attention_fwd(res, dims, causal, 0, kv_tile, prefill_waves=w)
        o16 = hf.attention_fwd(kv_only, dims, causal, 0, kv_tile, q16=q16, prefill_waves=w)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), auto.view(torch.int16)), w
        assert torch.equal(o16.view(torch.int16), auto.view(torch.int16)), w


def test_tile_stats_match_oracle():
    cfg, q, k, v, cal = gen(1, B=1, Hq=4, Hkv=1, Lq=200, Lk=200)
    print("case stats", flush=True)
    got, want, qq, diag, st = run_case(q, k, v, True, 64, calib=cal, stats=True)
    compare_out(got, want, "stats-out")
    for h in range(4):
        for rb, t, sph, sp in A.tile_stats_p(qq, True, 64, 0, h):
            assert np.isclose(st[0, h, rb, t, 0], sph, rtol=1e-5), (h, rb, t)
            assert np.isclose(st[0, h, rb, t, 1], sp, rtol=1e-5), (h, rb, t)
    # tiles above the causal diagonal of a row block are zero
    assert st[0, 0, 0, 3, 0] == 0 and st[0, 0, 0, 3, 1] == 0


def test_deterministic():
    import torch
    cfg, q, k, v, cal = gen(1, B=1, Hq=8, Hkv=2, Lq=300, Lk=300)
    res = gpu_quantize(q, k, v, None, None)
    dims = hf.make_dims(1, 8, 2, 128, 300, 300)
    a = hf.attention_fwd(res, dims, True, 0, 128).clone()
    b = hf.attention_fwd(res, dims, True, 0, 128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_quantizer_edge_values():
    """Zero blocks, signed zeros, tiny and huge FP16 values, ragged V tail: codes bit-exact."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 2, 40, 64)).astype(np.float16)
    k = rng.standard_normal((1, 1, 70, 64)).astype(np.float16)
    v = rng.standard_normal((1, 1, 70, 64)).astype(np.float16)
    q[0, 0, 0] = 0
    q[0, 0, 1] = -0.0
    q[0, 0, 2, :32] = np.float16(6e-8)
    q[0, 0, 3, :32] = np.float16(65504)
    q[0, 0, 3, 5] = -np.float16(1e-7)
    k[0, 0, 5] = np.float16(-0.0)
    v[0, 0, 60:] = 0
    v[0, 0, 3, :] = np.float16(-65504)
    res = gpu_quantize(q, k, v, None, None)
    assert_codes_equal(res, A.quantize_qkv(q, k, v))
    s = np.full((1, 64), 3.0, np.float32)
    inv = (1.0 / s.astype(np.float64)).astype(np.float32)
    res = gpu_quantize(q, k, v, s, inv)
    assert_codes_equal(res, A.quantize_qkv(q, k, v, s, inv))


def test_floor_scale_rule_saturation_and_attention():
    """The OCP floor scale rule (accuracy variant): block maxima in (6, 8) * 2^e saturate at code 6;
    codes bit-exact against the oracle's floor rule, attention from them within tolerance."""
    import torch
    from gpu_helpers import to_dev
    rng = np.random.default_rng(22)
    q = rng.standard_normal((1, 4, 96, 64)).astype(np.float16)
    k = rng.standard_normal((1, 2, 130, 64)).astype(np.float16)
    v = rng.standard_normal((1, 2, 130, 64)).astype(np.float16)
    for i, m in enumerate([7.0, 7.99, 6.5, 8.0, 6.0, 4.0, 5.99]):
        q[0, 0, i, 0] = m
        q[0, 1, i, 33] = -m
        k[0, 0, i, 7] = m
        v[0, 1, 32 + i, 9] = -m
    q[0, 2, 0] = 0
    print("case floor scale rule", flush=True)
    dims = hf.make_dims(1, 4, 2, 64, 96, 130)
    res = hf.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), dims=dims, scale_rule=hf.SCALE_FLOOR)
    qq = A.quantize_qkv(q, k, v, rule="floor")
    assert_codes_equal(res, qq)
    out = hf.attention_fwd(res, dims, True, 0, 64)
    torch.cuda.synchronize()
    compare_out(out.cpu().numpy(), A.attention_p(qq, True, 64, 0), "floor-rule")


@pytest.mark.parametrize("cfg_id,b,hq,hkv,lq,lk,d,causal,kv_tile", [
    (0, 1, 2, 2, 128, 128, 64, False, 64),     # the tiny non-causal workload
    (1, 1, 8, 2, 300, 300, 128, True, 128),    # Qwen-shaped, reduced
    (1, 3, 6, 3, 17, 129, 128, True, 64),      # ragged: a key past a tile, rows past a 16-row block
    (1, 1, 4, 1, 77, 333, 128, True, 128),     # causal with Lq < Lk
    (3, 1, 4, 2, 200, 200, 256, True, 128),    # Gemma-shaped d = 256
    (1, 1, 16, 1, 64, 96, 64, False, 64),      # GQA group of 16, d = 64
])
def test_round_to_nearest_running_max(cfg_id, b, hq, hkv, lq, lk, d, causal, kv_tile):
    """Accuracy variant HIFA4_MAX_NEAREST16: m is the FP16 value nearest to fp32(max S * C) and the
    rescale the FP16 exp2 of the difference; against the oracle's variant (both entry points)."""
    cfg, q, k, v, cal = gen(cfg_id, B=b, Hq=hq, Hkv=hkv, Lq=lq, Lk=lk, d=d)
    print("case nearest max", cfg_id, b, hq, hkv, lq, lk, d, causal, kv_tile, flush=True)
    got, want, *_ = run_case(q, k, v, causal, kv_tile, calib=cal, alpha=cfg["alpha"], max_rule=A.MAX_NEAREST16)
    compare_out(got, want, "nearest-max-%d-%d-%d" % (lq, lk, d))
    # the variant is a different function of the same codes: it must differ from the method's output
    _, want_ceil, *_ = run_case(q, k, v, causal, kv_tile, calib=cal, alpha=cfg["alpha"])
    assert np.count_nonzero(want_ceil.view(np.uint16) != want.view(np.uint16)) > 0


@pytest.mark.parametrize("cfg_id,b,hq,hkv,lq,lk,d,causal,kv_tile", [
    (0, 1, 2, 2, 128, 128, 64, False, 64),     # the tiny non-causal workload
    (1, 1, 8, 2, 300, 300, 128, True, 128),    # Qwen-shaped, reduced
    (1, 3, 6, 3, 17, 129, 128, True, 64),      # ragged: a key past a tile, rows past a 16-row block
    (1, 1, 4, 1, 77, 333, 128, True, 128),     # causal with Lq < Lk
    (1, 2, 2, 2, 100, 300, 128, False, 128),   # non-causal, ragged key tail
    (3, 1, 4, 2, 200, 200, 256, True, 128),    # Gemma-shaped d = 256
    (1, 3, 8, 2, 1, 1000, 128, True, 128),     # decode (split-KV)
    (3, 2, 4, 2, 1, 700, 256, True, 64),       # decode, d = 256, 64-key tiles
])
@pytest.mark.parametrize("variant", ["tile", "direct"])
def test_phat_variants(cfg_id, b, hq, hkv, lq, lk, d, causal, kv_tile, variant):
    """P-hat variants against the oracle's: one scale per (row, tile) (HIFA4_PHAT_TILE), and
    Direct-P codes built straight from the log2-domain score (HIFA4_PHAT_DIRECT); both entry
    points, prefill and split-KV decode.  Each must also differ from the method's output."""
    cfg, q, k, v, cal = gen(cfg_id, B=b, Hq=hq, Hkv=hkv, Lq=lq, Lk=lk, d=d)
    kw = dict(phat_scale=A.PHAT_TILE) if variant == "tile" else dict(phat_rule=A.PHAT_DIRECT)
    print("case phat", variant, cfg_id, b, hq, hkv, lq, lk, d, causal, kv_tile, flush=True)
    got, want, *_ = run_case(q, k, v, causal, kv_tile, calib=cal, alpha=cfg["alpha"], **kw)
    compare_out(got, want, "phat-%s-%d-%d-%d" % (variant, lq, lk, d))
    _, want_method, *_ = run_case(q, k, v, causal, kv_tile, calib=cal, alpha=cfg["alpha"])
    assert np.count_nonzero(want_method.view(np.uint16) != want.view(np.uint16)) > 0
