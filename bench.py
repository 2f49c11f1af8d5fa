#!/usr/bin/env python3
"""Benchmark of the 4-bit (HiFA4-style) attention forward on one MI355X.

A step is one pass of the hot path over one batch of resident synthetic input:
the Smooth-QK rescale + 4-bit quantization of K and V (HBM-bound kernels) followed
by the fused 4-bit attention forward, which rescales and quantizes its own query
rows on the way in (hifa4_attention_fwd_q16).  The default workload is the batched
causal prefill (B=8, L=4096, Hq=32/Hkv=8, d=128, P-Reordered normalizer, 128-key
tiles).  The JSON line also carries the memory-bound split-KV decode (B=64,
Lk=32768, pre-quantized cache; a step runs split, with the query token quantized
in-kernel, and merge).  The default warm-up (50 steps, about 40 ms) lets the GPU
clocks settle before the timed steps.  The line also carries the same prefill step from
pre-RoPE Q and K (rope_prefill: K/V quantized with RoPE by hifa4_quantize_qkv_rope, the query
quantized in the RoPE quantizer too, then the attention from the codes).

    python bench.py [--steps K] [--warmup W] [--no-decode] [--no-cpu-baseline]

Rates: algorithmic FLOPs are 4 * d per visible (query, key) pair (L(L+1)/2 pairs
per head when causal); decode bytes are the K-hat/V-hat codes and scales, the FP16
query, the Smooth-QK scales and the FP16 output.  Kernel durations come from HIP events recorded on the
stream the kernels run on.  Peaks: MI355X dense FP4 MFMA 10.1 PFLOP/s, HBM3E
8 TB/s (AMD's published figures).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0
HBM_PEAK_GBS = 8000.0
COPY_PROBE_BYTES = 512 << 20  # plain device copy run by --traffic-probe to calibrate the counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["attn_prefill.hip", "attn_decode.hip", "device_common.h", "quantize.hip"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-rope", action="store_true", help="skip the pre-RoPE (fused RoPE prologue) variant of the step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle timing sample")
    p.add_argument("--workload", default="prefill", choices=["prefill", "prefill-d256", "prefill-L2048"])
    p.add_argument("--traffic-probe", action="store_true",
                   help="also run one plain %d MiB device copy (counter calibration for HBM traffic)"
                        % (COPY_PROBE_BYTES >> 20))
    return p.parse_args()


def kernel_source_digest():
    """sha256 over the kernel sources: the HBM-traffic figures are valid only for these bytes."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_flashattention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(key):
    """HBM bytes per launch of a kernel from the committed counter summary, or None.

    profiles/traffic.json holds FETCH_SIZE / WRITE_SIZE per dispatch (KiB) of each kernel and
    of a plain copy of known size measured in the same runs; each counter is scaled by
    bytes_copied / counter(copy).  The figures are dropped when the kernel sources changed
    since they were taken.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest() or key not in t.get("kernels", {}):
        return None
    k = t["kernels"][key]
    cp = t["copy"]
    f_scale = cp["bytes"] / (cp["fetch_kib"] * 1024.0)
    w_scale = cp["bytes"] / (cp["write_kib"] * 1024.0)
    return int(round(k["fetch_kib"] * 1024.0 * f_scale + k["write_kib"] * 1024.0 * w_scale))


def copy_probe():
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def causal_pairs(lq, lk):
    shift = lk - lq
    return sum(min(lk, r + shift + 1) for r in range(lq))


def bench_prefill(args, cfg_id):
    import torch
    import bit_quantized_flashattention_amd as hf
    import synth

    cfg = synth.config(cfg_id)
    b, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    q, k, v = synth.make_qkv_device(cfg)
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    sd = torch.from_numpy(s).cuda()
    invd = torch.from_numpy(inv).cuda()
    dims = hf.make_dims(b, hq, hkv, d, lq, lk)
    qkv = hf.quantize_qkv(q, k, v, sd, invd, dims=dims)
    out = torch.empty((b, hq, lq, d), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        # K-hat, V-hat from the quantizer; Q is rescaled and quantized inside the attention kernel
        hf.quantize_qkv(None, k, v, sd, invd, dims=dims, out=qkv)
        if ev is not None:
            ev[0].record(stream)
        hf.attention_fwd(qkv, dims, cfg["causal"], hf.P_REORDERED, cfg["kv_tile"], out=out, q16=(q, sd))
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_ms = sum(a.elapsed_time(c) for a, c in evs) / args.steps
    step_ms = (t1 - t0) * 1e3 / args.steps
    pairs = causal_pairs(lq, lk) if cfg["causal"] else lq * lk
    flops = 4.0 * d * pairs * b * hq
    return dict(cfg=cfg, step_ms=step_ms, attn_ms=attn_ms, flops=flops, gate=gate,
                qkv_inputs=(q, k, v), qkv=qkv, out=out)


def bench_rope(args):
    """The same prefill step from pre-RoPE Q and K: hifa4_quantize_qkv_rope rotates, rescales and
    quantizes Q and K (and quantizes V) in streaming passes, then the attention from the codes."""
    import torch
    import bit_quantized_flashattention_amd as hf
    import synth

    cfg = synth.config(2)
    b, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    q, k, v = synth.make_qkv_device(cfg, pre_rope=True)
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    sd = torch.from_numpy(s).cuda()
    invd = torch.from_numpy(inv).cuda()
    cos32, sin32 = synth.rope_table(cfg["rope_theta"], lk, d)
    cosd, sind = torch.from_numpy(cos32).cuda(), torch.from_numpy(sin32).cuda()
    dims = hf.make_dims(b, hq, hkv, d, lq, lk)
    qkv = hf.quantize_qkv_rope(q, k, v, sd, invd, cosd, sind, dims=dims)
    out = torch.empty((b, hq, lq, d), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        hf.quantize_qkv_rope(q, k, v, sd, invd, cosd, sind, dims=dims, out=qkv)
        if ev is not None:
            ev[1].record(stream)
        hf.attention_fwd(qkv, dims, cfg["causal"], hf.P_REORDERED, cfg["kv_tile"], out=out)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    quant_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    step_ms = (t1 - t0) * 1e3 / args.steps
    flops = 4.0 * d * causal_pairs(lq, lk) * b * hq
    # algorithmic bytes of the Q, K (RoPE) and V quantizers: FP16 in, codes and scales out, the
    # tables and the Smooth-QK scales once
    elems = b * (hq + 2 * hkv) * lk * d
    q_bytes = elems * 2 + elems // 2 + elems // 32 + lk * d * 4 + 2 * hkv * d * 4
    res = {
        "workload": "%s from pre-RoPE Q/K: Q/K/V quantize with RoPE on Q and K, then attention" % cfg["name"],
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "ms_per_step": round(step_ms, 4),
        "attention_ms": round(attn_ms, 4),
        "quantize_qkv_rope": {"us": round(quant_ms * 1e3, 1), "bytes": q_bytes,
                             "achieved_gbs": round(q_bytes / (quant_ms * 1e-3) / 1e9, 1), "peak_gbs": HBM_PEAK_GBS},
    }
    del q, k, v, qkv, out
    torch.cuda.empty_cache()
    return res


def bench_append(args):
    """hifa4_cache_append of one key per sequence (the decode loop's cache update): B64 Hkv8 d128,
    RoPE and Smooth-QK on the key, the open V-hat block re-quantized from its FP16 stage.  The
    cost does not depend on the cache length, so a 1024-key cache is cycled through."""
    import torch
    import bit_quantized_flashattention_amd as hf
    import synth

    cfg = synth.config(4)
    b, hkv, d = cfg["B"], cfg["Hkv"], cfg["d"]
    cap = 1024
    cache = hf.make_cache(b, hkv, d, cap)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    kn = torch.randn((b, hkv, 1, d), generator=gen, device="cuda").to(torch.float16)
    vn = torch.randn((b, hkv, 1, d), generator=gen, device="cuda").to(torch.float16)
    invd = torch.ones((hkv, d), dtype=torch.float32, device="cuda")
    cos32, sin32 = synth.rope_table(cfg["rope_theta"], cap, d)
    cosd, sind = torch.from_numpy(cos32).cuda(), torch.from_numpy(sin32).cuda()

    def step():
        if cache["length"] == cap:
            cache["length"] = 0
        hf.cache_append(cache, kn, vn, invd, cosd, sind)

    for _ in range(64):
        step()
    torch.cuda.synchronize()
    n = 256  # eight full 32-key cycles of the open V-hat block
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    return {"workload": "append 1 key per sequence, B%d Hkv%d d%d, RoPE + Smooth-QK on K, V-hat block re-quantized"
                        % (b, hkv, d), "us_per_call": round(e0.elapsed_time(e1) / n * 1e3, 2)}


def bench_decode(args):
    import torch
    import bit_quantized_flashattention_amd as hf
    import synth

    cfg = synth.config(4)
    b, hq, hkv, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lk"], cfg["d"]
    q, k, v = synth.make_qkv_device(cfg)
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    sd = torch.from_numpy(s).cuda()
    invd = torch.from_numpy(inv).cuda()
    dims = hf.make_dims(b, hq, hkv, d, 1, lk)
    qkv = hf.quantize_qkv(q, k, v, sd, invd, dims=dims)  # the cache is quantized once
    # k and v (8.6 GB) stay allocated until the timing is done: freeing them here slowed the
    # timed steps by ~5 % for the next ~250 ms (measured), while the freed memory is reclaimed
    opts = hf.make_opts(True, hf.P_REORDERED, cfg["kv_tile"], 0)
    splits = hf.decode_num_splits(dims, opts)
    ws = torch.empty(hf.attention_workspace_bytes(dims, opts), dtype=torch.uint8, device="cuda")
    out = torch.empty((b, hq, 1, d), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        # the FP16 query is rescaled and quantized inside the split kernel
        hf.attention_fwd(qkv, dims, True, hf.P_REORDERED, cfg["kv_tile"], 0, out=out, workspace=ws, q16=(q, sd))
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n = max(args.steps, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_ms = sum(a.elapsed_time(c) for a, c in evs) / n
    step_ms = (t1 - t0) * 1e3 / n
    lk32 = -(-lk // 32) * 32
    kv_bytes = 2 * b * hkv * (lk * d // 2 + lk * d // 32)  # K-hat and V-hat codes + scales
    assert kv_bytes == b * hkv * (lk * (d // 2 + d // 32) + d * (lk32 // 2 + lk32 // 32))
    q_bytes = b * hq * d * 2 + hkv * d * 4  # FP16 query and the Smooth-QK scales
    out_bytes = b * hq * d * 2
    total = kv_bytes + q_bytes + out_bytes
    res = {
        "workload": "split-KV decode B%d Hq%d/Hkv%d d%d Lk%d, 4-bit cache, %d splits" % (b, hq, hkv, d, lk, splits),
        "metric": "decode HBM GB/s",
        "value": round(total / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "us_per_step": round(step_ms * 1e3, 1),
        "bytes_per_step": total,
        "roofline": {"bound": "hbm", "achieved": round(total / (attn_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(total / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("decode"), "kernel_us": round(attn_ms * 1e3, 1)},
    }
    del qkv, ws, out, q, k, v
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, pre):
    """The oracle, as it stands, timed on host cores on a bounded sample of the same workload."""
    import numpy as np
    import torch
    from oracle import attention as A
    from oracle import smooth

    cfg = pre["cfg"]
    q, k, v = pre["qkv_inputs"]
    d, lq, lk, hq, hkv = cfg["d"], cfg["Lq"], cfg["Lk"], cfg["Hq"], cfg["Hkv"]
    qh = q[0:1, 0:1].cpu().numpy()
    kh = k[0:1, 0:1].cpu().numpy()
    vh = v[0:1, 0:1].cpu().numpy()
    import synth
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, _ = smooth.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    qq = A.quantize_qkv(qh, kh, vh, s[:1], inv[:1])
    flops = 0.0
    rows_done = 0
    while time.perf_counter() - t0 < args.cpu_seconds:
        rows = np.sort(rng.choice(lq, size=16, replace=False))
        A.attention_head_p(qq, 0, 0, rows, cfg["causal"], cfg["kv_tile"], A.P_REORDERED)
        shift = lk - lq
        vis = np.minimum(lk, rows + shift + 1) if cfg["causal"] else np.full(len(rows), lk)
        flops += 4.0 * d * float(vis.sum())
        rows_done += len(rows)
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": "%d query rows of head (0,0) of the prefill workload incl. that head's quantization; %.1f s"
                      % (rows_done, el)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU; there is no multi-GPU path: use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    cfg_id = {"prefill": 2, "prefill-d256": 3, "prefill-L2048": 1}[args.workload]
    pre = bench_prefill(args, cfg_id)
    cfg = pre["cfg"]
    attn_tflops = pre["flops"] / (pre["attn_ms"] * 1e-3) / 1e12
    step_tflops = pre["flops"] / (pre["step_ms"] * 1e-3) / 1e12
    line = {
        "metric": "4-bit attention fwd TFLOP/s (+% FP4-MFMA peak); decode HBM GB/s",
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {
            "workload": "%s: causal=%s B%d Hq%d/Hkv%d d%d L%d, kv_tile %d, per step: K/V quantize + attention with Q quantized in-kernel"
                        % (cfg["name"], cfg["causal"], cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["Lq"],
                           cfg["kv_tile"]),
            "global_batch": cfg["B"], "seq_len": cfg["Lq"], "heads_q": cfg["Hq"], "heads_kv": cfg["Hkv"],
            "head_dim": cfg["d"], "normalizer": "p_reordered", "smooth_qk_gate": pre["gate"],
        },
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / FP4_PEAK_TFLOPS, 4), "traffic": traffic_for("prefill") if args.workload == "prefill" else None,
                     "kernel_ms": round(pre["attn_ms"], 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, pre)
    del pre
    torch.cuda.empty_cache()
    if not args.no_rope and args.workload == "prefill":
        line["rope_prefill"] = bench_rope(args)
    if not args.no_decode:
        line["decode"] = bench_decode(args)
        line["decode"]["cache_append"] = bench_append(args)
    if args.traffic_probe:
        copy_probe()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
