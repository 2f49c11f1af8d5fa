#!/usr/bin/env python3
"""Benchmark of the 4-bit (HiFA4-style) attention forward on one MI355X.

A step is one pass of the hot path over one batch of resident synthetic input: the Smooth-QK
rescale + 4-bit quantization of K and V (HBM-bound kernels) followed by the fused 4-bit attention
forward, which rescales and quantizes its own query rows on the way in
(hifa4_attention_fwd_q16).  The headline workload is the batched causal prefill (B=8, L=4096,
Hq=32/Hkv=8, d=128, P-Reordered normalizer, P-hat with one scale per 32-key block, 128-key
tiles).  The JSON line also carries, each with its own roofline:
  prefill_d256       the Gemma2-9B-shaped causal prefill (B=2, L=8192, Hq=16/Hkv=8, d=256);
  prefill_b1         the Qwen3-8B-shaped single-sequence causal prefill (B=1, L=2048,
                     Hq=32/Hkv=8, d=128), a grid too small to fill the chip;
  direct_p           the headline workload with Direct-P codes (no exponential per score);
  noncausal          the headline shapes without the causal mask, with the method's codes and
                     with Direct-P codes (the Direct-P page's setting is non-causal inference);
  rope_prefill       the headline step from pre-RoPE Q and K (RoPE fused into the quantizer);
  decode             the memory-bound split-KV decode (B=64, Lk=32768, pre-quantized cache),
                     with the cache append of one key per sequence;
  cpu_baseline       the oracle timed on the host's cores on a bounded sample, run last.

    python bench.py [--steps K] [--warmup W] [--no-decode] [--no-cpu-baseline] [--legs a,b,...]

Every leg runs W untimed warm-up steps and keeps warming up for at least 0.3 s (the GPU clocks
settle), then times exactly K steps between two device synchronizations.  Kernel durations come
from HIP events recorded on the stream the kernels run on; the line gives their mean and, per
leg, median, min and max.  Rates: algorithmic FLOPs are 4 * d per visible (query, key) pair
(L(L+1)/2 pairs per head when causal); decode bytes are the K-hat/V-hat codes and scales, the
FP16 query, the Smooth-QK scales and the FP16 output.  Peaks: MI355X dense FP4 MFMA
10.1 PFLOP/s, HBM3E 8 TB/s (AMD's published figures).

roofline.traffic (HBM bytes per launch of the leg's dominant kernels) and the matrix-core and
vector-ALU busy fractions come from three rocprofv3 --pmc runs of this script started after the
timed legs (FETCH_SIZE; WRITE_SIZE; SQ_VALU_MFMA_BUSY_CYCLES, SQ_ACTIVE_INST_VALU and
GRBM_GUI_ACTIVE), each two steps of the headline, d256, Direct-P and decode legs plus a plain
512 MiB device copy that scales the byte counters.  --counters stored takes them from
profiles/counters.json instead when its kernel sources are these; "counters.source" says which.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0
HBM_PEAK_GBS = 8000.0
MIN_WARM_S = 0.3
COPY_PROBE_BYTES = 512 << 20  # plain device copy run by --traffic-probe to calibrate the counters
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ["attn_prefill.hip", "attn_decode.hip", "device_common.h", "quantize.hip"]
ALL_LEGS = ["prefill_d256", "prefill_b1", "direct_p", "noncausal", "rope_prefill", "decode"]


def progress(msg):
    """One progress line on stderr (stdout carries only the JSON line)."""
    sys.stderr.write("bench: %s (%.0f s)\n" % (msg, time.perf_counter() - T0))
    sys.stderr.flush()


T0 = time.perf_counter()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--legs", default=",".join(ALL_LEGS), help="comma-separated extra legs (%s)" % ",".join(ALL_LEGS))
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-rope", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="per-worker budget of the oracle sample")
    p.add_argument("--traffic-probe", action="store_true",
                   help="also run one plain %d MiB device copy (counter calibration for HBM traffic)"
                        % (COPY_PROBE_BYTES >> 20))
    p.add_argument("--counters", choices=["live", "stored", "none"], default="live",
                   help="HBM traffic and busy fractions of the rooflines: measured now by rocprofv3 runs of "
                        "this script (live), taken from profiles/counters.json when its kernel sources match "
                        "(stored), or left out")
    a = p.parse_args()
    legs = [x for x in a.legs.split(",") if x]
    if a.no_decode and "decode" in legs:
        legs.remove("decode")
    if a.no_rope and "rope_prefill" in legs:
        legs.remove("rope_prefill")
    a.leg_list = legs
    return a


def kernel_source_digest():
    """sha256 over the kernel sources: counter figures are valid only for these bytes."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_flashattention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counters_for(key):
    """Counter figures of one kernel from the committed summary, or None.

    profiles/counters.json holds, per kernel and workload, FETCH_SIZE / WRITE_SIZE per dispatch
    (KiB; scaled by bytes_copied / counter(copy) of a plain copy of known size measured in the
    same runs) and the matrix-core / vector-ALU busy fractions of its issue-counter run.  The
    figures are dropped when the kernel sources changed since they were taken.
    """
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest() or key not in t.get("kernels", {}):
        return None
    k = t["kernels"][key]
    out = {}
    cp = t.get("copy")
    if cp and "fetch_kib" in k and "write_kib" in k:
        f_scale = cp["bytes"] / (cp["fetch_kib"] * 1024.0)
        w_scale = cp["bytes"] / (cp["write_kib"] * 1024.0)
        out["traffic"] = int(round(k["fetch_kib"] * 1024.0 * f_scale + k["write_kib"] * 1024.0 * w_scale))
    for name in ("mfma_busy", "valu_busy"):
        if name in k:
            out[name] = k[name]
    return out


def copy_probe():
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


# The dominant kernels of the legs whose rooflines carry counter figures (demangled-name
# substrings; decode counts its split and merge launches together).
COUNTER_KERNELS = {
    "prefill": ["attn_prefill_kernel<128, true, 0, false, 0, 8>"],
    "prefill_d256": ["attn_prefill_kernel<256, true, 0, false, 0, 8>"],
    "direct_p": ["attn_prefill_kernel<128, true, 0, false, 2, 8>"],
    "decode": ["attn_decode_split_kernel<128, 0, 0, 2>", "attn_decode_merge_kernel<128>"],
}
COUNTER_RUNS = [["FETCH_SIZE"], ["WRITE_SIZE"], ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"]]
N_SIMDS = 1024  # 256 compute units x 4


def profiled_run(counters, timeout_s=150):
    """Runs this script (the headline, d256, Direct-P and decode legs, two timed steps each, and
    the copy probe) under rocprofv3 --pmc with the given counters; returns {kernel name: {counter:
    [value per dispatch]}} or None.  The child's own JSON line is discarded."""
    import glob
    import shutil
    import signal
    import subprocess
    import tempfile
    exe = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(exe):
        return None
    out = tempfile.mkdtemp(prefix="hifa4_ctr_")
    cmd = [exe, "--pmc"] + counters + ["--output-format", "csv", "-d", out, "-o", "c", "--",
                                       sys.executable, os.path.abspath(__file__), "--steps", "2", "--warmup", "1",
                                       "--no-cpu-baseline", "--counters", "none", "--traffic-probe",
                                       "--legs", "prefill_d256,direct_p,decode"]
    env = dict(os.environ, TMPDIR=out)
    progress("counter run %s" % " ".join(counters))
    proc = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, env=env, cwd=out,
                            start_new_session=True)
    try:
        _, err = proc.communicate(timeout=timeout_s)
    except subprocess.TimeoutExpired:
        os.killpg(proc.pid, signal.SIGKILL)  # the profiler and the child it started, nothing else
        proc.communicate()
        shutil.rmtree(out, ignore_errors=True)
        return None
    files = glob.glob(os.path.join(out, "**", "*counter_collection.csv"), recursive=True)
    if proc.returncode != 0 or not files:
        sys.stderr.write("counter run %s failed (rc %d): %s\n" % (counters, proc.returncode, err.decode()[-500:]))
        shutil.rmtree(out, ignore_errors=True)
        return None
    res = parse_counter_csv(files[0])
    shutil.rmtree(out, ignore_errors=True)
    return res


def parse_counter_csv(path):
    """{kernel name: {counter: [value per dispatch, in dispatch order]}} of a rocprofv3
    counter_collection.csv; a dispatch's rows (one per counter and hardware instance) are summed."""
    import csv
    per_disp, names = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = per_disp.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
    res = {}
    for disp in sorted(per_disp, key=int):
        for c, v in per_disp[disp].items():
            res.setdefault(names[disp], {}).setdefault(c, []).append(v)
    return res


def live_counters():
    """HBM bytes per launch and matrix/vector busy fractions of each leg's dominant kernel(s),
    measured in this run: three profiled runs of this script, one per counter group (a counter
    group needs a run of its own).  None when the profiler is missing or a run fails."""
    runs = []
    for counters in COUNTER_RUNS:
        r = profiled_run(counters)
        if r is None:
            return None
        runs.append(r)
    return derive_counters(runs)


def derive_counters(runs):
    """From the three parsed runs (FETCH_SIZE; WRITE_SIZE; the busy counters): per leg, the mean
    per dispatch of FETCH_SIZE and WRITE_SIZE (KiB) scaled by bytes / counter of the run's largest
    device copy (the 512 MiB probe), summed over the leg's kernels, and the busy fractions of its
    first kernel over 1024 SIMDs and the kernel's cycles (GRBM_GUI_ACTIVE / 8 XCDs)."""

    def mean(run, sub, counter):
        vals = [v for name, cs in run.items() if sub in name for v in cs.get(counter, [])]
        return sum(vals) / len(vals) if vals else None

    # the probe is the run's largest device copy: its dispatch, not a mean over smaller copies
    f_copy = max([v for name, cs in runs[0].items() if "copyBuffer" in name for v in cs.get("FETCH_SIZE", [])] or [0.0])
    w_copy = max([v for name, cs in runs[1].items() if "copyBuffer" in name for v in cs.get("WRITE_SIZE", [])] or [0.0])
    if f_copy <= 0.0 or w_copy <= 0.0:
        return None
    f_scale, w_scale = COPY_PROBE_BYTES / (f_copy * 1024.0), COPY_PROBE_BYTES / (w_copy * 1024.0)
    out = {}
    for key, subs in COUNTER_KERNELS.items():
        fetch = [mean(runs[0], sub, "FETCH_SIZE") for sub in subs]
        write = [mean(runs[1], sub, "WRITE_SIZE") for sub in subs]
        if None in fetch or None in write:
            continue
        k = {"traffic": int(round(sum(fetch) * 1024.0 * f_scale + sum(write) * 1024.0 * w_scale)),
             "fetch_bytes": int(round(sum(fetch) * 1024.0 * f_scale)), "write_bytes": int(round(sum(write) * 1024.0 * w_scale))}
        g = mean(runs[2], subs[0], "GRBM_GUI_ACTIVE")
        mb, va = mean(runs[2], subs[0], "SQ_VALU_MFMA_BUSY_CYCLES"), mean(runs[2], subs[0], "SQ_ACTIVE_INST_VALU")
        if g and mb is not None and va is not None:
            cyc = g / 8.0  # GRBM_GUI_ACTIVE is summed over the 8 XCDs
            k["mfma_busy"] = round(mb / (N_SIMDS * cyc), 4)
            k["valu_busy"] = round(4.0 * va / (N_SIMDS * cyc), 4)
        out[key] = k
    out["_scale"] = {"copy_bytes": COPY_PROBE_BYTES, "fetch_factor": round(f_scale, 4), "write_factor": round(w_scale, 4)}
    return out


def add_counters(line, mode):
    """Fills traffic (and the busy fractions) into the rooflines of the headline, d256, Direct-P
    and decode legs, from live counter runs or the stored ones; records which."""
    rooflines = {"prefill": line.get("roofline"), "prefill_d256": line.get("prefill_d256", {}).get("roofline"),
                 "direct_p": line.get("direct_p", {}).get("roofline"), "decode": line.get("decode", {}).get("roofline")}
    ctr, source = None, None
    if mode == "live":
        ctr = live_counters()
        source = "live: rocprofv3 --pmc runs of this script in this run" if ctr else None
    if ctr is None and mode in ("live", "stored"):
        ctr = {k: counters_for(k) for k in rooflines}
        if any(ctr.values()):
            source = "stored: profiles/counters.json (taken on these kernel sources)"
        else:
            ctr = None
    for key, rf in rooflines.items():
        c = (ctr or {}).get(key)
        if rf is None or not c:
            continue
        rf["traffic"] = c.get("traffic")
        for name in ("mfma_busy", "valu_busy"):
            if name in c:
                rf[name] = c[name]
    line["counters"] = {"source": source, "scale": (ctr or {}).get("_scale")}


def causal_pairs(lq, lk):
    shift = lk - lq
    return sum(min(lk, r + shift + 1) for r in range(lq))


def timed(step, n_events, args):
    """Warm up (args.warmup steps and at least MIN_WARM_S seconds), then time args.steps steps.

    step(ev) runs one step; ev is None or a list of n_events HIP events it records on its stream.
    Returns (wall ms per step, list per timed step of the n_events - 1 event intervals in ms)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < MIN_WARM_S:
        step(None)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(args.steps)]
    t1 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    gaps = [[e[j].elapsed_time(e[j + 1]) for j in range(n_events - 1)] for e in evs]
    return (t2 - t1) * 1e3 / args.steps, gaps


def spread(ms):
    """Mean, median, min and max of per-step times (ms)."""
    return {"mean": round(statistics.fmean(ms), 4), "median": round(statistics.median(ms), 4),
            "min": round(min(ms), 4), "max": round(max(ms), 4)}


def mfma_roofline(flops, kernel_ms):
    """Roofline against the dense FP4 peak; traffic (and the busy fractions) are filled in by
    add_counters once the counter runs are done."""
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": None, "kernel_ms": round(kernel_ms, 4)}


def bench_prefill(args, cfg_id, causal=None, phat_rule=0):
    """One prefill leg: per step, K/V quantize, then the attention with Q quantized in-kernel."""
    import torch
    import bit_quantized_flashattention_amd as hf
    import synth

    cfg = synth.config(cfg_id)
    causal = cfg["causal"] if causal is None else causal
    b, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    q, k, v = synth.make_qkv_device(cfg)
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    sd = torch.from_numpy(s).cuda()
    invd = torch.from_numpy(inv).cuda()
    dims = hf.make_dims(b, hq, hkv, d, lq, lk)
    qkv = hf.quantize_qkv(None, k, v, sd, invd, dims=dims)
    out = torch.empty((b, hq, lq, d), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev):
        # K-hat, V-hat from the quantizer; Q is rescaled and quantized inside the attention kernel
        if ev is not None:
            ev[0].record(stream)
        hf.quantize_qkv(None, k, v, sd, invd, dims=dims, out=qkv)
        if ev is not None:
            ev[1].record(stream)
        hf.attention_fwd(qkv, dims, causal, hf.P_REORDERED, cfg["kv_tile"], out=out, q16=(q, sd), phat_rule=phat_rule)
        if ev is not None:
            ev[2].record(stream)

    step_ms, gaps = timed(step, 3, args)
    quant = [g[0] for g in gaps]
    attn = [g[1] for g in gaps]
    attn_ms = statistics.fmean(attn)
    pairs = causal_pairs(lq, lk) if causal else lq * lk
    flops = 4.0 * d * pairs * b * hq
    res = {
        "workload": "%s: %s B%d Hq%d/Hkv%d d%d L%d, kv_tile %d, P-hat %s; per step: K/V quantize + attention with Q quantized in-kernel"
                    % (cfg["name"], "causal" if causal else "non-causal", b, hq, hkv, d, lq, cfg["kv_tile"],
                       "Direct-P codes" if phat_rule else "exp16 codes, one scale per 32-key block"),
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(step_ms, 4),
        "attention_ms": spread(attn),
        "quantize_kv_ms": spread(quant),
        "roofline": mfma_roofline(flops, attn_ms),
    }
    extra = dict(cfg=cfg, gate=gate, step_ms=step_ms, flops=flops)
    del q, k, v, qkv, out
    torch.cuda.empty_cache()
    return res, extra


def bench_rope(args):
    """The headline step from pre-RoPE Q and K: hifa4_quantize_qkv_rope rotates, rescales and
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

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        hf.quantize_qkv_rope(q, k, v, sd, invd, cosd, sind, dims=dims, out=qkv)
        if ev is not None:
            ev[1].record(stream)
        hf.attention_fwd(qkv, dims, cfg["causal"], hf.P_REORDERED, cfg["kv_tile"], out=out)
        if ev is not None:
            ev[2].record(stream)

    step_ms, gaps = timed(step, 3, args)
    quant = [g[0] for g in gaps]
    attn = [g[1] for g in gaps]
    flops = 4.0 * d * causal_pairs(lq, lk) * b * hq
    # algorithmic bytes of the Q, K (RoPE) and V quantizers: FP16 in, codes and scales out, the
    # tables and the Smooth-QK scales once
    elems = b * (hq + 2 * hkv) * lk * d
    q_bytes = elems * 2 + elems // 2 + elems // 32 + lk * d * 4 + 2 * hkv * d * 4
    quant_ms = statistics.fmean(quant)
    res = {
        "workload": "%s from pre-RoPE Q/K: Q/K/V quantize with RoPE on Q and K, then attention" % cfg["name"],
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(step_ms, 4),
        "attention_ms": spread(attn),
        "quantize_qkv_rope": {"us": round(quant_ms * 1e3, 1), "us_median": round(statistics.median(quant) * 1e3, 1),
                              "us_min": round(min(quant) * 1e3, 1), "us_max": round(max(quant) * 1e3, 1),
                              "bytes": q_bytes, "achieved_gbs": round(q_bytes / (quant_ms * 1e-3) / 1e9, 1),
                              "peak_gbs": HBM_PEAK_GBS},
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

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        # the FP16 query is rescaled and quantized inside the split kernel
        hf.attention_fwd(qkv, dims, True, hf.P_REORDERED, cfg["kv_tile"], 0, out=out, workspace=ws, q16=(q, sd))
        if ev is not None:
            ev[1].record(stream)

    step_ms, gaps = timed(step, 2, args)
    attn = [g[0] for g in gaps]
    attn_ms = statistics.fmean(attn)
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
        "kernel_ms": spread(attn),
        "roofline": {"bound": "hbm", "achieved": round(total / (attn_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(total / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel_us": round(attn_ms * 1e3, 1)},
    }
    del qkv, ws, out, q, k, v
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- CPU oracle baseline

def _cpu_unit(job):
    """One (batch, KV head) unit of the prefill workload on one core: the oracle quantizes the KV
    head's K and V and its query heads, then attends sample rows until the budget is spent."""
    from threadpoolctl import threadpool_limits
    import numpy as np
    from oracle import attention as A
    with threadpool_limits(1):
        q, k, v, s, inv, cfg, seconds, seed = job
        d, lq, lk = cfg["d"], cfg["Lq"], cfg["Lk"]
        t0 = time.perf_counter()
        qq = A.quantize_qkv(q, k, v, s, inv)
        rng = np.random.default_rng(seed)
        flops = 0.0
        rows_done = 0
        hq = q.shape[1]
        while time.perf_counter() - t0 < seconds:
            h = int(rng.integers(hq))
            rows = np.sort(rng.choice(lq, size=16, replace=False))
            A.attention_head_p(qq, 0, h, rows, cfg["causal"], cfg["kv_tile"], A.P_REORDERED)
            vis = np.minimum(lk, rows + (lk - lq) + 1) if cfg["causal"] else np.full(len(rows), lk)
            flops += 4.0 * d * float(vis.sum())
            rows_done += len(rows)
        return flops, rows_done, time.perf_counter() - t0


def cpu_baseline(args):
    """The oracle, as it stands, on the host's cores: one process per (batch, KV head) unit of the
    headline workload (one BLAS thread each), as many units as cores; each unit quantizes its
    K/V head and query heads, then attends randomly drawn query rows for a fixed budget.
    Rate = sum of the units' algorithmic FLOPs / wall time of the pool."""
    import multiprocessing as mp
    import numpy as np
    import synth
    from oracle import smooth

    cfg = synth.config(2)
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    group = cfg["Hq"] // cfg["Hkv"]
    q_cal, k_cal = synth.make_calibration(cfg)
    s, inv, _ = smooth.calibrate(q_cal, k_cal, cfg["alpha"], 4.0)
    jobs = []
    b = 0
    while len(jobs) < cores:
        q, k, v = synth.make_qkv(cfg, batch_slice=(b, b + 1))
        for g in range(cfg["Hkv"]):
            if len(jobs) == cores:
                break
            jobs.append((np.ascontiguousarray(q[:, g * group:(g + 1) * group]), np.ascontiguousarray(k[:, g:g + 1]),
                         np.ascontiguousarray(v[:, g:g + 1]), s[g:g + 1], inv[g:g + 1], cfg, args.cpu_seconds,
                         1000 * b + g))
        b += 1
    ctx = mp.get_context("spawn")  # fresh interpreters: the workers never touch the GPU
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.map(_cpu_unit, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    flops = sum(r[0] for r in res)
    rows = sum(r[1] for r in res)
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(wall, 2), "gflops": round(flops / wall / 1e9, 3),
            "sample": "%d (batch, KV head) units of the headline workload in parallel (one process and one BLAS "
                      "thread per core); each quantizes its K/V head and %d query heads, then attends randomly "
                      "drawn query rows for %.0f s: %d rows in all" % (cores, group, args.cpu_seconds, rows)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU; there is no multi-GPU path: use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    pre, ex = bench_prefill(args, 2)
    progress("headline prefill leg done")
    cfg = ex["cfg"]
    line = {
        "metric": "4-bit attention fwd TFLOP/s (+% FP4-MFMA peak); decode HBM GB/s",
        "value": pre["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {
            "workload": pre["workload"],
            "global_batch": cfg["B"], "seq_len": cfg["Lq"], "heads_q": cfg["Hq"], "heads_kv": cfg["Hkv"],
            "head_dim": cfg["d"], "normalizer": "p_reordered", "phat": "per 32-key block, exp16 codes",
            "smooth_qk_gate": ex["gate"],
        },
        "roofline": pre["roofline"],
        "attention_ms": pre["attention_ms"],
        "quantize_kv_ms": pre["quantize_kv_ms"],
    }
    if "prefill_d256" in args.leg_list:
        line["prefill_d256"] = bench_prefill(args, 3)[0]
    if "prefill_b1" in args.leg_list:
        line["prefill_b1"] = bench_prefill(args, 1)[0]
    if "direct_p" in args.leg_list:
        line["direct_p"] = bench_prefill(args, 2, phat_rule=1)[0]
    if "noncausal" in args.leg_list:
        line["noncausal"] = {"exp16": bench_prefill(args, 2, causal=False)[0],
                             "direct_p": bench_prefill(args, 2, causal=False, phat_rule=1)[0]}
    if "rope_prefill" in args.leg_list:
        line["rope_prefill"] = bench_rope(args)
    if "decode" in args.leg_list:
        line["decode"] = bench_decode(args)
        line["decode"]["cache_append"] = bench_append(args)
    progress("legs done: %s" % ",".join(args.leg_list))
    if args.traffic_probe:
        copy_probe()
    if args.counters != "none":
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        add_counters(line, args.counters)
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline")
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
