"""Seeded synthetic workloads shaped like the pages' models.

This module only draws inputs; it holds none of the method's arithmetic and is
shared by the oracle tests, the GPU parity tests and the benchmark.

The pages ([HiFA4] Abstract) evaluate Qwen3-8B, Gemma2-9B, LLaMA3.1-8B,
Mistral-7B and Phi-4B; no weights or datasets are used here.  Inputs are
post-RoPE Q/K with outlier channels in K (the case Smooth-QK targets) and
N(0, 1) values:

  config 0  tiny, non-causal: B=1, 2 heads, L=128, d=64, 64x64 tiles;
            K channels {5, 20, 37, 60} x20, no RoPE; 256 calibration tokens
  config 1  Qwen3-8B-shaped causal prefill: B=1, Hq=32/Hkv=8, d=128, L=2048;
            pre-RoPE N(0,1), K channel pairs i=56..63 x15, RoPE theta=1e6;
            512 calibration tokens
  config 2  batched causal prefill: B=8, L=4096, same generator as config 1
  config 3  Gemma2-9B-shaped causal prefill: B=2, Hq=16/Hkv=8, d=256, L=8192;
            K magnitude per (KV head, channel pair) exp(z), z ~ N(0,1);
            RoPE theta=1e4; mild smoothing (alpha = 0.25)
  config 4  decode: B=64, one query at position 32767, Lk=32768, Hq=32/Hkv=8,
            d=128, same generator as config 1, split-KV

Seeds: data 1000+i, calibration 2000+i, channel profile 3000+i.  Draws are
float32 standard normals; scaling and RoPE are applied in FP64 and the result
is rounded once to FP16.  RoPE is rotate-half: pair (i, i + d/2) rotates by
position * theta**(-2i/d).
"""

import numpy as np

CONFIGS = {
    0: dict(name="tiny-noncausal-d64", B=1, Hq=2, Hkv=2, Lq=128, Lk=128, d=64, causal=False, kv_tile=64,
            rope_theta=None, outliers="fixed4", calib_tokens=256, alpha=0.5),
    1: dict(name="qwen3-8b-prefill-L2048", B=1, Hq=32, Hkv=8, Lq=2048, Lk=2048, d=128, causal=True, kv_tile=128,
            rope_theta=1e6, outliers="pairs56_63", calib_tokens=512, alpha=0.5),
    2: dict(name="batched-prefill-B8-L4096", B=8, Hq=32, Hkv=8, Lq=4096, Lk=4096, d=128, causal=True, kv_tile=128,
            rope_theta=1e6, outliers="pairs56_63", calib_tokens=512, alpha=0.5),
    3: dict(name="gemma2-9b-prefill-L8192-d256", B=2, Hq=16, Hkv=8, Lq=8192, Lk=8192, d=256, causal=True,
            kv_tile=128, rope_theta=1e4, outliers="lognormal", calib_tokens=512, alpha=0.25),
    4: dict(name="decode-B64-Lk32768", B=64, Hq=32, Hkv=8, Lq=1, Lk=32768, d=128, causal=True, kv_tile=128,
            rope_theta=1e6, outliers="pairs56_63", calib_tokens=512, alpha=0.5),
}


def config(i, **override):
    c = dict(CONFIGS[i])
    c.update(override)
    c["id"] = i
    return c


def _channel_gain(cfg, hkv, d):
    """Per (KV head, channel) magnitude multiplier for K, shape [Hkv, d]."""
    gain = np.ones((hkv, d))
    kind = cfg["outliers"]
    if kind == "fixed4":
        gain[:, [5, 20, 37, 60]] = 20.0
    elif kind == "pairs56_63":
        half = d // 2
        idx = np.arange(56, 64)
        idx = idx[idx < half]
        gain[:, idx] = 15.0
        gain[:, idx + half] = 15.0
    elif kind == "lognormal":
        rng = np.random.default_rng(3000 + cfg["id"])
        z = rng.standard_normal((hkv, d // 2))
        g = np.exp(1.0 * z)
        gain[:, : d // 2] = g
        gain[:, d // 2:] = g
    return gain


def _rope(x, positions, theta):
    """Rotate-half RoPE on the last axis; x [..., L, d] float64, positions [L]."""
    if theta is None:
        return x
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half)
    omega = theta ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_table(theta, n_pos, d):
    """cos and sin of the rotate-half RoPE angles, FP32 [n_pos, d/2]: angle (p, i) = p * theta**(-2i/d),
    computed in FP64 and rounded once.  These tables are an input of the fused RoPE prologue, as a
    model runtime's cached cos/sin would be."""
    half = d // 2
    omega = theta ** (-2.0 * np.arange(half) / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * omega[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _draw(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float64)


def make_qkv(cfg, batch_slice=None, seed_offset=0, pre_rope=False):
    """Q [B, Hq, Lq, d], K, V [B, Hkv, Lk, d] as float16 arrays.

    ``batch_slice`` (start, stop) draws only those batch entries, each from its
    own child seed, so large configs can be generated in chunks with the same
    result as a whole draw.  ``pre_rope`` returns Q and K before the rotation
    (the same draws, rounded to FP16), the input of the fused RoPE prologue.
    """
    b_n, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    lo, hi = batch_slice if batch_slice is not None else (0, b_n)
    children = np.random.SeedSequence(1000 + cfg["id"] + seed_offset).spawn(b_n)
    gain = _channel_gain(cfg, hkv, d)
    qpos = np.arange(lk - lq, lk)
    kpos = np.arange(lk)
    qs, ks, vs = [], [], []
    for b in range(lo, hi):
        rng = np.random.default_rng(children[b])
        q = _draw(rng, (hq, lq, d))
        k = _draw(rng, (hkv, lk, d)) * gain[:, None, :]
        v = _draw(rng, (hkv, lk, d))
        theta = None if pre_rope else cfg["rope_theta"]
        qs.append(_rope(q, qpos, theta).astype(np.float16))
        ks.append(_rope(k, kpos, theta).astype(np.float16))
        vs.append(v.astype(np.float16))
    return np.stack(qs), np.stack(ks), np.stack(vs)


def make_calibration(cfg, seed_offset=0):
    """Calibration draw from the same generator: q_cal [Hq, N, d], k_cal [Hkv, N, d] float16."""
    hq, hkv, d, n = cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["calib_tokens"]
    rng = np.random.default_rng(2000 + cfg["id"] + seed_offset)
    gain = _channel_gain(cfg, hkv, d)
    pos = np.arange(n)
    q = _rope(_draw(rng, (hq, n, d)), pos, cfg["rope_theta"])
    k = _rope(_draw(rng, (hkv, n, d)) * gain[:, None, :], pos, cfg["rope_theta"])
    return q.astype(np.float16), k.astype(np.float16)


def small(cfg_id, **override):
    """A reduced-size version of a config (same generator) for tests that the oracle finishes quickly."""
    return config(cfg_id, **override)


def make_qkv_device(cfg, device="cuda", with_q=True, with_kv=True, pre_rope=False):
    """Same distributions as make_qkv, drawn on the GPU with torch's seeded generator.

    Used for the full-size workloads (the decode cache alone is 8.6 GB of FP16); the
    values differ from make_qkv's (another random stream) but the recipe is identical.
    Returns float16 CUDA tensors (None for parts not requested); ``pre_rope`` as in make_qkv.
    """
    import torch
    b_n, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + cfg["id"])
    gain = torch.tensor(_channel_gain(cfg, hkv, d), dtype=torch.float32, device=device)

    def rope(x, positions):
        if cfg["rope_theta"] is None or pre_rope:
            return x
        half = d // 2
        i = torch.arange(half, device=device, dtype=torch.float64)
        omega = cfg["rope_theta"] ** (-2.0 * i / d)
        ang = (positions.to(torch.float64)[:, None] * omega[None, :])
        c, s = torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)
        a, bb = x[..., :half], x[..., half:]
        return torch.cat([a * c - bb * s, bb * c + a * s], dim=-1)

    q = torch.empty((b_n, hq, lq, d), dtype=torch.float16, device=device) if with_q else None
    k = torch.empty((b_n, hkv, lk, d), dtype=torch.float16, device=device) if with_kv else None
    v = torch.empty((b_n, hkv, lk, d), dtype=torch.float16, device=device) if with_kv else None
    qpos = torch.arange(lk - lq, lk, device=device)
    kpos = torch.arange(lk, device=device)
    for b in range(b_n):
        if with_q:
            q[b] = rope(torch.randn((hq, lq, d), generator=gen, device=device), qpos).to(torch.float16)
        if with_kv:
            kk = torch.randn((hkv, lk, d), generator=gen, device=device) * gain[:, None, :]
            k[b] = rope(kk, kpos).to(torch.float16)
            v[b] = torch.randn((hkv, lk, d), generator=gen, device=device).to(torch.float16)
    return q, k, v
