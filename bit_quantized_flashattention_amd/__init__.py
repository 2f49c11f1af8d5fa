"""Python binding of libhifa4 (MI355X / gfx950 4-bit FlashAttention forward).

Argument marshalling only: every step of the computation runs in the HIP library
(``libhifa4.so``, built in-tree by ``build.py``).  PyTorch supplies device memory and
the current HIP stream.  The functions mirror the C ABI in ``include/hifa4.h``:

    calibrate(q_cal, k_cal, alpha, tau)            -> (s, inv_s, gate_on)     host
    quantize_qkv(q, k, v, s, inv_s)                -> dict of code/scale tensors
    attention_fwd(qkv_q, dims..., causal, ...)     -> FP16 output (+ tile statistics)
    decode_num_splits(...), attention_workspace_bytes(...)

There is no fallback: if the library is missing or fails, a RuntimeError is raised.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhifa4.so")

P_REORDERED = 0
INCONSISTENT = 1
MAX_CEIL, MAX_NEAREST16 = 0, 1  # running-max rules (hifa4.h)
PHAT_BLOCK32, PHAT_TILE = 0, 1  # P-hat scale granularity (hifa4.h)
PHAT_EXP16, PHAT_DIRECT = 0, 1  # P-hat code rule (hifa4.h)


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("len_q", ctypes.c_int64), ("len_kv", ctypes.c_int64)]


class Opts(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("normalizer", ctypes.c_int32), ("kv_tile", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("kv_capacity", ctypes.c_int64), ("max_rule", ctypes.c_int32),
                ("phat_scale", ctypes.c_int32), ("phat_rule", ctypes.c_int32), ("prefill_waves", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhifa4.so is not built (run python -m bit_quantized_flashattention_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.hifa4_calibrate.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_float, ctypes.c_float, _vp, _vp, _vp]
        L.hifa4_calibrate.restype = ctypes.c_int
        L.hifa4_quantize_qkv.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 11
        L.hifa4_quantize_qkv.restype = ctypes.c_int
        L.hifa4_quantize_qkv_rule.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32] + [_vp] * 12
        L.hifa4_quantize_qkv_rule.restype = ctypes.c_int
        L.hifa4_quantize_qkv_rope.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 7 + [ctypes.c_int64] + [_vp] * 7
        L.hifa4_quantize_qkv_rope.restype = ctypes.c_int
        L.hifa4_cache_append.argtypes = [ctypes.POINTER(Dims), ctypes.c_int64] + [_vp] * 5 + [ctypes.c_int64] + [_vp] * 6
        L.hifa4_cache_append.restype = ctypes.c_int
        L.hifa4_decode_num_splits.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts)]
        L.hifa4_decode_num_splits.restype = ctypes.c_int32
        L.hifa4_attention_workspace_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts)]
        L.hifa4_attention_workspace_bytes.restype = ctypes.c_size_t
        L.hifa4_attention_fwd.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts)] + [_vp] * 8 + \
            [ctypes.c_size_t, _vp, _vp]
        L.hifa4_attention_fwd.restype = ctypes.c_int
        L.hifa4_attention_fwd_q16.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts)] + [_vp] * 4 + \
            [ctypes.c_int64] + [_vp] * 6 + \
            [ctypes.c_size_t, _vp, _vp]
        L.hifa4_attention_fwd_q16.restype = ctypes.c_int
        L.hifa4_attention_fwd_q16_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts)] + [_vp] * 4 + \
            [ctypes.c_int64] + [_vp] * 7
        L.hifa4_attention_fwd_q16_noalloc.restype = ctypes.c_int
        L.hifa4_status_string.argtypes = [ctypes.c_int]
        L.hifa4_status_string.restype = ctypes.c_char_p
        L.hifa4_last_error.argtypes = []
        L.hifa4_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


class Hifa4Error(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("hifa4 status %d (%s): %s" % (status, lib().hifa4_status_string(status).decode(), detail))


def _check(status):
    if status != 0:
        raise Hifa4Error(status, lib().hifa4_last_error().decode())


def make_dims(batch, heads_q, heads_kv, head_dim, len_q, len_kv):
    return Dims(batch, heads_q, heads_kv, head_dim, len_q, len_kv)


def make_opts(causal=False, normalizer=P_REORDERED, kv_tile=128, num_splits=0, kv_capacity=0, max_rule=0,
              phat_scale=PHAT_BLOCK32, phat_rule=PHAT_EXP16, prefill_waves=0):
    return Opts(int(causal), int(normalizer), int(kv_tile), int(num_splits), int(kv_capacity), int(max_rule),
                int(phat_scale), int(phat_rule), int(prefill_waves))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def calibrate(q_cal, k_cal, alpha=0.5, tau=4.0):
    """Smooth-QK scales on the host from FP16 calibration activations.

    q_cal [Hq, N, d], k_cal [Hkv, N, d] (numpy float16 or CPU torch float16).
    Returns (s, inv_s) float32 numpy [Hkv, d] and the gate flag.
    """
    q = np.ascontiguousarray(np.asarray(q_cal, dtype=np.float16))
    k = np.ascontiguousarray(np.asarray(k_cal, dtype=np.float16))
    hq, n, d = q.shape
    hkv = k.shape[0]
    if k.shape != (hkv, n, d):
        raise ValueError("k_cal must be [Hkv, N, d] with the same N and d as q_cal")
    s = np.empty((hkv, d), dtype=np.float32)
    inv = np.empty((hkv, d), dtype=np.float32)
    gate = ctypes.c_int32(0)
    _check(lib().hifa4_calibrate(q.ctypes.data, k.ctypes.data, n, hq, hkv, d, float(alpha), float(tau),
                                 s.ctypes.data, inv.ctypes.data, ctypes.addressof(gate)))
    return s, inv, bool(gate.value)


def quantized_shapes(batch, heads_q, heads_kv, head_dim, len_q, len_kv):
    lk32 = -(-len_kv // 32) * 32
    return {
        "q_codes": (batch, heads_q, len_q, head_dim // 2), "q_scales": (batch, heads_q, len_q, head_dim // 32),
        "k_codes": (batch, heads_kv, len_kv, head_dim // 2), "k_scales": (batch, heads_kv, head_dim // 32, lk32),
        "v_codes": (batch, heads_kv, lk32 // 32, head_dim, 16), "v_scales": (batch, heads_kv, lk32 // 32, head_dim),
    }


SCALE_NO_CLIP, SCALE_FLOOR = 0, 1


def quantize_qkv(q=None, k=None, v=None, s=None, inv_s=None, dims=None, out=None, stream=None, scale_rule=SCALE_NO_CLIP):
    """Smooth-QK rescale + 4-bit quantization on the GPU.

    q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d]: contiguous CUDA float16 tensors (any may be None
    when ``dims`` is given).  s, inv_s: CUDA float32 [Hkv, d] or None.  Returns a dict of uint8
    tensors named as in the C ABI (allocated unless ``out`` provides them).
    """
    import torch
    if dims is None:
        b, hq, lq, d = q.shape
        hkv, lk = k.shape[1], k.shape[2]
        dims = make_dims(b, hq, hkv, d, lq, lk)
    for t in (q, k, v):
        if t is not None and (not t.is_cuda or t.dtype != torch.float16 or not t.is_contiguous()):
            raise ValueError("q, k, v must be contiguous CUDA float16 tensors")
    shapes = quantized_shapes(dims.batch, dims.heads_q, dims.heads_kv, dims.head_dim, dims.len_q, dims.len_kv)
    dev = next(t for t in (q, k, v) if t is not None).device
    res = dict(out) if out is not None else {}
    for name, shp in shapes.items():
        src = {"q": q, "k": k, "v": v}[name[0]]
        if src is not None and name not in res:
            res[name] = torch.empty(shp, dtype=torch.uint8, device=dev)
    if (s is None) != (inv_s is None):
        raise ValueError("pass both s and inv_s or neither")
    _check(lib().hifa4_quantize_qkv_rule(
        ctypes.byref(dims), int(scale_rule), _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(inv_s),
        _ptr(res.get("q_codes") if q is not None else None), _ptr(res.get("q_scales") if q is not None else None),
        _ptr(res.get("k_codes") if k is not None else None), _ptr(res.get("k_scales") if k is not None else None),
        _ptr(res.get("v_codes") if v is not None else None), _ptr(res.get("v_scales") if v is not None else None),
        _stream(stream)))
    return res


def quantize_qkv_rope(q=None, k=None, v=None, s=None, inv_s=None, rope_cos=None, rope_sin=None, dims=None,
                      out=None, stream=None):
    """RoPE + Smooth-QK + 4-bit quantization of pre-RoPE q, k (and plain v) on the GPU.

    rope_cos, rope_sin: CUDA float32 [n_pos, d/2] tables (n_pos >= Lk).  Otherwise as quantize_qkv.
    """
    import torch
    if dims is None:
        b, hq, lq, d = q.shape
        hkv, lk = k.shape[1], k.shape[2]
        dims = make_dims(b, hq, hkv, d, lq, lk)
    for t in (q, k, v):
        if t is not None and (not t.is_cuda or t.dtype != torch.float16 or not t.is_contiguous()):
            raise ValueError("q, k, v must be contiguous CUDA float16 tensors")
    for t in (rope_cos, rope_sin):
        if t is not None and (not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("rope tables must be contiguous CUDA float32 tensors")
    shapes = quantized_shapes(dims.batch, dims.heads_q, dims.heads_kv, dims.head_dim, dims.len_q, dims.len_kv)
    dev = next(t for t in (q, k, v) if t is not None).device
    res = dict(out) if out is not None else {}
    for name, shp in shapes.items():
        src = {"q": q, "k": k, "v": v}[name[0]]
        if src is not None and name not in res:
            res[name] = torch.empty(shp, dtype=torch.uint8, device=dev)
    n_pos = rope_cos.shape[0] if rope_cos is not None else 0
    _check(lib().hifa4_quantize_qkv_rope(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(inv_s), _ptr(rope_cos), _ptr(rope_sin), n_pos,
        _ptr(res.get("q_codes") if q is not None else None), _ptr(res.get("q_scales") if q is not None else None),
        _ptr(res.get("k_codes") if k is not None else None), _ptr(res.get("k_scales") if k is not None else None),
        _ptr(res.get("v_codes") if v is not None else None), _ptr(res.get("v_scales") if v is not None else None),
        _stream(stream)))
    return res


def cache_shapes(batch, heads_kv, head_dim, capacity):
    """Shapes of the 4-bit K-hat / V-hat cache buffers of hifa4_cache_append (and of the stage)."""
    c32 = -(-capacity // 32) * 32
    return {
        "k_codes": (batch, heads_kv, capacity, head_dim // 2),
        "k_scales": (batch, heads_kv, head_dim // 32, c32),
        "v_codes": (batch, heads_kv, c32 // 32, head_dim, 16),
        "v_scales": (batch, heads_kv, c32 // 32, head_dim),
        "v_stage": (batch, heads_kv, 32, head_dim),
    }


def make_cache(batch, heads_kv, head_dim, capacity, device="cuda"):
    """Empty cache buffers (dict) for cache_append / attention_fwd(kv_capacity=...)."""
    import torch
    out = {}
    for name, shp in cache_shapes(batch, heads_kv, head_dim, capacity).items():
        dt = torch.float16 if name == "v_stage" else torch.uint8
        out[name] = torch.zeros(shp, dtype=dt, device=device)
    out["capacity"] = capacity
    out["length"] = 0
    return out


def cache_append(cache, k_new, v_new, inv_s=None, rope_cos=None, rope_sin=None, heads_q=None, stream=None):
    """Append k_new, v_new (CUDA float16 [B, Hkv, n, d]) to ``cache``; returns the new length."""
    import torch
    b, hkv, n, d = k_new.shape
    for t in (k_new, v_new):
        if not t.is_cuda or t.dtype != torch.float16 or not t.is_contiguous():
            raise ValueError("k_new, v_new must be contiguous CUDA float16 tensors")
    dims = make_dims(b, heads_q or hkv, hkv, d, n, cache["length"])
    n_pos = rope_cos.shape[0] if rope_cos is not None else 0
    _check(lib().hifa4_cache_append(
        ctypes.byref(dims), cache["capacity"], _ptr(k_new), _ptr(v_new), _ptr(inv_s), _ptr(rope_cos), _ptr(rope_sin),
        n_pos, _ptr(cache["k_codes"]), _ptr(cache["k_scales"]), _ptr(cache["v_codes"]), _ptr(cache["v_scales"]),
        _ptr(cache["v_stage"]), _stream(stream)))
    cache["length"] += n
    return cache["length"]


def decode_num_splits(dims, opts):
    return int(lib().hifa4_decode_num_splits(ctypes.byref(dims), ctypes.byref(opts)))


def attention_workspace_bytes(dims, opts):
    return int(lib().hifa4_attention_workspace_bytes(ctypes.byref(dims), ctypes.byref(opts)))


STATS_ROWS = 16  # query rows per tile-statistics block


def stats_shape(dims, kv_tile):
    return (dims.batch, dims.heads_q, -(-dims.len_q // STATS_ROWS), -(-dims.len_kv // kv_tile), 2)


def attention_fwd(qkv, dims, causal=False, normalizer=P_REORDERED, kv_tile=128, num_splits=0,
                  out=None, workspace=None, tile_stats=None, stream=None, q16=None, kv_capacity=0,
                  max_rule=MAX_CEIL, phat_scale=PHAT_BLOCK32, phat_rule=PHAT_EXP16, prefill_waves=0):
    """4-bit attention forward from quantized operands (a dict as returned by quantize_qkv).

    ``q16=(q, s)`` or ``(q, s, rope_cos, rope_sin)``: take FP16 Q (before RoPE when the tables are
    given) and the Smooth-QK scales (device tensor or None) instead of qkv's Q-hat and quantize Q
    inside the kernel (hifa4_attention_fwd_q16); qkv then needs only the K-hat and V-hat entries.
    ``kv_capacity``: the key rows allocated per (batch, KV head) when qkv's K-hat / V-hat live in a
    cache (make_cache / cache_append); 0 = Lk.  ``max_rule``: MAX_CEIL (the method) or MAX_NEAREST16
    (round-to-nearest running max, an accuracy variant; prefill, P-Reordered, no tile statistics).
    ``phat_scale``: PHAT_BLOCK32 (the method) or PHAT_TILE; ``phat_rule``: PHAT_EXP16 (the method) or
    PHAT_DIRECT (Direct-P codes); the variants run P-Reordered without tile statistics.
    ``prefill_waves``: 0 (automatic), 4 or 8 waves per prefill work-group (the output does not
    depend on it).

    Returns the FP16 output [B, Hq, Lq, d] (``out`` if given).  ``tile_stats``: True to allocate,
    or an FP32 tensor of ``stats_shape`` to fill (prefill only); returned as a second value.
    """
    import torch
    opts = make_opts(causal, normalizer, kv_tile, num_splits, kv_capacity, max_rule, phat_scale, phat_rule,
                     prefill_waves)
    dev = qkv["k_codes"].device
    if out is None:
        out = torch.empty((dims.batch, dims.heads_q, dims.len_q, dims.head_dim), dtype=torch.float16, device=dev)
    need = attention_workspace_bytes(dims, opts)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stats = None
    if tile_stats is True:
        stats = torch.empty(stats_shape(dims, kv_tile), dtype=torch.float32, device=dev)
    elif tile_stats is not None:
        stats = tile_stats
    if q16 is None:
        _check(lib().hifa4_attention_fwd(
            ctypes.byref(dims), ctypes.byref(opts), _ptr(qkv["q_codes"]), _ptr(qkv["q_scales"]), _ptr(qkv["k_codes"]),
            _ptr(qkv["k_scales"]), _ptr(qkv["v_codes"]), _ptr(qkv["v_scales"]), _ptr(out), _ptr(workspace),
            workspace.numel() if workspace is not None else 0, _ptr(stats), _stream(stream)))
    else:
        q, s = q16[0], q16[1]
        rc, rs = (q16[2], q16[3]) if len(q16) > 2 else (None, None)
        n_pos = rc.shape[0] if rc is not None else 0
        _check(lib().hifa4_attention_fwd_q16(
            ctypes.byref(dims), ctypes.byref(opts), _ptr(q), _ptr(s), _ptr(rc), _ptr(rs), n_pos, _ptr(qkv["k_codes"]),
            _ptr(qkv["k_scales"]), _ptr(qkv["v_codes"]), _ptr(qkv["v_scales"]), _ptr(out), _ptr(workspace),
            workspace.numel() if workspace is not None else 0, _ptr(stats), _stream(stream)))
    return (out, stats) if tile_stats is not None else out


NOALLOC_SCRATCH_BYTES = 8 << 20  # the library's fixed decode scratch per GPU (hifa4.h)


def attention_fwd_q16_noalloc(kv, q, s, dims, causal=False, normalizer=P_REORDERED, kv_tile=128, num_splits=0,
                              out=None, stream=None, rope_cos=None, rope_sin=None, kv_capacity=0, max_rule=MAX_CEIL,
                              phat_scale=PHAT_BLOCK32, phat_rule=PHAT_EXP16):
    """hifa4_attention_fwd_q16_noalloc: the fused-Q forward with decode partials in the library's fixed
    device scratch (no workspace).  kv: dict with the K-hat / V-hat tensors; q FP16 [B, Hq, Lq, d];
    s the Smooth-QK scales or None.  ``out`` must be given by callers that cannot allocate."""
    import torch
    opts = make_opts(causal, normalizer, kv_tile, num_splits, kv_capacity, max_rule, phat_scale, phat_rule)
    if out is None:
        out = torch.empty((dims.batch, dims.heads_q, dims.len_q, dims.head_dim), dtype=torch.float16,
                          device=kv["k_codes"].device)
    n_pos = rope_cos.shape[0] if rope_cos is not None else 0
    _check(lib().hifa4_attention_fwd_q16_noalloc(
        ctypes.byref(dims), ctypes.byref(opts), _ptr(q), _ptr(s), _ptr(rope_cos), _ptr(rope_sin), n_pos,
        _ptr(kv["k_codes"]), _ptr(kv["k_scales"]), _ptr(kv["v_codes"]), _ptr(kv["v_scales"]), _ptr(out), None,
        _stream(stream)))
    return out
