"""C ABI checks that need no GPU: the library loads, exports what include/hifa4.h declares,
rejects invalid arguments before launching anything, and calibrates like the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
from oracle import smooth
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hf.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hf.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hifa4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hifa4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.hifa4_status_string(0) == b"ok"
    assert L.hifa4_status_string(5) == b"HIP runtime error"
    assert b"16-byte" in L.hifa4_status_string(6)


def test_misaligned_device_pointers_are_rejected(L):
    dims = hf.make_dims(1, 4, 2, 128, 64, 64)
    ok, off = ctypes.c_void_p(256), ctypes.c_void_p(264)  # never dereferenced
    for i in range(7):
        args = [ok] * 7
        args[i] = off
        st = L.hifa4_attention_fwd(ctypes.byref(dims), ctypes.byref(hf.make_opts(causal=True)), *args, None, 0, None, None)
        assert st == 6 and b"aligned" in L.hifa4_last_error(), i
    dec = hf.make_dims(1, 4, 2, 128, 1, 64)  # in-kernel RoPE is a decode feature

    def q16(args, n_pos=64, dm=dec):
        # q, s, cos, sin | n_pos | K-hat, V-hat (4), out, workspace
        return L.hifa4_attention_fwd_q16(ctypes.byref(dm), ctypes.byref(hf.make_opts(causal=True)),
                                         *args[:4], n_pos, *args[4:], 0, None, None)
    for i in range(10):
        args = [ok] * 10
        args[i] = off
        assert q16(args) == 6, i
    args = [ok] * 10
    args[0] = None  # q is required; s may be NULL
    assert q16(args) == 1
    args = [ok] * 10
    args[3] = None  # one RoPE table without the other
    assert q16(args) == 1
    assert q16([ok] * 10, n_pos=63) == 2  # tables shorter than Lk
    assert q16([ok] * 10, dm=dims) == 3  # RoPE tables with a prefill shape
    for i in range(11):
        args = [ok] * 11
        args[i] = off
        st = L.hifa4_quantize_qkv(ctypes.byref(dims), *args, None)
        assert st == 6, i


def test_attention_rejects_bad_arguments_without_launching(L):
    dims = hf.make_dims(1, 4, 2, 128, 64, 64)
    opts = hf.make_opts(causal=True)
    dummy = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    args = [dummy] * 7
    st = L.hifa4_attention_fwd(ctypes.byref(dims), ctypes.byref(opts), None, *args[:5], args[5], None, 0, None, None)
    assert st == 1 and b"NULL" in L.hifa4_last_error()
    bad = [hf.make_dims(1, 4, 3, 128, 64, 64), hf.make_dims(1, 4, 2, 96, 64, 64), hf.make_dims(0, 4, 2, 128, 64, 64),
           hf.make_dims(1, 4, 2, 128, 65, 64), hf.make_dims(1, 24, 2, 128, 64, 64)]
    want = [2, 3, 2, 2, 3]
    for dm, w in zip(bad, want):
        o = hf.make_opts(causal=True)
        st = L.hifa4_attention_fwd(ctypes.byref(dm), ctypes.byref(o), *([dummy] * 7), None, 0, None, None)
        assert st == w, (dm.heads_q, dm.heads_kv, dm.head_dim, dm.len_q, st, L.hifa4_last_error())
    for o, w in [(hf.make_opts(kv_tile=96), 3), (hf.make_opts(normalizer=2), 2), (hf.Opts(2, 0, 128, 0), 2)]:
        st = L.hifa4_attention_fwd(ctypes.byref(dims), ctypes.byref(o), *([dummy] * 7), None, 0, None, None)
        assert st == w
    # decode without workspace
    dd = hf.make_dims(2, 8, 2, 128, 1, 4096)
    o = hf.make_opts(causal=True)
    assert L.hifa4_attention_workspace_bytes(ctypes.byref(dd), ctypes.byref(o)) > 0
    st = L.hifa4_attention_fwd(ctypes.byref(dd), ctypes.byref(o), *([dummy] * 7), None, 0, None, None)
    assert st == 4 and b"workspace" in L.hifa4_last_error()
    assert L.hifa4_attention_workspace_bytes(ctypes.byref(dims), ctypes.byref(opts)) == 0


def test_max_rule_is_validated_and_limited_to_prefill(L):
    # hifa4_attn_opts: four int32, the int64 capacity at offset 16, max_rule at 24, phat_scale at
    # 28, phat_rule at 32, prefill_waves at 36: 40 bytes
    assert ctypes.sizeof(hf.Opts) == 40 and hf.Opts.max_rule.offset == 24
    assert hf.Opts.phat_scale.offset == 28 and hf.Opts.phat_rule.offset == 32 and hf.Opts.prefill_waves.offset == 36
    dummy = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    pre = hf.make_dims(1, 4, 2, 128, 64, 64)
    st = L.hifa4_attention_fwd(ctypes.byref(pre), ctypes.byref(hf.make_opts(max_rule=2)), *([dummy] * 7), None, 0, None, None)
    assert st == 2 and b"max_rule" in L.hifa4_last_error()
    near = hf.make_opts(causal=True, max_rule=hf.MAX_NEAREST16)
    dec = hf.make_dims(2, 8, 2, 128, 1, 4096)
    st = L.hifa4_attention_fwd(ctypes.byref(dec), ctypes.byref(near), *([dummy] * 7), dummy, 1 << 30, None, None)
    assert st == 3 and b"prefill-only" in L.hifa4_last_error()
    inc = hf.make_opts(causal=True, normalizer=hf.INCONSISTENT, max_rule=hf.MAX_NEAREST16)
    st = L.hifa4_attention_fwd(ctypes.byref(pre), ctypes.byref(inc), *([dummy] * 7), None, 0, None, None)
    assert st == 3
    stats = ctypes.cast(dummy, ctypes.POINTER(ctypes.c_float))
    st = L.hifa4_attention_fwd(ctypes.byref(pre), ctypes.byref(near), *([dummy] * 7), None, 0, stats, None)
    assert st == 3 and b"statistics" in L.hifa4_last_error()


def test_phat_options_are_validated(L):
    dummy = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    pre = hf.make_dims(1, 4, 2, 128, 64, 64)

    def call(o, stats=None):
        return L.hifa4_attention_fwd(ctypes.byref(pre), ctypes.byref(o), *([dummy] * 7), None, 0, stats, None)
    assert call(hf.make_opts(phat_scale=2)) == 2 and b"phat_scale" in L.hifa4_last_error()
    assert call(hf.make_opts(phat_rule=5)) == 2 and b"phat_rule" in L.hifa4_last_error()
    # Direct-P takes per-block scales; the variants run P-Reordered with the integer running max
    assert call(hf.make_opts(phat_scale=hf.PHAT_TILE, phat_rule=hf.PHAT_DIRECT)) == 3
    for o in [hf.make_opts(normalizer=hf.INCONSISTENT, phat_rule=hf.PHAT_DIRECT),
              hf.make_opts(normalizer=hf.INCONSISTENT, phat_scale=hf.PHAT_TILE),
              hf.make_opts(max_rule=hf.MAX_NEAREST16, phat_rule=hf.PHAT_DIRECT)]:
        assert call(o) == 3 and b"P-Reordered" in L.hifa4_last_error()
    stats = ctypes.cast(dummy, ctypes.POINTER(ctypes.c_float))
    assert call(hf.make_opts(phat_rule=hf.PHAT_DIRECT), stats) == 3 and b"statistics" in L.hifa4_last_error()


def test_prefill_waves_is_validated(L):
    dummy = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    pre = hf.make_dims(1, 4, 2, 128, 64, 64)

    def call(o, dims=pre, stats=None):
        return L.hifa4_attention_fwd(ctypes.byref(dims), ctypes.byref(o), *([dummy] * 7), None, 0, stats, None)
    for w in (1, 2, 6, 16, -4):
        assert call(hf.make_opts(prefill_waves=w)) == 2 and b"prefill_waves" in L.hifa4_last_error()
    # 4-wave work-groups exist for the method's P-Reordered instance only
    for o in [hf.make_opts(prefill_waves=4, normalizer=hf.INCONSISTENT),
              hf.make_opts(prefill_waves=4, max_rule=hf.MAX_NEAREST16),
              hf.make_opts(prefill_waves=4, phat_rule=hf.PHAT_DIRECT),
              hf.make_opts(prefill_waves=4, phat_scale=hf.PHAT_TILE)]:
        assert call(o) == 3 and b"prefill_waves" in L.hifa4_last_error()
    stats = ctypes.cast(dummy, ctypes.POINTER(ctypes.c_float))
    assert call(hf.make_opts(prefill_waves=4), stats=stats) == 3 and b"statistics" in L.hifa4_last_error()


def test_noalloc_rejects_partials_beyond_the_fixed_scratch(L):
    dummy = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    big = hf.make_dims(256, 64, 8, 256, 1, 1 << 16)
    o = hf.make_opts(causal=True, num_splits=4)
    need = hf.attention_workspace_bytes(big, o)
    assert need > hf.NOALLOC_SCRATCH_BYTES
    st = L.hifa4_attention_fwd_q16_noalloc(ctypes.byref(big), ctypes.byref(o), dummy, None, None, None, 0,
                                           *([dummy] * 5), None, None)
    assert st == 4 and b"scratch" in L.hifa4_last_error()


def test_size_limits_are_rejected(L):
    dummy = ctypes.c_void_p(256)
    o = hf.make_opts(causal=False)
    for dm in [hf.make_dims(1, 4, 2, 256, 16, 1 << 24),  # a K-hat slice of 2^31 bytes
               hf.make_dims(1, 4, 2, 128, 1 << 31, 64),
               hf.make_dims(70000, 4, 2, 128, 16, 64),
               hf.make_dims(1, 70000 * 8, 8, 128, 16, 64)]:
        st = L.hifa4_attention_fwd(ctypes.byref(dm), ctypes.byref(o), *([dummy] * 7), None, 0, None, None)
        assert st in (2, 3), (dm.batch, dm.heads_q, dm.len_q, dm.len_kv, st)
    ok = hf.make_dims(1, 4, 2, 256, 16, (1 << 24) - 32)
    assert L.hifa4_attention_workspace_bytes(ctypes.byref(ok), ctypes.byref(o)) == 0  # valid prefill


def test_decode_splits_resolution(L):
    d = hf.make_dims(64, 32, 8, 128, 1, 32768)
    assert hf.decode_num_splits(d, hf.make_opts(causal=True, num_splits=0)) >= 1
    assert hf.decode_num_splits(d, hf.make_opts(causal=True, num_splits=7)) == 7
    small = hf.make_dims(1, 4, 1, 64, 1, 200)  # 2 tiles of 128: at most 2 splits
    assert hf.decode_num_splits(small, hf.make_opts(num_splits=16)) == 2
    assert hf.decode_num_splits(hf.make_dims(1, 4, 1, 64, 9, 200), hf.make_opts()) == 1


def test_automatic_decode_splits():
    """The automatic split count at Lk = 32768 (256 tiles of 128 keys), Hkv = 8: one wave per SIMD
    (1024 waves) for up to 32 (batch, KV head) units, two per SIMD (2048) above, at most 64
    splits and at least 8 tiles per split."""
    want = {1: 32, 2: 32, 4: 32, 8: 32, 16: 16, 32: 8, 64: 4, 128: 2}
    for b, n in want.items():
        d = hf.make_dims(b, 32, 8, 128, 1, 32768)
        assert hf.decode_num_splits(d, hf.make_opts(causal=True)) == n, b
    # a short cache: at least 8 tiles per split
    assert hf.decode_num_splits(hf.make_dims(1, 32, 8, 128, 1, 2048), hf.make_opts(causal=True)) == 2


def test_quantize_rejects_bad_arguments(L):
    dims = hf.make_dims(1, 4, 2, 128, 64, 64)
    dummy = ctypes.c_void_p(16)
    st = L.hifa4_quantize_qkv(ctypes.byref(dims), dummy, None, None, dummy, None, None, None, None, None, None, None, None)
    assert st == 1  # s without inv_s
    st = L.hifa4_quantize_qkv(ctypes.byref(dims), dummy, None, None, None, None, None, None, None, None, None, None, None)
    assert st == 1  # q present, outputs missing
    bad = hf.make_dims(1, 4, 2, 80, 64, 64)
    st = L.hifa4_quantize_qkv(ctypes.byref(bad), dummy, None, None, None, None, dummy, dummy, None, None, None, None, None)
    assert st == 3
    st = L.hifa4_quantize_qkv_rule(ctypes.byref(dims), 2, dummy, None, None, None, None, dummy, dummy, None, None, None,
                                   None, None)
    assert st == 2 and b"scale_rule" in L.hifa4_last_error()


def test_quantize_rope_rejects_bad_arguments(L):
    dims = hf.make_dims(1, 4, 2, 128, 64, 64)
    ok = ctypes.c_void_p(256)
    outs = [ok] * 6
    # q, k, v, s, inv_s, cos, sin, n_pos, outputs..., stream
    st = L.hifa4_quantize_qkv_rope(ctypes.byref(dims), ok, ok, None, ok, ok, None, None, 64, *outs, None)
    assert st == 1 and b"RoPE" in L.hifa4_last_error()
    st = L.hifa4_quantize_qkv_rope(ctypes.byref(dims), ok, ok, None, ok, ok, ok, ok, 63, *outs, None)
    assert st == 2 and b"positions" in L.hifa4_last_error()
    longq = hf.make_dims(1, 4, 2, 128, 65, 64)
    st = L.hifa4_quantize_qkv_rope(ctypes.byref(longq), ok, ok, None, ok, ok, ok, ok, 64, *outs, None)
    assert st == 2
    st = L.hifa4_quantize_qkv_rope(ctypes.byref(dims), ok, ok, None, ok, ok, ctypes.c_void_p(260), ok, 64, *outs,
                                   None)
    assert st == 6
    # V alone needs no tables
    st = L.hifa4_quantize_qkv_rope(ctypes.byref(dims), None, None, ok, None, None, None, None, 0, None, None, None,
                                   None, None, None, None)
    assert st == 1  # v outputs missing, checked before any launch


def test_cache_append_rejects_bad_arguments(L):
    ok = ctypes.c_void_p(256)
    ptrs = [ok] * 2 + [None, None, None] + [ok] * 5  # k_new, v_new, inv_s, cos, sin | 5 cache buffers
    dims = hf.make_dims(2, 8, 2, 128, 1, 100)  # len_q = keys appended, len_kv = keys present

    def app(dm, cap, p, n_pos=0):
        return L.hifa4_cache_append(ctypes.byref(dm), cap, *p[:5], n_pos, *p[5:], None)
    assert app(dims, 100, ptrs) == 2  # 100 + 1 > capacity
    assert app(hf.make_dims(2, 8, 2, 96, 1, 10), 128, ptrs) == 3  # head_dim
    bad = list(ptrs)
    bad[9] = None  # stage missing
    assert app(dims, 128, bad) == 1
    rope = list(ptrs)
    rope[3] = ok
    assert app(dims, 128, rope) == 1  # one table without the other
    rope[4] = ok
    assert app(dims, 128, rope, n_pos=100) == 2  # tables must cover position 100
    mis = list(ptrs)
    mis[7] = ctypes.c_void_p(264)
    assert app(dims, 128, mis) == 6
    o = hf.make_opts(causal=True, kv_capacity=99)
    assert L.hifa4_attention_workspace_bytes(ctypes.byref(dims), ctypes.byref(o)) == 0  # capacity < len_kv


@pytest.mark.parametrize("cfg_id", [0, 1, 3])
def test_calibrate_matches_oracle_bit_exactly(L, cfg_id):
    cfg = synth.config(cfg_id)
    qc, kc = synth.make_calibration(cfg)
    s, inv, gate = hf.calibrate(qc, kc, cfg["alpha"], 4.0)
    so, invo, gateo = smooth.calibrate(qc, kc, cfg["alpha"], 4.0)
    assert gate == gateo and gate
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(inv.view(np.uint32), invo.view(np.uint32))


def test_calibrate_gate_off_and_errors(L):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 32, 64)).astype(np.float16)
    k = rng.standard_normal((2, 32, 64)).astype(np.float16)
    s, inv, gate = hf.calibrate(q, k, 0.5, 4.0)
    assert not gate and np.all(s == 1) and np.all(inv == 1)
    with pytest.raises(hf.Hifa4Error):
        hf.calibrate(q, k, 1.5, 4.0)
    with pytest.raises(hf.Hifa4Error):
        hf.calibrate(q[:3], k, 0.5, 4.0)
