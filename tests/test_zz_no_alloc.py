"""hifa4_attention_fwd_q16_noalloc through the C ABI: the fused-Q forward whose decode partials
live in the library's fixed per-GPU scratch must reproduce hifa4_attention_fwd_q16 (with a caller
workspace) bit for bit, on two decode calls in a row (the second with a smaller input, so the
scratch still holds the first call's partials) and on a prefill call; both also match the oracle
within the parity tolerance."""
import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
import synth
from oracle import attention as A
from gpu_helpers import compare_out, gpu_quantize, to_dev

pytestmark = pytest.mark.gpu


def _case(cfg_id, splits=0, **over):
    import torch
    cfg = synth.config(cfg_id, **over)
    q, k, v = synth.make_qkv(cfg)
    b, hq, hkv, lq, lk, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"], cfg["Lk"], cfg["d"]
    res = gpu_quantize(q, k, v, None, None)
    kv = {n: res[n] for n in ("k_codes", "k_scales", "v_codes", "v_scales")}
    dims = hf.make_dims(b, hq, hkv, d, lq, lk)
    qd = to_dev(q)
    ref = hf.attention_fwd(kv, dims, True, hf.P_REORDERED, 128, splits, q16=(qd, None))
    out = torch.full_like(ref, float("nan"))
    got = hf.attention_fwd_q16_noalloc(kv, qd, None, dims, True, hf.P_REORDERED, 128, splits, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "no-alloc output differs from the workspace path"
    qq = A.quantize_qkv(q, k, v)
    used = hf.decode_num_splits(dims, hf.make_opts(True, 0, 128, splits)) if lq == 1 else 1
    want = A.attention_p(qq, True, 128, num_splits=used)
    compare_out(got.cpu().numpy(), want, "no-alloc B%d Hq%d d%d Lq%d Lk%d" % (b, hq, d, lq, lk))
    return used


def test_noalloc_decode_twice_then_prefill():
    print("case no-alloc decode B3 Hq8 Hkv2 d128 Lk1000", flush=True)
    s1 = _case(1, 3, B=3, Hq=8, Hkv=2, Lq=1, Lk=1000, d=128)
    print("case no-alloc decode B2 Hq4 Hkv1 d64 Lk300 (smaller, after the first)", flush=True)
    s2 = _case(0, 2, B=2, Hq=4, Hkv=1, Lq=1, Lk=300, d=64)
    assert (s1, s2) == (3, 2)  # both calls run split-KV partials through the scratch
    print("case no-alloc prefill (no scratch)", flush=True)
    _case(1, B=1, Hq=4, Hkv=2, Lq=130, Lk=200, d=128)
