"""Exhaustive GPU pins of the elementwise P-hat helpers of the library against the oracle.

tests/mfma_probe runs the library's own device helpers (device_common.h) on every FP16 bit
pattern:
* exp2_h2, the FP16 exponential of the P-hat codes (R10: rn16(2^h) for the FP16 value h), in
  both halves of its packed form, against oracle.attention.exp2_16;
* the E2M1 conversions at scale 1 of an FP16 value (the P-hat codes) and of an FP32 value (the
  quantizers and Direct-P), against oracle.mx.rne_code (RNE onto the E2M1 grid, ties to the even
  code, saturating at 6, sign copied).
NaN inputs are left out (no NaN reaches these helpers on the path); infinities are included.
"""
import ctypes
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import mx

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "mfma_probe", "libmfmaprobe.so")


def _run():
    import torch
    if not os.path.exists(LIB):
        raise RuntimeError("tests/mfma_probe/libmfmaprobe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.prim_probe_run.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    lib.prim_probe_run.restype = ctypes.c_int
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    keep = ~np.isnan(vals)
    bits, vals = bits[keep], vals[keep]
    n = bits.size
    h = torch.from_numpy(bits.view(np.int16).copy()).cuda()
    e = torch.zeros(2 * n, dtype=torch.int16, device="cuda")
    c16 = torch.zeros(n, dtype=torch.uint8, device="cuda")
    c32 = torch.zeros(n, dtype=torch.uint8, device="cuda")
    print("case primitives probe, %d FP16 inputs" % n, flush=True)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.prim_probe_run(ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(e.data_ptr()),
                              ctypes.c_void_p(c16.data_ptr()), ctypes.c_void_p(c32.data_ptr()), n,
                              ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    return vals, e.cpu().numpy().view(np.uint16).reshape(n, 2), c16.cpu().numpy(), c32.cpu().numpy()


def test_fp16_exponential_matches_oracle_on_every_input():
    vals, e, _, _ = _run()
    want = A.exp2_16(vals.astype(np.float32)).astype(np.float16).view(np.uint16)
    for half in range(2):
        bad = np.flatnonzero(e[:, half] != want)
        print("exp2_h2 half %d: %d mismatches" % (half, bad.size))
        assert bad.size == 0, [(float(vals[i]), hex(e[i, half]), hex(want[i])) for i in bad[:5]]


def test_e2m1_conversions_match_oracle_on_every_input():
    vals, _, c16, c32 = _run()
    want = mx.rne_code(vals.astype(np.float64))
    for name, got in (("fp16", c16), ("fp32", c32)):
        lo, hi = got & 0xF, got >> 4
        bad = np.flatnonzero((lo != want) | (hi != want))
        print("E2M1 from %s: %d mismatches" % (name, bad.size))
        assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]
