"""Exhaustive GPU pin of the output quotient (R13: out = fp16(O / l), IEEE division).

The prefill epilogue divides with hifa4::quot_h (device_common.h): q = x r with the hardware
FP32 reciprocal r of l, corrected once with the exact residual.  tests/mfma_probe runs it for
every finite FP16 x and every positive finite FP16 l (2,015,299,584 pairs) and compares the FP16
result with the correctly rounded quotient, taken from the FP64 quotient by one exact integer
rounding to FP16.  The test requires no mismatch.  (A single multiply x r without the
correction misses 10,528 of these pairs, all with subnormal quotients.)
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "mfma_probe", "libmfmaprobe.so")


def test_quotient_is_correctly_rounded_for_every_fp16_pair():
    import torch
    if not os.path.exists(LIB):
        raise RuntimeError("tests/mfma_probe/libmfmaprobe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.quot_probe_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.quot_probe_run.restype = ctypes.c_int
    counts = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(1, dtype=torch.int32, device="cuda")
    print("case quotient probe, all FP16 pairs", flush=True)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.quot_probe_run(ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(first.data_ptr()),
                              ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    n = int(counts.item())
    f = int(first.item()) & 0xFFFFFFFF
    print("quotient mismatches:", n, "first (l bits, x bits): 0x%04x 0x%04x" % (f >> 16, f & 0xFFFF))
    assert n == 0
