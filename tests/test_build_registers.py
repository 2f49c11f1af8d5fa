"""No kernel of the library spills registers (compile-only check, no GPU).

The prefill kernels are register-capped (80 VGPRs for d <= 128) to fit six waves per SIMD; a
change that makes an instance spill costs far more than the cap saves (a spilled value reloaded
inside the tile loop also waits on the in-flight tile loads).  Every device source is compiled
for gfx950 with the resource-usage remarks and each kernel must report no VGPR spills and no
scratch.
"""
import concurrent.futures
import os
import shutil
import subprocess
import tempfile

import pytest

from bit_quantized_flashattention_amd import build as B

DEVICE_SOURCES = ["quantize.hip", "attn_prefill.hip", "attn_decode.hip"]


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_no_kernel_spills_registers():
    tmp = tempfile.mkdtemp()

    def remarks(src):
        cmd = [B.HIPCC] + B.FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(B.CSRC, src),
                                     "-o", os.path.join(tmp, src + ".o")]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return r.stderr

    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=3) as ex:
            outs = list(ex.map(remarks, DEVICE_SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    kernels = sum(o.count("Function Name:") for o in outs)
    assert kernels >= 30, "expected the kernel instances' remarks, got %d" % kernels
    spills = [s for o in outs for s in B.kernel_spills(o)]
    assert not spills, "kernels that spill: %s" % spills
