"""Build libhifa4.so for gfx950 with hipcc (in-tree, next to this file).

    python -m bit_quantized_flashattention_amd.build
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libhifa4.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["hifa4_api.cpp", "quantize.hip", "attn_prefill.hip", "attn_decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # the kernels' FP32 rounding sequence is part of their definition: no implicit fma
    "-ffp-contract=off",
    # packed FP32 arithmetic is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def kernel_spills(remarks):
    """(kernel, VGPR spills, scratch bytes per lane) for every kernel of a compile's
    kernel-resource-usage remarks that spills or uses scratch."""
    out = []
    name = None
    spill = scratch = 0
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
        if text.startswith("Function Name:"):
            if name is not None and (spill or scratch):
                out.append((name, spill, scratch))
            name, spill, scratch = text.split(":", 1)[1].strip(), 0, 0
        elif text.startswith("VGPRs Spill:"):
            spill = int(text.split(":", 1)[1])
        elif text.startswith("ScratchSize [bytes/lane]:"):
            scratch = int(text.split(":", 1)[1])
    if name is not None and (spill or scratch):
        out.append((name, spill, scratch))
    return out


def _compile(src):
    obj = os.path.join(OBJDIR, src + ".o")
    # the resource remarks report register spills, which cost the kernels far more than the
    # registers they save (a spilling loop also waits on its in-flight tile loads)
    cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):  # host-only C++: the HIP runtime API, no device code
        cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
               "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    for name, spill, scratch in kernel_spills(r.stderr):
        print("warning: %s spills %d VGPRs (%d scratch bytes per lane)" % (name, spill, scratch), file=sys.stderr)
    return obj


PROBE_SRC = os.path.join(ROOT, "tests", "mfma_probe", "mfma_probe.hip")
PROBE_OUT = os.path.join(ROOT, "tests", "mfma_probe", "libmfmaprobe.so")


def build_test_probe(verbose=False):
    """The GPU tests' probes (tests/mfma_probe): one scaled FP4 MFMA per wave on buffer operands,
    and the exhaustive check of the output quotient.  Test infrastructure, not part of
    libhifa4.so."""
    tmp = PROBE_OUT + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SRC, " ".join(cmd), r.stderr))
    os.replace(tmp, PROBE_OUT)
    if verbose:
        print("built", PROBE_OUT)
    return PROBE_OUT


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    if os.path.exists(PROBE_SRC):
        build_test_probe(verbose)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
