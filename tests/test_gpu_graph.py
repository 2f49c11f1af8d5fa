"""The library's device calls can be captured in a HIP graph: no allocation, synchronization or
memset happens inside them.  A captured quantize + attention step is replayed several times,
with other eager work of the same library in between, and every replay must equal the eager
result bit for bit."""
import numpy as np
import pytest

import bit_quantized_flashattention_amd as hf
import synth
from oracle import smooth
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _capture_and_replay(step, out, other):
    import torch
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        other()  # eager work of the library between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d differs" % i


@pytest.mark.parametrize("lq", [1, 200])
def test_graph_replay_of_quantize_and_attention(lq):
    import torch
    cfg = synth.config(1, B=2, Hq=8, Hkv=2, Lq=lq, Lk=700)
    q, k, v = synth.make_qkv(cfg)
    qc, kc = synth.make_calibration(cfg)
    s32, inv32, _ = smooth.calibrate(qc, kc, 0.5, 4.0)
    print("case graph replay lq", lq, flush=True)
    qd, kd, vd, sd, invd = to_dev(q), to_dev(k), to_dev(v), to_dev(s32), to_dev(inv32)
    dims = hf.make_dims(2, 8, 2, 128, lq, 700)
    opts = hf.make_opts(True, 0, 128, 0)
    qkv = hf.quantize_qkv(None, kd, vd, sd, invd, dims=dims)
    n_ws = hf.attention_workspace_bytes(dims, opts)
    ws = torch.empty(max(n_ws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, 8, lq, 128), dtype=torch.float16, device="cuda")
    other_out = torch.empty_like(out)

    def step():
        hf.quantize_qkv(None, kd, vd, sd, invd, dims=dims, out=qkv)
        hf.attention_fwd(qkv, dims, True, 0, 128, out=out, workspace=ws if n_ws else None, q16=(qd, sd))

    def other():
        hf.attention_fwd(qkv, dims, True, 1, 128, out=other_out, workspace=ws if n_ws else None, q16=(qd, None))

    _capture_and_replay(step, out, other)
