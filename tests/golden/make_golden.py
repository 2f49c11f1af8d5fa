"""Write tests/golden/regression_c0.json from the oracle alone (config 0: both normalizers, the
per-tile P-hat scale variant and the Direct-P code rule).

Usage: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import attention as A, smooth  # noqa: E402


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute():
    cfg = synth.config(0)
    q, k, v = synth.make_qkv(cfg)
    qc, kc = synth.make_calibration(cfg)
    s, inv, gate = smooth.calibrate(qc, kc, cfg["alpha"])
    qq = A.quantize_qkv(q, k, v, s, inv)
    packed = qq.packed()
    out = {"config": 0, "gate": gate, "s32": digest(s), "inv32": digest(inv)}
    for name, arr in zip(["q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"], packed):
        out[name] = digest(arr)
    out["out_p_reordered"] = digest(A.attention_p(qq, cfg["causal"], cfg["kv_tile"], A.P_REORDERED))
    out["out_inconsistent"] = digest(A.attention_p(qq, cfg["causal"], cfg["kv_tile"], A.INCONSISTENT))
    out["out_phat_tile"] = digest(A.attention_p(qq, cfg["causal"], cfg["kv_tile"], A.P_REORDERED,
                                                phat_scale=A.PHAT_TILE))
    out["out_direct_p"] = digest(A.attention_p(qq, cfg["causal"], cfg["kv_tile"], A.P_REORDERED,
                                               phat_rule=A.PHAT_DIRECT))
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "regression_c0.json"), "w") as f:
        json.dump(compute(), f, indent=1, sort_keys=True)
        f.write("\n")
