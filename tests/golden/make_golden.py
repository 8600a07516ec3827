"""Write tests/golden/tiny_oracle.json: digests of the oracle's intermediates on
the tiny configuration (T=16, H=256, I=128, E=8, k=2).

Calls only synth/ (inputs) and oracle/ (arithmetic).  Run from the repo root:
    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import mxfp4  # noqa: E402
from oracle.forward import forward  # noqa: E402

KEYS = ("xq", "xsf", "counts", "offsets", "sorted_rows", "pos", "hq", "hsf", "out")


def digest(a):
    a = np.ascontiguousarray(a)
    return hashlib.sha256(a.tobytes()).hexdigest()


def tiny_record():
    cfg = synth.CONFIGS[0]
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    parts = []
    for e in range(cfg.experts):
        w1, w2 = synth.expert_weights_f32(cfg, e)
        parts.append(mxfp4.quantize_packed(w1) + mxfp4.quantize_packed(w2))
    W = tuple(np.stack([p[i] for p in parts]) for i in range(4))
    res = forward(x, ids, w, W, cfg.experts, cfg.inter)
    rec = {k: digest(res[k].astype(np.int64) if res[k].dtype.kind == "i" else res[k]) for k in KEYS}
    rec["weights"] = [digest(a) for a in W]
    rec["out_first8_bits"] = [int(v) for v in res["out"][0, :8]]
    return rec


if __name__ == "__main__":
    rec = tiny_record()
    rec["_about"] = ("sha256 digests of oracle intermediates on the tiny layer; written by "
                     "tests/golden/make_golden.py (oracle + synthetic inputs only)")
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json"), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print("wrote tiny_oracle.json")
