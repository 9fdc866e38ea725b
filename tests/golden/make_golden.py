"""Writes oracle_regression.json: outputs of the CPU oracle (and nothing else)
on one small seeded input, so that an unintended change to the oracle's
arithmetic shows up as a test failure.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from long_context_attn_amd import synth  # noqa: E402

KEY = (synth.SEED, 99, 0)
H, D, SEG = 2, 4, [0, 5, 12]


def inputs():
    T = SEG[-1]
    q, k, v, g = (synth.normal(KEY + (j,), (T, H, D)) for j in range(4))
    w = synth.normal(KEY + (4,), (H * D,), scale=0.02, mean=1.0)
    s0 = synth.normal(KEY + (5,), (len(SEG) - 1, H, D, D), scale=0.5, bf16=False)
    return q, k, v, g, w, s0


def main():
    q, k, v, g, w, s0 = inputs()
    out, st = oracle.prefill(q, k, v, g, w, cu_seqlens=SEG, eps=1e-6, init_state=s0,
                             return_state=True)
    doc = {"_about": "CPU-oracle regression values, written by tests/golden/make_golden.py "
                     "(calls only oracle/). Inputs: long_context_attn_amd.synth key "
                     "[2025, 99, 0, tensor]; H=2, D=4, segments [0, 5, 12], eps 1e-6, "
                     "initial states given.",
           "H": H, "D": D, "seg": SEG, "eps": 1e-6,
           "out": [float("%.15e" % x) for x in out.reshape(-1)],
           "final_state": [float("%.15e" % x) for x in st.reshape(-1)]}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
