"""Writes oracle_small_varlen.json: the fp64 oracle's output on a small seeded
varlen case (2 heads, two sequences over 20 tokens, K=4, V=3, random initial
state). It calls only the oracle, and the file guards the oracle's arithmetic
against unnoticed drift; the pages print no worked example of their own.

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from linear_attention_04_amd import inputs  # noqa: E402

WORKLOAD = inputs.custom_workload("golden_small_varlen", 4242, heads=2, total_tokens=20, head_k=4,
                                  head_v=3, io_dtype="f32", has_initial_state=True, num_seqs=2)


def compute():
    x = inputs.generate(WORKLOAD)
    o, fs = oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=x["cu_seqlens"],
                           initial_state=x["initial_state"])
    return x, o, fs


if __name__ == "__main__":
    x, o, fs = compute()
    doc = {
        "about": "fp64 oracle output for the seeded workload in make_golden.py",
        "cu_seqlens": x["cu_seqlens"].tolist(),
        "out": o.tolist(),
        "final_state": fs.tolist(),
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_varlen.json"), "w") as f:
        json.dump(doc, f, indent=0)
