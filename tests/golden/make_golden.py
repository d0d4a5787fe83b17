"""Writes tests/golden/tiny_fp32_oracle.json from the fp64 oracle only.

Inputs: the seeded tiny fp32 workload (B1 T64 H2 K=V=16, sigmoid gates, seed 1).
Stored: the oracle's output at a few tokens (both heads, all channels) and the
full final state, as exact float64 reprs.  This is a regression fixture of the
oracle (it must not drift), and a stored expectation the GPU tests can use.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from linear_attention_sequence_chunked_amd.workloads import workload_inputs  # noqa: E402

TOKENS = [0, 1, 15, 16, 31, 47, 63]


def main():
    inp = workload_inputs("tiny_fp32")
    o, sf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    doc = {
        "what": "fp64 token-oracle outputs for the seeded tiny fp32 workload",
        "workload": "tiny_fp32: B=1 T=64 H=2 K=V=16 chunk=16 seed=1, q,k L2-normalised "
                    "N(0,1), v N(0,1), alpha=sigmoid(N), beta=sigmoid(N), zero initial state",
        "written_by": "tests/golden/make_golden.py (calls oracle/ only)",
        "tokens": TOKENS,
        "o_at_tokens": [[[float(x) for x in o[0, t, h]] for h in range(2)] for t in TOKENS],
        "final_state": [[[float(x) for x in row] for row in sf[0, h]] for h in range(2)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
