"""The oracle reproduces its committed fixture bit for bit (regression pin)."""
import json
import os

import numpy as np

import oracle
from linear_attention_sequence_chunked_amd.workloads import workload_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_fp32_oracle.json")


def test_oracle_matches_fixture():
    doc = json.load(open(GOLDEN))
    inp = workload_inputs("tiny_fp32")
    o, sf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    for i, t in enumerate(doc["tokens"]):
        np.testing.assert_array_equal(o[0, t], np.array(doc["o_at_tokens"][i]))
    np.testing.assert_array_equal(sf[0], np.array(doc["final_state"]))
