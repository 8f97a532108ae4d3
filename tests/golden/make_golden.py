"""Writes tests/golden/tiny_oracle.json: the FP64 oracle's result on the tiny
workload (batch 2, lengths {37, 100}, 16 heads, one new token), with a digest
of the inputs so a change in the generator is told apart from a change in the
oracle. Calls only the oracle and the input generator.

    python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import make_workload_inputs  # noqa: E402


def input_digest(inp):
    h = hashlib.sha256()
    for a in (inp.seqlens, inp.block_table, inp.q_bits, inp.kv_bits):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def main():
    inp = make_workload_inputs("tiny")
    out, lse = oracle.mla_decode_ref(inp.q_bits, inp.kv_bits, inp.block_table,
                                     inp.seqlens, inp.scale, inp.causal)
    doc = {
        "workload": "tiny: batch 2, seqlens {37,100}, s_q=1, h_q=16, seed 1",
        "writer": "tests/golden/make_golden.py (oracle.mla_decode_ref only)",
        "input_sha256": input_digest(inp),
        "lse": lse.tolist(),
        "out_first8": out[..., :8].tolist(),
        "out_row_sums": out.sum(axis=-1).tolist(),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
