"""Write the oracle regression fixtures in this folder.

The pages print no worked example with numbers (no intermediate values, no
selected indices), so these fixtures are not the pages' values: they freeze
what the pinned oracle computes on small seeded inputs, so that any later
change to the oracle's arithmetic shows up as a diff that must be justified.
This script calls only the oracle and the seeded input generator.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from hash_hierarchical_top_amd import synth  # noqa: E402
from oracle import hhr as O  # noqa: E402
from oracle import hisa as OH  # noqa: E402


def hhr_fixture():
    inp = synth.make_hhr_inputs(1, 4, 1, [300], 304, "bf16", seed=77)
    q = inp["q"][0]
    K = synth.kv_values(inp["K"][0, 0, :300], "bf16")
    V = synth.kv_values(inp["V"][0, 0, :300], "bf16")
    res = O.select(q, K, inp["R"][0], inp["W"][0], 16, 1, 4, 0, 32)
    o = O.attend(q, K[res["sel"]], V[res["sel"]])
    return {
        "source": "HHR abstract (GKR page bounds, LHP Hamming selection, sparse attention); "
                  "generator: make_hhr_inputs(1, 4, 1, [300], 304, 'bf16', seed=77); "
                  "page_size 16, keep 1/4 of pages, top_k 32",
        "n_keep": int(res["n_keep"]),
        "kept": res["kept"].tolist(),
        "sel": res["sel"].tolist(),
        "qcodes": res["qcodes"].tolist(),
        "codes_first4": res["enc"]["codes"][:4].tolist(),
        "scores_first4": res["scores"][:4].tolist(),
        "out_row0_first8": o[0, :8].tolist(),
    }


def hisa_fixture():
    inp = synth.make_hisa_inputs(8, 1000, 1000, 4, 78, head_dim=32, make_kv=False)
    res = OH.select(inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], 1000,
                    block=64, keep_blocks=4, top_k=50)
    return {
        "source": "HISA abstract (pooled block filter, token refinement); generator: "
                  "make_hisa_inputs(8, 1000, 1000, 4, 78, head_dim=32); block 64, keep 4, top_k 50",
        "blocks": res["blocks"].tolist(),
        "sel": res["sel"].tolist(),
        "block_scores_first4": res["block_scores"][:4].tolist(),
    }


if __name__ == "__main__":
    for name, fx in (("hhr_small.json", hhr_fixture()), ("hisa_small.json", hisa_fixture())):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fx, f, indent=1)
        print("wrote", name)
