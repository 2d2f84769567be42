"""Oracle regression against the fixtures written by tests/golden/make_golden.py."""
import json
import os

import numpy as np

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_hhr_fixture_unchanged():
    want = _load("hhr_small.json")
    got = make_golden.hhr_fixture()
    for key in ("n_keep", "kept", "sel", "qcodes", "codes_first4"):
        assert got[key] == want[key], key
    assert np.allclose(got["scores_first4"], want["scores_first4"], rtol=1e-12, atol=0)
    assert np.allclose(got["out_row0_first8"], want["out_row0_first8"], rtol=1e-12, atol=1e-15)


def test_hisa_fixture_unchanged():
    want = _load("hisa_small.json")
    got = make_golden.hisa_fixture()
    assert got["blocks"] == want["blocks"] and got["sel"] == want["sel"]
    assert np.allclose(got["block_scores_first4"], want["block_scores_first4"], rtol=1e-12)
