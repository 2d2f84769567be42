"""The reference selections behind the reported quality figures (hash_hierarchical_top_amd
/quality.py: torch fp64) equal the oracle's exact top-k and flat indexer, on the CPU."""
import numpy as np
import torch

from hash_hierarchical_top_amd import quality as Q
from hash_hierarchical_top_amd import synth
from oracle import hhr as O
from oracle import hisa as OS


def test_exact_topk_matches_oracle_with_ties():
    inp = synth.make_hhr_inputs(1, 8, 2, [3000], 3008, "bf16", seed=3)
    for g in range(2):
        K = torch.from_numpy(inp["K"][0, g, :3000]).view(torch.bfloat16)
        q = torch.from_numpy(inp["q"][0, 4 * g:4 * g + 4])
        want = O.exact_topk(inp["q"][0, 4 * g:4 * g + 4],
                            synth.kv_values(inp["K"][0, g, :3000], "bf16"), 256)
        assert np.array_equal(Q.exact_topk(q, K, 256).numpy(), want)
    # forced ties: duplicated keys are taken at the lower position
    Kd = np.repeat(np.random.default_rng(0).standard_normal((50, 128)), 2, axis=0)
    qd = np.random.default_rng(1).standard_normal((2, 128))
    got = Q.exact_topk(torch.from_numpy(qd), torch.from_numpy(Kd), 7).numpy()
    assert np.array_equal(got, O.exact_topk(qd, Kd, 7))


def test_flat_indexer_matches_oracle():
    rng = np.random.default_rng(2)
    Hi, L = 8, 3000
    q8, qs = synth.quantize_rows_e4m3(rng.standard_normal((Hi, 128)).astype(np.float32))
    k8, ks = synth.quantize_rows_e4m3(rng.standard_normal((L, 128)).astype(np.float32))
    wt = rng.uniform(0, 1, Hi).astype(np.float32)
    got = Q.flat_indexer_topk(q8, qs, wt, k8, ks, 2500, 300, "cpu")
    assert np.array_equal(got, OS.flat_select(q8, qs, wt, k8, ks, 2500, 300))


def test_overlap_and_iou():
    assert Q.overlap([1, 2, 3], [2, 3, 4, 5]) == 0.5 and Q.overlap([], []) == 1.0
    assert Q.iou([1, 2, 3], [2, 3, 4]) == 0.5 and Q.iou([], []) == 1.0
