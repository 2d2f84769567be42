"""GPU exactness of the page top-P on scores built to exercise every path of the
selection: ties at the cut (the lower page wins), a threshold bin with more
members than the exact-rank list holds (the radix fallback), all-equal scores
(zero range), a far outlier that squeezes the bulk into a few histogram bins,
signed zeros, and P from 1 to every page.  hhr_top_pages takes the scores as
input, so each case feeds them directly; the expected kept pages come from the
oracle's sort by (score descending, page ascending).
"""
import numpy as np
import pytest
import torch

from oracle import hhr as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

LCAP = 262144  # the largest context: 16384 pages of 16
PATTERNS = ["normal", "equal", "few_values", "ties_at_cut", "outlier", "signed_zeros"]
SIZES = [1, 5, 777, 4096, 8193, 16384]


def _scores(pattern: str, n: int, P: int, rng: np.random.Generator) -> np.ndarray:
    if pattern == "normal":
        s = rng.normal(1000.0, 50.0, n)
    elif pattern == "equal":
        s = np.full(n, 3.25)
    elif pattern == "few_values":
        s = rng.integers(0, 4, n).astype(np.float64) * 0.5
    elif pattern == "ties_at_cut":
        s = rng.normal(0.0, 1.0, n)
        if n > 1:
            cut = np.sort(s)[::-1][P - 1]
            near = np.argsort(np.abs(s - cut))[:min(n, 24)]
            s[near] = cut
    elif pattern == "outlier":
        s = rng.normal(10.0, 1.0, n)
        s[rng.integers(0, n)] = 1e6
    else:  # signed zeros among small values of both signs
        s = rng.choice(np.array([-0.0, 0.0, -1.5, 2.0]), n)
    return s.astype(np.float32)


def test_top_pages_exact_on_constructed_scores(gpu_lib):
    H = gpu_lib
    shape = H.make_shape(1, 4, 1, LCAP, "bf16")
    dev = torch.device("cuda", 0)
    rng = np.random.Generator(np.random.PCG64(2024))
    scores = torch.zeros((1, 1, LCAP // 16), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    checked = 0
    for pattern in PATTERNS:
        for n in SIZES:
            for P in sorted({1, max(1, n // 8), max(1, n - 1), n}):
                s = _scores(pattern, n, P, rng)
                scores.zero_()
                scores[0, 0, :n] = torch.from_numpy(s).to(dev)
                seq = torch.tensor([n * 16], dtype=torch.int32, device=dev)
                kept = torch.full((1, 1, P), 12345, dtype=torch.int32, device=dev)
                kc = torch.full((1, 1), -3, dtype=torch.int32, device=dev)
                H.hhr_top_pages(shape, scores, seq, 0, 1, P, kept, kc, status)
                torch.cuda.synchronize()
                want = O.top_pages(s.astype(np.float64), P)
                got = kept[0, 0].cpu().numpy()
                assert int(kc[0, 0]) == P, (pattern, n, P)
                assert got.tolist() == want.tolist(), (pattern, n, P)
                checked += 1
    assert int(status.item()) == 0
    print(f"checked {checked} selections")
