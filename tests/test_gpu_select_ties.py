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


@pytest.mark.parametrize("group,Lcap,lens,ramp", [(4, 8192, [8192, 5000], False),
                                                  (3, 8192, [8192, 5000], False),
                                                  (8192, 8192, [8192, 5000], False),
                                                  (1, 98304, [98304, 80000], False),
                                                  (3, 98304, [98304, 80000], False),
                                                  (98304, 98304, [98304, 80000], False),
                                                  (1, 98304, [98304, 80000], True),
                                                  (1, 163840, [80000, 66000], False),
                                                  (3, 163840, [80000, 66000], True)])
def test_duplicate_pages_composite_equals_stages(gpu_lib, group, Lcap, lens, ramp):
    """Keys copied page by page in runs of `group` pages give equal page bounds in runs,
    so the cut of the top-P falls inside a run of ties (group = Lcap: every page equal).
    The one-launch coarse stage of hhr_decode and hhr_select (top-P in the last scoring
    workgroup) must keep the same pages as the staged top-P, both breaking ties to the
    lower page: the selections and outputs are bit-identical, and the staged kept pages
    equal the oracle's top-P of the GPU's own bounds.  The 98304-key cache (6144 and 5000
    pages) takes the one-launch top-P through its lower-bound pre-filter, the second
    sequence with a partly filled last scoring workgroup.  ramp: keys scaled up with their
    page index, so the largest bounds crowd into the last scoring workgroups and the
    pre-filter keeps most pages (its widest compaction).  The 163840-key cache (10240
    pages) holds sequences of 5000 and 4125 pages, under half of it: the scoring
    workgroups take their 16-page blocks round robin, and the pre-filter still runs."""
    print(f"\n[gpu duplicate pages] group={group} Lcap={Lcap} ramp={ramp}", flush=True)
    from hash_hierarchical_top_amd import synth

    B, Hq, Hkv = 2, 8, 2
    inp = synth.make_hhr_inputs(B, Hq, Hkv, lens, Lcap, "bf16", seed=77)
    K = inp["K"].reshape(B, Hkv, Lcap // 16, 16, 128)
    src = (np.arange(Lcap // 16) // group) * group
    inp["K"] = np.ascontiguousarray(K[:, :, src].reshape(B, Hkv, Lcap, 128))
    if ramp:  # bf16 keys times 1 + 3 p / pages, truncated back to bf16
        Kf = (inp["K"].astype(np.uint32) << 16).view(np.float32)
        scale = 1.0 + 3.0 * (np.arange(Lcap) // 16) / (Lcap // 16)
        Kf = (Kf * scale[None, None, :, None].astype(np.float32)).astype(np.float32)
        inp["K"] = np.ascontiguousarray((Kf.view(np.uint32) >> 16).astype(np.uint16))
    for b, L in enumerate(lens):
        inp["K"][b, :, L:] = 0
    p = U.Pipeline(gpu_lib, inp, "bf16", Hq, Hkv, Lcap, 1, 8, 0, 256)
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        Np = O.n_pages(L, 16)
        P = O.keep_count(Np, 1, 8, 0)
        for g in range(Hkv):
            s = p.scores[b, g, :Np].cpu().numpy().astype(np.float64)
            assert p.kept[b, g, :P].cpu().tolist() == O.top_pages(s, P).tolist(), (b, g)
    sel = torch.zeros_like(p.sel)
    sc = torch.zeros_like(p.sel_count)
    out = torch.zeros_like(p.out)
    p.decode(sel, sc, out)
    torch.cuda.synchronize()
    assert torch.equal(sc, p.sel_count) and torch.equal(sel, p.sel)
    assert torch.equal(out, p.out)
    sel2, sc2 = p.select()
    assert torch.equal(sc2, p.sel_count) and torch.equal(sel2, p.sel)
    kept, kc, _ = p.select_pages()
    assert torch.equal(kc, p.kept_count) and torch.equal(kept, p.kept)
    assert p.status() == 0
