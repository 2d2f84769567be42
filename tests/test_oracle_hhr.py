"""Pins for the HHR oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formulas: each checks it against an
independent characterisation (brute force over orders or box corners, a closed
form, an invariant, or a library routine), chosen so a dropped term, a wrong
sign, a transposed operand or a wrong index fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import hhr as O
from hash_hierarchical_top_amd import synth


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------- rotation
def test_generated_rotation_is_orthogonal_and_preserves_logits():
    """q.k = (qR).(kR) for orthogonal R (GKR's rotation must not change logits)."""
    inp = synth.make_hhr_inputs(1, 4, 2, [64], 64, "f32", seed=3)
    for g in range(2):
        R = inp["R"][g].astype(np.float64)
        assert np.abs(R @ R.T - np.eye(128)).max() < 1e-6
        q = inp["q"][0, 2 * g: 2 * g + 2]
        K = inp["K"][0, g]
        direct = q.astype(np.float64) @ K.astype(np.float64).T
        rotated = O.rotate(q, R) @ O.rotate(K, R).T
        assert np.allclose(direct, rotated, rtol=0, atol=1e-4 * np.abs(direct).max())


def test_rotation_orientation_convention():
    """X = K R with R stored [input dim][output dim]: a 4-cycle permutation, worked by hand.

    R[i][j] = 1 iff j == (i + 1) % 4 sends coordinate i of k to coordinate i+1 of kR.
    k = (1, 2, 3, 4) -> kR = (4, 1, 2, 3); with R^T instead it would be (2, 3, 4, 1).
    """
    R = np.zeros((4, 4))
    for i in range(4):
        R[i, (i + 1) % 4] = 1.0
    assert np.array_equal(O.rotate(np.array([[1.0, 2.0, 3.0, 4.0]]), R), [[4.0, 1.0, 2.0, 3.0]])


# --------------------------------------------------------------------------- codes
def test_sign_and_packing_worked_examples():
    """Bit j = [y_j >= 0] in word j//32 at bit j%32; worked by hand for 128-bit codes."""
    def words_for(nonneg):
        y = -np.ones(128)
        for j in nonneg:
            y[j] = 0.5
        return O.pack_bits(O.sign_bits(y)).tolist()

    assert words_for([]) == [0, 0, 0, 0]
    assert words_for(range(128)) == [0xFFFFFFFF] * 4
    assert words_for([0]) == [1, 0, 0, 0]
    assert words_for([33]) == [0, 2, 0, 0]
    assert words_for([127]) == [0, 0, 0, 0x80000000]
    assert words_for([3, 64, 65]) == [8, 0, 3, 0]
    # zero and negative zero both count as non-negative
    y = -np.ones(128)
    y[5] = -0.0
    y[6] = 0.0
    assert O.pack_bits(O.sign_bits(y)).tolist() == [(1 << 5) | (1 << 6), 0, 0, 0]


def test_unpack_inverts_pack():
    bits = _rng(1).random((7, 128)) < 0.5
    assert np.array_equal(O.unpack_bits(O.pack_bits(bits)), bits)


@pytest.mark.parametrize("nbits", [64, 128, 256])
def test_hamming_closed_form(nbits):
    """H = sum_h (b - <sigma_qh, sigma_k>)/2 with sigma in {+-1}^b taken from the float
    projections, for b-bit codes."""
    rng = _rng(2 + nbits)
    for G in (1, 4, 16):
        W = rng.standard_normal((128, nbits))
        q = rng.standard_normal((G, 128))
        K = rng.standard_normal((50, 128))
        qc, kc = O.hash_codes(q, W), O.hash_codes(K, W)
        assert qc.shape == (G, nbits // 32) and kc.shape == (50, nbits // 32)
        H = O.hamming(qc, kc)
        sq = np.where(q @ W >= 0, 1.0, -1.0)
        sk = np.where(K @ W >= 0, 1.0, -1.0)
        closed = ((nbits - sk @ sq.T) / 2.0).sum(axis=1)
        assert np.array_equal(H, closed.astype(np.int64))
        assert H.max() <= nbits * G


def test_hamming_extremes_at_every_width():
    """Identical codes give 0, complementary codes give the full width per query head."""
    for nbits in (64, 128, 256):
        bits = _rng(nbits).random((3, nbits)) < 0.5
        c = O.pack_bits(bits)
        assert O.hamming(c[:1], c[:1]).tolist() == [0]
        assert O.hamming(c[:1], O.pack_bits(~bits[:1])).tolist() == [nbits]
        # three query heads against the complement of head 0: nbits + the two others'
        # distances to head 0's complement, counted bit by bit
        want = nbits + int((bits[1] == bits[0]).sum()) + int((bits[2] == bits[0]).sum())
        assert O.hamming(c, O.pack_bits(~bits[:1])).tolist() == [want]


def test_codes_scale_invariant():
    """Positive scaling of the input or of the projection leaves sign codes unchanged."""
    rng = _rng(3)
    W = rng.standard_normal((128, 128))
    K = rng.standard_normal((40, 128))
    base = O.hash_codes(K, W)
    assert np.array_equal(O.hash_codes(3.7 * K, W), base)
    assert np.array_equal(O.hash_codes(K, 0.01 * W), base)
    assert not np.array_equal(O.hash_codes(-K, W), base)


# --------------------------------------------------------------------------- page bound
def _corner_max(q, mn, mx):
    """max over the bounding box [mn, mx]^d of q.x, by enumerating all 2^d corners."""
    best = -np.inf
    for pick in itertools.product((0, 1), repeat=len(q)):
        corner = np.where(np.array(pick) == 1, mx, mn)
        best = max(best, float(q @ corner))
    return best


def test_page_score_is_sum_of_box_maxima():
    """Per head, the page bound is the max of q'.x over the page's bounding box (corner brute force)."""
    rng = _rng(4)
    for _ in range(20):
        d, ps, G = 4, 3, 2
        X = rng.standard_normal((7, d))
        q = rng.standard_normal((G, d))
        meta = O.page_minmax(X, ps)
        s = O.page_scores(q, meta)
        for p in range(meta.shape[0]):
            expect = sum(_corner_max(q[h], meta[p, :, 0], meta[p, :, 1]) for h in range(G))
            assert abs(s[p] - expect) <= 1e-12 * (1 + abs(expect))


def test_page_minmax_brute_force_partial_pages():
    """min/max over exactly the page's valid rows (partial last page included), by row loops."""
    rng = _rng(5)
    X = rng.standard_normal((37, 6))
    meta = O.page_minmax(X, 16)
    assert meta.shape == (3, 6, 2)
    for p in range(3):
        for j in range(6):
            vals = [X[t, j] for t in range(37) if t // 16 == p]
            assert meta[p, j, 0] == min(vals) and meta[p, j, 1] == max(vals)


@pytest.mark.parametrize("G,L", [(1, 100), (4, 333), (8, 64)])
def test_page_bound_at_least_true_group_logit(G, L):
    """Every page score >= max over its keys of sum_h q_h.k (unrotated logits, brute force)."""
    inp = synth.make_hhr_inputs(1, G, 1, [L], L, "f32", seed=6 + G)
    q = inp["q"][0].astype(np.float64)
    K = inp["K"][0, 0].astype(np.float64)
    R, W = inp["R"][0], inp["W"][0]
    enc = O.encode_keys(K, R, W, 16)
    s = O.page_scores(O.rotate(q, R), enc["meta"])
    for p in range(s.shape[0]):
        rows = K[p * 16: min(L, (p + 1) * 16)]
        true = (rows @ q.T).sum(axis=1)
        slack = np.array([_orth_slack(R, q, r) for r in rows])
        assert s[p] >= (true - slack).max()


def _orth_slack(R, q, k):
    """|sum_h q_h.k - sum_h (q_h R).(k R)| <= ||I - R R^T||_2 * sum_h |q_h| |k| (R is f32-stored)."""
    R = np.asarray(R, np.float64)
    defect = np.linalg.norm(np.eye(R.shape[0]) - R @ R.T, 2)
    return (defect * np.linalg.norm(q, axis=1).sum() * np.linalg.norm(k)) * 1.01 + 1e-12


def test_page_bound_tight_on_single_key_pages():
    """A page holding one key (a partial last page here) has bound == its group logit."""
    inp = synth.make_hhr_inputs(1, 4, 1, [33], 48, "f32", seed=9)
    q = inp["q"][0].astype(np.float64)
    K = inp["K"][0, 0, :33].astype(np.float64)
    R, W = inp["R"][0], inp["W"][0]
    enc = O.encode_keys(K, R, W, 16)
    s = O.page_scores(O.rotate(q, R), enc["meta"])
    exact = float((q @ K[32]).sum())
    assert abs(s[2] - exact) <= _orth_slack(R, q, K[32])
    # page size 1: every page is a single key
    enc1 = O.encode_keys(K, R, W, 1)
    s1 = O.page_scores(O.rotate(q, R), enc1["meta"])
    exact1 = (K @ q.T).sum(axis=1)
    for t in range(33):
        assert abs(s1[t] - exact1[t]) <= _orth_slack(R, q, K[t])


# --------------------------------------------------------------------------- counts and top-k
@pytest.mark.parametrize("np_,num,den,absn,expect", [
    (256, 0, 1, 64, 64), (2048, 1, 4, 0, 512), (8192, 1, 8, 0, 1024), (2049, 1, 4, 0, 513),
    (1, 1, 4, 0, 1), (0, 1, 4, 0, 0), (3, 1, 8, 0, 1), (10, 3, 8, 0, 4), (40, 0, 1, 64, 40),
    (4096, 1, 4, 0, 1024), (513, 1, 4, 0, 129),
])
def test_keep_count_worked_values(np_, num, den, absn, expect):
    assert O.keep_count(np_, num, den, absn) == expect


def _brute_top_largest(scores, k):
    n = len(scores)
    keep = []
    for i in range(n):
        better = sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if better < k:
            keep.append(i)
    return keep


def _brute_top_smallest(H, pos, k):
    n = len(H)
    keep = []
    for i in range(n):
        better = sum(1 for j in range(n) if H[j] < H[i] or (H[j] == H[i] and pos[j] < pos[i]))
        if better < k:
            keep.append(pos[i])
    return sorted(keep)


def test_top_pages_brute_force_with_ties():
    rng = _rng(10)
    for trial in range(50):
        n = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, n).astype(np.float64)  # heavy ties
        if trial % 5 == 0:
            s[:] = 1.0
        if trial % 7 == 0:
            s = s * 0.0  # signed zeros compare equal
            s[::2] = -0.0
        for k in (1, n // 2, n):
            assert O.top_pages(s, k).tolist() == _brute_top_largest(list(s), k)


def test_topk_smallest_brute_force_with_ties():
    rng = _rng(11)
    for trial in range(50):
        n = int(rng.integers(1, 64))
        pos = np.sort(rng.choice(1000, n, replace=False))
        H = rng.integers(0, 5, n)
        if trial % 4 == 0:
            H[:] = 7  # all equal: lowest positions must win
        for k in (1, n // 3 + 1, n, n + 5):
            assert O.topk_smallest(H, pos, k).tolist() == _brute_top_smallest(list(H), list(pos), k)
    # all-equal case, explicit
    assert O.topk_smallest(np.full(10, 3), np.arange(10) * 5, 4).tolist() == [0, 5, 10, 15]


def test_candidates_respect_seq_len():
    assert O.candidates(np.array([0, 2]), 40, 16).tolist() == list(range(16)) + list(range(32, 40))


# --------------------------------------------------------------------------- attention
def test_attend_matches_library_sdpa():
    """Dense reduction: attend over all keys == torch CPU scaled_dot_product_attention (fp64)."""
    import torch

    rng = _rng(12)
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((300, 128))
    V = rng.standard_normal((300, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(K)[None, None].expand(1, 4, 300, 128),
        torch.from_numpy(V)[None, None].expand(1, 4, 300, 128))[0, :, 0, :].numpy()
    assert np.abs(O.attend(q, K, V) - ref).max() < 1e-12


def test_attend_single_key_returns_its_value_and_empty_is_zero():
    rng = _rng(13)
    q = rng.standard_normal((3, 128))
    K = rng.standard_normal((1, 128))
    V = rng.standard_normal((1, 128))
    assert np.allclose(O.attend(q, K, V), np.repeat(V, 3, axis=0), atol=1e-15)
    assert np.array_equal(O.attend(q, K[:0], V[:0]), np.zeros((3, 128)))


def test_keep_all_and_k_equal_L_reproduces_dense_attention():
    """Special case from the method: keeping every page and k = L selects every key."""
    import torch

    inp = synth.make_hhr_inputs(1, 4, 1, [200], 208, "bf16", seed=14)
    q = inp["q"][0].astype(np.float64)
    K = synth.kv_values(inp["K"][0, 0, :200], "bf16").astype(np.float64)
    V = synth.kv_values(inp["V"][0, 0, :200], "bf16").astype(np.float64)
    res = O.select(q, K, inp["R"][0], inp["W"][0], 16, 1, 1, 0, 200)
    assert res["n_keep"] == 13 and res["sel"].tolist() == list(range(200))
    o = O.attend(q, K[res["sel"]], V[res["sel"]])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], torch.from_numpy(K)[None].expand(4, 200, 128),
        torch.from_numpy(V)[None].expand(4, 200, 128))[:, 0, :].numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_exact_topk_brute_force():
    rng = _rng(15)
    q = rng.integers(-2, 3, (2, 8)).astype(np.float64)
    K = rng.integers(-2, 3, (30, 8)).astype(np.float64)
    logits = list((K @ q.T).sum(axis=1))
    for k in (1, 5, 30):
        assert O.exact_topk(q, K, k).tolist() == _brute_top_largest(logits, k)


# --------------------------------------------------------------------------- pipeline
def test_pipeline_shapes_on_tiny_workload():
    """Composed pipeline on the tiny 4K f32 recipe: counts, ordering, and better-than-chance recall.

    Recall itself is a property of the synthetic data (not a parity pin); chance level for
    256 of 4096 keys would be 1/16.
    """
    inp = synth.make_hhr_inputs(1, 4, 1, [4096], 4096, "f32", seed=1000)
    q = inp["q"][0]
    K = inp["K"][0, 0]
    res = O.select(q, K, inp["R"][0], inp["W"][0], 16, 0, 1, 64, 256)
    assert res["n_keep"] == 64 and len(res["sel"]) == 256
    assert np.all(np.diff(res["sel"]) > 0)
    assert O.recall(res["sel"], O.exact_topk(q, K, 256)) > 0.2


def test_pipeline_degenerate_lengths():
    inp = synth.make_hhr_inputs(1, 4, 1, [1], 16, "f32", seed=16)
    res = O.select(inp["q"][0], inp["K"][0, 0, :1], inp["R"][0], inp["W"][0], 16, 1, 4, 0, 8)
    assert res["n_keep"] == 1 and res["sel"].tolist() == [0]
    res0 = O.select(inp["q"][0], inp["K"][0, 0, :0], inp["R"][0], inp["W"][0], 16, 1, 4, 0, 8)
    assert res0["n_keep"] == 0 and res0["sel"].size == 0


# --------------------------------------------------------------------------- #
# bfloat16 page metadata (outward rounding)
# --------------------------------------------------------------------------- #
def _bf16_neighbours(v):
    """bfloat16 values around v from torch's round-to-nearest-even conversion
    (an independent library routine): the nearest one and the next grid points
    on both sides, as float64."""
    import torch

    near = torch.tensor(v, dtype=torch.float64).to(torch.bfloat16)
    bits = near.view(torch.int16).to(torch.int32) & 0xFFFF
    out = []
    for dbits in (-1, 0, 1):
        b = bits + dbits * torch.where(near >= 0, 1, -1)
        b = b & 0xFFFF
        out.append(torch.tensor(b.numpy().astype(np.uint16).view(np.int16)).view(torch.bfloat16)
                   .to(torch.float64).numpy())
    return np.stack(out)


def test_bf16_round_is_the_nearest_grid_point_in_each_direction():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 7, 4000),
                        [0.0, 1.0, -1.0, 2.0 ** -130, -3.0 * 2.0 ** -133, 1.0 + 2.0 ** -8]])
    down, up = O.bf16_round(v, up=False), O.bf16_round(v, up=True)
    # representable in bfloat16: the float32 bit pattern has zero low half
    for r in (down, up):
        f = r.astype(np.float32)
        assert np.all(f.astype(np.float64) == r)
        assert np.all((f.view(np.uint32) & 0xFFFF) == 0)
    assert np.all(down <= v) and np.all(up >= v)
    # no bfloat16 value lies strictly between: check against torch's grid
    nb = _bf16_neighbours(v)  # [3][n]
    below = np.where(nb <= v, nb, -np.inf).max(axis=0)
    above = np.where(nb >= v, nb, np.inf).min(axis=0)
    assert np.all(down == below) and np.all(up == above)
    exact = v == down
    assert np.all(up[exact] == v[exact])


def test_bf16_outward_metadata_keeps_the_bound_valid():
    rng = np.random.default_rng(6)
    d, G = 32, 3
    Q = rng.standard_normal((G, d))
    K = rng.standard_normal((50, d)) * np.array([8.0 if i < 2 else 1.0 for i in range(d)])
    R = np.linalg.qr(rng.standard_normal((d, d)))[0]
    W = rng.standard_normal((d, d))
    enc32 = O.encode_keys(K, R, W, 16)
    enc16 = O.encode_keys(K, R, W, 16, meta_dtype="bf16")
    assert np.all(enc16["meta"][..., 0] <= enc32["meta"][..., 0])
    assert np.all(enc16["meta"][..., 1] >= enc32["meta"][..., 1])
    qr = O.rotate(Q, R)
    s16 = O.page_scores(qr, enc16["meta"])
    s32 = O.page_scores(qr, enc32["meta"])
    assert np.all(s16 >= s32 - 1e-9 * np.abs(s32))
    true = (K @ Q.T).sum(axis=1)
    for p in range(s16.size):
        assert s16[p] >= true[p * 16:(p + 1) * 16].max() - 1e-9


def test_recall_worked_values():
    """recall = |selected & exact| / |exact| (HHR Figure 4: top-k key recall)."""
    assert O.recall([1, 2, 3, 4], [2, 4, 6, 8]) == 0.5
    # more or fewer selected than exact: the denominator is the exact set
    assert O.recall([5], [1, 2, 3, 5]) == 0.25
    assert O.recall([1, 2, 3, 4, 5, 6], [1, 2]) == 1.0
    assert O.recall([7, 9], [1, 2, 3]) == 0.0
    assert O.recall([], [1]) == 0.0
    assert O.recall([3], []) == 1.0
