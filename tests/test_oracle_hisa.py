"""Pins for the HISA oracle: library fp8 decode, special cases that reduce to the flat indexer,
the ReLU scale factoring, and brute-force ordering."""
import numpy as np
import pytest

from oracle import hisa as O
from hash_hierarchical_top_amd import synth


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_e4m3fn_decode_matches_library_for_all_256_codes():
    import torch

    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    # worked values: 0x38 = 1.0, 0x7E = 448 (largest finite), 0x01 = 2^-9, 0xB8 = -1.0
    assert O.e4m3fn_decode(np.array([0x38, 0x7E, 0x01, 0xB8], np.uint8)).tolist() == \
        [1.0, 448.0, 2.0 ** -9, -1.0]


def test_pooled_reps_worked_and_special_cases():
    keys = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 9.0], [7.0, -1.0], [2.0, 2.0]])
    # blocks of 2 over 5 rows: means (2,3), (6,4), (2,2) -- the last block has one valid row
    assert O.pooled_reps(keys, 2).tolist() == [[2.0, 3.0], [6.0, 4.0], [2.0, 2.0]]
    assert np.array_equal(O.pooled_reps(keys, 1), keys)


def test_indexer_scores_worked_example_and_relu_factoring():
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([0.5, 2.0])
    x = np.array([[2.0, -3.0], [-1.0, 1.0]])
    # t0: 0.5*relu(2) + 2*relu(-3) = 1.0 ; t1: 0.5*relu(-1) + 2*relu(1) = 2.0
    assert O.indexer_scores(q, w, x).tolist() == [1.0, 2.0]
    rng = _rng(1)
    q = rng.standard_normal((8, 16))
    w = rng.random(8)
    x = rng.standard_normal((30, 16))
    base = O.indexer_scores(q, w, x)
    assert np.allclose(O.indexer_scores(3.0 * q, w, x), 3.0 * base)
    assert np.allclose(O.indexer_scores(q, w, 0.25 * x), 0.25 * base)
    assert np.all(base >= 0)


def _brute_top_largest(scores, ids, k):
    keep = []
    for i in range(len(ids)):
        better = sum(1 for j in range(len(ids))
                     if scores[j] > scores[i] or (scores[j] == scores[i] and ids[j] < ids[i]))
        if better < k:
            keep.append(ids[i])
    return sorted(keep)


def test_top_largest_brute_force():
    rng = _rng(2)
    for _ in range(40):
        n = int(rng.integers(1, 50))
        s = rng.integers(0, 4, n).astype(float)
        ids = np.arange(n) * 3
        for k in (1, n // 2 + 1, n + 2):
            assert O.top_largest(s, ids, k).tolist() == _brute_top_largest(list(s), list(ids), k)


def _small_inputs(ctx, seed):
    return synth.make_hisa_inputs(8, ctx, ctx, 4, seed, head_dim=32, make_kv=False)


def test_keep_all_blocks_equals_flat_indexer():
    inp = _small_inputs(1000, 3)
    args = (inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], 1000)
    res = O.select(*args, block=64, keep_blocks=16, top_k=100)
    flat = O.flat_select(*args, top_k=100)
    assert res["sel"].tolist() == flat.tolist()
    assert O.iou(res["sel"], flat) == 1.0


def test_block_size_one_coarse_equals_fine():
    inp = _small_inputs(300, 4)
    args = (inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], 300)
    res = O.select(*args, block=1, keep_blocks=40, top_k=40)
    assert res["blocks"].tolist() == res["sel"].tolist()
    assert res["sel"].tolist() == O.flat_select(*args, top_k=40).tolist()


def test_iou_definition():
    assert O.iou([1, 2, 3], [2, 3, 4]) == pytest.approx(0.5)
    assert O.iou([], []) == 1.0


# --------------------------------------------------------------------------- #
# prefill rows (one shared cache, causal prefixes)
# --------------------------------------------------------------------------- #
def _prefill_inputs(seed=31, Hi=8, L=900):
    rng = np.random.default_rng(seed)
    q8, qs = synth.quantize_rows_e4m3(rng.standard_normal((Hi, 128)).astype(np.float32))
    k8, ks = synth.quantize_rows_e4m3(rng.standard_normal((L, 128)).astype(np.float32))
    return q8, qs, rng.uniform(0, 1, Hi).astype(np.float32), k8, ks


def test_prefill_row_at_the_cache_end_is_the_decode_selection():
    q8, qs, wt, k8, ks = _prefill_inputs()
    for L in (900, 896, 1):
        a = O.prefill_select(q8, qs, wt, k8, ks, L, L, 64, 5, 100)
        b = O.select(q8, qs, wt, k8, ks, L, 64, 5, 100)
        assert np.array_equal(a["sel"], b["sel"]) and np.array_equal(a["blocks"], b["blocks"])


@pytest.mark.parametrize("q_len", [1, 63, 64, 65, 500, 900])
def test_prefill_row_is_the_decode_selection_at_its_length(q_len):
    """Causal prefill: row r of a chunk over a 900-key cache selects exactly what a decode
    query with a sequence of q_len[r] tokens selects (the decode path pools the prefix
    keys[:q_len] itself, so a partly visible last block is pooled over its visible rows)."""
    q8, qs, wt, k8, ks = _prefill_inputs()
    a = O.prefill_select(q8, qs, wt, k8, ks, 900, q_len, 64, 3, 150)
    b = O.select(q8, qs, wt, k8, ks, q_len, 64, 3, 150)
    assert a["reps"].shape == b["reps"].shape
    assert np.allclose(a["reps"], b["reps"], rtol=1e-12, atol=1e-14)
    assert np.allclose(a["block_scores"], b["block_scores"], rtol=1e-12, atol=1e-14)
    assert np.array_equal(a["blocks"], b["blocks"])
    assert np.array_equal(a["cand"], b["cand"])
    assert np.array_equal(a["sel"], b["sel"])


def test_prefill_row_does_not_see_future_keys():
    """Rewriting every key at or after the row's position (the rest of its last block
    included) leaves the row's representatives, block scores and selection unchanged."""
    q8, qs, wt, k8, ks = _prefill_inputs()
    rng = np.random.default_rng(77)
    for q_len in (1, 40, 64, 100, 511):
        k8b, ksb = k8.copy(), ks.copy()
        junk8, junks = synth.quantize_rows_e4m3(
            (5.0 * rng.standard_normal((900 - q_len, 128))).astype(np.float32))
        k8b[q_len:], ksb[q_len:] = junk8, junks
        a = O.prefill_select(q8, qs, wt, k8, ks, 900, q_len, 64, 2, 40)
        b = O.prefill_select(q8, qs, wt, k8b, ksb, 900, q_len, 64, 2, 40)
        assert np.array_equal(a["reps"], b["reps"])
        assert np.array_equal(a["block_scores"], b["block_scores"])
        assert np.array_equal(a["sel"], b["sel"])


def test_prefill_row_sees_only_its_prefix():
    q8, qs, wt, k8, ks = _prefill_inputs()
    keys = O.dequantize(k8[:900], ks[:900])
    full = O.pooled_reps(keys, 64)
    for q_len in (1, 63, 64, 65, 500):
        r = O.prefill_select(q8, qs, wt, k8, ks, 900, q_len, 64, 4, 300)
        assert r["sel"].size == min(300, r["cand"].size) and np.all(r["sel"] < q_len)
        assert r["blocks"].size == min(4, -(-q_len // 64)) and np.all(r["blocks"] * 64 < q_len)
        # blocks wholly inside the prefix keep the cache's pooled representative; a partly
        # visible last block is the mean of its visible rows (worked: q_len = 1 is row 0)
        nf = q_len // 64
        assert np.array_equal(r["reps"][:nf], full[:nf])
        if q_len % 64:
            assert np.allclose(r["reps"][nf], keys[nf * 64:q_len].mean(axis=0), rtol=0,
                               atol=1e-15)
    assert np.array_equal(O.prefill_select(q8, qs, wt, k8, ks, 900, 1, 64, 4, 300)["reps"],
                          keys[:1])


def test_prefill_keep_all_blocks_is_the_flat_indexer_on_the_prefix():
    q8, qs, wt, k8, ks = _prefill_inputs()
    for q_len in (1, 100, 640, 900):
        r = O.prefill_select(q8, qs, wt, k8, ks, 900, q_len, 64, 15, 50)
        assert np.array_equal(r["sel"], O.flat_select(q8, qs, wt, k8, ks, q_len, 50))
