"""Each plausible oracle mistake must be caught by at least one pin.

The mutants are planted into the oracle on the CPU only (monkeypatched copies of
its functions); the pins are the unmodified tests in test_oracle_hhr.py and
test_oracle_hisa.py, re-run against each mutant.
"""
import numpy as np
import pytest

from oracle import hhr as O
from oracle import hisa as OH
import tests.test_oracle_hhr as P
import tests.test_oracle_hisa as PH


def _pins(module):
    out = []
    for name in dir(module):
        if not name.startswith("test_"):
            continue
        fn = getattr(module, name)
        params = getattr(fn, "pytestmark", [])
        cases = [()]
        for m in params:
            if m.name == "parametrize":
                cases = [c if isinstance(c, tuple) else (c,) for c in m.args[1]]
        for c in cases:
            out.append((name, fn, c))
    return out


def _caught(module, monkeypatch_target, attr, mutant):
    original = getattr(monkeypatch_target, attr)
    setattr(monkeypatch_target, attr, mutant)
    try:
        for name, fn, args in _pins(module):
            try:
                fn(*args)
            except Exception:
                return name
        return None
    finally:
        setattr(monkeypatch_target, attr, original)


def _scores_drop_head(qrot, meta):
    qrot = np.asarray(qrot, np.float64)
    meta = np.asarray(meta, np.float64)
    s = np.zeros(meta.shape[0])
    for h in range(max(qrot.shape[0] - 1, 1)):
        s += np.maximum(qrot[h] * meta[..., 0], qrot[h] * meta[..., 1]).sum(-1)
    return s


def _scores_swapped(qrot, meta):
    qrot = np.asarray(qrot, np.float64)
    meta = np.asarray(meta, np.float64)
    s = np.zeros(meta.shape[0])
    for h in range(qrot.shape[0]):
        s += np.minimum(qrot[h] * meta[..., 0], qrot[h] * meta[..., 1]).sum(-1)
    return s


def _scores_sum_query(qrot, meta):  # bound of sum_h q_h instead of the sum of per-head bounds
    q = np.asarray(qrot, np.float64).sum(0)
    meta = np.asarray(meta, np.float64)
    return np.maximum(q * meta[..., 0], q * meta[..., 1]).sum(-1)


def _pack_msb_first(bits):
    bits = np.asarray(bits, bool)
    g = bits.reshape(bits.shape[:-1] + (bits.shape[-1] // 32, 32)).astype(np.uint64)
    w = np.left_shift(np.uint64(1), np.arange(31, -1, -1, dtype=np.uint64))
    return (g * w).sum(-1).astype(np.uint32)


def _sign_strict(y):
    return np.asarray(y, np.float64) > 0.0


def _hamming_one_head(qc, kc):
    return np.bitwise_count(np.bitwise_xor(np.asarray(kc, np.uint32),
                                           np.asarray(qc, np.uint32)[0][None])).sum(-1).astype(np.int64)


def _top_pages_high_index_ties(s, n):
    s = np.asarray(s, np.float64)
    idx = np.arange(s.shape[0])
    return np.sort(np.lexsort((-idx, -s))[:n])


def _topk_high_pos_ties(H, pos, k):
    H = np.asarray(H, np.int64)
    pos = np.asarray(pos, np.int64)
    return np.sort(pos[np.lexsort((-pos, H))[:k]])


def _keep_floor(np_, num, den, absn=0):
    if np_ <= 0:
        return 0
    if absn > 0:
        return min(np_, absn)
    return min(np_, max(1, num * np_ // den))


def _attend_no_scale(q, K, V, scale=None):
    return O.__dict__["_attend_orig"](q, K, V, 1.0)


def _minmax_whole_last_page(X, ps):
    X = np.asarray(X, np.float64)
    L, d = X.shape
    pad = -(-L // ps) * ps
    Xp = np.zeros((pad, d))
    Xp[:L] = X
    return np.stack([Xp.reshape(-1, ps, d).min(1), Xp.reshape(-1, ps, d).max(1)], axis=-1)


def _rotate_transposed(x, R):
    return np.asarray(x, np.float64) @ np.asarray(R, np.float64).T


def _bf16_round_fine(v, up):
    """one bit too many: a grid of 9 significant bits"""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(np.abs(v))
    ulp = np.exp2(np.maximum(e - 1, -126) - 8.0)
    return (np.ceil(v / ulp) if up else np.floor(v / ulp)) * ulp


def _bf16_round_toward_zero(v, up):
    """directions applied to the magnitude: negative values round the wrong way"""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    ulp = np.exp2(np.maximum(e - 1, -126) - 7.0)
    return np.sign(v) * (np.ceil(a / ulp) if up else np.floor(a / ulp)) * ulp


def _outward_inward(meta):
    meta = np.asarray(meta, np.float64)
    out = np.empty_like(meta)
    out[..., 0] = O.bf16_round(meta[..., 0], up=True)
    out[..., 1] = O.bf16_round(meta[..., 1], up=False)
    return out


def _recall_over_selected(selected, exact):
    """divides by the number selected instead of the exact set's size"""
    selected = np.asarray(selected)
    if selected.size == 0:
        return 1.0
    return float(np.intersect1d(selected, np.asarray(exact)).size) / float(selected.size)


MUTANTS = [
    ("recall", _recall_over_selected),
    ("bf16_round", _bf16_round_fine),
    ("bf16_round", _bf16_round_toward_zero),
    ("bf16_outward", _outward_inward),
    ("page_scores", _scores_drop_head),
    ("page_scores", _scores_swapped),
    ("page_scores", _scores_sum_query),
    ("pack_bits", _pack_msb_first),
    ("sign_bits", _sign_strict),
    ("hamming", _hamming_one_head),
    ("top_pages", _top_pages_high_index_ties),
    ("topk_smallest", _topk_high_pos_ties),
    ("keep_count", _keep_floor),
    ("attend", _attend_no_scale),
    ("page_minmax", _minmax_whole_last_page),
    ("rotate", _rotate_transposed),
]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[f"{a}:{m.__name__}" for a, m in MUTANTS])
def test_hhr_pins_catch_mutant(attr, mutant):
    O._attend_orig = O.attend.__wrapped__ if hasattr(O.attend, "__wrapped__") else O.attend
    assert _caught(P, O, attr, mutant) is not None, f"no pin catches mutant {mutant.__name__}"


def _decode_no_subnormal(codes):
    u = np.asarray(codes, np.uint8).astype(np.int64)
    e = (u >> 3) & 0xF
    m = u & 7
    mag = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where((u >> 7) & 1, -mag, mag)


def _decode_bias8(codes):
    return OH.__dict__["_dec_orig"](codes) / 2.0


def _reps_sum(keys, block):
    keys = np.asarray(keys, np.float64)
    nb = -(-keys.shape[0] // block)
    return np.stack([keys[b * block:(b + 1) * block].sum(0) for b in range(nb)])


def _scores_no_relu(q, w, x):
    return (np.asarray(x, np.float64) @ np.asarray(q, np.float64).T) @ np.asarray(w, np.float64)


def _top_largest_high_ties(s, ids, k):
    s = np.asarray(s, np.float64)
    ids = np.asarray(ids, np.int64)
    return np.sort(ids[np.lexsort((-ids, -s))[:k]])


def _prefill_whole_block_mean(q8, q_scale, w, k8, k_scale, cache_len, q_len, block,
                              keep_blocks, top_k):
    """the non-causal reading: the row's partly visible last block is scored with the mean
    of the whole cache block, keys after the row's position included"""
    q = OH.dequantize(q8, q_scale)
    keys = OH.dequantize(np.asarray(k8)[:cache_len], np.asarray(k_scale)[:cache_len])
    reps = OH.pooled_reps(keys, block)[:(q_len + block - 1) // block]
    S = OH.indexer_scores(q, w, reps)
    blocks = OH.top_largest(S, np.arange(reps.shape[0]), keep_blocks)
    cand = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    cand = cand[cand < q_len]
    s = OH.indexer_scores(q, w, keys[cand])
    return dict(reps=reps, block_scores=S, blocks=blocks, cand=cand, token_scores=s,
                sel=OH.top_largest(s, cand, top_k))


def _prefill_no_causal_mask(q8, q_scale, w, k8, k_scale, cache_len, q_len, block, keep_blocks,
                            top_k):
    """the token stage scans the kept blocks up to the cache end"""
    r = OH.__dict__["_prefill_orig"](q8, q_scale, w, k8, k_scale, cache_len, q_len, block,
                                     keep_blocks, top_k)
    q = OH.dequantize(q8, q_scale)
    keys = OH.dequantize(np.asarray(k8)[:cache_len], np.asarray(k_scale)[:cache_len])
    cand = (r["blocks"][:, None] * block + np.arange(block)[None, :]).reshape(-1)
    cand = cand[cand < cache_len]
    s = OH.indexer_scores(q, w, keys[cand])
    return dict(r, cand=cand, token_scores=s, sel=OH.top_largest(s, cand, top_k))


def _prefill_prefix_of_cache_rows(q8, q_scale, w, k8, k_scale, cache_len, q_len, block,
                                  keep_blocks, top_k):
    """an off-by-one on the row's prefix: it sees tokens t <= q_len (one key too many)"""
    return OH.__dict__["_prefill_orig"](q8, q_scale, w, k8, k_scale, cache_len,
                                        min(q_len + 1, cache_len), block, keep_blocks, top_k)


HISA_MUTANTS = [
    ("prefill_select", _prefill_whole_block_mean),
    ("prefill_select", _prefill_no_causal_mask),
    ("prefill_select", _prefill_prefix_of_cache_rows),
    ("e4m3fn_decode", _decode_no_subnormal),
    ("e4m3fn_decode", _decode_bias8),
    ("pooled_reps", _reps_sum),
    ("indexer_scores", _scores_no_relu),
    ("top_largest", _top_largest_high_ties),
]


@pytest.mark.parametrize("attr,mutant", HISA_MUTANTS,
                         ids=[f"{a}:{m.__name__}" for a, m in HISA_MUTANTS])
def test_hisa_pins_catch_mutant(attr, mutant):
    OH._dec_orig = OH.e4m3fn_decode
    OH._prefill_orig = OH.prefill_select
    assert _caught(PH, OH, attr, mutant) is not None, f"no pin catches mutant {mutant.__name__}"
