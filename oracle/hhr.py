"""Oracle: coarse-to-fine hash retrieval and sparse decode attention (HHR / HATA).

TEST INFRASTRUCTURE ONLY (see the package docstring): plain, slow, fp64.

The method, as the HHR abstract states it: queries and keys are encoded into
binary codes and keys are selected by Hamming distance; a head-wise orthogonal
transform R_h (Geometry-Aware Key Routing, GKR) yields page-level logit bounds
that prune low-logit pages; a head-wise learned projection W_h (Learned Hash
Projection, LHP) gives the codes that rank keys inside the surviving pages;
attention then runs over only the selected keys.  Figure 1 ("Overview") orders
the stages coarse (GKR) then fine (LHP).  Figure 2's caption fixes the hash as
a projection followed by sign(.).  Appendix Table 4 fixes 128-bit codes and
appendix Figure 10 varies the number of bits; the functions here take any multiple
of 32 bits, the width of W's last axis.  The
HATA abstract adds that codes only need to give the relative q.k order,
which is what a top-k needs.

Readings where the pages are silent (each also listed in the design notes):
  * page bound: per page and per rotated dimension, the min and max of the
    rotated keys; the bound for one query head is sum_d max(q'_d*mn_d, q'_d*mx_d),
    the plainest valid upper bound of q'.x over the page;
  * GQA: one selection per KV head; per-head bounds and per-head Hamming
    distances are summed over the query heads of the group;
  * sign(0): code bit j is 1 iff y_j >= 0 (so -0.0 also gives 1);
  * bit packing: bit j of a code sits in 32-bit word j // 32 at bit j % 32;
  * tie-breaks: pages by larger bound then lower page index; keys by smaller
    Hamming distance then lower position; exact top-k by larger logit then
    lower position;
  * kept page count P = min(Np, max(1, ceil(num * Np / den))), or
    min(Np, P_abs) when an absolute count is given;
  * softmax scale 1/sqrt(d) on exact q.k (hashes only select, never weight).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- #
# Hash codes  [HHR abstract: binary codes; Figure 2 caption: projection + sign]
# --------------------------------------------------------------------------- #
def sign_bits(y) -> np.ndarray:
    """Bit of each projected coordinate: 1 where y >= 0 (IEEE: -0.0 >= 0 holds)."""
    return _f64(y) >= 0.0


def pack_bits(bits) -> np.ndarray:
    """Pack [..., nbits] booleans into [..., nbits/32] uint32: bit j -> word j//32, bit j%32."""
    bits = np.asarray(bits, dtype=bool)
    nbits = bits.shape[-1]
    if nbits % 32:
        raise ValueError("code length must be a multiple of 32")
    grouped = bits.reshape(bits.shape[:-1] + (nbits // 32, 32)).astype(np.uint64)
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    return (grouped * weights).sum(axis=-1).astype(np.uint32)


def unpack_bits(words) -> np.ndarray:
    """Inverse of pack_bits: [..., nwords] uint32 -> [..., 32*nwords] bool."""
    w = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    shifts = np.arange(32, dtype=np.uint64)
    bits = (w[..., None] >> shifts) & np.uint64(1)
    return bits.reshape(w.shape[:-1] + (w.shape[-1] * 32,)).astype(bool)


def hash_codes(x, W) -> np.ndarray:
    """Codes of rows x under projection W: pack(sign(x @ W))  [HHR abstract, LHP]."""
    return pack_bits(sign_bits(_f64(x) @ _f64(W)))


def hamming(q_codes, key_codes) -> np.ndarray:
    """Summed Hamming distance of each key code to the group's query codes.

    q_codes [G][w] (one row per query head of the GQA group), key_codes [n][w]
    -> H [n] = sum_h popcount(q_codes[h] XOR key_codes[t])   [HHR abstract].
    """
    q = np.asarray(q_codes, dtype=np.uint32)
    k = np.asarray(key_codes, dtype=np.uint32)
    total = np.zeros(k.shape[0], dtype=np.int64)
    for h in range(q.shape[0]):
        total += np.bitwise_count(np.bitwise_xor(k, q[h][None, :])).sum(axis=-1).astype(np.int64)
    return total


# --------------------------------------------------------------------------- #
# Key encoding: rotated keys and page metadata  [HHR abstract, GKR]
# --------------------------------------------------------------------------- #
def rotate(x, R) -> np.ndarray:
    """x @ R: keys (or queries) in the head's orthogonally rotated frame."""
    return _f64(x) @ _f64(R)


def page_minmax(X, page_size: int) -> np.ndarray:
    """Per page and per dimension, [min, max] of the rotated keys over the page's valid rows.

    X [L][d] holds only valid rows; the last page may be partial.
    Returns meta [ceil(L/page_size)][d][2].
    """
    X = _f64(X)
    L, d = X.shape
    n_pages = -(-L // page_size)
    meta = np.empty((n_pages, d, 2), dtype=np.float64)
    for p in range(n_pages):
        rows = X[p * page_size: min((p + 1) * page_size, L)]
        meta[p, :, 0] = rows.min(axis=0)
        meta[p, :, 1] = rows.max(axis=0)
    return meta


def bf16_round(v, up: bool) -> np.ndarray:
    """Each value rounded to bfloat16 toward +inf (up) or -inf (down).

    bfloat16 keeps 8 significant bits, so in the binade [2^e, 2^(e+1)) its grid
    spacing is 2^(e-7) (2^-133 below the normal range).  Dividing by a power of
    two, floor / ceil and multiplying back are exact in fp64.
    """
    v = _f64(v)
    _, e = np.frexp(np.abs(v))  # |v| = m 2^e with m in [0.5, 1): binade 2^(e-1)
    ulp = np.exp2(np.maximum(e - 1, -126) - 7.0)
    q = v / ulp
    return (np.ceil(q) if up else np.floor(q)) * ulp


def bf16_outward(meta) -> np.ndarray:
    """Compressed page metadata: every min rounded down and every max rounded up
    to bfloat16, so the page bound built from it still bounds every key
    (looser by at most one bfloat16 step per dimension)."""
    meta = _f64(meta)
    out = np.empty_like(meta)
    out[..., 0] = bf16_round(meta[..., 0], up=False)
    out[..., 1] = bf16_round(meta[..., 1], up=True)
    return out


def encode_keys(K, R, W, page_size: int, meta_dtype: str = "f32") -> Dict[str, np.ndarray]:
    """What appending keys K [L][d] (valid rows only) to the cache produces.

    Returns X = K R (fp64), codes = pack(sign(K W)), meta = page min/max of X
    (outward-rounded to bfloat16 when meta_dtype is "bf16").
    """
    X = rotate(K, R)
    meta = page_minmax(X, page_size)
    if meta_dtype == "bf16":
        meta = bf16_outward(meta)
    return dict(X=X, codes=hash_codes(K, W), meta=meta)


def encode_query(q_group, R, W) -> Dict[str, np.ndarray]:
    """Rotated queries q' = q R and query codes pack(sign(q W)) for each head of the group."""
    return dict(qrot=rotate(q_group, R), qcodes=hash_codes(q_group, W))


# --------------------------------------------------------------------------- #
# Page scoring and pruning  [HHR abstract: page-level logit bounds, pruning]
# --------------------------------------------------------------------------- #
def page_scores(qrot_group, meta) -> np.ndarray:
    """Upper bound of the group's summed logits over each page.

    s(p) = sum_h sum_d max(q'_{h,d} * mn_{p,d}, q'_{h,d} * mx_{p,d}).
    For every key x of page p and every head h, q'_h . x <= sum_d max(...),
    so s(p) >= max_t sum_h q'_h . x_t (scale omitted: it does not change ranks).
    """
    qrot = _f64(qrot_group)
    meta = _f64(meta)
    mn, mx = meta[..., 0], meta[..., 1]
    s = np.zeros(meta.shape[0], dtype=np.float64)
    for h in range(qrot.shape[0]):
        s += np.maximum(qrot[h][None, :] * mn, qrot[h][None, :] * mx).sum(axis=-1)
    return s


def n_pages(seq_len: int, page_size: int) -> int:
    return -(-int(seq_len) // page_size) if seq_len > 0 else 0


def keep_count(n_pages_: int, keep_num: int, keep_den: int, keep_abs: int = 0) -> int:
    """Number of kept pages: min(Np, keep_abs) if keep_abs > 0, else
    min(Np, max(1, ceil(keep_num * Np / keep_den))) in integer arithmetic; 0 when Np == 0."""
    if n_pages_ <= 0:
        return 0
    if keep_abs > 0:
        return min(n_pages_, keep_abs)
    p = -(-(keep_num * n_pages_) // keep_den)
    return min(n_pages_, max(1, p))


def top_pages(scores, n_keep: int) -> np.ndarray:
    """The n_keep pages with the largest score (ties: lower page index), ascending ids."""
    s = _f64(scores)
    idx = np.arange(s.shape[0])
    order = np.lexsort((idx, -s))          # primary: larger score; secondary: lower index
    return np.sort(order[:n_keep]).astype(np.int64)


# --------------------------------------------------------------------------- #
# Fine selection inside kept pages  [HHR abstract, LHP; HATA abstract]
# --------------------------------------------------------------------------- #
def candidates(kept_pages, seq_len: int, page_size: int) -> np.ndarray:
    """Valid key positions of the kept pages, ascending."""
    pos = (np.asarray(kept_pages, dtype=np.int64)[:, None] * page_size
           + np.arange(page_size)[None, :]).reshape(-1)
    return pos[pos < seq_len]


def topk_smallest(H, positions, k: int) -> np.ndarray:
    """First min(k, n) positions in (H ascending, position ascending) order, returned ascending."""
    H = np.asarray(H, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    order = np.lexsort((positions, H))
    return np.sort(positions[order[:k]])


def select(q_group, K_valid, R, W, page_size: int, keep_num: int, keep_den: int,
           keep_abs: int, top_k: int, meta_dtype: str = "f32") -> Dict[str, np.ndarray]:
    """The whole selection for one (sequence, KV head), from raw inputs.

    q_group [G][d] queries of the group, K_valid [L][d] the sequence's keys;
    meta_dtype "bf16" stores the page metadata outward-rounded (bf16_outward).
    """
    L = K_valid.shape[0]
    enc = encode_keys(K_valid, R, W, page_size, meta_dtype)
    qe = encode_query(q_group, R, W)
    s = page_scores(qe["qrot"], enc["meta"])
    P = keep_count(n_pages(L, page_size), keep_num, keep_den, keep_abs)
    kept = top_pages(s, P)
    cand = candidates(kept, L, page_size)
    H = hamming(qe["qcodes"], enc["codes"][cand])
    sel = topk_smallest(H, cand, top_k)
    return dict(enc=enc, qrot=qe["qrot"], qcodes=qe["qcodes"], scores=s, n_keep=P, kept=kept,
                cand=cand, H=H, sel=sel)


def select_from_codes(q_codes, key_codes, kept_pages, seq_len: int, page_size: int,
                      top_k: int) -> Dict[str, np.ndarray]:
    """Fine stage alone, on given query codes, key codes [L][w] and kept pages."""
    cand = candidates(kept_pages, seq_len, page_size)
    H = hamming(q_codes, np.asarray(key_codes)[cand])
    return dict(cand=cand, H=H, sel=topk_smallest(H, cand, top_k))


# --------------------------------------------------------------------------- #
# Attention over the selected keys  [HHR abstract: hash-based sparse attention]
# --------------------------------------------------------------------------- #
def attend(q_group, K_rows, V_rows, scale: Optional[float] = None) -> np.ndarray:
    """o_h = sum_i softmax_i(q_h . K_i * scale) V_i over the given rows, fp64.

    An empty row set gives o = 0.
    """
    q = _f64(q_group)
    K = _f64(K_rows)
    V = _f64(V_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[-1] if V.ndim == 2 else q.shape[-1]))
    logits = (q @ K.T) * scale
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ V


# --------------------------------------------------------------------------- #
# Measurement helpers  [HHR Figure 4: per-KV-head top-k key recall]
# --------------------------------------------------------------------------- #
def exact_topk(q_group, K_valid, k: int) -> np.ndarray:
    """The k positions with the largest summed group logit sum_h q_h . K_t (ties: lower t)."""
    logits = (_f64(K_valid) @ _f64(q_group).T).sum(axis=-1)
    t = np.arange(logits.shape[0])
    order = np.lexsort((t, -logits))
    return np.sort(order[:k])


def recall(selected, exact) -> float:
    """|selected & exact| / |exact|."""
    exact = np.asarray(exact)
    if exact.size == 0:
        return 1.0
    return float(np.intersect1d(np.asarray(selected), exact).size) / float(exact.size)
