"""Oracle: HISA hierarchical indexer (block-pooled coarse filter, token refinement).

TEST INFRASTRUCTURE ONLY (see the package docstring): plain, slow, fp64.

The HISA abstract describes the path: a DSA-style lightweight indexer scores
every past token for the query and keeps a token-level top-k; HISA replaces the
flat scan by (1) a block-level coarse filter that scores pooled block
representatives and drops the rest, then (2) the original indexer applied only
inside the remaining blocks, giving an exact token-level top-k among them.

Readings where the pages are silent:
  * indexer score of token t: sum_h w_h * ReLU(q_h . k_t) with non-negative
    per-head weights w_h (the DSA lightweight-indexer form);
  * pooled representative of a block: the mean of its valid (dequantized) keys;
  * the block score uses the same indexer formula on the representative;
  * fp8 storage: OCP e4m3fn codes with one positive f32 scale per row,
    dequantized value = scale * e4m3fn(code);
  * ties: larger score first, then lower block / token index;
  * "exact" top-k means exact within the kept blocks (the coarse stage is a
    heuristic; its agreement with the flat indexer is measured by IoU);
  * a prefill query row at position p is causal in both stages: it sees tokens
    t <= p only, so its partly visible last block is pooled over its visible rows,
    and it selects what a decode query with p + 1 tokens in the cache selects.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def e4m3fn_decode(codes) -> np.ndarray:
    """Value of OCP fp8 e4m3fn bytes: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0.

    Exponent field 0 is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; there is no infinity.
    """
    u = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (u >> 7) & 1
    exp = (u >> 3) & 0xF
    man = u & 0x7
    mag = np.where(exp == 0, (man / 8.0) * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def dequantize(codes, scale) -> np.ndarray:
    """Rows of fp8 codes times their per-row scale."""
    return _f64(scale)[..., None] * e4m3fn_decode(codes)


def pooled_reps(keys, block: int) -> np.ndarray:
    """Mean of each block's valid keys: keys [L][d] (valid rows only) -> [ceil(L/block)][d]."""
    keys = _f64(keys)
    L = keys.shape[0]
    nb = -(-L // block)
    reps = np.empty((nb, keys.shape[1]))
    for b in range(nb):
        reps[b] = keys[b * block: min((b + 1) * block, L)].mean(axis=0)
    return reps


def indexer_scores(q, w, x) -> np.ndarray:
    """sum_h w_h * ReLU(q_h . x_t) for every row x_t."""
    q = _f64(q)
    w = _f64(w)
    x = _f64(x)
    total = np.zeros(x.shape[0])
    for h in range(q.shape[0]):
        total += w[h] * np.maximum(x @ q[h], 0.0)
    return total


def top_largest(scores, ids, k: int) -> np.ndarray:
    """First min(k, n) ids in (score descending, id ascending) order, returned ascending."""
    s = _f64(scores)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -s))
    return np.sort(ids[order[:k]])


def select(q8, q_scale, w, k8, k_scale, seq_len: int, block: int, keep_blocks: int,
           top_k: int) -> Dict[str, np.ndarray]:
    """HISA selection for one query from raw fp8 inputs."""
    q = dequantize(q8, q_scale)
    keys = dequantize(np.asarray(k8)[:seq_len], np.asarray(k_scale)[:seq_len])
    reps = pooled_reps(keys, block)
    S = indexer_scores(q, w, reps)
    blocks = top_largest(S, np.arange(reps.shape[0]), keep_blocks)
    cand = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    cand = cand[cand < seq_len]
    s = indexer_scores(q, w, keys[cand])
    sel = top_largest(s, cand, top_k)
    return dict(reps=reps, block_scores=S, blocks=blocks, cand=cand, token_scores=s, sel=sel)


def prefill_select(q8, q_scale, w, k8, k_scale, cache_len: int, q_len: int, block: int,
                   keep_blocks: int, top_k: int) -> Dict[str, np.ndarray]:
    """HISA selection for one query row of a prefill chunk [HISA abstract: the
    indexer's per-layer O(L^2) case, where every query scans its whole prefix].

    The index-key cache holds cache_len rows; the row sits at position q_len - 1 and
    sees only tokens t < q_len, in both stages.  Coarse stage: a block wholly inside
    the prefix is represented by the mean of all its rows (what pooling the shared
    cache gives); the row's last block, when only partly visible, by the mean of its
    visible rows t < q_len alone.  So no key after the row's position enters its
    selection, and the row selects what a decode query with a sequence of q_len
    tokens would.  Fine stage: the indexer on the kept blocks' tokens t < q_len.
    """
    q = dequantize(q8, q_scale)
    keys = dequantize(np.asarray(k8)[:cache_len], np.asarray(k_scale)[:cache_len])
    n_full = q_len // block                          # blocks wholly visible to the row
    reps = pooled_reps(keys, block)[:n_full]
    if q_len % block:                                # the row's partly visible last block
        partial = keys[n_full * block:q_len].mean(axis=0)
        reps = np.concatenate([reps, partial[None, :]], axis=0)
    S = indexer_scores(q, w, reps)
    blocks = top_largest(S, np.arange(reps.shape[0]), keep_blocks)
    cand = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    cand = cand[cand < q_len]
    s = indexer_scores(q, w, keys[cand])
    sel = top_largest(s, cand, top_k)
    return dict(reps=reps, block_scores=S, blocks=blocks, cand=cand, token_scores=s, sel=sel)


def flat_select(q8, q_scale, w, k8, k_scale, seq_len: int, top_k: int) -> np.ndarray:
    """The flat DSA-style indexer: exact top-k over every valid token."""
    q = dequantize(q8, q_scale)
    keys = dequantize(np.asarray(k8)[:seq_len], np.asarray(k_scale)[:seq_len])
    return top_largest(indexer_scores(q, w, keys), np.arange(seq_len), top_k)


def iou(a, b) -> float:
    a = np.asarray(a)
    b = np.asarray(b)
    union = np.union1d(a, b).size
    return 1.0 if union == 0 else np.intersect1d(a, b).size / union
