"""Helpers for the GPU parity tests: device uploads of generated inputs, the
HIP pipeline run stage by stage through the C ABI, and the excused-mismatch
accounting that compares it with the oracle.

Excuse bands (the only places where GPU and oracle may differ in a discrete
result, both coming from fp32 vs fp64 rounding):
  * a code bit j of vector x may differ iff |(xW)_j| <= 1e-4 * sum_d |x_d W_dj|;
  * a kept page may differ iff |s(p) - s_(P)| <= 1e-4 * |s_(P)|, with s the
    oracle's page bound and s_(P) the P-th largest.
Downstream stages are compared against the oracle run on the GPU's own
upstream outputs (conditioned oracle), where results must be exact.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from hash_hierarchical_top_amd import synth
from oracle import hhr as O

CODE_EXCUSE = 1e-4
PAGE_EXCUSE = 1e-4

# Excused mismatches per test, written to a JSON file at the end of the session
# (tests/conftest.py): {test name: {counter: total}}.
EXCUSED: dict = {}


def record_excused(name: str, **counts) -> None:
    """Adds counts of excused mismatches (code bits, pages, blocks, tokens, ...) under name."""
    rec = EXCUSED.setdefault(name, {})
    for k, v in counts.items():
        rec[k] = rec.get(k, 0) + int(v)


def dev():
    return torch.device("cuda", 0)


def kv_to_device(store: np.ndarray, kv_dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(store))
    if kv_dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(dev())


def upload_hhr(inp: dict, kv_dtype: str) -> dict:
    d = {
        "K": kv_to_device(inp["K"], kv_dtype),
        "q": torch.from_numpy(inp["q"]).to(dev()),
        "R": torch.from_numpy(inp["R"]).to(dev()),
        "W": torch.from_numpy(inp["W"]).to(dev()),
        "seq_len": torch.from_numpy(inp["seq_len"].astype(np.int32)).to(dev()),
    }
    if "V" in inp:
        d["V"] = kv_to_device(inp["V"], kv_dtype)
    return d


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


class Pipeline:
    """Buffers and stage-by-stage calls of the HIP path for one workload."""

    def __init__(self, H, inp, kv_dtype, n_q_heads, n_kv_heads, max_ctx, keep_num, keep_den,
                 keep_abs, top_k, with_v=True, meta_dtype="f32", code_bits=128):
        self.H = H
        self.inp = inp
        self.kv_dtype = kv_dtype
        B = inp["q"].shape[0]
        self.B, self.Hq, self.Hkv, self.Lcap = B, n_q_heads, n_kv_heads, max_ctx
        self.G = n_q_heads // n_kv_heads
        self.keep = (keep_num, keep_den, keep_abs)
        self.top_k = top_k
        self.meta_dtype = meta_dtype
        self.NW = code_bits // 32
        assert inp["W"].shape[-1] == code_bits
        self.shape = H.make_shape(B, n_q_heads, n_kv_heads, max_ctx, kv_dtype,
                                  code_bits=code_bits, meta_dtype=meta_dtype)
        self.d = upload_hhr(inp if with_v else {k: v for k, v in inp.items() if k != "V"},
                            kv_dtype)
        NpCap = max_ctx // 16
        self.NpCap = NpCap
        self.p_max = H.hhr_keep_count(NpCap, keep_num, keep_den, keep_abs)
        i32 = dict(dtype=torch.int32, device=dev())
        f32 = dict(dtype=torch.float32, device=dev())
        self.codes = torch.zeros((B, n_kv_heads, max_ctx, self.NW), **i32)
        self.meta = torch.zeros(H.meta_shape(self.shape),
                                **(f32 if meta_dtype == "f32" else i32))
        self.q_rot = torch.zeros((B, n_q_heads, 128), **f32)
        self.q_codes = torch.zeros((B, n_q_heads, self.NW), **i32)
        self.scores = torch.full((B, n_kv_heads, NpCap), float("nan"), **f32)
        self.kept = torch.zeros((B, n_kv_heads, self.p_max), **i32)
        self.kept_count = torch.zeros((B, n_kv_heads), **i32)
        self.sel = torch.zeros((B, n_kv_heads, top_k), **i32)
        self.sel_count = torch.zeros((B, n_kv_heads), **i32)
        self.dist = torch.zeros((B, n_kv_heads, self.p_max * 16), dtype=torch.int16, device=dev())
        self.out = torch.zeros((B, n_q_heads, 128), **f32)
        self.ws_bytes = H.hhr_workspace_size(self.shape, keep_num, keep_den, keep_abs, top_k)
        assert self.ws_bytes > 0
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev())
        self.scale = 1.0 / math.sqrt(128.0)

    # ---- stages
    def append_all(self):
        start = torch.zeros(self.B, dtype=torch.int32, device=dev())
        self.H.hhr_append_keys(self.shape, self.d["K"], start, self.d["seq_len"],
                               int(self.inp["seq_len"].max()), self.d["R"], self.d["W"],
                               self.codes, self.meta, self.ws)

    def encode_queries(self):
        self.H.hhr_encode_queries(self.shape, self.d["q"], self.d["R"], self.d["W"], self.q_rot,
                                  self.q_codes)

    def page_scores(self):
        self.H.hhr_page_scores(self.shape, self.q_rot, self.d["seq_len"], self.meta, self.scores,
                               self.ws)

    def top_pages(self):
        self.H.hhr_top_pages(self.shape, self.scores, self.d["seq_len"], *self.keep, self.kept,
                             self.kept_count, self.ws)

    def hamming_topk(self):
        self.H.hhr_hamming_topk(self.shape, self.q_codes, self.codes, self.d["seq_len"],
                                self.kept, self.kept_count, self.p_max, self.top_k, self.sel,
                                self.sel_count, self.dist, self.ws)

    def sparse_decode(self):
        self.H.hhr_sparse_decode(self.shape, self.d["q"], self.d["K"], self.d["V"], self.sel,
                                 self.sel_count, self.top_k, self.scale, self.out, self.ws)

    def decode(self, sel, sel_count, out):
        self.H.hhr_decode(self.shape, self.d["q"], self.d["seq_len"], self.d["R"], self.d["W"],
                          self.codes, self.meta, self.d["K"], self.d["V"], *self.keep, self.top_k,
                          self.scale, sel, sel_count, out, self.ws)

    def select_pages(self):
        """hhr_select_pages into fresh buffers (and a workspace of its own)."""
        kept = torch.full_like(self.kept, 12345)
        kc = torch.full_like(self.kept_count, -3)
        qc = torch.zeros_like(self.q_codes)
        ws = torch.zeros(self.H.hhr_workspace_size(self.shape, *self.keep, 1), dtype=torch.uint8,
                         device=dev())
        self.H.hhr_select_pages(self.shape, self.d["q"], self.d["seq_len"], self.d["R"],
                                self.d["W"], self.meta, *self.keep, kept, kc, qc, ws)
        torch.cuda.synchronize()
        assert self.H.hhr_read_device_status(ws) == 0
        return kept, kc, qc

    def select(self):
        """hhr_select into fresh buffers (and a workspace of its own)."""
        sel = torch.full_like(self.sel, 12345)
        sc = torch.full_like(self.sel_count, -3)
        ws = torch.zeros(self.H.hhr_workspace_size(self.shape, *self.keep, self.top_k),
                         dtype=torch.uint8, device=dev())
        self.H.hhr_select(self.shape, self.d["q"], self.d["seq_len"], self.d["R"], self.d["W"],
                          self.codes, self.meta, *self.keep, self.top_k, sel, sc, ws)
        torch.cuda.synchronize()
        assert self.H.hhr_read_device_status(ws) == 0
        return sel, sc

    def status(self):
        return self.H.hhr_read_device_status(self.ws)

    # ---- host views
    def meta_host(self, b, g, Np=None):
        """Page metadata of (b, g) as float64 [Np][128][2] ({min, max}), decoding the
        bfloat16 words of the compressed format."""
        m = self.meta[b, g] if Np is None else self.meta[b, g, :Np]
        if self.meta_dtype == "f32":
            return m.cpu().numpy().astype(np.float64)
        w = m.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        lo = ((w & 0xFFFF) << 16).astype(np.uint32).view(np.float32)
        hi = (w & 0xFFFF0000).astype(np.uint32).view(np.float32)
        return np.stack([lo, hi], axis=-1).astype(np.float64)

    def K_valid(self, b, g):
        L = int(self.inp["seq_len"][b])
        return synth.kv_values(self.inp["K"][b, g, :L], self.kv_dtype).astype(np.float64)

    def V_valid(self, b, g):
        L = int(self.inp["seq_len"][b])
        return synth.kv_values(self.inp["V"][b, g, :L], self.kv_dtype).astype(np.float64)

    def q_group(self, b, g):
        return self.inp["q"][b, g * self.G:(g + 1) * self.G].astype(np.float64)


def check_code_bits(x: np.ndarray, W: np.ndarray, got_words: np.ndarray) -> int:
    """GPU codes of rows x must equal sign(x W) except within the rounding band; returns
    the number of excused mismatching bits."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    Y = x @ W
    scale = np.abs(x) @ np.abs(W)
    want = Y >= 0
    got = O.unpack_bits(got_words)
    mism = want != got
    bad = mism & ~(np.abs(Y) <= CODE_EXCUSE * scale)
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} unexcused code-bit mismatches, e.g. row {r} bit "
                             f"{c}: Y={Y[r, c]!r} scale={scale[r, c]!r} gpu={got[r, c]}")
    return int(mism.sum())


def check_kept_pages(oracle_scores: np.ndarray, P: int, got: np.ndarray) -> int:
    """GPU kept pages may differ from the oracle's only among pages whose oracle bound is
    within the excuse band of the P-th largest; returns the number of excused differences."""
    want = O.top_pages(oracle_scores, P)
    got = np.asarray(got, np.int64)
    assert got.size == P and np.all(np.diff(got) > 0)
    diff = np.setxor1d(want, got)
    if diff.size == 0:
        return 0
    sP = np.sort(oracle_scores)[::-1][P - 1]
    band = PAGE_EXCUSE * abs(sP)
    far = diff[np.abs(oracle_scores[diff] - sP) > band]
    assert far.size == 0, f"kept pages differ outside the excuse band: {far[:8]}"
    return int(diff.size)


def _threshold(H: np.ndarray, k: int) -> int:
    """The k-th smallest value of H (the cut of a top-k by smallest H), or a value above
    every H when there are at most k of them."""
    if H.size <= k:
        return 1 << 30
    return int(np.sort(H)[k - 1])


def explain_selection(res: dict, sel_gpu, kept_gpu, codes_gpu, qcodes_gpu, L: int,
                      top_k: int) -> dict:
    """Every difference between the GPU selection and the oracle's selection from raw
    inputs (res = oracle.hhr.select(...)) must be explained by an excused item: a kept
    page inside the page band; a key whose code differs from the oracle's (bits inside the
    code band, checked by check_code_bits); a query code that differs; or the displacement
    of the top-k cut that such an item causes (a position whose distance lies between the
    GPU's and the oracle's cut).  With no excused item the selections must be identical.
    Returns the counts: excused pages, keys with excused code bits among the candidates,
    query code words, and the differing selected positions by explanation."""
    P = res["n_keep"]
    n_pages = check_kept_pages(res["scores"], P, kept_gpu)
    ex_pages = set(np.setxor1d(res["kept"], kept_gpu).tolist())
    codes_or = res["enc"]["codes"]
    key_mis = np.flatnonzero(np.any(np.asarray(codes_gpu)[:L] != codes_or[:L], axis=-1))
    cand_gpu = O.candidates(np.asarray(kept_gpu, np.int64), L, 16)
    cand_or = res["cand"]
    ex_keys = set(key_mis.tolist()) & (set(cand_gpu.tolist()) | set(cand_or.tolist()))
    q_mis = int(np.sum(np.asarray(qcodes_gpu) != res["qcodes"]))
    H_gpu = O.hamming(qcodes_gpu, np.asarray(codes_gpu)[cand_gpu])
    hg = dict(zip(cand_gpu.tolist(), H_gpu.tolist()))
    ho = dict(zip(cand_or.tolist(), res["H"].tolist()))
    T_lo, T_hi = sorted((_threshold(H_gpu, top_k), _threshold(res["H"], top_k)))
    any_excused = bool(ex_pages) or bool(ex_keys) or q_mis > 0
    diff = np.setxor1d(np.asarray(sel_gpu, np.int64), res["sel"])
    counts = dict(pages=n_pages, key_codes=len(ex_keys), query_code_words=q_mis,
                  sel_diff=int(diff.size), by_page=0, by_key_code=0, by_query_code=0,
                  by_cut=0)
    if not any_excused:
        assert diff.size == 0, f"selection differs with nothing excused: {diff[:8]}"
        return counts
    for t in diff.tolist():
        if t // 16 in ex_pages:
            counts["by_page"] += 1
        elif t in ex_keys:
            counts["by_key_code"] += 1
        elif q_mis:
            counts["by_query_code"] += 1
        elif any(T_lo <= h.get(t, -1) <= T_hi for h in (hg, ho)):
            counts["by_cut"] += 1
        else:
            raise AssertionError(f"unexplained selection difference at position {t}: H gpu "
                                 f"{hg.get(t)}, oracle {ho.get(t)}, cuts {T_lo}..{T_hi}")
    return counts
