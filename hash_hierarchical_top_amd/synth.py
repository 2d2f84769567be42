"""Seeded synthetic inputs for hierarchical hash retrieval decode.

This module only draws random inputs and stores them in the formats the
kernels read (f32, bf16 bit patterns, OCP fp8 e4m3fn bytes).  It holds none of
the method's arithmetic: no projection, no code, no bound, no selection and no
attention.  Both the HIP path (through the Python binding) and the CPU oracle
consume what it returns.

Workload shapes follow the Llama-3.1-8B row of the HHR appendix model table
(32 query heads, 8 KV heads, hidden 4096, so head_dim 128, max context 131072)
and the HISA abstract's 128K indexer setting.  The value recipe:

* keys  ~ N(0, 1) per channel, with 4 seeded "outlier" channels per KV head
  multiplied by 8 (the uneven per-dimension magnitudes that HHR's Figure 3
  shows for real keys);
* values ~ N(0, 1);
* each query head of a GQA group is 0.5 * (sum of 8 planted keys) / sqrt(8)
  plus N(0, 0.5^2) noise (0.5 is the standard deviation); the 8 planted keys
  sit at distinct seeded positions of that (sequence, KV head);
* R_h: a Haar-random orthogonal 128x128 matrix (QR of a Gaussian in fp64,
  columns multiplied by the sign of diag(R)), stored as f32;
* W_h: a Gaussian 128 x code_bits matrix, f32;
* bf16 workloads store K and V as bf16 (round to nearest even) and round q to
  bf16-representable values (q stays an f32 array).

All draws come from numpy's PCG64 generator with an explicit seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
CODE_BITS = 128
PAGE_SIZE = 16


# --------------------------------------------------------------------------- #
# storage formats
# --------------------------------------------------------------------------- #
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the f32 values they denote (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """f32 array whose values are the bf16 roundings of ``x``."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def f32_to_e4m3fn_bytes(x: np.ndarray) -> np.ndarray:
    """Encode f32 values as OCP fp8 e4m3fn bytes: saturate to +-448, round to nearest even.

    The rounding itself is torch's CPU float8_e4m3fn conversion; values are
    clamped first because that conversion maps overflow to NaN.
    """
    import torch

    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def kv_values(store: np.ndarray, kv_dtype: str) -> np.ndarray:
    """The f32 values held by a K or V storage array (bf16 bits or f32)."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f32(store)
    if kv_dtype == "f32":
        return np.asarray(store, dtype=np.float32)
    raise ValueError(kv_dtype)


# --------------------------------------------------------------------------- #
# HHR decode workloads
# --------------------------------------------------------------------------- #
@dataclasses.dataclass(frozen=True)
class HHRWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    max_ctx: int
    kv_dtype: str                 # "f32" or "bf16"
    keep_num: int                 # kept pages P = min(Np, max(1, ceil(keep_num*Np/keep_den)))
    keep_den: int
    keep_pages_abs: int           # > 0 overrides the ratio
    top_k: int
    seed: int
    min_len: Optional[int] = None  # ragged lengths ~ U{min_len..max_ctx}; None -> all max_ctx
    fixed_len: Optional[int] = None  # every sequence this long (a partly filled cache)
    head_dim: int = HEAD_DIM
    code_bits: int = CODE_BITS
    page_size: int = PAGE_SIZE


WORKLOADS: Dict[str, HHRWorkload] = {
    # tiny fp32 single decode step, 4K context
    "tiny_f32_4k": HHRWorkload("tiny_f32_4k", 1, 4, 1, 4096, "f32", 0, 1, 64, 256, 1000),
    # Llama-3.1-8B-shaped single-layer decode, 32K context, keep 25% of pages
    "llama8b_32k": HHRWorkload("llama8b_32k", 1, 32, 8, 32768, "bf16", 1, 4, 0, 2048, 1001),
    # same shape at 128K context, keep 12.5% of pages
    "llama8b_128k": HHRWorkload("llama8b_128k", 1, 32, 8, 131072, "bf16", 1, 8, 0, 4096, 1002),
    # same shape at 64K context (a test size between the two: 4096 pages per KV head)
    "llama8b_64k": HHRWorkload("llama8b_64k", 1, 32, 8, 65536, "bf16", 1, 8, 0, 4096, 1005),
    # a 16K sequence in a 128K cache (the one-launch path on a partly filled cache: only
    # the sequence's own pages are read), keep 25% of pages
    "llama8b_16k_in_128k": HHRWorkload("llama8b_16k_in_128k", 1, 32, 8, 131072, "bf16", 1, 4, 0,
                                       2048, 1006, fixed_len=16384),
    # batched ragged decode, 16 sequences of 8K..64K
    "llama8b_ragged_b16": HHRWorkload("llama8b_ragged_b16", 16, 32, 8, 65536, "bf16", 1, 4, 0,
                                      2048, 1003, min_len=8192),
}


def seq_lens_for(w: HHRWorkload) -> np.ndarray:
    """Per-sequence context lengths (seeded; ragged when min_len is set)."""
    if w.fixed_len is not None:
        return np.full(w.batch, w.fixed_len, dtype=np.int32)
    if w.min_len is None:
        return np.full(w.batch, w.max_ctx, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(w.seed + 7919))
    return rng.integers(w.min_len, w.max_ctx, size=w.batch, endpoint=True).astype(np.int32)


def random_orthogonal(rng: np.random.Generator, n: int) -> np.ndarray:
    """Haar-random orthogonal n x n matrix, fp64 (QR of a Gaussian, sign-fixed)."""
    a = rng.standard_normal((n, n))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def make_hhr_inputs(batch: int, n_q_heads: int, n_kv_heads: int, seq_lens: Sequence[int],
                    max_ctx: int, kv_dtype: str, seed: int, head_dim: int = HEAD_DIM,
                    code_bits: int = CODE_BITS, n_planted: int = 8, n_outliers: int = 4,
                    outlier_scale: float = 8.0, q_signal: float = 0.5, q_noise: float = 0.5,
                    make_v: bool = True) -> Dict[str, np.ndarray]:
    """Draw one decode workload.

    Returns a dict with
      K, V      [B][Hkv][max_ctx][d]  uint16 bf16 bits or float32 (rows >= seq_len are 0)
      q         [B][Hq][d]            float32
      R         [Hkv][d][d]           float32 (orthogonal)
      W         [Hkv][d][code_bits]   float32
      seq_len   [B]                   int32
      planted   [B][Hkv][n_planted]   int32 positions of the planted keys
      outliers  [Hkv][n_outliers]     int32 outlier channels
    """
    assert n_q_heads % n_kv_heads == 0
    assert kv_dtype in ("f32", "bf16")
    G = n_q_heads // n_kv_heads
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,) and int(seq_lens.max()) <= max_ctx
    rng = np.random.Generator(np.random.PCG64(seed))

    R = np.stack([random_orthogonal(rng, head_dim) for _ in range(n_kv_heads)]).astype(np.float32)
    W = rng.standard_normal((n_kv_heads, head_dim, code_bits)).astype(np.float32)
    outliers = np.stack([rng.choice(head_dim, n_outliers, replace=False)
                         for _ in range(n_kv_heads)]).astype(np.int32)
    chan_scale = np.ones((n_kv_heads, head_dim), dtype=np.float32)
    for g in range(n_kv_heads):
        chan_scale[g, outliers[g]] = outlier_scale

    sdt = np.uint16 if kv_dtype == "bf16" else np.float32
    K = np.zeros((batch, n_kv_heads, max_ctx, head_dim), dtype=sdt)
    V = np.zeros((batch, n_kv_heads, max_ctx, head_dim), dtype=sdt) if make_v else None
    q = np.empty((batch, n_q_heads, head_dim), dtype=np.float32)
    planted = np.empty((batch, n_kv_heads, n_planted), dtype=np.int32)

    def store(x):
        return f32_to_bf16_bits(x) if kv_dtype == "bf16" else x

    for b in range(batch):
        L = int(seq_lens[b])
        for g in range(n_kv_heads):
            k = rng.standard_normal((L, head_dim), dtype=np.float32) * chan_scale[g][None, :]
            K[b, g, :L] = store(k)
            if make_v:
                V[b, g, :L] = store(rng.standard_normal((L, head_dim), dtype=np.float32))
            if L >= n_planted:
                pos = np.sort(rng.choice(L, n_planted, replace=False)).astype(np.int32)
            else:
                pos = np.arange(n_planted, dtype=np.int32) % max(L, 1)
            planted[b, g] = pos
            kv = kv_values(K[b, g, pos], kv_dtype).astype(np.float32) if L > 0 else \
                np.zeros((n_planted, head_dim), np.float32)
            signal = q_signal * kv.sum(0) / math.sqrt(n_planted)
            for j in range(G):
                noise = rng.normal(0.0, q_noise, head_dim).astype(np.float32)
                q[b, g * G + j] = (signal + noise).astype(np.float32)
    if kv_dtype == "bf16":
        q = round_to_bf16(q)
    out = dict(K=K, q=q, R=R, W=W, seq_len=seq_lens, planted=planted, outliers=outliers)
    if make_v:
        out["V"] = V
    return out


def make_workload_inputs(name: str, make_v: bool = True,
                         code_bits: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of a named workload; code_bits overrides its projection width."""
    w = WORKLOADS[name]
    return make_hhr_inputs(w.batch, w.n_q_heads, w.n_kv_heads, seq_lens_for(w), w.max_ctx,
                           w.kv_dtype, w.seed, w.head_dim,
                           w.code_bits if code_bits is None else code_bits, make_v=make_v)


# --------------------------------------------------------------------------- #
# HISA indexer workload (block-pooled coarse filter over a DSA-style indexer)
# --------------------------------------------------------------------------- #
@dataclasses.dataclass(frozen=True)
class HISAWorkload:
    name: str
    n_index_heads: int
    ctx: int
    block: int
    keep_blocks: int
    top_k: int
    n_attn_heads: int
    seed: int
    head_dim: int = HEAD_DIM


HISA_WORKLOADS: Dict[str, HISAWorkload] = {
    # 64 index heads x 128 dims, 131072 fp8 index keys in 1024 blocks of 128, top 64 blocks,
    # token top-2048, then 16 attention heads on one bf16 KV head
    "hisa_128k": HISAWorkload("hisa_128k", 64, 131072, 128, 64, 2048, 16, 1004),
}


# Prefill chunks for the HISA indexer: `rows` query rows (index-query draws of their own)
# at positions spread evenly over the context of a decode workload's shared cache, so the
# mean row sees half the context, as over a whole prefill.
HISA_PREFILL_WORKLOADS: Dict[str, Tuple[str, int]] = {
    "hisa_prefill_128k": ("hisa_128k", 512),
}


def make_hisa_prefill_rows(name: str, ctx: int = 0) -> Dict[str, np.ndarray]:
    """q8 [M][Hi][d], q_scale [M][Hi], w [M][Hi] and q_len [M]: the rows' positions + 1,
    drawn uniformly over [1, ctx] (seeded, ascending; the last row is the prompt's last
    token), so most rows end inside a block; ctx defaults to the workload's."""
    base, rows = HISA_PREFILL_WORKLOADS[name]
    w = HISA_WORKLOADS[base]
    ctx = ctx or w.ctx
    parts = [make_hisa_inputs(w.n_index_heads, 1, 16, 0, w.seed + 1000 + r, w.head_dim,
                              block=16, make_kv=False) for r in range(rows)]
    rng = np.random.Generator(np.random.PCG64(w.seed + 999))
    q_len = np.sort(rng.integers(1, ctx + 1, rows)).astype(np.int32)
    q_len[-1] = ctx
    return dict(q8=np.stack([x["q8"] for x in parts]),
                q_scale=np.stack([x["q_scale"] for x in parts]),
                w=np.stack([x["w"] for x in parts]), q_len=q_len)


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row symmetric fp8 e4m3fn storage: scale = amax/448, bytes = e4m3(x/scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = f32_to_e4m3fn_bytes(x / scale[..., None])
    return codes, scale


def make_hisa_inputs(n_index_heads: int, ctx: int, max_ctx: int, n_attn_heads: int, seed: int,
                     head_dim: int = HEAD_DIM, planted_blocks: int = 0, block: int = 128,
                     make_kv: bool = True) -> Dict[str, np.ndarray]:
    """Draw one HISA decode workload.

    Returns
      q8 [Hi][d] uint8 (e4m3fn), q_scale [Hi] f32, w [Hi] f32 ~ U(0,1)
      k8 [max_ctx][d] uint8, k_scale [max_ctx] f32 (rows >= ctx are 0 / scale 0)
      q_attn [Ha][d] f32 (bf16-representable), K, V [1][max_ctx][d] uint16 bf16 bits
      seq_len [1] int32
    With planted_blocks > 0, that many seeded blocks get keys correlated with the
    index queries' mean direction (a variant with meaningful recall).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    qf = rng.standard_normal((n_index_heads, head_dim), dtype=np.float32)
    w = rng.uniform(0.0, 1.0, n_index_heads).astype(np.float32)
    kf = rng.standard_normal((ctx, head_dim), dtype=np.float32)
    if planted_blocks > 0:
        nb = (ctx + block - 1) // block
        blocks = rng.choice(nb, planted_blocks, replace=False)
        direction = qf.mean(0)
        direction /= np.linalg.norm(direction)
        for blk in blocks:
            lo, hi = blk * block, min((blk + 1) * block, ctx)
            kf[lo:hi] += 2.0 * direction[None, :] * np.sqrt(head_dim) / 4.0
    q8, q_scale = quantize_rows_e4m3(qf)
    k8 = np.zeros((max_ctx, head_dim), dtype=np.uint8)
    k_scale = np.zeros(max_ctx, dtype=np.float32)
    k8[:ctx], k_scale[:ctx] = quantize_rows_e4m3(kf)
    out = dict(q8=q8, q_scale=q_scale, w=w, k8=k8, k_scale=k_scale,
               seq_len=np.array([ctx], dtype=np.int32))
    if make_kv:
        out["q_attn"] = round_to_bf16(rng.standard_normal((n_attn_heads, head_dim),
                                                          dtype=np.float32))
        K = np.zeros((1, 1, max_ctx, head_dim), dtype=np.uint16)
        V = np.zeros((1, 1, max_ctx, head_dim), dtype=np.uint16)
        K[0, 0, :ctx] = f32_to_bf16_bits(rng.standard_normal((ctx, head_dim), dtype=np.float32))
        V[0, 0, :ctx] = f32_to_bf16_bits(rng.standard_normal((ctx, head_dim), dtype=np.float32))
        out["K"], out["V"] = K, V
    return out


def make_hisa_workload_inputs(name: str, planted_blocks: int = 0, make_kv: bool = True):
    w = HISA_WORKLOADS[name]
    return make_hisa_inputs(w.n_index_heads, w.ctx, w.ctx, w.n_attn_heads, w.seed, w.head_dim,
                            planted_blocks=planted_blocks, block=w.block, make_kv=make_kv)


def small_hhr_cases() -> List[dict]:
    """Parity cases the oracle finishes in seconds: several tiles, ragged tails, GQA 1/4/8."""
    return [
        dict(name="f32_g4_ragged", batch=2, n_q_heads=4, n_kv_heads=1, seq_lens=[1000, 4096],
             max_ctx=4096, kv_dtype="f32", seed=11, keep_num=0, keep_den=1, keep_abs=64,
             top_k=256),
        dict(name="bf16_g4_ragged", batch=3, n_q_heads=8, n_kv_heads=2, seq_lens=[5003, 1, 2049],
             max_ctx=6144, kv_dtype="bf16", seed=12, keep_num=1, keep_den=4, keep_abs=0,
             top_k=512),
        dict(name="bf16_g1", batch=1, n_q_heads=2, n_kv_heads=2, seq_lens=[3000], max_ctx=3008,
             kv_dtype="bf16", seed=13, keep_num=3, keep_den=8, keep_abs=0, top_k=300),
        dict(name="bf16_g8_bigk", batch=2, n_q_heads=16, n_kv_heads=2, seq_lens=[700, 333],
             max_ctx=1024, kv_dtype="bf16", seed=14, keep_num=1, keep_den=2, keep_abs=0,
             top_k=4096),
    ]


def small_code_bits_cases() -> List[dict]:
    """Parity cases at the other code widths: 64 bits, and 256 bits with G = 16 (the
    largest summed distance, 4096) and with top_k above the candidate count."""
    return [
        dict(name="bf16_g4_c64", batch=3, n_q_heads=8, n_kv_heads=2, seq_lens=[5003, 1, 2049],
             max_ctx=6144, kv_dtype="bf16", seed=21, keep_num=1, keep_den=4, keep_abs=0,
             top_k=512, code_bits=64),
        dict(name="f32_g16_c256", batch=2, n_q_heads=16, n_kv_heads=1, seq_lens=[3000, 777],
             max_ctx=3008, kv_dtype="f32", seed=22, keep_num=0, keep_den=1, keep_abs=48,
             top_k=300, code_bits=256),
        dict(name="bf16_g8_c256_bigk", batch=2, n_q_heads=16, n_kv_heads=2,
             seq_lens=[700, 333], max_ctx=1024, kv_dtype="bf16", seed=23, keep_num=1,
             keep_den=2, keep_abs=0, top_k=4096, code_bits=256),
    ]
