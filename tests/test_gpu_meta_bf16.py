"""GPU parity of the bfloat16 page-metadata format (meta_dtype = HHR_BF16) through the
C ABI: the small seeded cases and the 128K Llama-3.1-8B-shaped decode step.

- The stored words are the f32 metadata of the same encoder rounded outward (min
  toward -inf, max toward +inf), bit for bit, and lie within one bfloat16 step of
  the oracle's outward-rounded exact min/max.
- Page bounds equal the oracle's bound recomputed from the GPU's own decoded
  metadata and rotated queries, and are never below the f32-metadata bounds.
- Top-P on those bounds is exact; the kept pages from raw inputs are a valid top-P
  for some value of every bound inside the interval that the rounding allows.
- hhr_decode (eager and replayed from a HIP graph) equals the stage-by-stage run.
"""
import numpy as np
import pytest
import torch

from hash_hierarchical_top_amd import synth
from oracle import hhr as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = synth.small_hhr_cases()
META_TOL = 3e-5  # f32 metadata error of the encoder, relative to sum_d |k_d R_dj|


def _run_pipeline(H, inp, w, meta_dtype):
    p = U.Pipeline(H, inp, w["kv_dtype"], w["n_q_heads"], w["n_kv_heads"], w["max_ctx"],
                   w["keep_num"], w["keep_den"], w["keep_abs"], w["top_k"],
                   meta_dtype=meta_dtype)
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    return p


def _case_params():
    out = [(c["name"], c) for c in CASES]
    w = synth.WORKLOADS["llama8b_128k"]
    out.append(("llama8b_128k", dict(kv_dtype=w.kv_dtype, n_q_heads=w.n_q_heads,
                                     n_kv_heads=w.n_kv_heads, max_ctx=w.max_ctx,
                                     keep_num=w.keep_num, keep_den=w.keep_den,
                                     keep_abs=w.keep_pages_abs, top_k=w.top_k)))
    return out


PARAMS = _case_params()


@pytest.fixture(scope="module", params=PARAMS, ids=[n for n, _ in PARAMS])
def pair(request, gpu_lib):
    """The same inputs through the bf16-metadata and the f32-metadata pipelines."""
    name, w = request.param
    print(f"\n[gpu bf16-metadata case] {name}", flush=True)
    if name == "llama8b_128k":
        inp = synth.make_workload_inputs(name)
    else:
        inp = synth.make_hhr_inputs(w["batch"], w["n_q_heads"], w["n_kv_heads"], w["seq_lens"],
                                    w["max_ctx"], w["kv_dtype"], w["seed"])
    p16 = _run_pipeline(gpu_lib, inp, w, "bf16")
    p32 = _run_pipeline(gpu_lib, inp, w, "f32")
    torch.cuda.synchronize()
    assert p16.status() == 0 and p32.status() == 0
    if p16.B == 1 and p16.Hkv > 2:
        pairs = [(0, g) for g in sorted({0, p16.Hkv // 2, p16.Hkv - 1})]
    else:
        pairs = [(b, g) for b in range(p16.B) for g in range(p16.Hkv)]
    return name, p16, p32, pairs


def _bf16_words(meta64):
    """{min, max} float64 values that are bfloat16-representable -> packed uint32 words."""
    f = meta64.astype(np.float32).view(np.uint32)
    return (f[..., 0] >> 16) | (f[..., 1] & 0xFFFF0000)


def _ab(qr):
    return np.maximum(qr, 0).sum(0), np.minimum(qr, 0).sum(0)


def test_meta_words_are_f32_meta_rounded_outward(pair):
    name, p16, p32, pairs = pair
    for b, g in pairs:
        Np = O.n_pages(int(p16.inp["seq_len"][b]), 16)
        got = p16.meta[b, g, :Np].cpu().numpy().view(np.uint32)
        f32 = p32.meta_host(b, g, Np)
        want = _bf16_words(O.bf16_outward(f32))
        assert np.array_equal(got, want), (b, g, np.argwhere(got != want)[:4])


def test_meta_within_one_rounding_of_exact(pair):
    name, p16, p32, pairs = pair
    rng = np.random.Generator(np.random.PCG64(3))
    for b, g in pairs:
        L = int(p16.inp["seq_len"][b])
        Np = O.n_pages(L, 16)
        K = p16.K_valid(b, g)
        R = p16.inp["R"][g].astype(np.float64)
        meta = p16.meta_host(b, g, Np)
        pages = np.unique(np.concatenate([rng.choice(Np, min(Np, 256), replace=False),
                                          [0, Np - 1]]))
        for pg in pages:
            Kp = K[pg * 16:min(L, pg * 16 + 16)]
            ex = O.page_minmax(O.rotate(Kp, R), 16)[0]
            tol = META_TOL * (np.abs(Kp) @ np.abs(R)).max()
            mn, mx = meta[pg, :, 0], meta[pg, :, 1]
            assert np.all(O.bf16_round(ex[:, 0] - tol, up=False) <= mn)
            assert np.all(mn <= O.bf16_round(ex[:, 0] + tol, up=False))
            assert np.all(O.bf16_round(ex[:, 1] - tol, up=True) <= mx)
            assert np.all(mx <= O.bf16_round(ex[:, 1] + tol, up=True))


def test_page_scores_conditioned_and_not_below_f32(pair):
    name, p16, p32, pairs = pair
    for b, g in pairs:
        Np = O.n_pages(int(p16.inp["seq_len"][b]), 16)
        if Np == 0:
            continue
        qr = p16.q_rot[b, g * p16.G:(g + 1) * p16.G].cpu().numpy().astype(np.float64)
        meta = p16.meta_host(b, g, Np)
        got = p16.scores[b, g, :Np].cpu().numpy().astype(np.float64)
        want = O.page_scores(qr, meta)
        mag = (np.abs(qr).sum(0)[None, :] * np.abs(meta).max(-1)).sum(-1)
        assert np.all(np.abs(got - want) <= 1e-5 * mag + 1e-30)
        s32 = p32.scores[b, g, :Np].cpu().numpy().astype(np.float64)
        assert np.all(got >= s32 - 2e-5 * mag)


def test_top_pages_conditioned_exact(pair):
    name, p16, p32, pairs = pair
    for b, g in pairs:
        Np = O.n_pages(int(p16.inp["seq_len"][b]), 16)
        P = O.keep_count(Np, *p16.keep)
        assert int(p16.kept_count[b, g]) == P
        s = p16.scores[b, g, :Np].cpu().numpy().astype(np.float64)
        assert p16.kept[b, g, :P].cpu().tolist() == O.top_pages(s, P).tolist()


def test_kept_pages_valid_within_rounding_intervals(pair):
    """From raw inputs: every bound lies in [s_lo, s_hi], the range its metadata can take
    once the encoder's f32 error moves a value across a bfloat16 grid point; the GPU's kept
    pages must be a top-P for some choice of bounds in those ranges."""
    name, p16, p32, pairs = pair
    for b, g in pairs[:3]:
        L = int(p16.inp["seq_len"][b])
        Np = O.n_pages(L, 16)
        if Np == 0:
            continue
        K = p16.K_valid(b, g)
        R = p16.inp["R"][g].astype(np.float64)
        ex = O.page_minmax(O.rotate(K, R), 16)
        rowscale = (np.abs(K) @ np.abs(R)).max(1)
        pad = np.full(Np * 16, 0.0)
        pad[:L] = rowscale
        tol = META_TOL * pad.reshape(Np, 16).max(1)[:, None]
        mn_lo = O.bf16_round(ex[..., 0] - tol, up=False)
        mn_hi = O.bf16_round(ex[..., 0] + tol, up=False)
        mx_lo = O.bf16_round(ex[..., 1] - tol, up=True)
        mx_hi = O.bf16_round(ex[..., 1] + tol, up=True)
        A, Bn = _ab(O.rotate(p16.q_group(b, g), R))
        mag = (A + np.abs(Bn)) @ np.maximum(np.abs(mn_lo), np.abs(mx_hi)).T
        s_hi = mx_hi @ A + mn_lo @ Bn + 2e-5 * mag
        s_lo = mx_lo @ A + mn_hi @ Bn - 2e-5 * mag
        P = O.keep_count(Np, *p16.keep)
        got = p16.kept[b, g, :P].cpu().numpy().astype(np.int64)
        assert got.size == P and np.all(np.diff(got) > 0) and got.max() < Np
        out = np.setdiff1d(np.arange(Np), got)
        # a kept page could not be beaten by P others; a dropped one could not beat P kept
        if out.size:
            assert np.all(s_hi[got] >= np.sort(s_lo)[::-1][P - 1])
            assert np.all(s_lo[out] <= np.sort(s_hi)[::-1][P - 1])


def test_select_pages_equals_stages(pair):
    name, p16, p32, pairs = pair
    kept, kc, qc = p16.select_pages()
    assert torch.equal(kept, p16.kept) and torch.equal(kc, p16.kept_count)
    assert torch.equal(qc, p16.q_codes)


def test_selection_and_attention_conditioned(pair):
    name, p16, p32, pairs = pair
    atol = 1e-5 if p16.kv_dtype == "f32" else 2e-3
    for b, g in pairs:
        L = int(p16.inp["seq_len"][b])
        P = int(p16.kept_count[b, g])
        res = O.select_from_codes(U.u32(p16.q_codes)[b, g * p16.G:(g + 1) * p16.G],
                                  U.u32(p16.codes)[b, g], p16.kept[b, g, :P].cpu().numpy(), L,
                                  16, p16.top_k)
        n = len(res["sel"])
        assert int(p16.sel_count[b, g]) == n
        idx = p16.sel[b, g, :n].cpu().numpy()
        assert idx.tolist() == res["sel"].tolist()
        K = synth.kv_values(p16.inp["K"][b, g, idx], p16.kv_dtype).astype(np.float64)
        V = synth.kv_values(p16.inp["V"][b, g, idx], p16.kv_dtype).astype(np.float64)
        want = O.attend(p16.q_group(b, g), K, V, p16.scale)
        got = p16.out[b, g * p16.G:(g + 1) * p16.G].cpu().numpy().astype(np.float64)
        assert np.abs(got - want).max() <= atol


def test_decode_and_graph_replays_equal_stages(pair):
    name, p16, p32, pairs = pair
    p = p16
    sel = torch.zeros_like(p.sel)
    sc = torch.zeros_like(p.sel_count)
    out = torch.zeros_like(p.out)
    p.decode(sel, sc, out)
    torch.cuda.synchronize()
    assert torch.equal(sel, p.sel) and torch.equal(sc, p.sel_count) and torch.equal(out, p.out)
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        p.decode(sel, sc, out)
    torch.cuda.current_stream().wait_stream(gs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        p.decode(sel, sc, out)
    for i in range(2):
        out.fill_(float(i + 1))
        sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, p.sel) and torch.equal(sc, p.sel_count)
        assert torch.equal(out, p.out), f"replay {i}"
    assert p.status() == 0


def test_chunked_append_equals_one_shot(gpu_lib):
    """Rounding happens per write, from the page's full f32 min/max, so appending in
    pieces gives the same words as appending at once."""
    c = CASES[1]
    inp = synth.make_hhr_inputs(c["batch"], c["n_q_heads"], c["n_kv_heads"], c["seq_lens"],
                                c["max_ctx"], c["kv_dtype"], c["seed"])
    p = U.Pipeline(gpu_lib, inp, c["kv_dtype"], c["n_q_heads"], c["n_kv_heads"], c["max_ctx"],
                   c["keep_num"], c["keep_den"], c["keep_abs"], c["top_k"], with_v=False,
                   meta_dtype="bf16")
    p.append_all()
    meta1 = p.meta.clone()
    p.meta.zero_()
    lens = p.inp["seq_len"].astype(np.int64)
    pts = np.stack([np.maximum.accumulate(np.clip([0, 37, 1000, L - 2, L - 1, L], 0, L))
                    for L in lens])
    for i in range(pts.shape[1] - 1):
        a, z = pts[:, i], pts[:, i + 1]
        start = torch.from_numpy(a.astype(np.int32)).cuda()
        n_new = torch.from_numpy((z - a).astype(np.int32)).cuda()
        gpu_lib.hhr_append_keys(p.shape, p.d["K"], start, n_new, int((z - a).max()), p.d["R"],
                                p.d["W"], p.codes, p.meta, p.ws)
    torch.cuda.synchronize()
    for b in range(p.B):
        Np = O.n_pages(int(lens[b]), 16)
        assert torch.equal(p.meta[b, :, :Np], meta1[b, :, :Np])
