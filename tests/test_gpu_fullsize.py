"""GPU parity at the full workload sizes, on sampled outputs the oracle computes one
by one: the 4K f32 single-head case, the 32K, 64K and 128K Llama-3.1-8B-shaped
decode steps (the 128K one as bench.py times it) and the 16-sequence ragged
batch.  The coarse launch scores 64, 128 and 256 pages per workgroup at 32K,
64K and 128K respectively.

For a few sampled (sequence, KV head) pairs: key codes and page metadata of
sampled keys and pages, the query encoding, every page bound (conditioned on
the GPU's metadata and rotated queries), the exact top-P and top-k selections
(conditioned), the selection from raw inputs within the excuse band, and the
attention output over the GPU's selection.  hhr_decode, eager and replayed
from a HIP graph, must equal the stage-by-stage run bit for bit.
"""
import numpy as np
import pytest
import torch

from hash_hierarchical_top_amd import synth
from oracle import hhr as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny_f32_4k", "llama8b_32k", "llama8b_64k", "llama8b_128k", "llama8b_ragged_b16"]


def _pairs(w, seq_len):
    """Sampled (b, g): every head for one sequence of one head group, else corners and the
    shortest and longest sequences."""
    if w.batch == 1:
        return [(0, g) for g in sorted({0, w.n_kv_heads // 2, w.n_kv_heads - 1})]
    order = np.argsort(seq_len, kind="stable")
    return [(0, 0), (int(order[0]), 2), (int(order[-1]), w.n_kv_heads - 1),
            (w.batch - 1, w.n_kv_heads - 1)]


@pytest.fixture(scope="module", params=WORKLOADS)
def full(request, gpu_lib):
    name = request.param
    print(f"\n[gpu full-size workload] {name}", flush=True)
    w = synth.WORKLOADS[name]
    inp = synth.make_workload_inputs(name)
    p = U.Pipeline(gpu_lib, inp, w.kv_dtype, w.n_q_heads, w.n_kv_heads, w.max_ctx, w.keep_num,
                   w.keep_den, w.keep_pages_abs, w.top_k)
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    torch.cuda.synchronize()
    assert p.status() == 0
    host = dict(codes=U.u32(p.codes), q_rot=p.q_rot.cpu().numpy().astype(np.float64),
                q_codes=U.u32(p.q_codes), scores=p.scores.cpu().numpy().astype(np.float64),
                kept=p.kept.cpu().numpy(), kept_count=p.kept_count.cpu().numpy(),
                sel=p.sel.cpu().numpy(), sel_count=p.sel_count.cpu().numpy(),
                out=p.out.cpu().numpy().astype(np.float64))
    return name, w, p, host, _pairs(w, inp["seq_len"])


def test_codes_and_meta_sampled(full):
    name, w, p, h, pairs = full
    rng = np.random.Generator(np.random.PCG64(7))
    for b, g in pairs:
        L = int(p.inp["seq_len"][b])
        Np = O.n_pages(L, 16)
        K = p.K_valid(b, g)
        rows = np.unique(np.concatenate([rng.choice(L, min(L, 2048), replace=False), [L - 1]]))
        n = U.check_code_bits(K[rows], p.inp["W"][g], h["codes"][b, g, rows])
        U.record_excused(f"full_{name}_sampled_key_codes", keys=rows.size, code_bits=n)
        pages = np.unique(np.concatenate([rng.choice(Np, min(Np, 64), replace=False),
                                          [0, Np - 1]]))
        meta = p.meta[b, g].cpu().numpy().astype(np.float64)
        R = p.inp["R"][g].astype(np.float64)
        for pg in pages:
            Kp = K[pg * 16:min(L, pg * 16 + 16)]
            want = O.page_minmax(O.rotate(Kp, R), 16)[0]
            tol = 3e-5 * (np.abs(Kp) @ np.abs(R)).max()
            assert np.abs(meta[pg] - want).max() <= tol, (b, g, pg)


def test_query_encoding(full):
    name, w, p, h, pairs = full
    for b, g in pairs:
        qg = p.q_group(b, g)
        R = p.inp["R"][g].astype(np.float64)
        tol = 2e-6 * (np.abs(qg) @ np.abs(R))
        assert np.all(np.abs(h["q_rot"][b, g * p.G:(g + 1) * p.G] - O.rotate(qg, R)) <= tol + 1e-30)
        U.check_code_bits(qg, p.inp["W"][g], h["q_codes"][b, g * p.G:(g + 1) * p.G])


def test_page_bounds_and_top_pages_conditioned(full):
    name, w, p, h, pairs = full
    for b, g in pairs:
        Np = O.n_pages(int(p.inp["seq_len"][b]), 16)
        meta = p.meta[b, g, :Np].cpu().numpy().astype(np.float64)
        qr = h["q_rot"][b, g * p.G:(g + 1) * p.G]
        want = O.page_scores(qr, meta)
        mag = (np.abs(qr).sum(0)[None, :] * np.abs(meta).max(-1)).sum(-1)
        assert np.all(np.abs(h["scores"][b, g, :Np] - want) <= 1e-5 * mag + 1e-30)
        P = O.keep_count(Np, *p.keep)
        assert h["kept_count"][b, g] == P
        assert h["kept"][b, g, :P].tolist() == O.top_pages(h["scores"][b, g, :Np], P).tolist()


def test_end_to_end_against_unconditioned_oracle(full):
    """The oracle's whole selection from raw inputs on sampled (b, g): kept pages within the
    page band, and every selected position that differs explained by an excused page, an
    excused code bit or the cut displacement it causes (every key encoded by the oracle, so
    the codes of all candidates are compared); the counts are recorded."""
    name, w, p, h, pairs = full
    total = {}
    for b, g in pairs[:2]:
        L = int(p.inp["seq_len"][b])
        res = O.select(p.q_group(b, g), p.K_valid(b, g), p.inp["R"][g], p.inp["W"][g], 16,
                       *p.keep, p.top_k)
        n = int(h["sel_count"][b, g])
        assert n == len(res["sel"])
        c = U.explain_selection(res, h["sel"][b, g, :n], h["kept"][b, g, :res["n_keep"]],
                                h["codes"][b, g], h["q_codes"][b, g * p.G:(g + 1) * p.G], L,
                                p.top_k)
        for k, v in c.items():
            total[k] = total.get(k, 0) + v
    print(f"excused ({name}): {total}")
    U.record_excused(f"full_{name}_e2e", **total)


def test_hamming_topk_conditioned_exact(full):
    name, w, p, h, pairs = full
    for b, g in pairs:
        L = int(p.inp["seq_len"][b])
        P = h["kept_count"][b, g]
        res = O.select_from_codes(h["q_codes"][b, g * p.G:(g + 1) * p.G], h["codes"][b, g],
                                  h["kept"][b, g, :P], L, 16, p.top_k)
        n = len(res["sel"])
        assert h["sel_count"][b, g] == n
        assert h["sel"][b, g, :n].tolist() == res["sel"].tolist()
        assert np.all(h["sel"][b, g, n:] == -1)


def test_attention_conditioned(full):
    name, w, p, h, pairs = full
    atol = 1e-5 if w.kv_dtype == "f32" else 2e-3
    for b, g in pairs:
        idx = h["sel"][b, g, :h["sel_count"][b, g]]
        L = int(p.inp["seq_len"][b])
        K = synth.kv_values(p.inp["K"][b, g, idx], w.kv_dtype).astype(np.float64)
        V = synth.kv_values(p.inp["V"][b, g, idx], w.kv_dtype).astype(np.float64)
        assert idx.size == 0 or idx.max() < L
        want = O.attend(p.q_group(b, g), K, V, p.scale)
        assert np.abs(h["out"][b, g * p.G:(g + 1) * p.G] - want).max() <= atol


def test_select_pages_equals_stages(full):
    name, w, p, h, pairs = full
    kept, kc, qc = p.select_pages()
    assert torch.equal(kept, p.kept) and torch.equal(kc, p.kept_count)
    assert torch.equal(qc, p.q_codes)


def test_select_equals_stages(full):
    """hhr_select (one launch on all but the ragged batch) equals the staged selection."""
    name, w, p, h, pairs = full
    sel, sc = p.select()
    assert torch.equal(sc, p.sel_count) and torch.equal(sel, p.sel)


def test_decode_and_graph_replays_equal_stages(full):
    """The bench launch configuration: hhr_decode captured in a HIP graph and replayed."""
    name, w, p, h, pairs = full
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
    for i in range(3):
        out.fill_(float(i + 1))
        sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, p.sel) and torch.equal(sc, p.sel_count)
        assert torch.equal(out, p.out), f"replay {i}"
    assert p.status() == 0
