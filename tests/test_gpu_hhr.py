"""GPU parity: the HIP path through the C ABI against the CPU oracle, stage by
stage (conditioned oracle: each stage fed the GPU's own upstream outputs) and
end to end (with excused-mismatch accounting), on small seeded cases that span
several tiles, ragged tails, GQA 1/4/8/16, an empty-ish sequence, top_k above
the candidate count and 64-, 128- and 256-bit codes.
"""
import functools
import math

import numpy as np
import pytest
import torch

from hash_hierarchical_top_amd import synth
from oracle import hhr as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = synth.small_hhr_cases() + synth.small_code_bits_cases()


def _inputs(case):
    return synth.make_hhr_inputs(case["batch"], case["n_q_heads"], case["n_kv_heads"],
                                 case["seq_lens"], case["max_ctx"], case["kv_dtype"],
                                 case["seed"], code_bits=case.get("code_bits", 128))


def _pipeline(H, case, with_v=True, meta_dtype="f32"):
    return U.Pipeline(H, _inputs(case), case["kv_dtype"], case["n_q_heads"], case["n_kv_heads"],
                      case["max_ctx"], case["keep_num"], case["keep_den"], case["keep_abs"],
                      case["top_k"], with_v=with_v, meta_dtype=meta_dtype,
                      code_bits=case.get("code_bits", 128))


def _atol(kv_dtype):
    return 1e-5 if kv_dtype == "f32" else 2e-3


@pytest.fixture(scope="module", params=CASES, ids=[c["name"] for c in CASES])
def run(request, gpu_lib):
    case = request.param
    print(f"\n[gpu case] {case['name']}", flush=True)
    p = _pipeline(gpu_lib, case)
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    torch.cuda.synchronize()
    return case, p


def test_append_codes_and_meta(run):
    case, p = run
    codes = U.u32(p.codes)
    meta = p.meta.cpu().numpy().astype(np.float64)
    excused = 0
    for b in range(p.B):
        L = int(p.inp["seq_len"][b])
        Np = O.n_pages(L, 16)
        for g in range(p.Hkv):
            K = p.K_valid(b, g)
            excused += U.check_code_bits(K, p.inp["W"][g], codes[b, g, :L])
            enc = O.encode_keys(K, p.inp["R"][g], p.inp["W"][g], 16)
            scaleX = np.abs(K) @ np.abs(p.inp["R"][g].astype(np.float64))
            for pg in range(Np):
                rows = slice(pg * 16, min(L, pg * 16 + 16))
                tol = 3e-5 * scaleX[rows].max()
                err = np.abs(meta[b, g, pg] - enc["meta"][pg]).max()
                assert err <= tol, (b, g, pg, err, tol)
    print(f"excused code bits: {excused}")
    U.record_excused(f"hhr_codes_{case['name']}", code_bits=excused)


def test_encode_queries(run):
    case, p = run
    q_rot = p.q_rot.cpu().numpy().astype(np.float64)
    q_codes = U.u32(p.q_codes)
    for b in range(p.B):
        for g in range(p.Hkv):
            qg = p.q_group(b, g)
            want = O.rotate(qg, p.inp["R"][g])
            tol = 2e-6 * (np.abs(qg) @ np.abs(p.inp["R"][g].astype(np.float64)))
            assert np.all(np.abs(q_rot[b, g * p.G:(g + 1) * p.G] - want) <= tol + 1e-30)
            U.check_code_bits(qg, p.inp["W"][g], q_codes[b, g * p.G:(g + 1) * p.G])


def test_page_scores_conditioned(run):
    """GPU bounds vs fp64 bounds recomputed from the GPU's own rotated queries and metadata."""
    case, p = run
    q_rot = p.q_rot.cpu().numpy().astype(np.float64)
    meta = p.meta.cpu().numpy().astype(np.float64)
    scores = p.scores.cpu().numpy().astype(np.float64)
    for b in range(p.B):
        Np = O.n_pages(int(p.inp["seq_len"][b]), 16)
        for g in range(p.Hkv):
            qr = q_rot[b, g * p.G:(g + 1) * p.G]
            want = O.page_scores(qr, meta[b, g, :Np])
            mag = (np.abs(qr).sum(0)[None, :] * np.abs(meta[b, g, :Np]).max(-1)).sum(-1)
            err = np.abs(scores[b, g, :Np] - want)
            assert np.all(err <= 1e-5 * mag + 1e-30), err.max()


def test_top_pages_conditioned_exact(run):
    """Top-P on the GPU's f32 scores is exact (same values, same tie-break)."""
    case, p = run
    scores = p.scores.cpu().numpy().astype(np.float64)
    kept = p.kept.cpu().numpy()
    kc = p.kept_count.cpu().numpy()
    for b in range(p.B):
        Np = O.n_pages(int(p.inp["seq_len"][b]), 16)
        P = O.keep_count(Np, *p.keep)
        for g in range(p.Hkv):
            assert kc[b, g] == P
            assert kept[b, g, :P].tolist() == O.top_pages(scores[b, g, :Np], P).tolist()
            assert np.all(kept[b, g, P:] == -1)


def test_hamming_topk_conditioned_exact(run):
    """Distances and selected positions from the GPU's own codes and kept pages: bit-exact."""
    case, p = run
    codes = U.u32(p.codes)
    q_codes = U.u32(p.q_codes)
    kept = p.kept.cpu().numpy()
    kc = p.kept_count.cpu().numpy()
    sel = p.sel.cpu().numpy()
    sc = p.sel_count.cpu().numpy()
    dist = p.dist.cpu().numpy().view(np.uint16)
    for b in range(p.B):
        L = int(p.inp["seq_len"][b])
        for g in range(p.Hkv):
            P = kc[b, g]
            res = O.select_from_codes(q_codes[b, g * p.G:(g + 1) * p.G], codes[b, g],
                                      kept[b, g, :P], L, 16, p.top_k)
            n = len(res["sel"])
            assert sc[b, g] == n
            assert sel[b, g, :n].tolist() == res["sel"].tolist()
            assert np.all(sel[b, g, n:] == -1)
            slot_pos = (kept[b, g, :P, None] * 16 + np.arange(16)[None, :]).reshape(-1)
            d = dist[b, g, :P * 16]
            valid = slot_pos < L
            assert np.all(d[~valid] == 0xFFFF)
            assert d[valid].tolist() == res["H"].tolist()


def test_sparse_decode_conditioned(run):
    case, p = run
    sel = p.sel.cpu().numpy()
    sc = p.sel_count.cpu().numpy()
    out = p.out.cpu().numpy().astype(np.float64)
    for b in range(p.B):
        for g in range(p.Hkv):
            idx = sel[b, g, :sc[b, g]]
            K = p.K_valid(b, g)
            V = p.V_valid(b, g)
            want = O.attend(p.q_group(b, g), K[idx], V[idx], p.scale)
            got = out[b, g * p.G:(g + 1) * p.G]
            assert np.abs(got - want).max() <= _atol(case["kv_dtype"])


def test_end_to_end_against_unconditioned_oracle(run):
    """Selection from raw inputs: every position where the GPU's selection differs from the
    oracle's must be explained by an excused page, an excused code bit or the cut
    displacement one causes; the counts are recorded."""
    case, p = run
    sel = p.sel.cpu().numpy()
    sc = p.sel_count.cpu().numpy()
    kept = p.kept.cpu().numpy()
    codes = U.u32(p.codes)
    q_codes = U.u32(p.q_codes)
    total = {}
    for b in range(p.B):
        L = int(p.inp["seq_len"][b])
        for g in range(p.Hkv):
            K = p.K_valid(b, g)
            res = O.select(p.q_group(b, g), K, p.inp["R"][g], p.inp["W"][g], 16, *p.keep,
                           p.top_k)
            assert sc[b, g] == len(res["sel"])
            c = U.explain_selection(res, sel[b, g, :sc[b, g]], kept[b, g, :res["n_keep"]],
                                    codes[b, g], q_codes[b, g * p.G:(g + 1) * p.G], L, p.top_k)
            for k, v in c.items():
                total[k] = total.get(k, 0) + v
    print(f"excused: {total}")
    U.record_excused(f"hhr_e2e_{case['name']}", **total)


def test_decode_composite_equals_stages(run, gpu_lib):
    case, p = run
    sel = torch.zeros_like(p.sel)
    sc = torch.zeros_like(p.sel_count)
    out = torch.zeros_like(p.out)
    p.decode(sel, sc, out)
    torch.cuda.synchronize()
    assert torch.equal(sel, p.sel) and torch.equal(sc, p.sel_count)
    assert torch.equal(out, p.out)
    # deterministic: a second call is bit-identical
    out2 = torch.zeros_like(out)
    p.decode(sel, sc, out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert p.status() == 0


def test_select_pages_equals_stages(run):
    """The one-launch coarse stage writes what encode + page_scores + top_pages write."""
    case, p = run
    kept, kc, qc = p.select_pages()
    assert torch.equal(kept, p.kept) and torch.equal(kc, p.kept_count)
    assert torch.equal(qc, p.q_codes)


@pytest.mark.parametrize("L,keep", [(150000, (1, 16, 0)), (262144, (1, 8, 0)),
                                    (262000, (0, 1, 2000))])
def test_long_context_top_pages(gpu_lib, L, keep):
    """Contexts past 128K give every top-P thread 3 or 4 float4 runs of bounds: the staged
    and one-launch top-P both equal the oracle's top-P of the GPU's own bounds."""
    print(f"\n[gpu long-context top-P] L={L} keep={keep}", flush=True)
    Lcap = -(-L // 16) * 16
    inp = synth.make_hhr_inputs(1, 4, 1, [L], Lcap, "bf16", seed=31, make_v=False)
    p = U.Pipeline(gpu_lib, inp, "bf16", 4, 1, Lcap, *keep, 64, with_v=False)
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    torch.cuda.synchronize()
    Np = O.n_pages(L, 16)
    P = O.keep_count(Np, *keep)
    s = p.scores[0, 0, :Np].cpu().numpy().astype(np.float64)
    want = O.top_pages(s, P).tolist()
    assert int(p.kept_count[0, 0]) == P and p.kept[0, 0, :P].cpu().tolist() == want
    kept, kc, qc = p.select_pages()
    assert int(kc[0, 0]) == P and kept[0, 0, :P].cpu().tolist() == want
    assert torch.equal(qc, p.q_codes)


@functools.lru_cache(maxsize=1)
def _wide_inputs(B, Hq, Hkv, Lcap):
    rng = np.random.Generator(np.random.PCG64(41))
    lens = rng.integers(1, Lcap + 1, B)
    lens[0], lens[1] = Lcap, 17
    return lens, synth.make_hhr_inputs(B, Hq, Hkv, lens.tolist(), Lcap, "bf16", seed=42)


@pytest.mark.parametrize("meta_dtype", ["f32", "bf16"])
def test_wide_batch_decode(gpu_lib, meta_dtype):
    """33 sequences x 8 KV heads: 528 scoring workgroups and 1056 attention workgroups, past
    the sizes where hhr_decode encodes the queries in a launch of their own and selects
    before attending.  hhr_decode and hhr_select_pages equal the stage-by-stage run bit for
    bit; sampled (b, g) pairs match the conditioned oracle."""
    print(f"\n[gpu wide batch] meta={meta_dtype}", flush=True)
    B, Hq, Hkv, Lcap, top_k = 33, 32, 8, 8192, 256
    lens, inp = _wide_inputs(B, Hq, Hkv, Lcap)
    p = U.Pipeline(gpu_lib, inp, "bf16", Hq, Hkv, Lcap, 1, 4, 0, top_k, meta_dtype=meta_dtype)
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    torch.cuda.synchronize()
    sel = torch.zeros_like(p.sel)
    sc = torch.zeros_like(p.sel_count)
    out = torch.zeros_like(p.out)
    p.decode(sel, sc, out)
    torch.cuda.synchronize()
    assert p.status() == 0
    assert torch.equal(sel, p.sel) and torch.equal(sc, p.sel_count) and torch.equal(out, p.out)
    kept, kc, qc = p.select_pages()
    assert torch.equal(kept, p.kept) and torch.equal(kc, p.kept_count)
    assert torch.equal(qc, p.q_codes)
    codes, q_codes = U.u32(p.codes), U.u32(p.q_codes)
    for b, g in [(0, 0), (1, 3), (int(np.argmax(lens[2:])) + 2, 7), (B - 1, 5)]:
        L = int(lens[b])
        Np = O.n_pages(L, 16)
        qr = p.q_rot[b, g * p.G:(g + 1) * p.G].cpu().numpy().astype(np.float64)
        s = p.scores[b, g, :Np].cpu().numpy().astype(np.float64)
        meta = p.meta_host(b, g, Np)
        mag = (np.abs(qr).sum(0)[None, :] * np.abs(meta).max(-1)).sum(-1)
        assert np.all(np.abs(s - O.page_scores(qr, meta)) <= 1e-5 * mag + 1e-30)
        P = O.keep_count(Np, 1, 4, 0)
        assert p.kept[b, g, :P].cpu().tolist() == O.top_pages(s, P).tolist()
        res = O.select_from_codes(q_codes[b, g * p.G:(g + 1) * p.G], codes[b, g],
                                  p.kept[b, g, :P].cpu().numpy(), L, 16, top_k)
        n = len(res["sel"])
        assert int(p.sel_count[b, g]) == n and p.sel[b, g, :n].cpu().tolist() == res["sel"].tolist()
        want = O.attend(p.q_group(b, g), p.K_valid(b, g)[res["sel"]], p.V_valid(b, g)[res["sel"]],
                        p.scale)
        assert np.abs(p.out[b, g * p.G:(g + 1) * p.G].cpu().numpy() - want).max() <= 2e-3


def _check_decode_append(p, lens, meta_dtype, codes0, meta0, sel, sc, out, pairs):
    """After hhr_decode_append: the new rows' codes and their pages' metadata against the
    oracle, everything else untouched, and the staged stages on the updated cache equal
    the fused call's selection and output bit for bit."""
    codes, codes_before = U.u32(p.codes), U.u32(codes0)
    for b, g in pairs:
        L = int(lens[b])
        if L == 0:
            continue
        K = p.K_valid(b, g)
        U.check_code_bits(K[L - 1:L], p.inp["W"][g], codes[b, g, L - 1:L])
        assert np.array_equal(np.delete(codes[b, g], L - 1, axis=0),
                              np.delete(codes_before[b, g], L - 1, axis=0))
        Np = O.n_pages(L, 16)
        pn = Np - 1
        Kp = K[pn * 16:L]
        R = p.inp["R"][g].astype(np.float64)
        ex = O.page_minmax(O.rotate(Kp, R), 16)[0]
        tol = 3e-5 * (np.abs(Kp) @ np.abs(R)).max()
        got = p.meta_host(b, g, Np)[pn]
        if meta_dtype == "f32":
            assert np.abs(got - ex).max() <= tol, (b, g)
        else:
            assert np.all(O.bf16_round(ex[:, 0] - tol, up=False) <= got[:, 0])
            assert np.all(got[:, 0] <= O.bf16_round(ex[:, 0] + tol, up=False))
            assert np.all(O.bf16_round(ex[:, 1] - tol, up=True) <= got[:, 1])
            assert np.all(got[:, 1] <= O.bf16_round(ex[:, 1] + tol, up=True))
        assert torch.equal(p.meta[b, g, :pn], meta0[b, g, :pn]) and \
            torch.equal(p.meta[b, g, pn + 1:], meta0[b, g, pn + 1:])
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    torch.cuda.synchronize()
    assert torch.equal(sel, p.sel) and torch.equal(sc, p.sel_count) and torch.equal(out, p.out)


def _decode_append_run(H, p):
    """Encode every row but each sequence's last, then one fused append + decode step."""
    lens = p.inp["seq_len"].astype(np.int64)
    start = torch.zeros(p.B, dtype=torch.int32, device="cuda")
    n_new = torch.from_numpy(np.maximum(lens - 1, 0).astype(np.int32)).cuda()
    H.hhr_append_keys(p.shape, p.d["K"], start, n_new, int(max(lens.max() - 1, 0)), p.d["R"],
                      p.d["W"], p.codes, p.meta, p.ws)
    torch.cuda.synchronize()
    codes0, meta0 = p.codes.clone(), p.meta.clone()
    sel = torch.zeros_like(p.sel)
    sc = torch.zeros_like(p.sel_count)
    out = torch.zeros_like(p.out)
    H.hhr_decode_append(p.shape, p.d["q"], p.d["seq_len"], p.d["R"], p.d["W"], p.codes, p.meta,
                        p.d["K"], p.d["V"], *p.keep, p.top_k, p.scale, sel, sc, out, p.ws)
    torch.cuda.synchronize()
    assert p.status() == 0
    return lens, codes0, meta0, sel, sc, out


@pytest.mark.parametrize("meta_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_decode_append(gpu_lib, case, meta_dtype):
    """One fused append + decode step per sequence (one-launch coarse stage), including a
    one-key sequence, a key that opens a page and keys that extend a partial page."""
    print(f"\n[gpu decode_append] {case['name']} meta={meta_dtype}", flush=True)
    p = _pipeline(gpu_lib, case, meta_dtype=meta_dtype)
    lens, codes0, meta0, sel, sc, out = _decode_append_run(gpu_lib, p)
    pairs = [(b, g) for b in range(p.B) for g in range(p.Hkv)]
    _check_decode_append(p, lens, meta_dtype, codes0, meta0, sel, sc, out, pairs)


@pytest.mark.parametrize("meta_dtype", ["f32", "bf16"])
def test_wide_batch_decode_append(gpu_lib, meta_dtype):
    """The same on the 33-sequence batch, where the append runs in the encoder launch ahead
    of the staged coarse stage."""
    print(f"\n[gpu wide batch decode_append] meta={meta_dtype}", flush=True)
    B, Hq, Hkv, Lcap, top_k = 33, 32, 8, 8192, 256
    lens, inp = _wide_inputs(B, Hq, Hkv, Lcap)
    p = U.Pipeline(gpu_lib, inp, "bf16", Hq, Hkv, Lcap, 1, 4, 0, top_k, meta_dtype=meta_dtype)
    lens, codes0, meta0, sel, sc, out = _decode_append_run(gpu_lib, p)
    _check_decode_append(p, lens, meta_dtype, codes0, meta0, sel, sc, out,
                         [(0, 0), (1, 3), (5, 7), (B - 1, 2)])


def test_chunked_append_equals_one_shot(gpu_lib):
    case = CASES[1]
    p = _pipeline(gpu_lib, case, with_v=False)
    p.append_all()
    codes1, meta1 = p.codes.clone(), p.meta.clone()
    p.codes.zero_()
    p.meta.zero_()
    B = p.B
    lens = p.inp["seq_len"].astype(np.int64)
    # chunks with unaligned boundaries, then single-key appends at the end
    pts = np.stack([np.maximum.accumulate(np.clip([0, 37, 1000, L - 3, L - 2, L - 1, L], 0, L))
                    for L in lens])
    for i in range(pts.shape[1] - 1):
        a, z = pts[:, i], pts[:, i + 1]
        start = torch.from_numpy(a.astype(np.int32)).cuda()
        n_new = torch.from_numpy((z - a).astype(np.int32)).cuda()
        gpu_lib.hhr_append_keys(p.shape, p.d["K"], start, n_new, int((z - a).max()), p.d["R"],
                                p.d["W"], p.codes, p.meta, p.ws)
    torch.cuda.synchronize()
    assert torch.equal(p.codes, codes1)
    for b in range(B):
        Np = O.n_pages(int(lens[b]), 16)
        assert torch.equal(p.meta[b, :, :Np], meta1[b, :, :Np])


def test_bad_seq_len_sets_status_and_selects_nothing(gpu_lib):
    case = CASES[0]
    p = _pipeline(gpu_lib, case)
    p.append_all()
    bad = torch.tensor([-5, case["max_ctx"] + 16], dtype=torch.int32, device="cuda")
    sel = torch.zeros_like(p.sel)
    sc = torch.full_like(p.sel_count, 7)
    out = torch.full_like(p.out, 3.0)
    gpu_lib.hhr_decode(p.shape, p.d["q"], bad, p.d["R"], p.d["W"], p.codes, p.meta, p.d["K"],
                       p.d["V"], *p.keep, p.top_k, p.scale, sel, sc, out, p.ws)
    flags = p.status()
    assert flags & gpu_lib.HHR_DEV_BAD_SEQ_LEN
    assert torch.all(sc == 0) and torch.all(sel == -1) and torch.all(out == 0)
    assert p.status() == 0  # cleared by the read


def test_keep_all_pages_and_k_equal_L_is_dense_attention(gpu_lib):
    """Keeping every page with top_k >= L attends to every key: compare with dense SDPA."""
    inp = synth.make_hhr_inputs(1, 4, 1, [1000], 1024, "f32", seed=21)
    p = U.Pipeline(gpu_lib, inp, "f32", 4, 1, 1024, 1, 1, 0, 1024)
    p.append_all()
    sel = torch.zeros_like(p.sel)
    sc = torch.zeros_like(p.sel_count)
    p.decode(sel, sc, p.out)
    torch.cuda.synchronize()
    assert int(sc[0, 0]) == 1000 and sel[0, 0, :1000].tolist() == list(range(1000))
    q = torch.from_numpy(inp["q"][0]).double()
    K = torch.from_numpy(inp["K"][0, 0, :1000]).double()
    V = torch.from_numpy(inp["V"][0, 0, :1000]).double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], K[None].expand(4, -1, -1), V[None].expand(4, -1, -1))[:, 0]
    assert (p.out[0].double().cpu() - ref).abs().max().item() <= 1e-5


@pytest.mark.parametrize("code_bits", [64, 256])
def test_long_append_other_code_widths(gpu_lib, code_bits):
    """A 40,000-key append at 64- and 256-bit codes: the bf16 encoder runs several key tiles
    per workgroup (its LDS ring with tiles in flight), with its wave count and load waits
    for that width.  Sampled codes and page metadata against the oracle."""
    print(f"\n[gpu long append] code_bits={code_bits}", flush=True)
    L, Lcap, Hq, Hkv = 40000, 40960, 8, 2
    inp = synth.make_hhr_inputs(1, Hq, Hkv, [L], Lcap, "bf16", 31, code_bits=code_bits,
                                make_v=False)
    p = U.Pipeline(gpu_lib, inp, "bf16", Hq, Hkv, Lcap, 1, 8, 0, 256, with_v=False,
                   code_bits=code_bits)
    p.append_all()
    torch.cuda.synchronize()
    assert p.status() == 0
    codes = U.u32(p.codes)
    rng = np.random.Generator(np.random.PCG64(5))
    Np = O.n_pages(L, 16)
    for g in range(Hkv):
        K = p.K_valid(0, g)
        rows = np.unique(np.concatenate([rng.choice(L, 3000, replace=False), [0, L - 1]]))
        U.check_code_bits(K[rows], p.inp["W"][g], codes[0, g, rows])
        meta = p.meta[0, g].cpu().numpy().astype(np.float64)
        R = p.inp["R"][g].astype(np.float64)
        for pg in np.unique(np.concatenate([rng.choice(Np, 200, replace=False), [0, Np - 1]])):
            Kp = K[pg * 16:min(L, pg * 16 + 16)]
            want = O.page_minmax(O.rotate(Kp, R), 16)[0]
            tol = 3e-5 * (np.abs(Kp) @ np.abs(R)).max()
            assert np.abs(meta[pg] - want).max() <= tol, (g, pg)
