"""GPU parity of the HISA indexer path (H1..H5) through the C ABI against the CPU
oracle: pooled block representatives, block scores, top blocks, fp8 token
scores and the exact token top-k inside the kept blocks, then attention over
the selection (hhr_sparse_decode with one KV head).

Stages downstream of a floating-point result are checked on the GPU's own
upstream values (conditioned oracle), where the discrete results must be
exact; the end-to-end selection from raw inputs may differ only where the
oracle's score sits within 1e-4 (relative) of the cut-off score.  Cases span
block sizes 16 / 64 / 128, ragged and one-token and empty sequences, top_k
above the candidate count, and keep-all-blocks (which must equal the flat
indexer).
"""
import numpy as np
import pytest
import torch

from hash_hierarchical_top_amd import synth
from oracle import hhr as OH
from oracle import hisa as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCORE_EXCUSE = 1e-4
CASES = [
    dict(name="hi64_blk128_ragged", n_index_heads=64, block=128, max_ctx=16384,
         seq_lens=[10000, 16384], keep_blocks=16, top_k=1024, seed=21),
    dict(name="hi8_blk16_tiny", n_index_heads=8, block=16, max_ctx=4096, seq_lens=[1000, 1, 0],
         keep_blocks=20, top_k=200, seed=22),
    dict(name="hi32_blk64_bigk", n_index_heads=32, block=64, max_ctx=2048, seq_lens=[777],
         keep_blocks=8, top_k=2048, seed=23),
]


def _inputs(case):
    """Per-sequence draws stacked along the batch: q8 [B][Hi][d], k8 [B][Lcap][d], ..."""
    parts = [synth.make_hisa_inputs(case["n_index_heads"], L, case["max_ctx"], 4,
                                    case["seed"] + 7 * b, block=case["block"], make_kv=False)
             for b, L in enumerate(case["seq_lens"])]
    return {k: np.stack([p[k] for p in parts]) if k != "seq_len"
            else np.array([int(p[k][0]) for p in parts], dtype=np.int32)
            for k in parts[0]}


class HisaRun:
    def __init__(self, H, case):
        self.H, self.case = H, case
        self.inp = _inputs(case)
        B = len(case["seq_lens"])
        self.B, self.block, self.Lcap = B, case["block"], case["max_ctx"]
        self.keep, self.top_k = case["keep_blocks"], case["top_k"]
        self.NbCap = self.Lcap // self.block
        self.shape = H.make_hisa_shape(B, case["n_index_heads"], self.block, self.Lcap)
        dv = U.dev()
        self.d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dv) for k, v in self.inp.items()}
        i32 = dict(dtype=torch.int32, device=dv)
        f32 = dict(dtype=torch.float32, device=dv)
        self.reps = torch.zeros((B, self.NbCap, 128), **f32)
        self.block_scores = torch.full((B, self.NbCap), float("nan"), **f32)
        self.kept = torch.zeros((B, self.keep), **i32)
        self.kept_count = torch.zeros((B,), **i32)
        self.token_scores = torch.full((B, self.keep * self.block), float("nan"), **f32)
        self.sel = torch.zeros((B, self.top_k), **i32)
        self.sel_count = torch.zeros((B,), **i32)
        ws = H.hhr_hisa_workspace_size(self.shape, self.keep, self.top_k)
        assert ws > 0
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=dv)
        self.status = self.ws[:4].view(torch.int32)

    def run_stages(self):
        H, d = self.H, self.d
        zero = torch.zeros(self.B, dtype=torch.int32, device=U.dev())
        H.hhr_hisa_pool_keys(self.shape, d["k8"], d["k_scale"], zero, d["seq_len"],
                             max(1, int(self.inp["seq_len"].max())), self.reps, self.status)
        H.hhr_hisa_block_scores(self.shape, d["q8"], d["q_scale"], d["w"], self.reps,
                                d["seq_len"], self.block_scores, self.status)
        H.hhr_hisa_top_blocks(self.shape, self.block_scores, d["seq_len"], self.keep, self.kept,
                              self.kept_count, self.status)
        H.hhr_hisa_token_topk(self.shape, d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"],
                              d["seq_len"], self.kept, self.kept_count, self.keep, self.top_k,
                              self.sel, self.sel_count, self.token_scores, self.ws)
        torch.cuda.synchronize()

    # oracle-side views of one sequence
    def L(self, b):
        return int(self.inp["seq_len"][b])

    def q(self, b):
        return O.dequantize(self.inp["q8"][b], self.inp["q_scale"][b])

    def keys(self, b):
        L = self.L(b)
        return O.dequantize(self.inp["k8"][b, :L], self.inp["k_scale"][b, :L])

    def nb(self, b):
        return -(-self.L(b) // self.block)


@pytest.fixture(scope="module", params=CASES, ids=[c["name"] for c in CASES])
def run(request, gpu_lib):
    case = request.param
    print(f"\n[gpu hisa case] {case['name']}", flush=True)
    r = HisaRun(gpu_lib, case)
    r.run_stages()
    return r


def _abs_terms(q, w, x):
    """sum_h w_h * sum_d |q_hd x_td| per row: the scale of the rounding in the indexer score."""
    return (np.abs(x) @ np.abs(q).T) @ np.abs(np.asarray(w, dtype=np.float64))


def test_pool_reps(run):
    reps = run.reps.cpu().numpy().astype(np.float64)
    for b in range(run.B):
        if run.L(b) == 0:
            continue
        keys = run.keys(b)
        want = O.pooled_reps(keys, run.block)
        scale = np.stack([np.abs(keys[i * run.block:(i + 1) * run.block]).mean(0)
                          for i in range(run.nb(b))])
        assert np.all(np.abs(reps[b, :run.nb(b)] - want) <= 1e-5 * scale + 1e-30)


def test_block_scores_conditioned(run):
    got = run.block_scores.cpu().numpy().astype(np.float64)
    reps = run.reps.cpu().numpy().astype(np.float64)
    for b in range(run.B):
        nb = run.nb(b)
        q, w = run.q(b), run.inp["w"][b]
        want = O.indexer_scores(q, w, reps[b, :nb])
        tol = 1e-5 * _abs_terms(q, w, reps[b, :nb]) + 1e-30
        assert np.all(np.abs(got[b, :nb] - want) <= tol)


def test_top_blocks_conditioned_exact(run):
    sc = run.block_scores.cpu().numpy()
    kept = run.kept.cpu().numpy()
    cnt = run.kept_count.cpu().numpy()
    for b in range(run.B):
        nb = run.nb(b)
        want = O.top_largest(sc[b, :nb].astype(np.float64), np.arange(nb), run.keep)
        assert cnt[b] == min(run.keep, nb)
        np.testing.assert_array_equal(kept[b, :cnt[b]], want)
        assert np.all(kept[b, cnt[b]:] == -1)


def test_top_blocks_against_unconditioned_oracle(run):
    """Raw inputs: a kept-block difference is allowed only within the excuse band."""
    kept = run.kept.cpu().numpy()
    cnt = run.kept_count.cpu().numpy()
    for b in range(run.B):
        if run.L(b) == 0:
            assert cnt[b] == 0
            continue
        ref = O.select(run.inp["q8"][b], run.inp["q_scale"][b], run.inp["w"][b],
                       run.inp["k8"][b], run.inp["k_scale"][b], run.L(b), run.block, run.keep,
                       run.top_k)
        S = ref["block_scores"]
        cut = np.sort(S)[::-1][min(run.keep, S.size) - 1]
        diff = np.setxor1d(kept[b, :cnt[b]], ref["blocks"])
        for blk in diff:
            assert abs(S[blk] - cut) <= SCORE_EXCUSE * abs(cut), (b, blk)


def _candidates(run, b, kept_row, count):
    blocks = kept_row[:count].astype(np.int64)
    cand = (blocks[:, None] * run.block + np.arange(run.block)[None, :]).reshape(-1)
    return cand  # slot-major: slot i, row r -> kept[i] * block + r


def test_token_scores_conditioned(run):
    ts = run.token_scores.cpu().numpy().astype(np.float64)
    kept = run.kept.cpu().numpy()
    cnt = run.kept_count.cpu().numpy()
    for b in range(run.B):
        cand = _candidates(run, b, kept[b], cnt[b])
        valid = cand < run.L(b)
        got = ts[b, :cand.size]
        assert np.all(np.isneginf(got[~valid]))
        c = cand[valid]
        x = O.dequantize(run.inp["k8"][b, c], run.inp["k_scale"][b, c])
        q, w = run.q(b), run.inp["w"][b]
        want = O.indexer_scores(q, w, x)
        tol = 1e-5 * _abs_terms(q, w, x) + 1e-30
        assert np.all(np.abs(got[valid] - want) <= tol)


def test_token_topk_conditioned_exact(run):
    ts = run.token_scores.cpu().numpy()
    kept = run.kept.cpu().numpy()
    cnt = run.kept_count.cpu().numpy()
    sel = run.sel.cpu().numpy()
    sc = run.sel_count.cpu().numpy()
    for b in range(run.B):
        cand = _candidates(run, b, kept[b], cnt[b])
        valid = cand < run.L(b)
        want = O.top_largest(ts[b, :cand.size][valid].astype(np.float64), cand[valid], run.top_k)
        assert sc[b] == want.size
        np.testing.assert_array_equal(sel[b, :sc[b]], want)
        assert np.all(sel[b, sc[b]:] == -1)


def test_composite_equals_stages(run, gpu_lib):
    H, d = gpu_lib, run.d
    sel2 = torch.full_like(run.sel, 7)
    cnt2 = torch.full_like(run.sel_count, 7)
    H.hhr_hisa_select(run.shape, d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], run.reps,
                      d["seq_len"], run.keep, run.top_k, sel2, cnt2, run.ws)
    torch.cuda.synchronize()
    assert torch.equal(sel2, run.sel) and torch.equal(cnt2, run.sel_count)
    assert H.hhr_read_device_status(run.ws) == 0


def test_keep_all_blocks_equals_flat_indexer(gpu_lib):
    """Keeping every block, the selection is the flat indexer's exact top-k (IoU 1 against
    the oracle's flat selection, up to the excuse band around the k-th score)."""
    case = dict(CASES[1], name="keep_all", seq_lens=[3000, 4096], keep_blocks=4096 // 16,
                top_k=300, seed=31)
    r = HisaRun(gpu_lib, case)
    r.run_stages()
    ts = r.token_scores.cpu().numpy()
    sel = r.sel.cpu().numpy()
    sc = r.sel_count.cpu().numpy()
    for b in range(r.B):
        L = r.L(b)
        # conditioned: every valid token is a candidate, in position order
        np.testing.assert_array_equal(r.kept.cpu().numpy()[b, :r.nb(b)], np.arange(r.nb(b)))
        want = O.top_largest(ts[b, :L].astype(np.float64), np.arange(L), r.top_k)
        np.testing.assert_array_equal(sel[b, :sc[b]], want)
        # unconditioned: the flat oracle
        s = O.indexer_scores(r.q(b), r.inp["w"][b], r.keys(b))
        flat = O.flat_select(r.inp["q8"][b], r.inp["q_scale"][b], r.inp["w"][b], r.inp["k8"][b],
                             r.inp["k_scale"][b], L, r.top_k)
        cut = np.sort(s)[::-1][r.top_k - 1]
        for t in np.setxor1d(sel[b, :sc[b]], flat):
            assert abs(s[t] - cut) <= SCORE_EXCUSE * abs(cut)


def test_attention_over_hisa_selection(gpu_lib):
    """H5: 16 attention heads on one bf16 KV head over the HISA selection."""
    H = gpu_lib
    case = dict(CASES[0], name="attn", seq_lens=[9000], seed=41)
    r = HisaRun(H, case)
    r.run_stages()
    rng = np.random.Generator(np.random.PCG64(4242))
    Lcap, Ha = r.Lcap, 16
    K = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, Lcap, 128), dtype=np.float32))
    V = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, Lcap, 128), dtype=np.float32))
    q = synth.round_to_bf16(rng.standard_normal((1, Ha, 128), dtype=np.float32))
    shape = H.make_shape(1, Ha, 1, Lcap, "bf16")
    dv = U.dev()
    out = torch.zeros((1, Ha, 128), dtype=torch.float32, device=dv)
    ws = torch.zeros(H.hhr_workspace_size(shape, 1, 1, 0, r.top_k), dtype=torch.uint8, device=dv)
    sel = r.sel.view(1, 1, r.top_k)
    cnt = r.sel_count.view(1, 1)
    H.hhr_sparse_decode(shape, torch.from_numpy(q).to(dv), U.kv_to_device(K, "bf16"),
                        U.kv_to_device(V, "bf16"), sel, cnt, r.top_k, 1.0 / np.sqrt(128.0), out,
                        ws)
    torch.cuda.synchronize()
    idx = r.sel.cpu().numpy()[0, :int(r.sel_count[0])]
    Kf = synth.bf16_bits_to_f32(K[0, 0])
    Vf = synth.bf16_bits_to_f32(V[0, 0])
    want = OH.attend(q[0], Kf[idx], Vf[idx])
    assert np.abs(out.cpu().numpy()[0].astype(np.float64) - want).max() <= 2e-3


def test_bad_seq_len_sets_status_and_selects_nothing(gpu_lib):
    case = dict(CASES[1], name="bad_len", seq_lens=[1000, 2000], seed=51)
    r = HisaRun(gpu_lib, case)
    r.d["seq_len"][1] = r.Lcap + 1
    r.inp["seq_len"][1] = 0  # what the oracle should see: an empty sequence
    r.run_stages()
    assert gpu_lib.hhr_read_device_status(r.ws) & 0x1
    assert int(r.sel_count[1]) == 0 and int(r.kept_count[1]) == 0
    assert torch.all(r.sel[1] == -1)
    assert int(r.sel_count[0]) == min(r.top_k, 1000)


def test_full_size_hisa_128k(gpu_lib):
    """The full HISA decode workload: 131072 fp8 index keys, 64 index heads, 1024 blocks of 128,
    top 64 blocks, token top-2048; every block score and token score of the kept blocks checked,
    both selections exact on the GPU's scores, block selection within the excuse band on raw
    inputs."""
    w = synth.HISA_WORKLOADS["hisa_128k"]
    case = dict(name="hisa_128k", n_index_heads=w.n_index_heads, block=w.block, max_ctx=w.ctx,
                seq_lens=[w.ctx], keep_blocks=w.keep_blocks, top_k=w.top_k, seed=w.seed)
    r = HisaRun(gpu_lib, case)
    r.run_stages()
    q, wt = r.q(0), r.inp["w"][0]
    reps = r.reps.cpu().numpy().astype(np.float64)[0]
    keys = r.keys(0)
    want_reps = O.pooled_reps(keys, r.block)
    scale = np.abs(keys).reshape(-1, r.block, 128).mean(1)
    assert np.all(np.abs(reps - want_reps) <= 1e-5 * scale + 1e-30)
    bs = r.block_scores.cpu().numpy().astype(np.float64)[0]
    assert np.all(np.abs(bs - O.indexer_scores(q, wt, reps)) <= 1e-5 * _abs_terms(q, wt, reps))
    kept = r.kept.cpu().numpy()[0]
    np.testing.assert_array_equal(kept, O.top_largest(bs, np.arange(bs.size), r.keep))
    S = O.indexer_scores(q, wt, want_reps)
    cut = np.sort(S)[::-1][r.keep - 1]
    for blk in np.setxor1d(kept, O.top_largest(S, np.arange(S.size), r.keep)):
        assert abs(S[blk] - cut) <= SCORE_EXCUSE * abs(cut)
    cand = _candidates(r, 0, kept, r.keep)
    ts = r.token_scores.cpu().numpy().astype(np.float64)[0]
    x = keys[cand]
    assert np.all(np.abs(ts - O.indexer_scores(q, wt, x)) <= 1e-5 * _abs_terms(q, wt, x))
    sel = r.sel.cpu().numpy()[0]
    np.testing.assert_array_equal(sel, O.top_largest(ts, cand, r.top_k))
    assert int(r.sel_count[0]) == r.top_k
    assert gpu_lib.hhr_read_device_status(r.ws) == 0


# --------------------------------------------------------------------------- #
# prefill rows: one shared cache, causal prefixes
# --------------------------------------------------------------------------- #
def _kth_largest(s, k):
    s = np.sort(np.asarray(s, np.float64))[::-1]
    return s[min(k, s.size) - 1]


def _within_band(got, want, score_of, k_scores, k, what):
    """got and want (id sets) may differ only at ids whose fp64 score lies within the
    excuse band of the k-th largest of k_scores; returns how many ids differ."""
    diff = np.setxor1d(np.asarray(got, np.int64), np.asarray(want, np.int64))
    if diff.size:
        cut = _kth_largest(k_scores, k)
        for i in diff:
            assert abs(score_of(i) - cut) <= SCORE_EXCUSE * abs(cut), (what, int(i), cut)
    return int(diff.size)


class PrefillRun:
    """hhr_hisa_prefill_select for M query rows against one shared cache, and the decode
    path on per-row copies of the cache whose representatives are pooled over the row's own
    prefix (seq_len = q_len[r]): by the causal reading the two agree bit for bit.  The
    staged decode entry points expose the intermediates (each row's representatives, block
    scores, kept blocks and token scores) for the oracle checks."""

    def __init__(self, H, k8, ks, q8, q_scale, wt, q_len, blk, keep, top_k, copy_rows=None):
        dv = U.dev()
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dv)
        self.H, self.blk, self.keep, self.top_k = H, blk, keep, top_k
        self.q8, self.q_scale, self.wt, self.q_len = q8, q_scale, wt, q_len
        self.k8_np, self.ks_np = k8, ks
        Lcap = k8.shape[0]
        M = q_len.size
        self.Lcap, self.M = Lcap, M
        Hi = q8.shape[1]
        k8d, ksd = t(k8), t(ks)
        # the cache's shared representatives, pooled once over all of it
        shape1 = H.make_hisa_shape(1, Hi, blk, Lcap)
        self.reps = torch.zeros((1, Lcap // blk, 128), dtype=torch.float32, device=dv)
        st1 = torch.zeros(64, dtype=torch.int32, device=dv)
        H.hhr_hisa_pool_keys(shape1, k8d[None], ksd[None], torch.zeros(1, dtype=torch.int32,
                             device=dv), t(np.array([Lcap], np.int32)), Lcap, self.reps, st1)
        shape = H.make_hisa_shape(M, Hi, blk, Lcap)
        ws = torch.zeros(H.hhr_hisa_workspace_size(shape, keep, top_k), dtype=torch.uint8,
                         device=dv)
        self.sel = torch.zeros((M, top_k), dtype=torch.int32, device=dv)
        self.cnt = torch.zeros((M,), dtype=torch.int32, device=dv)
        print(f"[prefill] hhr_hisa_prefill_select M={M} Lcap={Lcap} keep={keep} k={top_k}",
              flush=True)
        H.hhr_hisa_prefill_select(shape, t(q8), t(q_scale), t(wt), k8d, ksd, self.reps,
                                  t(q_len), keep, top_k, self.sel, self.cnt, ws)
        torch.cuda.synchronize()
        assert H.hhr_read_device_status(ws) == 0
        # the decode path on per-row copies (all rows, or the sampled copy_rows)
        rows = np.arange(M) if copy_rows is None else np.asarray(copy_rows)
        self.rows = rows
        R = rows.size
        shape_r = H.make_hisa_shape(R, Hi, blk, Lcap)
        k8c = k8d[None].expand(R, -1, -1).contiguous()
        ksc = ksd[None].expand(R, -1).contiguous()
        ql = t(q_len[rows])
        qr8, qrs, qrw = t(q8[rows]), t(q_scale[rows]), t(wt[rows])
        self.reps_rows = torch.zeros((R, Lcap // blk, 128), dtype=torch.float32, device=dv)
        wsr = torch.zeros(H.hhr_hisa_workspace_size(shape_r, keep, top_k), dtype=torch.uint8,
                          device=dv)
        status = wsr[:4].view(torch.int32)
        H.hhr_hisa_pool_keys(shape_r, k8c, ksc, torch.zeros(R, dtype=torch.int32, device=dv), ql,
                             int(q_len[rows].max()), self.reps_rows, status)
        self.bs = torch.full((R, Lcap // blk), float("nan"), dtype=torch.float32, device=dv)
        self.kept = torch.zeros((R, keep), dtype=torch.int32, device=dv)
        self.kc = torch.zeros((R,), dtype=torch.int32, device=dv)
        self.ts = torch.full((R, keep * blk), float("nan"), dtype=torch.float32, device=dv)
        self.sel_r = torch.zeros((R, top_k), dtype=torch.int32, device=dv)
        self.cnt_r = torch.zeros((R,), dtype=torch.int32, device=dv)
        H.hhr_hisa_block_scores(shape_r, qr8, qrs, qrw, self.reps_rows, ql, self.bs, status)
        H.hhr_hisa_top_blocks(shape_r, self.bs, ql, keep, self.kept, self.kc, status)
        H.hhr_hisa_token_topk(shape_r, qr8, qrs, qrw, k8c, ksc, ql, self.kept, self.kc, keep,
                              top_k, self.sel_r, self.cnt_r, self.ts, wsr)
        sel_c = torch.zeros_like(self.sel_r)
        cnt_c = torch.zeros_like(self.cnt_r)
        H.hhr_hisa_select(shape_r, qr8, qrs, qrw, k8c, ksc, self.reps_rows, ql, keep, top_k,
                          sel_c, cnt_c, wsr)
        torch.cuda.synchronize()
        assert H.hhr_read_device_status(wsr) == 0
        self.sel_c, self.cnt_c = sel_c, cnt_c

    def check_decode_identity(self):
        """Prefill row r == the decode path at seq_len = q_len[r], bit for bit."""
        idx = torch.from_numpy(self.rows).to(self.sel.device)
        assert torch.equal(self.sel[idx], self.sel_r) and torch.equal(self.cnt[idx], self.cnt_r)
        assert torch.equal(self.sel_c, self.sel_r) and torch.equal(self.cnt_c, self.cnt_r)

    def check_row(self, i):
        """Row rows[i] against the oracle's causal prefill selection: the representatives and
        scores within their rounding tolerance, both top-k steps exact on the GPU's own
        scores, and from raw inputs the kept blocks (and then the tokens, on the GPU's kept
        blocks) differing only inside the excuse band.  Returns the excused counts."""
        r = int(self.rows[i])
        ql, blk = int(self.q_len[r]), self.blk
        res = O.prefill_select(self.q8[r], self.q_scale[r], self.wt[r], self.k8_np, self.ks_np,
                               self.Lcap, ql, blk, self.keep, self.top_k)
        q = O.dequantize(self.q8[r], self.q_scale[r])
        wt = self.wt[r]
        nb = -(-ql // blk)
        keys = O.dequantize(self.k8_np[:ql], self.ks_np[:ql])
        reps = self.reps_rows[i, :nb].cpu().numpy().astype(np.float64)
        scale = np.stack([np.abs(keys[j * blk:(j + 1) * blk]).mean(0) for j in range(nb)])
        assert np.all(np.abs(reps - res["reps"]) <= 1e-5 * scale + 1e-30), r
        bs = self.bs[i, :nb].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(bs - O.indexer_scores(q, wt, reps))
                      <= 1e-5 * _abs_terms(q, wt, reps) + 1e-30), r
        kc = int(self.kc[i])
        kept = self.kept[i, :kc].cpu().numpy()
        np.testing.assert_array_equal(kept, O.top_largest(bs, np.arange(nb), self.keep))
        S = res["block_scores"]
        n_blk = _within_band(kept, res["blocks"], lambda b: S[b], S, self.keep, ("block", r))
        cand = (kept.astype(np.int64)[:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
        valid = cand < ql
        ts = self.ts[i, :cand.size].cpu().numpy().astype(np.float64)
        assert np.all(np.isneginf(ts[~valid]))
        c = cand[valid]
        x = keys[c]
        s_or = O.indexer_scores(q, wt, x)
        assert np.all(np.abs(ts[valid] - s_or) <= 1e-5 * _abs_terms(q, wt, x) + 1e-30), r
        n = int(self.cnt_r[i])
        sel = self.sel_r[i, :n].cpu().numpy()
        np.testing.assert_array_equal(sel, O.top_largest(ts[valid], c, self.top_k))
        assert n == min(self.top_k, c.size) and torch.all(self.sel_r[i, n:] == -1)
        pos = dict(zip(c.tolist(), s_or.tolist()))
        n_tok = _within_band(sel, O.top_largest(s_or, c, self.top_k), lambda t: pos[int(t)],
                             s_or, self.top_k, ("token", r))
        if n_blk == 0:
            assert np.array_equal(c, res["cand"])
        return n_blk, n_tok


@pytest.mark.parametrize("n_rand", [41, 150], ids=["rows48", "rows150"])
@pytest.mark.parametrize("keep_all", [False, True])
def test_prefill_select(gpu_lib, keep_all, n_rand):
    """Query rows at positions across a 4000-key cache (first token, block edges, the end)
    against one shared cache: every row equals, bit for bit, the decode path at seq_len =
    its q_len on a copy of the cache pooled over its prefix (the causal reading), and
    every row is checked against the oracle's causal prefill selection (near-ties at a
    cut-off only inside the excuse band, counted); with every block kept, equal to the
    flat indexer on each row's prefix up to the band.  With 64 rows or more the block
    scores cover four 16-block groups per wave and the token scores map rows to XCDs in
    runs (a row count that is not a multiple of 8 leaves padding rows)."""
    H = gpu_lib
    print(f"\n[gpu hisa prefill] keep_all={keep_all} n_rand={n_rand}", flush=True)
    Hi, blk, Lcap, L, top_k = 16, 64, 4096, 4000, 300
    keep = Lcap // blk if keep_all else 8
    rng = np.random.default_rng(61)
    pos = np.unique(np.concatenate([[0, 62, 63, 64, 127, 128, L - 1],
                                    rng.integers(0, L, n_rand)]))
    while n_rand > 64 and pos.size % 8 != 3:  # > 64 rows, not a multiple of 8
        pos = np.delete(pos, pos.size // 2)
    q_len = (pos + 1).astype(np.int32)
    M = q_len.size
    src = synth.make_hisa_inputs(Hi, L, Lcap, 4, 62, block=blk, make_kv=False)
    qs = [synth.make_hisa_inputs(Hi, 1, 16, 4, 100 + r, block=16, make_kv=False)
          for r in range(M)]
    q8 = np.stack([x["q8"] for x in qs])
    q_scale = np.stack([x["q_scale"] for x in qs])
    wt = np.stack([x["w"] for x in qs])
    run = PrefillRun(H, src["k8"], src["k_scale"], q8, q_scale, wt, q_len, blk, keep, top_k)
    run.check_decode_identity()
    n_blk = n_tok = 0
    for i in range(M):
        b_, t_ = run.check_row(i)
        n_blk += b_
        n_tok += t_
        if keep_all:
            r = int(run.rows[i])
            s = O.indexer_scores(O.dequantize(q8[r], q_scale[r]), wt[r],
                                 O.dequantize(src["k8"][:q_len[r]], src["k_scale"][:q_len[r]]))
            flat = O.flat_select(q8[r], q_scale[r], wt[r], src["k8"], src["k_scale"],
                                 int(q_len[r]), top_k)
            n = int(run.cnt[r])
            _within_band(run.sel[r, :n].cpu().numpy(), flat, lambda t: s[t], s, top_k,
                         ("flat", r))
    print(f"excused blocks {n_blk}, tokens {n_tok} over {M} rows", flush=True)
    U.record_excused(f"hisa_prefill_4k_keepall{int(keep_all)}_rows{M}", rows=M,
                     blocks=n_blk, tokens=n_tok)


@pytest.mark.slow
@pytest.mark.parametrize("n_cap", [1024, 4096], ids=["blocks1024", "blocks4096"])
def test_top_blocks_exact_on_constructed_scores(gpu_lib, n_cap):
    """hhr_hisa_top_blocks on constructed block scores (the page top-P tests' patterns:
    ties at the cut, all equal, few values, an outlier, signed zeros) for several rows
    at once: one block per thread (up to 1024 blocks) and up to 16 per thread, each row
    equal to the oracle's (score descending, block ascending) order."""
    from tests.test_gpu_select_ties import PATTERNS, _scores
    H = gpu_lib
    dv = U.dev()
    blk = 16
    shape = H.make_hisa_shape(4, 8, blk, n_cap * blk)
    rng = np.random.Generator(np.random.PCG64(77))
    sizes = [1, 5, 777, n_cap] if n_cap == 1024 else [1, 1000, n_cap]
    checked = 0
    for pattern in PATTERNS:
        for P in (1, 5, 64, 1023):
            ns = rng.permutation(sizes * 2)[:4]
            scores = np.zeros((4, n_cap), np.float32)
            for r, n in enumerate(ns):
                scores[r, :n] = _scores(pattern, int(n), min(P, int(n)), rng)
            seq = torch.tensor(ns * blk, dtype=torch.int32, device=dv)
            kept = torch.full((4, P), 12345, dtype=torch.int32, device=dv)
            kc = torch.full((4,), -3, dtype=torch.int32, device=dv)
            status = torch.zeros(1, dtype=torch.int32, device=dv)
            H.hhr_hisa_top_blocks(shape, torch.from_numpy(scores).to(dv), seq, P, kept, kc,
                                  status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            for r, n in enumerate(ns):
                want = O.top_largest(scores[r, :n].astype(np.float64), np.arange(n), P)
                got = kept[r].cpu().numpy()
                cnt = int(kc[r])
                assert cnt == min(P, n), (pattern, n, P)
                assert got[:cnt].tolist() == want.tolist(), (pattern, n, P)
                assert (got[cnt:] == -1).all(), (pattern, n, P)
                checked += 1
    print(f"checked {checked} rows", flush=True)


def test_prefill_wide_selection(gpu_lib):
    """More than 64 rows over a cache of more than 1024 blocks, keeping more than 8192
    candidates per row: the many-row selections then hold up to 16 blocks and 16
    candidates per thread (the wide forms of k_hisa_top_blocks and k_hisa_topk).  Sampled
    rows equal the decode path at their q_len bit for bit and match the oracle's causal
    prefill selection within the band."""
    H = gpu_lib
    Hi, blk, Lcap, L, keep, top_k = 16, 16, 32768, 30000, 600, 1000
    rng = np.random.default_rng(71)
    pos = np.unique(np.concatenate([[0, 15, 16, 9599, 9600, 17000, L - 1],
                                    rng.integers(16384, L, 70)]))
    q_len = (pos + 1).astype(np.int32)
    M = q_len.size
    assert M > 64 and keep * blk > 8192 and Lcap // blk > 1024
    src = synth.make_hisa_inputs(Hi, L, Lcap, 4, 72, block=blk, make_kv=False)
    qs = [synth.make_hisa_inputs(Hi, 1, 16, 4, 300 + r, block=16, make_kv=False)
          for r in range(M)]
    q8 = np.stack([x["q8"] for x in qs])
    q_scale = np.stack([x["q_scale"] for x in qs])
    wt = np.stack([x["w"] for x in qs])
    mid = np.flatnonzero(q_len % blk != 0)
    sample = np.unique(np.concatenate([[0, 1, 2, 3, 4, M - 1], rng.choice(mid, 4, replace=False)]))
    print(f"\n[gpu hisa prefill wide] M={M} keep={keep} block={blk} sampled rows "
          f"{sample.tolist()}", flush=True)
    run = PrefillRun(H, src["k8"], src["k_scale"], q8, q_scale, wt, q_len, blk, keep, top_k,
                     copy_rows=sample)
    run.check_decode_identity()
    n_blk = n_tok = 0
    for i in range(sample.size):
        b_, t_ = run.check_row(i)
        n_blk += b_
        n_tok += t_
    print(f"excused blocks {n_blk}, tokens {n_tok} over {sample.size} rows", flush=True)
    U.record_excused("hisa_prefill_32k_wide_sampled", rows=int(sample.size), blocks=n_blk,
                     tokens=n_tok)


def test_prefill_bench_shape_sampled_rows(gpu_lib):
    """The bench's prefill shape: 512 rows at positions drawn over a 131072-key prompt
    (64 fp8 index heads, blocks of 128, 64 kept blocks, top-2048), in one call.  Sampled
    rows (the first, the last, and rows ending mid-block) equal the decode path at their
    q_len bit for bit and match the oracle's causal prefill selection within the band."""
    H = gpu_lib
    w = synth.HISA_WORKLOADS["hisa_128k"]
    rows = synth.make_hisa_prefill_rows("hisa_prefill_128k")
    src = synth.make_hisa_workload_inputs("hisa_128k", make_kv=False)
    q_len = rows["q_len"]
    M = q_len.size
    rng = np.random.default_rng(5)
    mid = np.flatnonzero(q_len % w.block != 0)
    sample = np.unique(np.concatenate([[0, M - 1], rng.choice(mid, 10, replace=False)]))
    print(f"\n[gpu hisa prefill bench shape] M={M} sampled rows {sample.tolist()}", flush=True)
    run = PrefillRun(H, src["k8"], src["k_scale"], rows["q8"], rows["q_scale"], rows["w"], q_len,
                     w.block, w.keep_blocks, w.top_k, copy_rows=sample)
    run.check_decode_identity()
    n_blk = n_tok = 0
    for i in range(sample.size):
        b_, t_ = run.check_row(i)
        n_blk += b_
        n_tok += t_
    print(f"excused blocks {n_blk}, tokens {n_tok} over {sample.size} rows", flush=True)
    U.record_excused("hisa_prefill_128k_sampled", rows=int(sample.size), blocks=n_blk,
                     tokens=n_tok)
