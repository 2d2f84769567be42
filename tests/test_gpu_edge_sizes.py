"""GPU parity at the edges of the supported sizes, through the C ABI:

- the candidate limit: the 32K Llama-3.1-8B-shaped step with every page kept
  (2048 pages x 16 = 32768 candidates per KV head, exactly the largest supported
  count) and top_k 4096 -- the LHP-only point of the stage sweep;
- the fused one-token append at the full 128K shape (256 pages per scoring
  workgroup, the appended key encoded inside the coarse launch), with f32 and
  bf16 page metadata.
"""
import numpy as np
import pytest
import torch

from hash_hierarchical_top_amd import synth
from oracle import hhr as O
from tests import gpu_util as U
from tests.test_gpu_hhr import _check_decode_append, _decode_append_run

pytestmark = pytest.mark.gpu


def test_hamming_topk_at_the_candidate_limit(gpu_lib):
    """32768 candidates per KV head: the staged stages, hhr_select (one launch) and hhr_decode
    (every attention workgroup picking its keys from 128 cumulative-histogram blocks) agree
    bit for bit; the selection of every KV head is exact against the oracle on the GPU's
    codes, and attention on sampled heads is within 2e-3 of fp64."""
    print("\n[gpu candidate limit] llama8b_32k, keep all pages, top_k 4096", flush=True)
    w = synth.WORKLOADS["llama8b_32k"]
    inp = synth.make_workload_inputs("llama8b_32k")
    p = U.Pipeline(gpu_lib, inp, w.kv_dtype, w.n_q_heads, w.n_kv_heads, w.max_ctx, 1, 1, 0, 4096)
    assert p.p_max * 16 == 32768
    p.append_all()
    p.encode_queries()
    p.page_scores()
    p.top_pages()
    p.hamming_topk()
    p.sparse_decode()
    torch.cuda.synchronize()
    assert p.status() == 0
    kept, kc = p.kept.cpu().numpy(), p.kept_count.cpu().numpy()
    codes, q_codes = U.u32(p.codes), U.u32(p.q_codes)
    sel, sc = p.sel.cpu().numpy(), p.sel_count.cpu().numpy()
    L = int(inp["seq_len"][0])
    for g in range(p.Hkv):
        assert kc[0, g] == 2048 and kept[0, g].tolist() == list(range(2048))
        res = O.select_from_codes(q_codes[0, g * p.G:(g + 1) * p.G], codes[0, g], kept[0, g], L,
                                  16, p.top_k)
        assert res["cand"].size == 32768
        assert sc[0, g] == 4096 and sel[0, g].tolist() == res["sel"].tolist()
    s2, c2 = p.select()
    assert torch.equal(s2, p.sel) and torch.equal(c2, p.sel_count)
    s3, c3, o3 = torch.zeros_like(p.sel), torch.zeros_like(p.sel_count), torch.zeros_like(p.out)
    p.decode(s3, c3, o3)
    torch.cuda.synchronize()
    assert p.status() == 0
    assert torch.equal(s3, p.sel) and torch.equal(c3, p.sel_count) and torch.equal(o3, p.out)
    out = p.out.cpu().numpy().astype(np.float64)
    for g in (0, p.Hkv - 1):
        idx = sel[0, g]
        want = O.attend(p.q_group(0, g), p.K_valid(0, g)[idx], p.V_valid(0, g)[idx], p.scale)
        assert np.abs(out[0, g * p.G:(g + 1) * p.G] - want).max() <= 2e-3


@pytest.mark.parametrize("meta_dtype", ["f32", "bf16"])
def test_decode_append_128k(gpu_lib, meta_dtype):
    """hhr_decode_append on the 128K Llama-shaped step: every row but the last encoded by
    hhr_append_keys, then one fused append + decode.  The new key's code and its page's
    metadata on sampled KV heads against the oracle, every other row and page untouched,
    and the staged stages on the updated cache equal the fused call bit for bit."""
    print(f"\n[gpu decode_append 128k] meta={meta_dtype}", flush=True)
    w = synth.WORKLOADS["llama8b_128k"]
    inp = synth.make_workload_inputs("llama8b_128k")
    p = U.Pipeline(gpu_lib, inp, w.kv_dtype, w.n_q_heads, w.n_kv_heads, w.max_ctx, w.keep_num,
                   w.keep_den, w.keep_pages_abs, w.top_k, meta_dtype=meta_dtype)
    lens, codes0, meta0, sel, sc, out = _decode_append_run(gpu_lib, p)
    _check_decode_append(p, lens, meta_dtype, codes0, meta0, sel, sc, out,
                         [(0, 0), (0, 3), (0, p.Hkv - 1)])
