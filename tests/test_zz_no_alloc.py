"""hhr_decode_no_alloc (the decode step with the library's static scratch instead of a
caller workspace) against hhr_decode on the same inputs, bit for bit, on two calls in a row
whose second one is smaller: first the 33-sequence batch (the staged composition, 8 KV
heads, 8192-key cache), then a 2-sequence single-launch case; then the first shape again,
so the scratch left by a smaller call is cleared where it must be."""
import numpy as np
import pytest
import torch

from hash_hierarchical_top_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _pipeline(H, B, Hq, Hkv, Lcap, top_k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(1, Lcap + 1, B)
    lens[0] = Lcap
    inp = synth.make_hhr_inputs(B, Hq, Hkv, lens.tolist(), Lcap, "bf16", seed=seed)
    p = U.Pipeline(H, inp, "bf16", Hq, Hkv, Lcap, 1, 4, 0, top_k)
    p.append_all()
    torch.cuda.synchronize()
    return p


def _compare(H, p):
    ref_sel, ref_sc = torch.zeros_like(p.sel), torch.zeros_like(p.sel_count)
    ref_out = torch.zeros_like(p.out)
    p.decode(ref_sel, ref_sc, ref_out)
    sel = torch.full_like(p.sel, 77)
    sc = torch.full_like(p.sel_count, -5)
    out = torch.full_like(p.out, 9.0)
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    H.hhr_decode_no_alloc(p.shape, p.d["q"], p.d["seq_len"], p.d["R"], p.d["W"], p.codes, p.meta,
                          p.d["K"], p.d["V"], *p.keep, p.top_k, p.scale, sel, sc, out, status)
    torch.cuda.synchronize()
    assert p.status() == 0 and int(status[0]) == 0
    assert torch.equal(sel, ref_sel) and torch.equal(sc, ref_sc) and torch.equal(out, ref_out)
    assert int(sc.min()) > 0


def test_no_alloc_decode_equals_decode(gpu_lib):
    H = gpu_lib
    print("\n[gpu no-alloc decode] 33 x 8 heads x 8192, then 2 x 2 heads x 2048", flush=True)
    wide = _pipeline(H, 33, 32, 8, 8192, 256, 41)
    small = _pipeline(H, 2, 8, 2, 2048, 128, 42)
    assert H.hhr_workspace_size(small.shape, 1, 4, 0, 128) < \
        H.hhr_workspace_size(wide.shape, 1, 4, 0, 256)
    _compare(H, wide)
    _compare(H, small)
    _compare(H, wide)


def test_no_alloc_decode_reports_device_errors(gpu_lib):
    """A seq_len past max_ctx empties that sequence and sets HHR_DEV_BAD_SEQ_LEN in the
    caller's status word; the next call (clean) reports nothing."""
    H = gpu_lib
    p = _pipeline(H, 2, 8, 2, 2048, 128, 43)
    bad = torch.tensor([p.Lcap + 16, 100], dtype=torch.int32, device="cuda")
    sel, sc = torch.zeros_like(p.sel), torch.full_like(p.sel_count, 7)
    out = torch.full_like(p.out, 3.0)
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    H.hhr_decode_no_alloc(p.shape, p.d["q"], bad, p.d["R"], p.d["W"], p.codes, p.meta, p.d["K"],
                          p.d["V"], *p.keep, p.top_k, p.scale, sel, sc, out, status)
    torch.cuda.synchronize()
    assert int(status[0]) & H.HHR_DEV_BAD_SEQ_LEN
    assert int(sc[0].max()) == 0 and torch.all(out[0] == 0)
    assert int(sc[1].min()) > 0 and int(sc[1].max()) <= 100
    _compare(H, p)
