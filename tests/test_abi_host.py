"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before anything reaches the GPU.

Nothing here launches a kernel: every call either is a pure host function or
fails argument validation (fake but aligned addresses are never dereferenced).
"""
import ctypes
import os
import re

import pytest

from oracle import hhr as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hhr.h")


@pytest.fixture(scope="module")
def H():
    from hash_hierarchical_top_amd import hhr

    if not os.path.exists(hhr.LIB_PATH):
        pytest.fail("libhhr.so is not built (run __graft_entry__.build())")
    hhr.load()
    return hhr


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hhr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("hhr_append_keys", "hhr_select", "hhr_sparse_decode", "hhr_decode",
              "hhr_hisa_select", "hhr_page_scores", "hhr_top_pages", "hhr_hamming_topk"):
        assert n in names


def test_every_declared_symbol_is_exported(H):
    lib = ctypes.CDLL(H.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol(H):
    assert sorted(H.EXPORTED) == _declared()
    for n in _declared():
        if n not in ("hhr_status_string", "hhr_last_error", "hhr_abi_version"):
            assert callable(getattr(H, n)), n


def test_status_strings_and_version(H):
    lib = H.load()
    assert lib.hhr_status_string(0) == b"HHR_OK"
    assert lib.hhr_status_string(-3) == b"HHR_ERR_WORKSPACE"
    assert lib.hhr_abi_version() == H.ABI_VERSION


@pytest.mark.parametrize("n", [0, 1, 2, 3, 10, 255, 256, 513, 2048, 2049, 8192, 16384])
@pytest.mark.parametrize("num,den,absn", [(1, 4, 0), (1, 8, 0), (3, 8, 0), (1, 1, 0), (0, 1, 64),
                                          (5, 7, 0)])
def test_keep_count_matches_oracle(H, n, num, den, absn):
    assert H.hhr_keep_count(n, num, den, absn) == O.keep_count(n, num, den, absn)


def test_workspace_size(H):
    s = H.make_shape(1, 32, 8, 131072, "bf16")
    ws = H.hhr_workspace_size(s, 1, 8, 0, 4096)
    # q_rot + q codes + scores (8 x 8192 f32) + kept (8 x 1024) + split-K partials
    assert ws > 8 * 8192 * 4 + 8 * 1024 * 4
    assert ws % 256 == 0
    assert H.hhr_workspace_size(H.make_shape(1, 32, 8, 131072, "bf16"), 0, 8, 0, 4096) == 0
    assert H.hhr_workspace_size(H.make_shape(1, 32, 8, 131072, "bf16"), 1, 8, 0, 0) == 0
    assert H.hhr_workspace_size(H.make_shape(1, 32, 8, 1000, "bf16"), 1, 8, 0, 64) == 0
    # more than 32768 candidates per KV head is unsupported
    assert H.hhr_workspace_size(H.make_shape(1, 4, 1, 262144, "bf16"), 1, 4, 0, 64) == 0
    hs = H.make_hisa_shape(1, 64, 128, 131072)
    assert H.hhr_hisa_workspace_size(hs, 64, 2048) > 1024 * 4
    assert H.hhr_hisa_workspace_size(hs, 1000, 2048) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation rejects first


def _status(fn, *args, **kw):
    from hash_hierarchical_top_amd import hhr

    with pytest.raises(hhr.HHRError) as ei:
        fn(*args, **kw)
    return ei.value.status


def test_shape_errors(H):
    good = dict(batch=1, n_q_heads=8, n_kv_heads=2, max_ctx=1024, kv_dtype="bf16")
    cases = [
        (dict(good, n_q_heads=6, n_kv_heads=4), H.HHR_ERR_INVALID_ARG),
        (dict(good, batch=0), H.HHR_ERR_INVALID_ARG),
        (dict(good, max_ctx=1000), H.HHR_ERR_INVALID_ARG),
        (dict(good, max_ctx=1 << 20), H.HHR_ERR_UNSUPPORTED),
        (dict(good, n_q_heads=64, n_kv_heads=2), H.HHR_ERR_UNSUPPORTED),
        (dict(good, kv_dtype=7), H.HHR_ERR_INVALID_ARG),
        (dict(good, meta_dtype=2), H.HHR_ERR_INVALID_ARG),
    ]
    for kw, want in cases:
        s = H.make_shape(**kw)
        assert _status(H.hhr_encode_queries, s, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0) == want
    s = H.make_shape(**good)
    s.head_dim = 64
    assert _status(H.hhr_encode_queries, s, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0) == \
        H.HHR_ERR_UNSUPPORTED
    s = H.make_shape(**good)
    s.page_size = 32
    assert _status(H.hhr_encode_queries, s, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0) == \
        H.HHR_ERR_UNSUPPORTED
    for bits in (0, 32, 96, 192, 512):
        s = H.make_shape(**good, code_bits=bits)
        assert _status(H.hhr_encode_queries, s, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0) == \
            H.HHR_ERR_UNSUPPORTED, bits


def test_workspace_grows_with_code_bits(H):
    """Query codes (nw words per query head) and the H histograms (code_bits * G + 1 bins per
    KV head) scale with the code width; every other region is the same."""
    sizes = {bits: H.hhr_workspace_size(H.make_shape(2, 32, 8, 131072, "bf16", code_bits=bits),
                                        1, 8, 0, 4096)
             for bits in (64, 128, 256)}
    assert 0 < sizes[64] < sizes[128] < sizes[256]


def test_pointer_errors(H):
    s = H.make_shape(1, 8, 2, 1024, "bf16")
    assert _status(H.hhr_encode_queries, s, None, FAKE, FAKE, FAKE, FAKE, stream=0) == \
        H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_encode_queries, s, FAKE + 4, FAKE, FAKE, FAKE, FAKE, stream=0) == \
        H.HHR_ERR_INVALID_ARG
    assert "q is not 16-byte aligned" in H.load().hhr_last_error().decode()
    assert _status(H.hhr_append_keys, s, FAKE, FAKE, FAKE, 10, FAKE, FAKE, None, FAKE,
                   stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_append_keys, s, FAKE, FAKE, FAKE, 5000, FAKE, FAKE, FAKE, FAKE,
                   stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_page_scores, s, FAKE, None, FAKE, FAKE, stream=0) == \
        H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_sparse_decode, s, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0.0, FAKE, FAKE,
                   workspace_bytes=1 << 20, stream=0) == H.HHR_ERR_INVALID_ARG


def test_selection_parameter_errors(H):
    s = H.make_shape(1, 8, 2, 1024, "bf16")
    args = (s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _status(H.hhr_select, *args, 0, 4, 0, 16, FAKE, FAKE, FAKE, workspace_bytes=1 << 30,
                   stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_select, *args, 5, 4, 0, 16, FAKE, FAKE, FAKE, workspace_bytes=1 << 30,
                   stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_select, *args, 1, 4, 0, 0, FAKE, FAKE, FAKE, workspace_bytes=1 << 30,
                   stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_select, *args, 1, 4, -1, 16, FAKE, FAKE, FAKE, workspace_bytes=1 << 30,
                   stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_top_pages, s, FAKE, FAKE, 2, 1, 0, FAKE, FAKE, stream=0) == \
        H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_hamming_topk, s, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, FAKE, FAKE, None,
                   FAKE, workspace_bytes=4096, stream=0) == H.HHR_ERR_INVALID_ARG


def test_workspace_errors(H):
    s = H.make_shape(1, 8, 2, 1024, "bf16")
    need = H.hhr_workspace_size(s, 1, 4, 0, 128)
    assert need > 0
    assert _status(H.hhr_select, s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 0, 128, FAKE, FAKE,
                   FAKE, workspace_bytes=need - 1, stream=0) == H.HHR_ERR_WORKSPACE
    assert _status(H.hhr_decode, s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 0, 128,
                   0.088, FAKE, FAKE, FAKE, FAKE, workspace_bytes=need - 256, stream=0) == \
        H.HHR_ERR_WORKSPACE
    assert _status(H.hhr_sparse_decode, s, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 0.088, FAKE, FAKE,
                   workspace_bytes=512, stream=0) == H.HHR_ERR_WORKSPACE
    # the fine top-k keeps per-chunk histograms (and, without dist, the
    # distances) in the workspace: a control block alone is too small
    p_max = H.hhr_keep_count(1024 // 16, 1, 4, 0)
    for dist in (None, FAKE):
        assert _status(H.hhr_hamming_topk, s, FAKE, FAKE, FAKE, FAKE, FAKE, p_max, 128, FAKE,
                       FAKE, dist, FAKE, workspace_bytes=4096, stream=0) == H.HHR_ERR_WORKSPACE


def test_select_pages_errors(H):
    s = H.make_shape(1, 8, 2, 1024, "bf16", meta_dtype="bf16")
    need = H.hhr_workspace_size(s, 1, 4, 0, 1)
    assert need > 0
    args = (s, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _status(H.hhr_select_pages, *args, 1, 4, 0, FAKE, FAKE, None, FAKE,
                   workspace_bytes=need - 1, stream=0) == H.HHR_ERR_WORKSPACE
    assert _status(H.hhr_select_pages, *args, 1, 4, 0, None, FAKE, None, FAKE,
                   workspace_bytes=need, stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_select_pages, *args, 1, 4, 0, FAKE, FAKE, FAKE + 8, FAKE,
                   workspace_bytes=need, stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_select_pages, *args, 3, 2, 0, FAKE, FAKE, None, FAKE,
                   workspace_bytes=need, stream=0) == H.HHR_ERR_INVALID_ARG


def test_metadata_layouts(H):
    s = H.make_shape(2, 8, 2, 1024, "bf16")
    assert H.meta_shape(s) == (2, 2, 64, 128, 2)
    s = H.make_shape(2, 8, 2, 1024, "bf16", meta_dtype="bf16")
    assert H.meta_shape(s) == (2, 2, 64, 128)


def test_hisa_errors(H):
    good = H.make_hisa_shape(1, 64, 128, 131072)
    bad_heads = H.make_hisa_shape(1, 65, 128, 131072)
    bad_block = H.make_hisa_shape(1, 64, 100, 131000)
    bad_ctx = H.make_hisa_shape(1, 64, 128, 131000)
    for s, want in ((bad_heads, H.HHR_ERR_UNSUPPORTED), (bad_block, H.HHR_ERR_UNSUPPORTED),
                    (bad_ctx, H.HHR_ERR_INVALID_ARG)):
        assert _status(H.hhr_hisa_block_scores, s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                       stream=0) == want
    assert _status(H.hhr_hisa_select, good, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2048,
                   FAKE, FAKE, FAKE, workspace_bytes=64, stream=0) == H.HHR_ERR_WORKSPACE
    assert _status(H.hhr_hisa_select, good, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 200, 2048,
                   FAKE, FAKE, FAKE, workspace_bytes=1 << 30, stream=0) == H.HHR_ERR_UNSUPPORTED
    assert _status(H.hhr_hisa_pool_keys, good, FAKE, FAKE, FAKE, FAKE, -1, FAKE,
                   stream=0) == H.HHR_ERR_INVALID_ARG


def test_documented_selection_limits(H):
    """The header's selection limits: p_max * 16 <= 32768 candidates per (b, g) and
    top_k <= 32768 (HISA: keep_blocks * block and top_k <= 16384).  At the limit the
    workspace size is positive; one step past it every entry point returns
    HHR_ERR_UNSUPPORTED and hhr_workspace_size returns 0."""
    at = H.make_shape(1, 32, 8, 32768, "bf16")       # 2048 pages, all kept: 32768 candidates
    past = H.make_shape(1, 32, 8, 32784, "bf16")     # 2049 pages: 32784 candidates
    assert H.hhr_workspace_size(at, 1, 1, 0, 4096) > 0
    assert H.hhr_workspace_size(at, 1, 1, 0, 32768) > 0
    assert H.hhr_workspace_size(past, 1, 1, 0, 4096) == 0
    assert H.hhr_workspace_size(past, 0, 1, 2049, 4096) == 0
    assert H.hhr_workspace_size(past, 0, 1, 2048, 4096) > 0
    assert H.hhr_workspace_size(at, 1, 1, 0, 32769) == 0
    # 262144 keys: keeping 1/8 of the pages is the most that fits
    assert H.hhr_workspace_size(H.make_shape(1, 32, 8, 262144, "bf16"), 1, 8, 0, 4096) > 0
    assert H.hhr_workspace_size(H.make_shape(1, 32, 8, 262144, "bf16"), 1, 4, 0, 4096) == 0
    big = 1 << 34
    sel = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for shape, keep, k in ((past, (1, 1, 0), 4096), (past, (0, 1, 2049), 4096),
                           (at, (1, 1, 0), 32769)):
        assert _status(H.hhr_select, shape, *sel, *keep, k, FAKE, FAKE, FAKE,
                       workspace_bytes=big, stream=0) == H.HHR_ERR_UNSUPPORTED
        assert _status(H.hhr_decode, shape, *sel, FAKE, FAKE, *keep, k, 0.088, FAKE, FAKE, FAKE,
                       FAKE, workspace_bytes=big, stream=0) == H.HHR_ERR_UNSUPPORTED
        if shape is past:  # hhr_select_pages takes no top_k: only the page limit applies
            assert _status(H.hhr_select_pages, shape, FAKE, FAKE, FAKE, FAKE, FAKE, *keep, FAKE,
                           FAKE, None, FAKE, workspace_bytes=big, stream=0) == \
                H.HHR_ERR_UNSUPPORTED
    assert _status(H.hhr_sparse_decode, at, FAKE, FAKE, FAKE, FAKE, FAKE, 32769, 0.088, FAKE,
                   FAKE, workspace_bytes=big, stream=0) == H.HHR_ERR_UNSUPPORTED
    assert _status(H.hhr_hamming_topk, past, FAKE, FAKE, FAKE, FAKE, FAKE, 2049, 64, FAKE, FAKE,
                   None, FAKE, workspace_bytes=big, stream=0) == H.HHR_ERR_UNSUPPORTED
    hs = H.make_hisa_shape(1, 64, 128, 131072)
    assert H.hhr_hisa_workspace_size(hs, 128, 2048) > 0       # 16384 candidates
    assert H.hhr_hisa_workspace_size(hs, 129, 2048) == 0
    assert H.hhr_hisa_workspace_size(hs, 64, 16385) == 0
    assert _status(H.hhr_hisa_select, hs, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 16385,
                   FAKE, FAKE, FAKE, workspace_bytes=big, stream=0) == H.HHR_ERR_UNSUPPORTED


def test_no_alloc_decode_host_checks(H):
    """hhr_decode_no_alloc: the static scratch holds 64 MiB; a shape whose workspace is larger
    is rejected with HHR_ERR_UNSUPPORTED before anything reaches the GPU, as are bad
    arguments (the ragged 16-sequence 64K workload, 63.8 MiB, fits)."""
    assert H.hhr_no_alloc_scratch_bytes() == 64 << 20
    fits = H.make_shape(16, 32, 8, 65536, "bf16")
    assert 0 < H.hhr_workspace_size(fits, 1, 4, 0, 2048) <= 64 << 20
    big = H.make_shape(32, 32, 8, 65536, "bf16")
    assert H.hhr_workspace_size(big, 1, 4, 0, 2048) > 64 << 20
    args = (FAKE,) * 8
    assert _status(H.hhr_decode_no_alloc, big, *args, 1, 4, 0, 2048, 0.088, FAKE, FAKE, FAKE,
                   None, stream=0) == H.HHR_ERR_UNSUPPORTED
    assert "static scratch" in H.load().hhr_last_error().decode()
    assert _status(H.hhr_decode_no_alloc, fits, *args, 1, 4, 0, 2048, 0.0, FAKE, FAKE, FAKE,
                   None, stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_decode_no_alloc, fits, *args, 1, 4, 0, 2048, 0.088, FAKE, None, FAKE,
                   None, stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_decode_no_alloc, fits, *args, 1, 4, 0, 2048, 0.088, FAKE, FAKE, FAKE,
                   FAKE + 4, stream=0) == H.HHR_ERR_INVALID_ARG
    assert _status(H.hhr_decode_no_alloc, fits, *args, 0, 4, 0, 2048, 0.088, FAKE, FAKE, FAKE,
                   None, stream=0) == H.HHR_ERR_INVALID_ARG
