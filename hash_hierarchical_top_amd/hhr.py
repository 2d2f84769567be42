"""Thin ctypes binding of libhhr.so.

Every function here has the name of the C entry point it calls (declared in
include/hhr.h) and only marshals arguments: torch tensors become device
pointers, a torch stream becomes its hipStream_t, and a non-OK status becomes
an HHRError.  All computation happens in the library's HIP kernels; there is
no fallback path, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libhhr.so")

HHR_OK = 0
HHR_ERR_INVALID_ARG = -1
HHR_ERR_UNSUPPORTED = -2
HHR_ERR_WORKSPACE = -3
HHR_ERR_HIP = -4
HHR_F32 = 0
HHR_BF16 = 1
ABI_VERSION = 5  # the include/hhr.h declarations this binding mirrors
HHR_DEV_BAD_SEQ_LEN = 0x1
HHR_DEV_BAD_INDEX = 0x2

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t
c_f32 = ctypes.c_float


class hhr_shape(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("code_bits", c_i32), ("page_size", c_i32),
                ("max_ctx", c_i32), ("kv_dtype", c_i32), ("meta_dtype", c_i32)]


class hhr_hisa_shape(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("n_index_heads", c_i32), ("head_dim", c_i32),
                ("block", c_i32), ("max_ctx", c_i32)]


class HHRError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {_status_name(status)}: {detail}")


_LIB: Optional[ctypes.CDLL] = None

# name -> (restype, argtypes)
_SIGS = {
    "hhr_status_string": (ctypes.c_char_p, [c_i32]),
    "hhr_last_error": (ctypes.c_char_p, []),
    "hhr_abi_version": (c_i32, []),
    "hhr_keep_count": (c_i32, [c_i32, c_i32, c_i32, c_i32]),
    "hhr_workspace_size": (c_size, [c_vp, c_i32, c_i32, c_i32, c_i32]),
    "hhr_read_device_status": (c_i32, [c_vp, c_vp, ctypes.POINTER(ctypes.c_uint32)]),
    "hhr_append_keys": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "hhr_encode_queries": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "hhr_page_scores": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "hhr_top_pages": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "hhr_hamming_topk": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp,
                                 c_vp, c_vp, c_size, c_vp]),
    "hhr_sparse_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_f32, c_vp, c_vp,
                                  c_size, c_vp]),
    "hhr_select_pages": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp,
                                 c_vp, c_vp, c_vp, c_size, c_vp]),
    "hhr_select": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                           c_vp, c_vp, c_vp, c_size, c_vp]),
    "hhr_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                           c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "hhr_decode_append": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                  c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_size,
                                  c_vp]),
    "hhr_decode_no_alloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                    c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "hhr_no_alloc_scratch_bytes": (c_size, []),
    "hhr_hisa_workspace_size": (c_size, [c_vp, c_i32, c_i32]),
    "hhr_hisa_pool_keys": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "hhr_hisa_block_scores": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "hhr_hisa_top_blocks": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "hhr_hisa_token_topk": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                    c_i32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "hhr_hisa_prefill_select": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                        c_i32, c_vp, c_vp, c_vp, c_size, c_vp]),
    "hhr_hisa_select": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                c_vp, c_vp, c_vp, c_size, c_vp]),
}

EXPORTED = tuple(_SIGS)


def load() -> ctypes.CDLL:
    """Load libhhr.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise HHRError(HHR_ERR_HIP, "load",
                           f"{LIB_PATH} is missing; build it with "
                           "`python -m hash_hierarchical_top_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.hhr_abi_version() != ABI_VERSION:
            raise HHRError(HHR_ERR_INVALID_ARG, "load",
                           f"{LIB_PATH} has ABI version {lib.hhr_abi_version()}, this binding "
                           f"expects {ABI_VERSION}; rebuild it")
        _LIB = lib
    return _LIB


def _status_name(st: int) -> str:
    return {0: "HHR_OK", -1: "HHR_ERR_INVALID_ARG", -2: "HHR_ERR_UNSUPPORTED",
            -3: "HHR_ERR_WORKSPACE", -4: "HHR_ERR_HIP"}.get(st, f"status {st}")


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name: str, *args) -> None:
    st = getattr(load(), name)(*args)
    if st != HHR_OK:
        raise HHRError(st, name, load().hhr_last_error().decode())


def make_shape(batch, n_q_heads, n_kv_heads, max_ctx, kv_dtype, head_dim=128, code_bits=128,
               page_size=16, meta_dtype="f32") -> hhr_shape:
    dt = {"f32": HHR_F32, "bf16": HHR_BF16}
    return hhr_shape(batch, n_q_heads, n_kv_heads, head_dim, code_bits, page_size, max_ctx,
                     dt.get(kv_dtype, kv_dtype), dt.get(meta_dtype, meta_dtype))


def meta_shape(shape: hhr_shape) -> tuple:
    """Shape of the page-metadata tensor for `shape` (f32 elements for HHR_F32,
    int32 words for HHR_BF16: one {min, max} bfloat16 pair each)."""
    base = (shape.batch, shape.n_kv_heads, shape.max_ctx // shape.page_size, shape.head_dim)
    return base + (2,) if shape.meta_dtype == HHR_F32 else base


def make_hisa_shape(batch, n_index_heads, block, max_ctx, head_dim=128) -> hhr_hisa_shape:
    return hhr_hisa_shape(batch, n_index_heads, head_dim, block, max_ctx)


# --------------------------------------------------------------------- host queries
def hhr_keep_count(n_pages: int, keep_num: int, keep_den: int, keep_pages_abs: int = 0) -> int:
    return int(load().hhr_keep_count(n_pages, keep_num, keep_den, keep_pages_abs))


def hhr_workspace_size(shape: hhr_shape, keep_num: int, keep_den: int, keep_pages_abs: int,
                       top_k: int) -> int:
    return int(load().hhr_workspace_size(ctypes.byref(shape), keep_num, keep_den,
                                         keep_pages_abs, top_k))


def hhr_hisa_workspace_size(shape: hhr_hisa_shape, keep_blocks: int, top_k: int) -> int:
    return int(load().hhr_hisa_workspace_size(ctypes.byref(shape), keep_blocks, top_k))


def hhr_read_device_status(workspace, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _call("hhr_read_device_status", _ptr(workspace), _stream(stream), ctypes.byref(flags))
    return int(flags.value)


# --------------------------------------------------------------------- HHR steps
def hhr_append_keys(shape, k_cache, start, n_new, max_new, R, W, codes, page_meta,
                    status_word=None, stream=None) -> None:
    _call("hhr_append_keys", ctypes.byref(shape), _ptr(k_cache), _ptr(start), _ptr(n_new),
          int(max_new), _ptr(R), _ptr(W), _ptr(codes), _ptr(page_meta), _ptr(status_word),
          _stream(stream))


def hhr_encode_queries(shape, q, R, W, q_rot, q_codes, stream=None) -> None:
    _call("hhr_encode_queries", ctypes.byref(shape), _ptr(q), _ptr(R), _ptr(W), _ptr(q_rot),
          _ptr(q_codes), _stream(stream))


def hhr_page_scores(shape, q_rot, seq_len, page_meta, scores, status_word=None,
                    stream=None) -> None:
    _call("hhr_page_scores", ctypes.byref(shape), _ptr(q_rot), _ptr(seq_len), _ptr(page_meta),
          _ptr(scores), _ptr(status_word), _stream(stream))


def hhr_top_pages(shape, scores, seq_len, keep_num, keep_den, keep_pages_abs, kept, kept_count,
                  status_word=None, stream=None) -> None:
    _call("hhr_top_pages", ctypes.byref(shape), _ptr(scores), _ptr(seq_len), keep_num, keep_den,
          keep_pages_abs, _ptr(kept), _ptr(kept_count), _ptr(status_word), _stream(stream))


def hhr_hamming_topk(shape, q_codes, codes, seq_len, kept, kept_count, p_max, top_k, sel_idx,
                     sel_count, dist, workspace, workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_hamming_topk", ctypes.byref(shape), _ptr(q_codes), _ptr(codes), _ptr(seq_len),
          _ptr(kept), _ptr(kept_count), int(p_max), int(top_k), _ptr(sel_idx), _ptr(sel_count),
          _ptr(dist), _ptr(workspace), wb, _stream(stream))


def hhr_sparse_decode(shape, q, k_cache, v_cache, sel_idx, sel_count, top_k, scale, out,
                      workspace, workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_sparse_decode", ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
          _ptr(sel_idx), _ptr(sel_count), int(top_k), float(scale), _ptr(out), _ptr(workspace),
          wb, _stream(stream))


def hhr_select_pages(shape, q, seq_len, R, W, page_meta, keep_num, keep_den, keep_pages_abs,
                     kept, kept_count, q_codes, workspace, workspace_bytes=None,
                     stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_select_pages", ctypes.byref(shape), _ptr(q), _ptr(seq_len), _ptr(R), _ptr(W),
          _ptr(page_meta), keep_num, keep_den, keep_pages_abs, _ptr(kept), _ptr(kept_count),
          _ptr(q_codes), _ptr(workspace), wb, _stream(stream))


def hhr_select(shape, q, seq_len, R, W, codes, page_meta, keep_num, keep_den, keep_pages_abs,
               top_k, sel_idx, sel_count, workspace, workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_select", ctypes.byref(shape), _ptr(q), _ptr(seq_len), _ptr(R), _ptr(W),
          _ptr(codes), _ptr(page_meta), keep_num, keep_den, keep_pages_abs, int(top_k),
          _ptr(sel_idx), _ptr(sel_count), _ptr(workspace), wb, _stream(stream))


def hhr_decode(shape, q, seq_len, R, W, codes, page_meta, k_cache, v_cache, keep_num, keep_den,
               keep_pages_abs, top_k, scale, sel_idx, sel_count, out, workspace,
               workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_decode", ctypes.byref(shape), _ptr(q), _ptr(seq_len), _ptr(R), _ptr(W),
          _ptr(codes), _ptr(page_meta), _ptr(k_cache), _ptr(v_cache), keep_num, keep_den,
          keep_pages_abs, int(top_k), float(scale), _ptr(sel_idx), _ptr(sel_count), _ptr(out),
          _ptr(workspace), wb, _stream(stream))

def hhr_decode_append(shape, q, seq_len, R, W, codes, page_meta, k_cache, v_cache, keep_num,
                      keep_den, keep_pages_abs, top_k, scale, sel_idx, sel_count, out, workspace,
                      workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_decode_append", ctypes.byref(shape), _ptr(q), _ptr(seq_len), _ptr(R), _ptr(W),
          _ptr(codes), _ptr(page_meta), _ptr(k_cache), _ptr(v_cache), keep_num, keep_den,
          keep_pages_abs, int(top_k), float(scale), _ptr(sel_idx), _ptr(sel_count), _ptr(out),
          _ptr(workspace), wb, _stream(stream))


def hhr_decode_no_alloc(shape, q, seq_len, R, W, codes, page_meta, k_cache, v_cache, keep_num,
                        keep_den, keep_pages_abs, top_k, scale, sel_idx, sel_count, out,
                        status_word=None, stream=None) -> None:
    _call("hhr_decode_no_alloc", ctypes.byref(shape), _ptr(q), _ptr(seq_len), _ptr(R), _ptr(W),
          _ptr(codes), _ptr(page_meta), _ptr(k_cache), _ptr(v_cache), keep_num, keep_den,
          keep_pages_abs, int(top_k), float(scale), _ptr(sel_idx), _ptr(sel_count), _ptr(out),
          _ptr(status_word), _stream(stream))


def hhr_no_alloc_scratch_bytes() -> int:
    return int(load().hhr_no_alloc_scratch_bytes())


# --------------------------------------------------------------------- HISA steps
def hhr_hisa_pool_keys(shape, k8, k_scale, start, n_new, max_new, reps, status_word=None,
                       stream=None) -> None:
    _call("hhr_hisa_pool_keys", ctypes.byref(shape), _ptr(k8), _ptr(k_scale), _ptr(start),
          _ptr(n_new), int(max_new), _ptr(reps), _ptr(status_word), _stream(stream))


def hhr_hisa_block_scores(shape, q8, q_scale, w, reps, seq_len, block_scores, status_word=None,
                          stream=None) -> None:
    _call("hhr_hisa_block_scores", ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w),
          _ptr(reps), _ptr(seq_len), _ptr(block_scores), _ptr(status_word), _stream(stream))


def hhr_hisa_top_blocks(shape, block_scores, seq_len, keep_blocks, kept_blocks, kept_count,
                        status_word=None, stream=None) -> None:
    _call("hhr_hisa_top_blocks", ctypes.byref(shape), _ptr(block_scores), _ptr(seq_len),
          int(keep_blocks), _ptr(kept_blocks), _ptr(kept_count), _ptr(status_word),
          _stream(stream))


def hhr_hisa_token_topk(shape, q8, q_scale, w, k8, k_scale, seq_len, kept_blocks, kept_count,
                        keep_blocks, top_k, sel_idx, sel_count, token_scores, workspace,
                        workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_hisa_token_topk", ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8),
          _ptr(k_scale), _ptr(seq_len), _ptr(kept_blocks), _ptr(kept_count), int(keep_blocks),
          int(top_k), _ptr(sel_idx), _ptr(sel_count), _ptr(token_scores), _ptr(workspace), wb,
          _stream(stream))


def hhr_hisa_select(shape, q8, q_scale, w, k8, k_scale, reps, seq_len, keep_blocks, top_k,
                    sel_idx, sel_count, workspace, workspace_bytes=None, stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_hisa_select", ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8),
          _ptr(k_scale), _ptr(reps), _ptr(seq_len), int(keep_blocks), int(top_k), _ptr(sel_idx),
          _ptr(sel_count), _ptr(workspace), wb, _stream(stream))


def hhr_hisa_prefill_select(shape, q8, q_scale, w, k8, k_scale, reps, q_len, keep_blocks, top_k,
                            sel_idx, sel_count, workspace, workspace_bytes=None,
                            stream=None) -> None:
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _call("hhr_hisa_prefill_select", ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w),
          _ptr(k8), _ptr(k_scale), _ptr(reps), _ptr(q_len), int(keep_blocks), int(top_k),
          _ptr(sel_idx), _ptr(sel_count), _ptr(workspace), wb, _stream(stream))
