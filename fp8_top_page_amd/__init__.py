"""MI355X (gfx950) MSA sparse-prefill path: thin Python binding over libmsa.so.

The four calls keep the C names declared in include/msa.h and only marshal
arguments (torch tensors -> device pointers, strides, the caller's current HIP
stream).  All computation happens in the library's HIP kernels; there is no
fallback: if the library is missing, importing a call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MsaError", "Varlen", "lib", "msa_index_score", "msa_index_score_workspace_size",
    "msa_topk_select", "msa_build_k2q_csr", "msa_k2q_schedule_size", "msa_sparse_attn_prefill",
    "msa_sparse_attn_workspace_size", "msa_status_string", "msa_last_error", "msa_abi_version",
    "msa_quantize_e4m3", "msa_insert_index_k", "msa_insert_kv", "msa_index_score_mxfp4",
    "msa_insert_index_k_mxfp4", "msa_index_score_noalloc", "msa_index_score_per_head",
    "msa_sparse_attn_prefill_mxfp4", "msa_index_score_topk", "msa_index_score_topk_workspace_size",
    "msa_check_varlen", "BAD_FLAGS",
    "LIB_PATH", "PAGE", "HEAD_DIM", "TOPK",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")
PAGE = 128
HEAD_DIM = 128
TOPK = 16

_c_i32, _c_i64, _c_size, _c_p, _c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                        ctypes.c_void_p, ctypes.c_float)


class _VarlenC(ctypes.Structure):
    _fields_ = [
        ("batch", _c_i32), ("total_q", _c_i32), ("max_seqlen_q", _c_i32),
        ("max_seqlen_k", _c_i32), ("total_rows", _c_i32), ("max_pages", _c_i32),
        ("cu_seqlens_q", _c_p), ("cu_seqlens_k", _c_p), ("block_table", _c_p),
        ("block_table_stride", _c_i64),
    ]


class MsaError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_status_name(status)}: {detail}")


_LIB = None


def lib():
    """Load libmsa.so (built in-tree by fp8_top_page_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmsa.so not built ({LIB_PATH}); run fp8_top_page_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.POINTER(_VarlenC)
        L.msa_index_score_workspace_size.argtypes = [vp, _c_i32]
        L.msa_index_score_workspace_size.restype = _c_size
        L.msa_index_score.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p,
                                      _c_i64, _c_p, _c_size, _c_p]
        L.msa_index_score.restype = ctypes.c_int
        L.msa_topk_select.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_i64, _c_p]
        L.msa_topk_select.restype = ctypes.c_int
        L.msa_k2q_schedule_size.argtypes = [vp, _c_i32, _c_i32]
        L.msa_k2q_schedule_size.restype = _c_size
        L.msa_build_k2q_csr.argtypes = [vp, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_p, _c_p,
                                        _c_p, _c_size, _c_p]
        L.msa_build_k2q_csr.restype = ctypes.c_int
        L.msa_check_varlen.argtypes = [vp, _c_i32, _c_p, _c_p]
        L.msa_check_varlen.restype = ctypes.c_int
        L.msa_sparse_attn_workspace_size.argtypes = [vp, _c_i32, _c_i32, _c_i32, _c_i32]
        L.msa_sparse_attn_workspace_size.restype = _c_size
        L.msa_sparse_attn_prefill.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_i32, _c_i32,
                                              _c_p, _c_p, _c_i32, _c_p, _c_size, _c_i32, _c_f,
                                              _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_size, _c_p]
        L.msa_sparse_attn_prefill.restype = ctypes.c_int
        L.msa_sparse_attn_prefill_mxfp4.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_p, _c_i32,
                                                    _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_size,
                                                    _c_i32, _c_f, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                                    _c_p, _c_size, _c_p]
        L.msa_sparse_attn_prefill_mxfp4.restype = ctypes.c_int
        L.msa_index_score_topk_workspace_size.argtypes = [vp, _c_i32]
        L.msa_index_score_topk_workspace_size.restype = _c_size
        L.msa_index_score_topk.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_i32, _c_p, _c_p,
                                           _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_size, _c_p]
        L.msa_index_score_topk.restype = ctypes.c_int
        L.msa_quantize_e4m3.argtypes = [_c_p, _c_i32, _c_i64, _c_i32, _c_i64, _c_p, _c_p, _c_i64,
                                        _c_p]
        L.msa_quantize_e4m3.restype = ctypes.c_int
        L.msa_insert_index_k.argtypes = [_c_p, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_i32,
                                         _c_p]
        L.msa_insert_index_k.restype = ctypes.c_int
        L.msa_insert_kv.argtypes = [_c_p, _c_p, _c_i32, _c_i64, _c_i32, _c_i64, _c_i64, _c_p, _c_p,
                                    _c_p, _c_p, _c_i32, _c_p]
        L.msa_insert_kv.restype = ctypes.c_int
        L.msa_index_score_mxfp4.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_p, _c_i32, _c_p,
                                            _c_p, _c_p, _c_i64, _c_p, _c_size, _c_p]
        L.msa_index_score_mxfp4.restype = ctypes.c_int
        L.msa_insert_index_k_mxfp4.argtypes = [_c_p, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                               _c_i32, _c_p]
        L.msa_insert_index_k_mxfp4.restype = ctypes.c_int
        L.msa_index_score_per_head.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_i32, _c_p, _c_p,
                                               _c_p, _c_i64, _c_i64, _c_p, _c_size, _c_p]
        L.msa_index_score_per_head.restype = ctypes.c_int
        L.msa_index_score_noalloc.argtypes = [vp, _c_p, _c_i64, _c_i32, _c_p, _c_i32, _c_p, _c_p,
                                              _c_p, _c_i64, _c_p]
        L.msa_index_score_noalloc.restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_abi_version.argtypes = []
        L.msa_abi_version.restype = _c_i32
        _LIB = L
    return _LIB


def _status_name(st: int) -> str:
    return lib().msa_status_string(st).decode()


def _check(st: int, fn: str):
    if st != 0:
        raise MsaError(st, fn, lib().msa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Varlen:
    """Var-len batch descriptor: device cu_seqlens/block_table plus host-side sizes."""

    def __init__(self, cu_seqlens_q, cu_seqlens_k, block_table, *, total_q, max_seqlen_q,
                 max_seqlen_k, total_rows, max_pages):
        self.cu_seqlens_q = cu_seqlens_q
        self.cu_seqlens_k = cu_seqlens_k
        self.block_table = block_table
        self.c = _VarlenC(
            batch=int(cu_seqlens_q.shape[0]) - 1, total_q=int(total_q),
            max_seqlen_q=int(max_seqlen_q), max_seqlen_k=int(max_seqlen_k),
            total_rows=int(total_rows), max_pages=int(max_pages),
            cu_seqlens_q=_ptr(cu_seqlens_q), cu_seqlens_k=_ptr(cu_seqlens_k),
            block_table=_ptr(block_table),
            block_table_stride=int(block_table.stride(0)) if block_table.dim() == 2 else int(max_pages))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def msa_abi_version() -> int:
    return int(lib().msa_abi_version())


def msa_status_string(status: int) -> str:
    return _status_name(status)


def msa_last_error() -> str:
    return lib().msa_last_error().decode()


def msa_index_score_workspace_size(vl: Varlen, num_index_heads: int) -> int:
    return int(lib().msa_index_score_workspace_size(vl.ref, num_index_heads))


def msa_index_score(vl: Varlen, q, num_index_heads, k_cache, num_pages, q_scale, k_scale,
                    scores, workspace, stream=None):
    """q: uint8 [total_q, H*128] (row stride in bytes = q.stride(0)); scores: f32 [total_q, ld]."""
    st = lib().msa_index_score(vl.ref, _ptr(q), q.stride(0), num_index_heads, _ptr(k_cache),
                               num_pages, _ptr(q_scale), _ptr(k_scale), _ptr(scores),
                               scores.stride(0), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(st, "msa_index_score")


def msa_topk_select(vl: Varlen, scores, topk, n_local, topk_idx, stream=None):
    st = lib().msa_topk_select(vl.ref, _ptr(scores), scores.stride(0), topk, n_local,
                               _ptr(topk_idx), topk_idx.stride(0), _stream(stream))
    _check(st, "msa_topk_select")


def msa_k2q_schedule_size(vl: Varlen, n_sel_heads: int, topk: int) -> int:
    return int(lib().msa_k2q_schedule_size(vl.ref, n_sel_heads, topk))


# flag bits of msa_check_varlen (include/msa.h, MSA_BAD_*)
BAD_FLAGS = {"cu_q": 1, "cu_k": 2, "max_q": 4, "max_k": 8, "pages": 16, "rows": 32, "block": 64}


def msa_check_varlen(vl: Varlen, num_pages, flags, stream=None):
    """flags: int32 device tensor of at least one element; flags[0] gets the OR of
    the MSA_BAD_* bits the batch's device metadata violates (0: consistent)."""
    assert flags.dtype == torch.int32 and flags.is_cuda and flags.numel() >= 1
    _check(lib().msa_check_varlen(vl.ref, int(num_pages), _ptr(flags), _stream(stream)),
           "msa_check_varlen")


def msa_build_k2q_csr(vl: Varlen, topk_idx, n_sel_heads, topk, row_ptr, q_indices, schedule,
                      stream=None):
    """topk_idx: int32 [total_q, 16] (shared) or [total_q, n_sel, 16] (any strides, last dim contiguous)."""
    if topk_idx.dim() == 2:
        tq, th = topk_idx.stride(0), 0
    else:
        tq, th = topk_idx.stride(0), topk_idx.stride(1)
    st = lib().msa_build_k2q_csr(vl.ref, _ptr(topk_idx), tq, th, n_sel_heads, topk, _ptr(row_ptr),
                                 _ptr(q_indices), _ptr(schedule), schedule.numel(), _stream(stream))
    _check(st, "msa_build_k2q_csr")


def msa_sparse_attn_workspace_size(vl: Varlen, num_q_heads, num_kv_heads, n_sel_heads, topk) -> int:
    return int(lib().msa_sparse_attn_workspace_size(vl.ref, num_q_heads, num_kv_heads,
                                                    n_sel_heads, topk))


def msa_sparse_attn_prefill(vl: Varlen, q, num_q_heads, kv_cache, num_pages, num_kv_heads,
                            row_ptr, q_indices, n_sel_heads, schedule, topk, softmax_scale,
                            q_scale, k_scale, v_scale, out, workspace, stream=None):
    """q: uint8 [total_q, Hq*128]; out: bf16 [total_q, Hq*128] (row stride out.stride(0))."""
    st = lib().msa_sparse_attn_prefill(
        vl.ref, _ptr(q), q.stride(0), num_q_heads, _ptr(kv_cache), num_pages, num_kv_heads,
        _ptr(row_ptr), _ptr(q_indices), n_sel_heads, _ptr(schedule), schedule.numel(), topk,
        float(softmax_scale), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(out),
        out.stride(0), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "msa_sparse_attn_prefill")


def msa_index_score_topk_workspace_size(vl: Varlen, num_index_heads):
    return lib().msa_index_score_topk_workspace_size(vl.ref, num_index_heads)


def msa_index_score_topk(vl: Varlen, q, num_index_heads, k_cache, num_pages, q_scale, k_scale,
                         topk, n_local, topk_out, workspace, stream=None):
    """Decode-like batches: index scores and top-k selection in one pass.
    q: uint8 [total_q, H*128]; topk_out: int32 [total_q, >= 16] (row stride topk_out.stride(0))."""
    st = lib().msa_index_score_topk(
        vl.ref, _ptr(q), q.stride(0), num_index_heads, _ptr(k_cache), num_pages, _ptr(q_scale),
        _ptr(k_scale), topk, n_local, _ptr(topk_out), topk_out.stride(0), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "msa_index_score_topk")


def msa_sparse_attn_prefill_mxfp4(vl: Varlen, q, num_q_heads, kv_data, kv_scales, num_pages,
                                  num_kv_heads, row_ptr, q_indices, n_sel_heads, schedule, topk,
                                  softmax_scale, q_scale, k_scale, v_scale, out, workspace,
                                  stream=None):
    """kv_data: uint8 [pages, Hkv, 128, 128] MXFP4 codes; kv_scales: uint8 [pages, Hkv, 128, 8]."""
    st = lib().msa_sparse_attn_prefill_mxfp4(
        vl.ref, _ptr(q), q.stride(0), num_q_heads, _ptr(kv_data), _ptr(kv_scales), num_pages,
        num_kv_heads, _ptr(row_ptr), _ptr(q_indices), n_sel_heads, _ptr(schedule),
        schedule.numel(), topk, float(softmax_scale), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
        _ptr(out), out.stride(0), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "msa_sparse_attn_prefill_mxfp4")


_DTYPES = {torch.bfloat16: 0, torch.float32: 1}     # MSA_DTYPE_BF16, MSA_DTYPE_F32


def _src_dtype(t):
    if t.dtype not in _DTYPES:
        raise TypeError(f"source must be bfloat16 or float32, got {t.dtype}")
    return _DTYPES[t.dtype]


def msa_quantize_e4m3(src, scale, dst, stream=None):
    """src: bf16/f32 [n, heads*128] (or [n, heads, 128]), rows contiguous; dst: uint8 same shape."""
    n = src.shape[0]
    inner = 1
    for d in src.shape[1:]:
        inner *= d
    heads = max(1, inner // HEAD_DIM)
    st = lib().msa_quantize_e4m3(_ptr(src), _src_dtype(src), n, heads, src.stride(0), _ptr(scale),
                                 _ptr(dst), dst.stride(0), _stream(stream))
    _check(st, "msa_quantize_e4m3")


def msa_insert_index_k(k, slot_mapping, scale, k_cache, num_pages, stream=None):
    """k: bf16/f32 [n_tokens, 128]; slot_mapping: int64 [n_tokens]; k_cache: uint8 [pages, 128, 128]."""
    st = lib().msa_insert_index_k(_ptr(k), _src_dtype(k), k.shape[0], k.stride(0),
                                  _ptr(slot_mapping), _ptr(scale), _ptr(k_cache), num_pages,
                                  _stream(stream))
    _check(st, "msa_insert_index_k")


def msa_insert_kv(k, v, slot_mapping, k_scale, v_scale, kv_cache, num_pages, num_kv_heads,
                  stream=None):
    """k, v: bf16/f32 [n_tokens, Hkv, 128] (heads contiguous); kv_cache: uint8 [pages, Hkv, 128, 256]."""
    st = lib().msa_insert_kv(_ptr(k), _ptr(v), _src_dtype(k), k.shape[0], num_kv_heads,
                             k.stride(0), v.stride(0), _ptr(slot_mapping), _ptr(k_scale),
                             _ptr(v_scale), _ptr(kv_cache), num_pages, _stream(stream))
    _check(st, "msa_insert_kv")


def msa_index_score_mxfp4(vl: Varlen, q, num_index_heads, k_data, k_scales, num_pages, q_scale,
                          k_scale, scores, workspace, stream=None):
    """msa_index_score over MXFP4 keys: k_data uint8 [pages, 128, 64], k_scales uint8 [pages, 128, 4]."""
    st = lib().msa_index_score_mxfp4(vl.ref, _ptr(q), q.stride(0), num_index_heads, _ptr(k_data),
                                     _ptr(k_scales), num_pages, _ptr(q_scale), _ptr(k_scale),
                                     _ptr(scores), scores.stride(0), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "msa_index_score_mxfp4")


def msa_insert_index_k_mxfp4(k, slot_mapping, k_data, k_scales, num_pages, stream=None):
    """k: bf16/f32 [n_tokens, 128]; k_data uint8 [pages, 128, 64]; k_scales uint8 [pages, 128, 4]."""
    st = lib().msa_insert_index_k_mxfp4(_ptr(k), _src_dtype(k), k.shape[0], k.stride(0),
                                        _ptr(slot_mapping), _ptr(k_data), _ptr(k_scales),
                                        num_pages, _stream(stream))
    _check(st, "msa_insert_index_k_mxfp4")



def msa_index_score_noalloc(vl: Varlen, q, num_index_heads, k_cache, num_pages, q_scale, k_scale,
                            scores, stream=None):
    """msa_index_score with the library's built-in work-list buffer (no workspace)."""
    st = lib().msa_index_score_noalloc(vl.ref, _ptr(q), q.stride(0), num_index_heads, _ptr(k_cache),
                                       num_pages, _ptr(q_scale), _ptr(k_scale), _ptr(scores),
                                       scores.stride(0), _stream(stream))
    _check(st, "msa_index_score_noalloc")


def msa_index_score_per_head(vl: Varlen, q, num_index_heads, k_cache, num_pages, q_scale, k_scale,
                             scores, workspace, stream=None):
    """Per-index-head scores: scores f32 [total_q, H, ld] (query stride scores.stride(0), head
    stride scores.stride(1))."""
    st = lib().msa_index_score_per_head(vl.ref, _ptr(q), q.stride(0), num_index_heads,
                                        _ptr(k_cache), num_pages, _ptr(q_scale), _ptr(k_scale),
                                        _ptr(scores), scores.stride(0), scores.stride(1),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream))
    _check(st, "msa_index_score_per_head")
