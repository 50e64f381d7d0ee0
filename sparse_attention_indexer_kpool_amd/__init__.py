"""Python binding of libkpool.so, the KPool DSA indexer for AMD MI355X (gfx950).

The functions below carry the names of the C entry points in include/kpool.h
and only marshal arguments: torch tensors supply device pointers and the
current HIP stream, every step of the indexer runs in the library's HIP
kernels. There is no fallback: when libkpool.so is missing, or a tensor is not
on the GPU, a call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkpool.so")

KPOOL_OK, KPOOL_E_INVALID, KPOOL_E_UNSUPPORTED, KPOOL_E_WORKSPACE, KPOOL_E_LAUNCH = range(5)


class KPoolError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"kpool status {status}: {detail}")
        self.status = status
        self.detail = detail


class _ProjParams(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("q_lora_rank", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


@dataclass
class ProjParams:
    """Mirror of kpool_proj_params (include/kpool.h)."""
    num_tokens: int
    hidden: int
    q_lora_rank: int
    num_heads: int
    head_dim: int = 128
    eps: float = 0.0

    def c(self) -> _ProjParams:
        return _ProjParams(int(self.num_tokens), int(self.hidden), int(self.q_lora_rank),
                           int(self.num_heads), int(self.head_dim), float(self.eps))


class _MlaParams(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("kv_rows", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("dim_qk", ctypes.c_int32),
        ("dim_v", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
    ]


@dataclass
class MlaParams:
    """Mirror of kpool_mla_params (include/kpool.h)."""
    num_tokens: int
    num_heads: int
    kv_rows: int
    width: int
    sm_scale: float
    dim_qk: int = 512
    dim_v: int = 512

    def c(self) -> _MlaParams:
        return _MlaParams(int(self.num_tokens), int(self.num_heads), int(self.kv_rows),
                          int(self.width), int(self.dim_qk), int(self.dim_v), float(self.sm_scale))


class _Params(ctypes.Structure):
    _fields_ = [
        ("num_docs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kpool", ctypes.c_int32),
        ("index_topk", ctypes.c_int32),
        ("always_select_tail", ctypes.c_int32),
        ("use_fp8", ctypes.c_int32),
        ("query_chunk", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


@dataclass
class Params:
    """Mirror of kpool_params (include/kpool.h)."""
    num_docs: int
    total_tokens: int
    max_seqlen: int
    num_heads: int
    head_dim: int
    kpool: int = 4
    index_topk: int = 2048
    always_select_tail: int = 1
    use_fp8: int = 0
    query_chunk: int = 0
    scale: float = 0.0

    def c(self) -> _Params:
        return _Params(int(self.num_docs), int(self.total_tokens), int(self.max_seqlen),
                       int(self.num_heads), int(self.head_dim), int(self.kpool),
                       int(self.index_topk), int(self.always_select_tail), int(self.use_fp8),
                       int(self.query_chunk), float(self.scale))

    @property
    def k_sel(self) -> int:
        return self.index_topk // self.kpool

    @property
    def width(self) -> int:
        return self.index_topk + self.kpool


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkpool.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_indexer_kpool_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(_Params)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.kpool_abi_version.restype = ctypes.c_int
        L.kpool_abi_version.argtypes = []
        L.kpool_workspace_bytes.restype = sz
        L.kpool_workspace_bytes.argtypes = [P]
        L.kpool_logits_ld.restype = ctypes.c_int64
        L.kpool_logits_ld.argtypes = [P]
        L.kpool_query_chunk_rows.restype = ctypes.c_int32
        L.kpool_query_chunk_rows.argtypes = [P]
        L.kpool_compress.restype = ctypes.c_int
        L.kpool_compress.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.kpool_indexer_topk.restype = ctypes.c_int
        L.kpool_indexer_topk.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.kpool_indexer_launches.restype = i32
        L.kpool_indexer_launches.argtypes = [P, vp, i32]
        L.kpool_indexer_scoring.restype = ctypes.c_int
        L.kpool_indexer_scoring.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, sz, i32, vp]
        L.kpool_indexer_selection.restype = ctypes.c_int
        L.kpool_indexer_selection.argtypes = [P, i32, vp, vp, vp, sz, vp, vp, vp]
        L.kpool_fused_max_ksel.restype = ctypes.c_int32
        L.kpool_fused_max_ksel.argtypes = [P]
        L.kpool_fused_workspace_bytes.restype = sz
        L.kpool_fused_workspace_bytes.argtypes = [P]
        L.kpool_indexer_topk_fused.restype = ctypes.c_int
        L.kpool_indexer_topk_fused.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.kpool_logits.restype = ctypes.c_int
        L.kpool_logits.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp, i32, vp]
        L.kpool_select.restype = ctypes.c_int
        L.kpool_select.argtypes = [P, vp, i32, i32, vp, vp, vp, vp]
        L.kpool_select_expand.restype = ctypes.c_int
        L.kpool_select_expand.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, vp]
        L.kpool_expand.restype = ctypes.c_int
        L.kpool_expand.argtypes = [P, vp, vp, vp, vp, vp]
        L.kpool_fp8_quantize.restype = ctypes.c_int
        L.kpool_fp8_quantize.argtypes = [vp, i32, vp, vp, vp]
        L.kpool_compress_pools.restype = ctypes.c_int
        L.kpool_compress_pools.argtypes = [P, vp, vp, vp, i32, vp, i32, vp, vp, vp]
        L.kpool_decode_workspace_bytes.restype = sz
        L.kpool_decode_workspace_bytes.argtypes = [P]
        L.kpool_decode_topk.restype = ctypes.c_int
        L.kpool_decode_topk.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.kpool_decode_noalloc_max_bytes.restype = sz
        L.kpool_decode_noalloc_max_bytes.argtypes = []
        L.kpool_decode_topk_noalloc.restype = ctypes.c_int
        L.kpool_decode_topk_noalloc.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
        PP = ctypes.POINTER(_ProjParams)
        L.kpool_proj_workspace_bytes.restype = sz
        L.kpool_proj_workspace_bytes.argtypes = [PP]
        L.kpool_indexer_projections.restype = ctypes.c_int
        L.kpool_indexer_projections.argtypes = [PP, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                vp, vp, vp, vp]
        L.kpool_check_cu_seqlens.restype = ctypes.c_int
        L.kpool_check_cu_seqlens.argtypes = [vp, i32, i32, i32, vp, vp]
        MP = ctypes.POINTER(_MlaParams)
        L.kpool_sparse_mla_fwd.restype = ctypes.c_int
        L.kpool_sparse_mla_fwd.argtypes = [MP, vp, vp, vp, vp, vp, vp]
        L.kpool_status_string.restype = ctypes.c_char_p
        L.kpool_status_string.argtypes = [ctypes.c_int]
        L.kpool_last_error.restype = ctypes.c_char_p
        L.kpool_last_error.argtypes = []
        _lib = L
    return _lib


EXPORTS = ["kpool_abi_version", "kpool_workspace_bytes", "kpool_logits_ld",
           "kpool_query_chunk_rows", "kpool_compress",
           "kpool_indexer_topk", "kpool_indexer_launches", "kpool_indexer_scoring",
           "kpool_indexer_selection", "kpool_fused_max_ksel", "kpool_fused_workspace_bytes",
           "kpool_indexer_topk_fused",
           "kpool_logits", "kpool_select", "kpool_select_expand",
           "kpool_expand",
           "kpool_fp8_quantize", "kpool_compress_pools", "kpool_decode_workspace_bytes",
           "kpool_decode_topk", "kpool_decode_noalloc_max_bytes", "kpool_decode_topk_noalloc",
           "kpool_proj_workspace_bytes", "kpool_indexer_projections", "kpool_sparse_mla_fwd",
           "kpool_check_cu_seqlens", "kpool_status_string", "kpool_last_error"]


def _check(status: int) -> None:
    if status != KPOOL_OK:
        raise KPoolError(status, lib().kpool_last_error().decode())


def _ptr(t) -> int:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def kpool_abi_version() -> int:
    return lib().kpool_abi_version()


def kpool_workspace_bytes(p: Params) -> int:
    return int(lib().kpool_workspace_bytes(ctypes.byref(p.c())))


def kpool_logits_ld(p: Params) -> int:
    return int(lib().kpool_logits_ld(ctypes.byref(p.c())))


def kpool_query_chunk_rows(p: Params) -> int:
    return int(lib().kpool_query_chunk_rows(ctypes.byref(p.c())))


def kpool_compress(p: Params, k, gate, ape, cu_seqlens, cu_pools, pooled, stream=None) -> None:
    _check(lib().kpool_compress(ctypes.byref(p.c()), _ptr(k), _ptr(gate), _ptr(ape),
                                _ptr(cu_seqlens), _ptr(cu_pools), _ptr(pooled), _stream(stream)))


def kpool_indexer_topk(p: Params, q, w, pooled, cu_seqlens, cu_pools, workspace,
                       out_token_idx, out_pool_idx=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_indexer_topk(ctypes.byref(p.c()), _ptr(q), _ptr(w), _ptr(pooled),
                                    _ptr(cu_seqlens), _ptr(cu_pools), _ptr(workspace), ws_bytes,
                                    _ptr(out_token_idx), _ptr(out_pool_idx), _stream(stream)))


def kpool_indexer_launches(p: Params) -> list:
    """The indexer's scoring launches: one (a0, a1, lda, b0, b1, ldb) tuple
    each (rows a0..a1-1 at row stride lda, then rows b0..b1-1 at ldb)."""
    n = int(lib().kpool_indexer_launches(ctypes.byref(p.c()), None, 0))
    if n <= 0:
        return []
    info = (ctypes.c_int32 * (6 * n))()
    lib().kpool_indexer_launches(ctypes.byref(p.c()), info, n)
    return [tuple(int(x) for x in info[6 * i:6 * i + 6]) for i in range(n)]


def kpool_indexer_scoring(p: Params, launch, q, w, pooled, cu_seqlens, cu_pools, workspace,
                          flags=0, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_indexer_scoring(ctypes.byref(p.c()), int(launch), _ptr(q), _ptr(w),
                                       _ptr(pooled), _ptr(cu_seqlens), _ptr(cu_pools),
                                       _ptr(workspace), ws_bytes, int(flags), _stream(stream)))


def kpool_indexer_selection(p: Params, launch, cu_seqlens, cu_pools, workspace, out_token_idx,
                            out_pool_idx=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_indexer_selection(ctypes.byref(p.c()), int(launch), _ptr(cu_seqlens),
                                         _ptr(cu_pools), _ptr(workspace), ws_bytes,
                                         _ptr(out_token_idx), _ptr(out_pool_idx),
                                         _stream(stream)))


def kpool_fused_max_ksel(p: Params) -> int:
    return int(lib().kpool_fused_max_ksel(ctypes.byref(p.c())))


def kpool_fused_workspace_bytes(p: Params) -> int:
    return int(lib().kpool_fused_workspace_bytes(ctypes.byref(p.c())))


def kpool_indexer_topk_fused(p: Params, q, w, pooled, cu_seqlens, cu_pools, workspace,
                             out_token_idx, out_pool_idx=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_indexer_topk_fused(ctypes.byref(p.c()), _ptr(q), _ptr(w), _ptr(pooled),
                                          _ptr(cu_seqlens), _ptr(cu_pools), _ptr(workspace),
                                          ws_bytes, _ptr(out_token_idx), _ptr(out_pool_idx),
                                          _stream(stream)))


KPOOL_LOGITS_FILL_MASKED = 1
KPOOL_LOGITS_SKIP_ALL_SELECTED = 2
KPOOL_LOGITS_INPUTS_QUANTIZED = 4
KPOOL_CU_FIRST_NOT_ZERO = 1
KPOOL_CU_DECREASING = 2
KPOOL_CU_TOO_LONG = 4
KPOOL_CU_LAST_NOT_TOTAL = 8


def kpool_logits(p: Params, q, w, pooled, cu_seqlens, cu_pools, q_begin, q_end, workspace,
                 out, flags=KPOOL_LOGITS_FILL_MASKED, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_logits(ctypes.byref(p.c()), _ptr(q), _ptr(w), _ptr(pooled),
                              _ptr(cu_seqlens), _ptr(cu_pools), int(q_begin), int(q_end),
                              _ptr(workspace), ws_bytes, _ptr(out), int(flags),
                              _stream(stream)))


def kpool_select(p: Params, logits, q_begin, q_end, cu_seqlens, cu_pools, out_pool_idx,
                 stream=None) -> None:
    _check(lib().kpool_select(ctypes.byref(p.c()), _ptr(logits), int(q_begin), int(q_end),
                              _ptr(cu_seqlens), _ptr(cu_pools), _ptr(out_pool_idx),
                              _stream(stream)))


def kpool_select_expand(p: Params, logits, q_begin, q_end, cu_seqlens, cu_pools, out_pool_idx,
                        out_token_idx, stream=None) -> None:
    _check(lib().kpool_select_expand(ctypes.byref(p.c()), _ptr(logits), int(q_begin), int(q_end),
                                     _ptr(cu_seqlens), _ptr(cu_pools), _ptr(out_pool_idx),
                                     _ptr(out_token_idx), _stream(stream)))


def kpool_expand(p: Params, pool_idx, cu_seqlens, cu_pools, out_token_idx, stream=None) -> None:
    _check(lib().kpool_expand(ctypes.byref(p.c()), _ptr(pool_idx), _ptr(cu_seqlens),
                              _ptr(cu_pools), _ptr(out_token_idx), _stream(stream)))


def kpool_fp8_quantize(x, rows, codes, row_scale, stream=None) -> None:
    _check(lib().kpool_fp8_quantize(_ptr(x), int(rows), _ptr(codes), _ptr(row_scale),
                                    _stream(stream)))


def kpool_compress_pools(p: Params, k, gate, ape, num_pools, dst_rows, pooled,
                         pooled_scale=None, stream=None) -> None:
    _check(lib().kpool_compress_pools(ctypes.byref(p.c()), _ptr(k), _ptr(gate), _ptr(ape),
                                      int(num_pools), _ptr(dst_rows), int(pooled.shape[0]),
                                      _ptr(pooled), _ptr(pooled_scale), _stream(stream)))


def kpool_decode_workspace_bytes(p: Params) -> int:
    return int(lib().kpool_decode_workspace_bytes(ctypes.byref(p.c())))


def kpool_decode_topk(p: Params, q, w, pooled, pool_start, seq_lens, workspace, out_token_idx,
                      out_pool_idx=None, token_base=None, pooled_scale=None,
                      stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_decode_topk(ctypes.byref(p.c()), _ptr(q), _ptr(w), _ptr(pooled),
                                   int(pooled.shape[0]), _ptr(pooled_scale), _ptr(pool_start), _ptr(seq_lens), _ptr(token_base),
                                   _ptr(workspace), ws_bytes, _ptr(out_token_idx),
                                   _ptr(out_pool_idx), _stream(stream)))


def kpool_decode_noalloc_max_bytes() -> int:
    return int(lib().kpool_decode_noalloc_max_bytes())


def kpool_decode_topk_noalloc(p: Params, q, w, pooled, pool_start, seq_lens, out_token_idx,
                              out_pool_idx=None, token_base=None, pooled_scale=None,
                              stream=None) -> None:
    _check(lib().kpool_decode_topk_noalloc(ctypes.byref(p.c()), _ptr(q), _ptr(w), _ptr(pooled),
                                           int(pooled.shape[0]), _ptr(pooled_scale),
                                           _ptr(pool_start), _ptr(seq_lens), _ptr(token_base),
                                           _ptr(out_token_idx), _ptr(out_pool_idx),
                                           _stream(stream)))


def kpool_proj_workspace_bytes(pp: ProjParams) -> int:
    return int(lib().kpool_proj_workspace_bytes(ctypes.byref(pp.c())))


def kpool_indexer_projections(pp: ProjParams, x, qr, wq_b, wk, k_norm_weight, k_norm_bias, wg,
                              ww, workspace, q_out, k_out, gate_out, w_out, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().kpool_indexer_projections(
        ctypes.byref(pp.c()), _ptr(x), _ptr(qr), _ptr(wq_b), _ptr(wk), _ptr(k_norm_weight),
        _ptr(k_norm_bias), _ptr(wg), _ptr(ww), _ptr(workspace), ws_bytes, _ptr(q_out),
        _ptr(k_out), _ptr(gate_out), _ptr(w_out), _stream(stream)))


def kpool_check_cu_seqlens(cu_seqlens, num_docs: int, total_tokens: int, max_seqlen: int,
                           flags_out, stream=None) -> None:
    _check(lib().kpool_check_cu_seqlens(_ptr(cu_seqlens), int(num_docs), int(total_tokens),
                                        int(max_seqlen), _ptr(flags_out), _stream(stream)))


def kpool_sparse_mla_fwd(mp: MlaParams, q, kv, indices, out, lse, stream=None) -> None:
    _check(lib().kpool_sparse_mla_fwd(ctypes.byref(mp.c()), _ptr(q), _ptr(kv), _ptr(indices),
                                      _ptr(out), _ptr(lse), _stream(stream)))


def kpool_status_string(status: int) -> str:
    return lib().kpool_status_string(int(status)).decode()


def kpool_last_error() -> str:
    return lib().kpool_last_error().decode()
