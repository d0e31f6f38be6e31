"""Python binding of libqsa.so: the four QSA decode calls on torch tensors.

Argument marshalling only -- every step runs in the HIP kernels of libqsa.so.
Tensors must be CUDA (HIP) tensors, contiguous, of the dtypes stated below;
the calls enqueue on the current torch stream (or `stream`) and return
without synchronising.  A non-OK status raises QSAError carrying the
library's own message.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

QSAError_codes = {
    _lib.QSA_ERR_INVALID_ARGUMENT: "INVALID_ARGUMENT",
    _lib.QSA_ERR_UNSUPPORTED: "UNSUPPORTED",
    _lib.QSA_ERR_WORKSPACE: "WORKSPACE",
    _lib.QSA_ERR_HIP: "HIP",
}


class QSAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{QSAError_codes.get(status, status)}: {msg}")
        self.status = status


@dataclass(frozen=True)
class QSAConfig:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    topk_blocks: int
    page_size: int
    max_pages_per_req: int
    kv_dtype: str = "bf16"  # "bf16" | "fp8"
    softmax_scale: float = 0.0  # 0 => 1/sqrt(head_dim)
    compress_ratio: int = 4
    ring_size: int = _lib.QSA_RING_SIZE

    def to_c(self) -> _lib.qsa_config:
        scale = self.softmax_scale if self.softmax_scale > 0 else self.head_dim ** -0.5
        dt = {"bf16": _lib.QSA_KV_BF16, "fp8": _lib.QSA_KV_FP8_E4M3}.get(self.kv_dtype, -1)
        return _lib.qsa_config(self.num_q_heads, self.num_kv_heads, self.head_dim, self.index_dim,
                               self.compress_ratio, self.topk_blocks, self.page_size,
                               self.max_pages_per_req, self.ring_size, dt, scale)


def _check(st: int) -> None:
    if st != _lib.QSA_OK:
        lib = _lib.load()
        raise QSAError(st, lib.qsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dt(t: Optional[torch.Tensor], *dtypes) -> None:
    if t is not None and t.dtype not in dtypes:
        raise TypeError(f"expected dtype in {dtypes}, got {t.dtype}")


def ckey_cache_bytes(cfg: QSAConfig, num_pages: int) -> int:
    c = cfg.to_c()
    return int(_lib.load().qsa_ckey_cache_bytes(ctypes.byref(c), num_pages))


def qsa_compress(cfg: QSAConfig, new_keys: torch.Tensor, new_cu: torch.Tensor,
                 seq_len_before: torch.Tensor, block_table: torch.Tensor, ring: torch.Tensor,
                 ckey_cache: torch.Tensor, max_new_tokens: int, stream=None) -> None:
    """Append new_keys (int8 [T, D]) per request; close micro-blocks into ckey_cache."""
    _dt(new_keys, torch.int8); _dt(ring, torch.int8); _dt(ckey_cache, torch.int8)
    _dt(new_cu, torch.int32); _dt(seq_len_before, torch.int32); _dt(block_table, torch.int32)
    c = cfg.to_c()
    B = seq_len_before.shape[0]
    _check(_lib.load().qsa_compress(ctypes.byref(c), B, int(max_new_tokens), _ptr(new_keys),
                                    _ptr(new_cu), _ptr(seq_len_before), _ptr(block_table),
                                    _ptr(ring), _ptr(ckey_cache), _stream(stream)))


def qsa_index_topk_workspace_size(cfg: QSAConfig, num_sel_rows: int, max_seq_len: int) -> int:
    c = cfg.to_c()
    return int(_lib.load().qsa_index_topk_workspace_size(ctypes.byref(c), num_sel_rows, max_seq_len))


def qsa_index_topk_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check(_lib.load().qsa_index_topk_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                                     _stream(stream)))


def qsa_index_topk(cfg: QSAConfig, q_index: torch.Tensor, sel_req: torch.Tensor,
                   sel_seq_len: torch.Tensor, block_table: torch.Tensor, ckey_cache: torch.Tensor,
                   topk: torch.Tensor, workspace: torch.Tensor, max_seq_len: int, stream=None) -> None:
    """Top-k micro-blocks per selecting row into topk (int32 [S, k], ascending, -1 padded).
    topk=None scores only (scores stay in the workspace)."""
    _dt(q_index, torch.int8); _dt(ckey_cache, torch.int8)
    if topk is not None:
        _dt(topk, torch.int32)
    _dt(sel_req, torch.int32); _dt(sel_seq_len, torch.int32); _dt(block_table, torch.int32)
    c = cfg.to_c()
    S = sel_req.shape[0]
    _check(_lib.load().qsa_index_topk(ctypes.byref(c), S, int(max_seq_len), _ptr(q_index), _ptr(sel_req),
                                      _ptr(sel_seq_len), _ptr(block_table), _ptr(ckey_cache),
                                      _ptr(topk), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))


def qsa_index_topk_noalloc(cfg: QSAConfig, q_index: torch.Tensor, sel_req: torch.Tensor,
                           sel_seq_len: torch.Tensor, block_table: torch.Tensor, ckey_cache: torch.Tensor,
                           topk: torch.Tensor, max_seq_len: int, stream=None) -> None:
    """qsa_index_topk over the library's own device scratch (no workspace argument, no allocation)."""
    _dt(q_index, torch.int8); _dt(ckey_cache, torch.int8); _dt(topk, torch.int32)
    _dt(sel_req, torch.int32); _dt(sel_seq_len, torch.int32); _dt(block_table, torch.int32)
    c = cfg.to_c()
    S = sel_req.shape[0]
    _check(_lib.load().qsa_index_topk_noalloc(ctypes.byref(c), S, int(max_seq_len), _ptr(q_index), _ptr(sel_req),
                                              _ptr(sel_seq_len), _ptr(block_table), _ptr(ckey_cache), _ptr(topk),
                                              _stream(stream)))


def qsa_compress_index_topk(cfg: QSAConfig, new_keys: torch.Tensor, new_cu: torch.Tensor,
                            seq_len_before: torch.Tensor, ring: torch.Tensor, q_index: torch.Tensor,
                            sel_req: torch.Tensor, sel_seq_len: torch.Tensor, block_table: torch.Tensor,
                            ckey_cache: torch.Tensor, topk: torch.Tensor, workspace: torch.Tensor,
                            max_new_tokens: int, max_seq_len: int, stream=None) -> None:
    """qsa_compress then qsa_index_topk in one scan (appends of at most 5 tokens per request)."""
    _dt(new_keys, torch.int8); _dt(ring, torch.int8); _dt(ckey_cache, torch.int8); _dt(q_index, torch.int8)
    _dt(new_cu, torch.int32); _dt(seq_len_before, torch.int32); _dt(block_table, torch.int32)
    _dt(sel_req, torch.int32); _dt(sel_seq_len, torch.int32); _dt(topk, torch.int32)
    c = cfg.to_c()
    B = seq_len_before.shape[0]
    S = sel_req.shape[0]
    _check(_lib.load().qsa_compress_index_topk(
        ctypes.byref(c), B, int(max_new_tokens), _ptr(new_keys), _ptr(new_cu), _ptr(seq_len_before), _ptr(ring),
        S, int(max_seq_len), _ptr(q_index), _ptr(sel_req), _ptr(sel_seq_len), _ptr(block_table),
        _ptr(ckey_cache), _ptr(topk), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def qsa_prefill_index_topk(cfg: QSAConfig, q_index: torch.Tensor, row_cu: torch.Tensor,
                           row_seq_len: torch.Tensor, block_table: torch.Tensor, ckey_cache: torch.Tensor,
                           topk: torch.Tensor, workspace: torch.Tensor, max_seq_len: int,
                           max_rows_per_req: int, stream=None) -> None:
    """Top-k per prefill query row (rows of request b: [row_cu[b], row_cu[b+1])), the scan as an
    int8 MFMA GEMM.  topk int32 [R, k] like qsa_index_topk; topk=None scores only."""
    _dt(q_index, torch.int8); _dt(ckey_cache, torch.int8)
    if topk is not None:
        _dt(topk, torch.int32)
    _dt(row_cu, torch.int32); _dt(row_seq_len, torch.int32); _dt(block_table, torch.int32)
    c = cfg.to_c()
    B = row_cu.shape[0] - 1
    R = row_seq_len.shape[0]
    _check(_lib.load().qsa_prefill_index_topk(ctypes.byref(c), B, R, int(max_rows_per_req), int(max_seq_len),
                                              _ptr(q_index), _ptr(row_cu), _ptr(row_seq_len), _ptr(block_table),
                                              _ptr(ckey_cache), _ptr(topk), _ptr(workspace),
                                              workspace.numel() * workspace.element_size(), _stream(stream)))


def _row_map(q: torch.Tensor, row_sel: Optional[torch.Tensor], sel_req: torch.Tensor,
             max_rows_per_sel: Optional[int]):
    R, S = q.shape[0], sel_req.shape[0]
    if row_sel is None:
        return R, S, 1
    _dt(row_sel, torch.int32)
    return R, S, int(max_rows_per_sel if max_rows_per_sel is not None else R)


def qsa_sparse_decode(cfg: QSAConfig, q: torch.Tensor, row_seq_len: torch.Tensor,
                      sel_req: torch.Tensor, sel_seq_len: torch.Tensor, topk: torch.Tensor,
                      block_table: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      o_part: torch.Tensor, lse_part: torch.Tensor, row_sel: Optional[torch.Tensor] = None,
                      max_rows_per_sel: Optional[int] = None, k_scale: Optional[torch.Tensor] = None,
                      v_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """Split partials of sparse attention: o_part fp32 [P, R, H_q, d], lse_part fp32 [P, R, H_q].
    Row r uses selecting row row_sel[r] (int32 [R]; None: row r is selecting row r)."""
    _dt(q, torch.bfloat16); _dt(o_part, torch.float32); _dt(lse_part, torch.float32)
    _dt(row_seq_len, torch.int32); _dt(sel_req, torch.int32); _dt(sel_seq_len, torch.int32)
    _dt(topk, torch.int32); _dt(block_table, torch.int32)
    c = cfg.to_c()
    R, S, mr = _row_map(q, row_sel, sel_req, max_rows_per_sel)
    P = o_part.shape[0]
    _check(_lib.load().qsa_sparse_decode(ctypes.byref(c), R, S, mr, P, _ptr(q), _ptr(row_sel), _ptr(row_seq_len),
                                         _ptr(sel_req), _ptr(sel_seq_len), _ptr(topk), _ptr(block_table),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                         _ptr(o_part), _ptr(lse_part), _stream(stream)))


def qsa_select_sparse_decode(cfg: QSAConfig, q: torch.Tensor, row_seq_len: torch.Tensor,
                             sel_req: torch.Tensor, sel_seq_len: torch.Tensor, block_table: torch.Tensor,
                             k_cache: torch.Tensor, v_cache: torch.Tensor, topk: torch.Tensor,
                             o_part: torch.Tensor, lse_part: torch.Tensor, workspace: torch.Tensor,
                             max_seq_len: int, row_sel: Optional[torch.Tensor] = None,
                             max_rows_per_sel: Optional[int] = None, k_scale: Optional[torch.Tensor] = None,
                             v_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """The selection of a scored workspace (left by an index call with topk=None) into topk, then
    qsa_sparse_decode on it: o_part fp32 [P, R, H_q, d], lse_part fp32 [P, R, H_q]."""
    _dt(q, torch.bfloat16); _dt(o_part, torch.float32); _dt(lse_part, torch.float32)
    _dt(row_seq_len, torch.int32); _dt(sel_req, torch.int32); _dt(sel_seq_len, torch.int32)
    _dt(topk, torch.int32); _dt(block_table, torch.int32)
    c = cfg.to_c()
    R, S, mr = _row_map(q, row_sel, sel_req, max_rows_per_sel)
    P = o_part.shape[0]
    _check(_lib.load().qsa_select_sparse_decode(
        ctypes.byref(c), R, S, mr, P, int(max_seq_len), _ptr(q), _ptr(row_sel), _ptr(row_seq_len), _ptr(sel_req),
        _ptr(sel_seq_len), _ptr(block_table), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(topk), _ptr(o_part), _ptr(lse_part), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def qsa_select_sparse_decode_launches(cfg: QSAConfig, num_sel_rows: int, max_rows_per_sel: int, num_splits: int,
                                      max_seq_len: int) -> int:
    """Kernel launches qsa_select_sparse_decode makes for this shape (1: fused, 2: finalize + attention)."""
    c = cfg.to_c()
    return int(_lib.load().qsa_select_sparse_decode_launches(ctypes.byref(c), num_sel_rows, max_rows_per_sel,
                                                             num_splits, max_seq_len))


def qsa_merge_partials(o_part: torch.Tensor, lse_part: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor, stream=None) -> None:
    """LSE merge: out fp32 or bf16 [R, H, d] (by out's dtype), lse fp32 [R, H]."""
    _dt(o_part, torch.float32); _dt(lse_part, torch.float32); _dt(out, torch.float32, torch.bfloat16)
    _dt(lse, torch.float32)
    P, R, H, d = o_part.shape
    od = _lib.QSA_OUT_BF16 if out.dtype == torch.bfloat16 else _lib.QSA_OUT_F32
    _check(_lib.load().qsa_merge_partials(P, R, H, d, _ptr(o_part), _ptr(lse_part), _ptr(out), od, _ptr(lse),
                                          _stream(stream)))


def qsa_indexer_project_workspace_size(num_tokens: int, hidden_dim: int, index_dim: int) -> int:
    return int(_lib.load().qsa_indexer_project_workspace_size(num_tokens, hidden_dim, index_dim))


def _project_args(hidden, positions, w_qk, g_q, g_k, q_index, keys, workspace, pos_shape):
    _dt(hidden, torch.bfloat16); _dt(w_qk, torch.bfloat16); _dt(positions, torch.int32)
    _dt(g_q, torch.float32); _dt(g_k, torch.float32); _dt(q_index, torch.int8); _dt(keys, torch.int8)
    T, H = hidden.shape
    D = q_index.shape[1]
    if w_qk.shape != (2 * D, H) or keys.shape != (T, D) or q_index.shape[0] != T:
        raise QSAError(_lib.QSA_ERR_INVALID_ARGUMENT, "shape mismatch between hidden, w_qk, q_index and keys")
    if tuple(positions.shape) != pos_shape(T) or not positions.is_contiguous():
        raise QSAError(_lib.QSA_ERR_INVALID_ARGUMENT, f"positions must be contiguous int32 {pos_shape(T)}")
    need = qsa_indexer_project_workspace_size(T, H, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=hidden.device)
    return T, H, D, workspace


def qsa_indexer_project(hidden: torch.Tensor, positions: torch.Tensor, w_qk: torch.Tensor, g_q: torch.Tensor,
                        g_k: torch.Tensor, q_index: torch.Tensor, keys: torch.Tensor, rope_base: float = 10000.0,
                        q_scale: float = 32.0, k_scale: float = 32.0, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """Indexer front end: hidden bf16 [T, H], w_qk bf16 [2D, H] -> q_index, keys int8 [T, D].
    workspace: device scratch of qsa_indexer_project_workspace_size bytes (allocated here if None)."""
    T, H, D, workspace = _project_args(hidden, positions, w_qk, g_q, g_k, q_index, keys, workspace, lambda t: (t,))
    _check(_lib.load().qsa_indexer_project(T, H, D, _ptr(hidden), _ptr(positions), _ptr(w_qk), _ptr(g_q),
                                           _ptr(g_k), float(rope_base), float(q_scale), float(k_scale),
                                           _ptr(q_index), _ptr(keys), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))


def qsa_indexer_project_mrope(hidden: torch.Tensor, positions: torch.Tensor, sections, w_qk: torch.Tensor,
                              g_q: torch.Tensor, g_k: torch.Tensor, q_index: torch.Tensor, keys: torch.Tensor,
                              rope_base: float = 10000.0, q_scale: float = 32.0, k_scale: float = 32.0,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """The front end with MRoPE: positions int32 [3, T] (temporal, height, width),
    sections (s_t, s_h, s_w) summing to D/2."""
    T, H, D, workspace = _project_args(hidden, positions, w_qk, g_q, g_k, q_index, keys, workspace,
                                       lambda t: (3, t))
    s_t, s_h, s_w = (int(v) for v in sections)
    _check(_lib.load().qsa_indexer_project_mrope(T, H, D, _ptr(hidden), _ptr(positions), s_t, s_h, s_w,
                                                 _ptr(w_qk), _ptr(g_q), _ptr(g_k), float(rope_base),
                                                 float(q_scale), float(k_scale), _ptr(q_index), _ptr(keys),
                                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _stream(stream)))
