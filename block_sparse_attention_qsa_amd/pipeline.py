"""One QSA layer's decode step on the GPU: buffers plus the four library calls.

QSALayer owns the device buffers one layer needs (compressed-key cache, ring,
top-k workspace, selection, split partials, output) for a Workload, and runs

    compress  ->  index_topk  ->  sparse_decode  ->  merge_partials

on one stream; when the step appends at most 5 tokens per request the first
two are one call, qsa_compress_index_topk (fuse_append=False keeps them apart),
and the selection step of index_topk runs with the attention, in
qsa_select_sparse_decode (select_decode=False keeps them apart).
It only allocates and sequences; all arithmetic is in libqsa.so.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import api
from .workloads import Workload


def config_for(wl: Workload) -> api.QSAConfig:
    s = wl.shape
    return api.QSAConfig(num_q_heads=s.num_q_heads, num_kv_heads=s.num_kv_heads, head_dim=s.head_dim,
                         index_dim=s.index_dim, topk_blocks=s.topk_blocks, page_size=s.page_size,
                         max_pages_per_req=int(wl.block_table.shape[1]), kv_dtype=s.kv_dtype,
                         softmax_scale=s.softmax_scale, compress_ratio=s.compress_ratio)


def _rows(keys: torch.Tensor, key_off: np.ndarray, lo: np.ndarray, hi: np.ndarray):
    """Concatenate keys[key_off[b]+lo[b] : key_off[b]+hi[b]] over requests -> (keys, cu)."""
    B = len(lo)
    parts, cu = [], np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        n = int(max(hi[b] - lo[b], 0))
        cu[b + 1] = cu[b] + n
        if n:
            a = int(key_off[b] + lo[b])
            parts.append(keys[a:a + n])
    D = keys.shape[1]
    out = torch.cat(parts) if parts else torch.zeros((0, D), dtype=torch.int8, device=keys.device)
    return out.contiguous(), cu


class QSALayer:
    def __init__(self, wl: Workload, num_splits: int = 1, poison: bool = False,
                 max_seq_len: Optional[int] = None, out_dtype: torch.dtype = torch.float32,
                 fuse_append: bool = True, select_decode: bool = True):
        dev = wl.q.device
        self.wl = wl
        self.cfg = config_for(wl)
        self.P = int(num_splits)
        s = wl.shape
        B, S, R = wl.num_reqs, wl.num_sel, wl.num_rows
        fill = (lambda t: t.fill_(0x7F) if t.dtype == torch.int8 else t.fill_(float("nan"))) if poison \
            else (lambda t: t.zero_())
        self.ckey = fill(torch.empty(api.ckey_cache_bytes(self.cfg, wl.num_pages), dtype=torch.int8, device=dev))
        self.ring = fill(torch.empty((B, 8, s.index_dim), dtype=torch.int8, device=dev))
        self.max_seq_len = int(max_seq_len if max_seq_len is not None else int(wl.final_len.max()))
        ws_bytes = api.qsa_index_topk_workspace_size(self.cfg, S, self.max_seq_len)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if poison:
            self.workspace.fill_(0x7F)
        api.qsa_index_topk_workspace_init(self.workspace)
        self.topk = torch.full((S, s.topk_blocks), -7, dtype=torch.int32, device=dev)
        self.o_part = fill(torch.empty((self.P, R, s.num_q_heads, s.head_dim), dtype=torch.float32, device=dev))
        self.lse_part = fill(torch.empty((self.P, R, s.num_q_heads), dtype=torch.float32, device=dev))
        self.out = torch.empty((R, s.num_q_heads, s.head_dim), dtype=out_dtype, device=dev)
        self.lse = torch.empty((R, s.num_q_heads), dtype=torch.float32, device=dev)
        # step inputs (the tokens appended in the step), prepared once
        self.step_keys, cu = _rows(wl.keys, wl.key_off, wl.prefix_len, wl.final_len)
        self.step_cu = torch.as_tensor(cu.astype(np.int32), device=dev)
        self.step_before = torch.as_tensor(wl.prefix_len.astype(np.int32), device=dev)
        self.step_max_new = int((wl.final_len - wl.prefix_len).max()) if B else 0
        self.fused = bool(fuse_append) and self.step_max_new <= 5
        self.select_decode = bool(select_decode)
        # one row per selecting row, in order: no row map (the library's identity)
        ident = wl.num_rows == wl.num_sel and wl.q_per_sel == 1 and bool(
            (wl.row_sel.cpu() == torch.arange(wl.num_rows, dtype=torch.int32)).all())
        self.row_sel = None if ident else wl.row_sel

    def prefill(self, chunk: Optional[int] = None) -> None:
        """Bulk-compress every request's prefix [0, prefix_len) (optionally in chunks)."""
        wl = self.wl
        B = wl.num_reqs
        total = wl.prefix_len
        step = int(total.max()) if chunk is None else int(chunk)
        done = np.zeros(B, dtype=np.int64)
        while (done < total).any():
            hi = np.minimum(done + max(step, 1), total)
            keys, cu = _rows(wl.keys, wl.key_off, done, hi)
            api.qsa_compress(self.cfg, keys, torch.as_tensor(cu.astype(np.int32), device=keys.device),
                             torch.as_tensor(np.where(hi > done, done, -1).astype(np.int32), device=keys.device),
                             wl.block_table, self.ring, self.ckey, int((hi - done).max()))
            done = hi

    def compress(self, stream=None) -> None:
        api.qsa_compress(self.cfg, self.step_keys, self.step_cu, self.step_before, self.wl.block_table,
                         self.ring, self.ckey, self.step_max_new, stream=stream)

    def index(self, stream=None, select: bool = True) -> None:
        """select=False scores only (the selection is left to select_attend)."""
        wl = self.wl
        api.qsa_index_topk(self.cfg, wl.q_index, wl.sel_req, wl.sel_seq_len, wl.block_table, self.ckey,
                           self.topk if select else None, self.workspace, self.max_seq_len, stream=stream)

    def compress_index(self, stream=None, select: bool = True) -> None:
        wl = self.wl
        api.qsa_compress_index_topk(self.cfg, self.step_keys, self.step_cu, self.step_before, self.ring,
                                    wl.q_index, wl.sel_req, wl.sel_seq_len, wl.block_table, self.ckey,
                                    self.topk if select else None, self.workspace, self.step_max_new,
                                    self.max_seq_len, stream=stream)

    def decode(self, stream=None) -> None:
        wl = self.wl
        api.qsa_sparse_decode(self.cfg, wl.q, wl.row_seq_len, wl.sel_req, wl.sel_seq_len, self.topk,
                              wl.block_table, wl.k_cache, wl.v_cache, self.o_part, self.lse_part,
                              row_sel=self.row_sel, max_rows_per_sel=wl.q_per_sel, k_scale=wl.k_scale,
                              v_scale=wl.v_scale, stream=stream)

    def select_attend(self, stream=None) -> None:
        """Selection of the scored workspace into topk, then the attention (one call)."""
        wl = self.wl
        api.qsa_select_sparse_decode(self.cfg, wl.q, wl.row_seq_len, wl.sel_req, wl.sel_seq_len, wl.block_table,
                                     wl.k_cache, wl.v_cache, self.topk, self.o_part, self.lse_part,
                                     self.workspace, self.max_seq_len, row_sel=self.row_sel,
                                     max_rows_per_sel=wl.q_per_sel, k_scale=wl.k_scale, v_scale=wl.v_scale,
                                     stream=stream)

    def merge(self, stream=None) -> None:
        api.qsa_merge_partials(self.o_part, self.lse_part, self.out, self.lse, stream=stream)

    def step(self, stream=None) -> None:
        """One decode step: the whole hot path."""
        sel = not self.select_decode
        if self.fused:
            self.compress_index(stream, select=sel)
        else:
            self.compress(stream)
            self.index(stream, select=sel)
        if self.select_decode:
            self.select_attend(stream)
        else:
            self.decode(stream)
        self.merge(stream)


class QSAPrefill(QSALayer):
    """Chunked prefill (a workload from make_prefill_workload): compress the chunk,
    select per query row with qsa_prefill_index_topk (the scan as an int8 GEMM),
    attend with qsa_sparse_decode (one selecting row per query row), merge."""

    def __init__(self, wl: Workload, num_splits: int = 1, poison: bool = False,
                 max_seq_len: Optional[int] = None, out_dtype: torch.dtype = torch.float32,
                 select_decode: bool = True):
        super().__init__(wl, num_splits=num_splits, poison=poison, max_seq_len=max_seq_len, out_dtype=out_dtype,
                         fuse_append=False, select_decode=select_decode)
        self.row_cu = wl.extra["row_cu"]
        self.max_rows = int(wl.extra["max_rows_per_req"])

    def index(self, stream=None, select: bool = True) -> None:
        wl = self.wl
        api.qsa_prefill_index_topk(self.cfg, wl.q_index, self.row_cu, wl.row_seq_len, wl.block_table, self.ckey,
                                   self.topk if select else None, self.workspace, self.max_seq_len, self.max_rows,
                                   stream=stream)

