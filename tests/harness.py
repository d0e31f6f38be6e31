"""Shared test plumbing: host copies of a workload and the oracle's expectations.

Expected values always come from the CPU oracle applied to the workload's own
inputs (raw indexer keys, paged K/V, q); never from the HIP path.
"""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np
import torch

from oracle import qsa_oracle as O

OUT_TOL = {"bf16": 5e-3, "fp8": 2e-2}
LSE_REL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class HostCopy:
    keys: np.ndarray
    key_off: np.ndarray
    block_table: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_scale: np.ndarray
    v_scale: np.ndarray
    q: np.ndarray
    q_index: np.ndarray
    sel_req: np.ndarray
    sel_seq_len: np.ndarray
    row_seq_len: np.ndarray
    row_sel: np.ndarray


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


def host_copy(wl) -> HostCopy:
    return HostCopy(
        keys=wl.keys.cpu().numpy(), key_off=wl.key_off, block_table=wl.block_table.cpu().numpy(),
        k_cache=_bits(wl.k_cache), v_cache=_bits(wl.v_cache),
        k_scale=None if wl.k_scale is None else wl.k_scale.cpu().numpy(),
        v_scale=None if wl.v_scale is None else wl.v_scale.cpu().numpy(),
        q=_bits(wl.q), q_index=wl.q_index.cpu().numpy(), sel_req=wl.sel_req.cpu().numpy(),
        sel_seq_len=wl.sel_seq_len.cpu().numpy(), row_seq_len=wl.row_seq_len.cpu().numpy(),
        row_sel=wl.row_sel.cpu().numpy())


def oracle_topk(wl, h: HostCopy, rows=None) -> np.ndarray:
    k = wl.shape.topk_blocks
    rows = range(wl.num_sel) if rows is None else rows
    out = np.full((wl.num_sel, k), -1, dtype=np.int32)
    for s in rows:
        b = int(h.sel_req[s])
        L = int(h.sel_seq_len[s])
        keys = h.keys[h.key_off[b]:h.key_off[b] + max(L, 0)]
        out[s] = O.index_topk_row(h.q_index[s], keys, L, k)
    return out


def oracle_decode(wl, h: HostCopy, topk: np.ndarray, num_splits: int, rows=None):
    return O.decode_rows(q=h.q, row_sel=h.row_sel, sel_req=h.sel_req, sel_seq_len=h.sel_seq_len,
                         row_seq_len=h.row_seq_len, topk=topk, block_table=h.block_table,
                         page_size=wl.shape.page_size, k_cache=h.k_cache, v_cache=h.v_cache,
                         kv_dtype=wl.shape.kv_dtype, scale=wl.shape.softmax_scale, num_splits=num_splits,
                         k_scale=h.k_scale, v_scale=h.v_scale, rows=rows)


def check_lse(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.float64)
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), f"{what}: -inf pattern differs"
    g, r = got[~ninf_ref], ref[~ninf_ref]
    if g.size:
        err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
        assert err.max() <= LSE_REL, f"{what}: lse rel err {err.max():.3e} > {LSE_REL}"


def check_out(got: np.ndarray, ref: np.ndarray, tol: float, what: str):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max() if got.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"
    return err


def ckey_blocks_from_cache(wl, ckey: np.ndarray, b: int, nb: int) -> np.ndarray:
    """Read the library's compressed-key storage back as int64 [nb, D] (the layout
    documented in include/qsa.h: s plane + two bit-masks, C = 256(2 b1 + b0) + s - 384)."""
    D, page = wl.shape.index_dim, wl.shape.page_size
    bpp = page // 4
    per_page = bpp * (D + D // 4)
    cache = ckey.reshape(-1, per_page)
    bt = wl.block_table[b].cpu().numpy()
    j = np.arange(nb)
    pages = bt[j // bpp]
    slots = j % bpp
    rows = cache[pages]                                     # [nb, per_page]
    splane = rows[:, : bpp * D].reshape(nb, D // 16, bpp, 16)
    sv = splane[np.arange(nb), :, slots, :].reshape(nb, D).astype(np.int64)
    masks = rows[:, bpp * D:].reshape(nb, bpp, D // 4)[np.arange(nb), slots].astype(np.uint8)
    bits = np.unpackbits(masks, axis=1, bitorder="little").astype(np.int64)  # [nb, 2D]
    b0, b1 = bits[:, :D], bits[:, D:]
    return 256 * (2 * b1 + b0) + sv - 384


def check_layer(wl, layer, h=None, rows=None, topk_ref=None):
    h = h or host_copy(wl)
    tol = OUT_TOL[wl.shape.kv_dtype]
    sel_rows = None if rows is None else sorted({int(h.row_sel[r]) for r in rows if h.row_sel[r] >= 0})
    ref_topk = oracle_topk(wl, h, sel_rows) if topk_ref is None else topk_ref
    got_topk = layer.topk.cpu().numpy()
    srows = range(wl.num_sel) if sel_rows is None else sel_rows
    for s in srows:
        assert np.array_equal(got_topk[s], ref_topk[s]), \
            f"{wl.name}: topk mismatch row {s}: first diff at {np.nonzero(got_topk[s] != ref_topk[s])[0][:5]}"
    ref = oracle_decode(wl, h, ref_topk, layer.P, rows=rows)
    rr = list(range(wl.num_rows)) if rows is None else list(rows)
    o_part = layer.o_part.cpu().numpy()[:, rr]
    lse_part = layer.lse_part.cpu().numpy()[:, rr]
    out = layer.out.float().cpu().numpy()[rr]
    lse = layer.lse.cpu().numpy()[rr]
    e1 = check_out(o_part, ref["o_part"], tol, f"{wl.name} o_part")
    check_lse(lse_part, ref["lse_part"], f"{wl.name} lse_part")
    e2 = check_out(out, ref["out"], tol, f"{wl.name} out")
    check_lse(lse, ref["lse"], f"{wl.name} lse")
    say(f"[gpu] {wl.name} ok: max|d o_part|={e1:.2e} max|d out|={e2:.2e}")
    return ref
