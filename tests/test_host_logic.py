"""Host-side logic without a GPU: the benchmark's algorithmic-byte accounting
against hand counts, and the structure of the seeded workloads (uneven draft
rows through the row map, chunked-prefill rows, the named shapes)."""
import numpy as np
import pytest
import torch

import bench
from block_sparse_attention_qsa_amd.workloads import (QSAShape, make_prefill_workload, make_workload,
                                                      mixed_lengths)


def test_algorithmic_parts_by_hand():
    """Two requests, one selecting row each, D = 64, 64-token pages, k = 4,
    16/2 heads of d = 128, bf16, 3 splits."""
    shape = QSAShape(16, 2, 128, 64, 4, 64)
    wl = make_workload(shape, [10, 1001], seed=3, name="bytes")
    p = bench.algorithmic_parts(wl, 3)
    # scan: floor(L/4) blocks x 80 B, ceil(L/64) page ids x 4 B, one query of 64 B per row
    assert p["scan"] == (2 * 80 + 250 * 80) + (1 + 16) * 4 + 2 * 64
    # K/V: row 0 has 2 closed blocks (< k: all kept) and 2 tail tokens -> 10 tokens;
    # row 1 keeps 4 blocks (16 tokens) plus a 1-token tail -> 17 tokens; 2 KV heads x 128 x 2 B, K and V
    assert p["kv"] == (10 + 17) * 2 * 128 * 2 * 2
    assert p["q"] == 2 * 16 * 128 * 2
    assert p["out"] == 2 * 16 * 128 * 4 + 2 * 16 * 4
    assert p["part"] == 3 * 2 * 16 * 129 * 4


def test_algorithmic_parts_fp8_adds_scales_and_reads_shared_kv_once():
    shape = QSAShape(16, 2, 128, 64, 512, 64, kv_dtype="fp8")
    wl = make_workload(shape, [40000], step_tokens=4, q_per_sel=4, seed=4, name="bytes-fp8")
    p = bench.algorithmic_parts(wl, 1)
    # the 4 rows share one selection: 512 blocks + the longest row's tail (40000 - 4*floor(39997/4) tokens)
    sel_len = int(wl.sel_seq_len[0])
    tail = 40000 - 4 * (sel_len // 4)
    ntok = 4 * 512 + tail
    assert p["kv"] == ntok * 2 * 128 * 1 * 2 + ntok * 4 * 2


@pytest.mark.parametrize("rows", [[1, 3, 0, 4, 2, 5], [0, 0, 1], [7]])
def test_uneven_draft_rows_map_to_their_requests_first_row(rows):
    shape = QSAShape(8, 2, 64, 32, 16, 16)
    lens = [300 + 37 * i for i in range(len(rows))]
    wl = make_workload(shape, lens, rows_per_req=rows, seed=5, name="uneven")
    row_sel = wl.row_sel.numpy()
    sel_req = wl.sel_req.numpy()
    row_len = wl.row_seq_len.numpy()
    sel_len = wl.sel_seq_len.numpy()
    active = [b for b, n in enumerate(rows) if n > 0]
    assert list(sel_req) == active and wl.num_rows == sum(rows) and wl.q_per_sel == max(rows)
    r = 0
    for s, b in enumerate(active):
        n = rows[b]
        assert list(row_sel[r:r + n]) == [s] * n
        # draft row j of request b sees the prefix plus j + 1 tokens; the first one is the selecting row
        assert list(row_len[r:r + n]) == [lens[b] - n + 1 + j for j in range(n)]
        assert sel_len[s] == row_len[r] and int(wl.final_len[b]) == lens[b]
        r += n


def test_prefill_rows_are_causal_and_delimited():
    shape = QSAShape(8, 2, 64, 32, 16, 16)
    wl = make_prefill_workload(shape, [100, 37, 64], [5, 37, 3], seed=6)
    cu = wl.extra["row_cu"].numpy()
    assert list(cu) == [0, 5, 42, 45]
    lens = wl.row_seq_len.numpy()
    assert list(lens[0:5]) == [96, 97, 98, 99, 100]
    assert list(lens[5:42]) == list(range(1, 38))
    assert list(wl.sel_req.numpy()) == [0] * 5 + [1] * 37 + [2] * 3
    assert torch.equal(wl.sel_seq_len, wl.row_seq_len)


def test_mixed_lengths_follow_the_stated_mix():
    L = np.asarray(mixed_lengths(3))
    assert L.shape == (128,) and L.min() >= 512 and L.max() <= 262144
    assert int((L <= 2048).sum()) == 13
