"""GPU parity of the chunked-prefill path (many query rows per request, each with
its own causal length).

Per-row selections from qsa_prefill_index_topk (the scan as an int8 MFMA GEMM)
are compared bit for bit with the oracle and with qsa_index_topk run on the
same rows; scores-only output is compared with the decode-path scores; the
attention of the whole prefill step (qsa_sparse_decode, one selecting row per
query row, then the merge) is held to the usual tolerances.  Expected values
come only from the oracle.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import api
from block_sparse_attention_qsa_amd.pipeline import QSALayer, QSAPrefill
from block_sparse_attention_qsa_amd.workloads import QSAShape, make_prefill_workload
from tests.harness import check_layer, host_copy, oracle_topk, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (index_dim D, page size, final lengths, chunk per request)
CASES = [
    (64, 64, [5000, 3001, 70], [64, 37, 70]),     # ragged chunks; one request is all chunk (L from 1)
    (32, 16, [2100, 999], [40, 16]),
    (128, 256, [12000, 6000], [33, 48]),
    (64, 16, [40000], [96]),
    (128, 64, [2051, 4096, 8], [17, 1, 8]),       # a one-row request; contexts below 4
]


def build(case, P=2):
    D, page, fl, ch = CASES[case]
    shape = QSAShape(16, 2, 128, D, 512, page)
    wl = make_prefill_workload(shape, fl, ch, seed=100 + case, device=DEV, name=f"prefill{case}")
    say(f"[gpu] prefill case {case}: D={D} page={page} lens={fl} chunks={ch} rows={wl.num_rows}")
    return wl


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_topk_matches_oracle_and_decode_path(case):
    wl = build(case)
    pf = QSAPrefill(wl, num_splits=2, poison=True)
    pf.prefill()
    pf.compress()
    pf.index()
    dec = QSALayer(wl, num_splits=2, poison=True)
    dec.prefill()
    dec.compress()
    dec.index()
    torch.cuda.synchronize()
    got = pf.topk.cpu().numpy()
    assert np.array_equal(got, dec.topk.cpu().numpy()), "prefill and decode-path selections differ"
    ref = oracle_topk(wl, host_copy(wl))
    bad = [r for r in range(wl.num_rows) if not np.array_equal(got[r], ref[r])]
    assert not bad, f"rows {bad[:5]} differ from the oracle"


@pytest.mark.parametrize("case", [0, 2])
def test_prefill_scores_only_equal_decode_scores(case):
    wl = build(case)
    pf = QSAPrefill(wl, num_splits=1, poison=True)
    dec = QSALayer(wl, num_splits=1, poison=True)
    for L in (pf, dec):
        L.prefill()
        L.compress()
    api.qsa_prefill_index_topk(pf.cfg, wl.q_index, pf.row_cu, wl.row_seq_len, wl.block_table, pf.ckey, None,
                               pf.workspace, pf.max_seq_len, pf.max_rows)
    api.qsa_index_topk(dec.cfg, wl.q_index, wl.sel_req, wl.sel_seq_len, wl.block_table, dec.ckey, None,
                       dec.workspace, dec.max_seq_len)
    torch.cuda.synchronize()
    stride = -(-(pf.max_seq_len // 4) // 1024) * 1024
    a = pf.workspace.view(torch.int32)[: wl.num_rows * stride].cpu().numpy().reshape(wl.num_rows, stride)
    b = dec.workspace.view(torch.int32)[: wl.num_rows * stride].cpu().numpy().reshape(wl.num_rows, stride)
    lens = wl.row_seq_len.cpu().numpy()
    for r in range(wl.num_rows):
        nb = int(lens[r]) // 4
        assert np.array_equal(a[r, :nb], b[r, :nb]), f"row {r}: scores differ"


@pytest.mark.parametrize("case,P", [(0, 1), (1, 3), (4, 2)])
def test_prefill_step_attention_parity(case, P):
    wl = build(case, P)
    pf = QSAPrefill(wl, num_splits=P, poison=True)
    pf.prefill()
    pf.step()
    torch.cuda.synchronize()
    check_layer(wl, pf)


def test_prefill_repeat_is_deterministic_and_workspace_clean():
    wl = build(0)
    pf = QSAPrefill(wl, num_splits=2)
    pf.prefill()
    pf.step()
    torch.cuda.synchronize()
    first = (pf.topk.clone(), pf.out.clone())
    for _ in range(3):
        pf.step()
    torch.cuda.synchronize()
    assert torch.equal(first[0], pf.topk)
    assert torch.equal(first[1], pf.out)
