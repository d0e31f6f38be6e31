"""GPU parity of the multi-step MTP flow ([PR53896]: step 0 of the draft model
selects, later draft steps reuse that selection while the side cache keeps
taking their tokens; rejected draft tokens are dropped).

Per request: step 0 appends one token, selects and attends; three draft steps
each append a draft token and attend with the step-0 selection plus their own
tail; then a random number of drafts is accepted, the rest is rolled back (the
next qsa_compress restarts at the accepted length) and a bonus token is
appended, selected and attended.  Selections are compared bit for bit, outputs
within tolerance, with the oracle run on the token sequence that is current at
each step (the accepted sequence after the rollback).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import api
from block_sparse_attention_qsa_amd.pipeline import QSALayer
from block_sparse_attention_qsa_amd.workloads import QSAShape, make_workload
from oracle import qsa_oracle as O
from tests.harness import OUT_TOL, check_lse, check_out, host_copy, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
DRAFT = 3


def _compress(layer, wl, toks, before):
    """Append toks[b] (np int8 [n_b, D] or None) at seq_len_before[b] for every request."""
    D = wl.shape.index_dim
    parts, cu, bef = [], [0], []
    for b, t in enumerate(toks):
        if t is None or len(t) == 0:
            bef.append(-1)
            cu.append(cu[-1])
        else:
            parts.append(torch.as_tensor(t, device=DEV))
            bef.append(int(before[b]))
            cu.append(cu[-1] + len(t))
    keys = torch.cat(parts) if parts else torch.zeros((0, D), dtype=torch.int8, device=DEV)
    api.qsa_compress(layer.cfg, keys.contiguous(), torch.as_tensor(np.array(cu, np.int32), device=DEV),
                     torch.as_tensor(np.array(bef, np.int32), device=DEV), wl.block_table, layer.ring, layer.ckey,
                     max(1, max(len(t) for t in toks if t is not None)))


def _attend_and_check(layer, wl, h, sel_len, row_len, topk, what):
    """qsa_sparse_decode + merge with the given selection and lengths; compare to the oracle."""
    sel_t = torch.as_tensor(np.asarray(sel_len, np.int32), device=DEV)
    row_t = torch.as_tensor(np.asarray(row_len, np.int32), device=DEV)
    api.qsa_sparse_decode(layer.cfg, wl.q, row_t, wl.sel_req, sel_t, torch.as_tensor(topk, device=DEV),
                          wl.block_table, wl.k_cache, wl.v_cache, layer.o_part, layer.lse_part)
    api.qsa_merge_partials(layer.o_part, layer.lse_part, layer.out, layer.lse)
    torch.cuda.synchronize()
    ref = O.decode_rows(q=h.q, row_sel=np.arange(wl.num_rows), sel_req=h.sel_req, sel_seq_len=np.asarray(sel_len),
                        row_seq_len=np.asarray(row_len), topk=topk, block_table=h.block_table,
                        page_size=wl.shape.page_size, k_cache=h.k_cache, v_cache=h.v_cache,
                        kv_dtype=wl.shape.kv_dtype, scale=wl.shape.softmax_scale, num_splits=layer.P,
                        k_scale=h.k_scale, v_scale=h.v_scale)
    tol = OUT_TOL[wl.shape.kv_dtype]
    check_out(layer.out.float().cpu().numpy(), ref["out"], tol, f"{what} out")
    check_lse(layer.lse.cpu().numpy(), ref["lse"], f"{what} lse")


def _select_and_check(layer, wl, seqs, L, q_index, what):
    k = wl.shape.topk_blocks
    api.qsa_index_topk(layer.cfg, q_index, wl.sel_req, torch.as_tensor(np.asarray(L, np.int32), device=DEV),
                       wl.block_table, layer.ckey, layer.topk, layer.workspace, layer.max_seq_len)
    torch.cuda.synchronize()
    got = layer.topk.cpu().numpy()
    qi = q_index.cpu().numpy()
    for b in range(wl.num_reqs):
        ref = O.index_topk_row(qi[b], seqs[b][:L[b]], int(L[b]), k)
        assert np.array_equal(got[b], ref), f"{what}: request {b} selection differs from the oracle"
    return got.copy()


@pytest.mark.parametrize("seed", [0, 1])
def test_mtp_draft_steps_reuse_selection_and_rollback(seed):
    shape = QSAShape(16, 2, 128, 64, 512, 64)
    L0 = np.array([9001, 6002, 3003, 4097, 2050, 30000, 4, 7])  # every L % 4, short rows too
    B = len(L0)
    cap = L0 + DRAFT + 2
    wl = make_workload(shape, list(cap), step_tokens=1, seed=50 + seed, device=DEV, name="mtp")
    say(f"[gpu] mtp seed={seed} B={B}")
    h = host_copy(wl)
    rng = np.random.default_rng(900 + seed)
    D = shape.index_dim
    layer = QSALayer(wl, num_splits=3, poison=True, max_seq_len=int(cap.max()))
    seqs = [h.keys[h.key_off[b]:h.key_off[b] + int(cap[b])].copy() for b in range(B)]  # current sequences

    # prefix [0, L0)
    _compress(layer, wl, [seqs[b][:L0[b]] for b in range(B)], np.zeros(B, np.int64))
    # step 0: token L0, selects
    _compress(layer, wl, [seqs[b][L0[b]:L0[b] + 1] for b in range(B)], L0)
    q0 = wl.q_index
    top0 = _select_and_check(layer, wl, seqs, L0 + 1, q0, "step 0")
    _attend_and_check(layer, wl, h, L0 + 1, L0 + 1, top0, "step 0")
    # draft steps: new (draft) keys, selection reused, tails grow
    drafts = rng.integers(-127, 128, size=(B, DRAFT, D)).astype(np.int8)
    for i in range(1, DRAFT + 1):
        _compress(layer, wl, [drafts[b, i - 1:i] for b in range(B)], L0 + i)
        for b in range(B):
            seqs[b][L0[b] + i] = drafts[b, i - 1]
        _attend_and_check(layer, wl, h, L0 + 1, L0 + 1 + i, top0, f"draft step {i}")
    # verification: accept a[b] drafts, roll the rest back, append a bonus token and select again
    acc = rng.integers(0, DRAFT + 1, size=B)
    L_acc = L0 + 1 + acc
    bonus = rng.integers(-127, 128, size=(B, 1, D)).astype(np.int8)
    for b in range(B):
        seqs[b][L_acc[b]] = bonus[b, 0]
    _compress(layer, wl, [bonus[b] for b in range(B)], L_acc)
    q1 = torch.randint(-127, 128, (B, D), dtype=torch.int8, device=DEV)
    top1 = _select_and_check(layer, wl, seqs, L_acc + 1, q1, "after rollback")
    _attend_and_check(layer, wl, h, L_acc + 1, L_acc + 1, top1, "after rollback")
    # the compressed cache equals the one built from the accepted sequence in one go
    from tests.harness import ckey_blocks_from_cache
    ck = layer.ckey.cpu().numpy()
    for b in range(B):
        nb = int(L_acc[b] + 1) // 4
        assert np.array_equal(ckey_blocks_from_cache(wl, ck, b, nb), O.compress_keys(seqs[b], int(L_acc[b] + 1)))
