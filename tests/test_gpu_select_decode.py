"""GPU parity of qsa_select_sparse_decode (the selection step and the attention
in one call).

Its contract is the selection half of qsa_index_topk followed by
qsa_sparse_decode.  Every case checks the selection bit for bit and the
partials / outputs within the bars against the oracle, and compares with the
two separate calls on the same inputs: the selection and the partials must
be identical (same kernels' arithmetic, same order), bit for bit.  Shapes cover the one-
launch kernel (few workgroups, head groups up to 16, d = 64 and 128, bf16 and
fp8, selecting rows whose query rows are spread over several workgroups,
uneven draft rows per request through row_sel) and the two-launch fallback
(large grids, one row with more heads than a workgroup holds, slices past
the LDS bitmap), rows with fewer than k blocks, rows with nothing scored, and
rows whose threshold bin holds more candidates than the LDS (massive ties),
coarse ties on both sides of the selection's key-count switch, and a row
whose selection clusters in its most recent chunks (score fallback).
Each case also asserts which of the two paths the library takes.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import api
from block_sparse_attention_qsa_amd.pipeline import QSALayer, QSAPrefill
from block_sparse_attention_qsa_amd.workloads import (SHAPE_FP8, SHAPE_MAIN, SHAPE_TINY, QSAShape, make_prefill_workload,
                                                      make_workload, named_workload)
from tests.harness import check_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(wl, P, cls=QSALayer, launches=None, **kw):
    a = cls(wl, P, poison=True, **kw)
    b = cls(wl, P, poison=True, select_decode=False, **kw)
    assert a.select_decode and not b.select_decode
    if launches is not None:  # which path the call takes (one kernel, or the finalize then the attention)
        got = api.qsa_select_sparse_decode_launches(a.cfg, wl.num_sel, wl.q_per_sel, P, a.max_seq_len)
        assert got == launches, f"expected {launches} launch(es), the library takes {got}"
    for layer in (a, b):
        layer.prefill()
        layer.step()
    torch.cuda.synchronize()
    return a, b


def _same(a, b):
    assert torch.equal(a.topk, b.topk), "selection differs from the separate calls"
    sh = a.wl.shape
    if a.wl.q_per_sel * (sh.num_q_heads // sh.num_kv_heads) > 16:
        # the separate decode then runs 4-wave workgroups (a different summation
        # order over the tiles) while the fused kernel spreads the rows over
        # 8-wave row groups: both are checked against the oracle instead
        check_layer(b.wl, b)
        return
    assert torch.equal(a.o_part, b.o_part), "o_part differs from the separate calls"
    assert torch.equal(a.lse_part, b.lse_part), "lse_part differs from the separate calls"
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


CASES = [
    # (name, shape, lengths, q_per_sel, P, seed, launches)
    ("main-mixed", SHAPE_MAIN, [70001, 9000, 2049, 13, 4, 3, 600, 40000], 1, 4, 401, 1),
    ("main-p16", SHAPE_MAIN, [65536, 30000], 1, 16, 402, 1),
    ("main-qps2", SHAPE_MAIN, [20001, 5000, 3], 2, 2, 403, 1),      # 16 heads x d=128: two row groups
    ("g16-fallback", QSAShape(16, 1, 128, 64, 512, 64), [20001, 5000, 3], 1, 2, 418, 2),  # 16 heads at d=128
    ("g16-d64", QSAShape(16, 1, 64, 64, 512, 64), [20001, 5000, 3], 1, 2, 420, 1),      # 16 heads at d=64
    ("g32-fallback", QSAShape(32, 1, 64, 64, 512, 64), [20001, 5000, 3], 1, 2, 419, 2),  # 32 heads of one row
    ("tiny-qps4", SHAPE_TINY, [3001, 100, 17, 2], 4, 3, 404, 1),           # 4 heads x 4 rows, d=64
    ("d64-g8-qps2", QSAShape(16, 2, 64, 128, 64, 32), [12000, 777], 2, 5, 405, 1),
    ("fp8", SHAPE_FP8, [50000, 1234, 9], 1, 8, 406, 1),
    ("k7-short", QSAShape(8, 2, 64, 32, 7, 16), [3, 17, 27, 28, 29, 100, 1000], 1, 2, 407, 1),
    ("fp8-d64-qps2", QSAShape(16, 2, 64, 64, 512, 64, kv_dtype="fp8"), [30000, 4099, 2], 2, 4, 408, 1),
    ("page128", QSAShape(16, 2, 128, 64, 512, 128), [50001, 777, 12345], 1, 8, 409, 1),
    ("k2048", QSAShape(16, 2, 128, 64, 2048, 64), [20000, 9003, 5000], 1, 4, 410, 1),   # the largest k
    ("p1", SHAPE_MAIN, [40000, 3001, 2], 1, 1, 411, 1),          # one split
    ("p32", SHAPE_MAIN, [90001, 20000, 7, 64], 1, 32, 412, 1),   # 32 splits (two rounds of the merge's loads)
    # 4 query rows x 8 heads = 32 heads per selecting row, more than one fused workgroup holds:
    # several row groups per KV head, each with its own query rows
    ("fp8-qps4-rowgroups", SHAPE_FP8, [70003, 9001, 4], 4, 4, 415, 1),
    ("bf16-qps2-rowgroups", SHAPE_MAIN, [30001, 6002], 2, 8, 416, 1),
    ("d64-qps4-rowgroups", QSAShape(16, 2, 64, 64, 512, 64), [40003, 5001], 4, 3, 417, 1),
    # 16-token pages: row 0 spans 18,751 pages, more than the LDS page-table copy (looked up in global memory)
    ("page16-long", QSAShape(16, 2, 128, 64, 512, 16), [300001, 5000, 65536], 1, 2, 414, 1),
]


@pytest.mark.parametrize("name,shape,lens,qps,P,seed,launches", CASES, ids=[c[0] for c in CASES])
def test_select_decode_matches_oracle_and_separate_calls(name, shape, lens, qps, P, seed, launches):
    wl = make_workload(shape, lens, q_per_sel=qps, seed=seed, device=DEV, name=f"seldec-{name}")
    say(f"[gpu] select+decode {name} S={wl.num_sel} R={wl.num_rows} P={P}")
    a, b = _pair(wl, P, launches=launches)
    check_layer(wl, a)
    _same(a, b)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_uneven_draft_rows_through_row_sel(kv):
    """Requests carry 1, 3, 0, 4, 2 and 5 draft tokens: one query row each, all
    sharing the selection of their request's first one (row_sel), with their
    own tails; an idle request has no rows.  One call, against the oracle and
    the separate calls."""
    shape = QSAShape(16, 2, 128, 64, 512, 64, kv_dtype=kv)
    wl = make_workload(shape, [40007, 9001, 5000, 70001, 2050, 30000], rows_per_req=[1, 3, 0, 4, 2, 5],
                       seed=421, device=DEV, name=f"seldec-uneven-{kv}")
    assert wl.num_sel == 5 and wl.num_rows == 15 and wl.q_per_sel == 5
    say(f"[gpu] uneven draft rows {kv}: S={wl.num_sel} R={wl.num_rows}")
    a, b = _pair(wl, 4, launches=1)
    check_layer(wl, a)
    check_layer(wl, b)
    assert torch.equal(a.topk, b.topk)


@pytest.mark.parametrize("L,kv", [(100003, "bf16"), (200003, "bf16"), (200003, "fp8"), (600003, "fp8")])
def test_row_map_at_each_key_count(L, kv):
    """Uneven draft rows through row_sel with the longest row at 100k, 200k and
    600k tokens: the fused selection's first round then reads 4, 6 and 8 list
    keys per thread (16, 8 and 2 threads per chunk)."""
    shape = QSAShape(16, 2, 128, 64, 512, 64, kv_dtype=kv)
    wl = make_workload(shape, [L, 9001, 5000], rows_per_req=[2, 3, 1], seed=424, device=DEV,
                       name=f"seldec-rowmap-{L}-{kv}")
    say(f"[gpu] row map with the longest row at {L} tokens ({kv})")
    a, b = _pair(wl, 4, launches=1)
    check_layer(wl, a)
    check_layer(wl, b)
    assert torch.equal(a.topk, b.topk)


@pytest.mark.parametrize("L,kv", [(200003, "bf16"), (600003, "fp8")])
def test_head_dim_64_at_six_and_eight_keys(L, kv):
    """d = 64 (16 heads of one KV group per workgroup) with rows long enough
    for 6 and 8 list keys per thread."""
    shape = QSAShape(16, 1, 64, 64, 512, 64, kv_dtype=kv)
    wl = make_workload(shape, [L, 20001, 3], seed=425, device=DEV, name=f"seldec-d64-{L}-{kv}")
    say(f"[gpu] d=64, longest row {L} tokens ({kv})")
    a, b = _pair(wl, 3, launches=1)
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_large_grid_uses_two_launches():
    """64 selecting rows x 2 KV heads x 4 splits = 512 workgroups: the fallback path."""
    lens = [3000 + 97 * i for i in range(64)]
    wl = make_workload(SHAPE_MAIN, lens, seed=31, device=DEV, name="seldec-grid512")
    a, b = _pair(wl, 4, launches=2)
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_massive_ties():
    """All keys equal: every block ties, so the threshold bin holds every block
    (5,000 candidates in row 0, more than the LDS keeps): the lowest ids win."""
    wl = make_workload(SHAPE_MAIN, [20000, 9000, 17000], seed=6, device=DEV, name="seldec-ties")
    wl.keys.fill_(3)
    a, b = _pair(wl, 2)
    got = a.topk.cpu().numpy()
    for s in range(3):
        assert np.array_equal(got[s], np.arange(512))
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_coarse_ties_over_several_chunks():
    """Keys in {-1, 0, 1}: scores in a narrow range, thousands of candidates in
    the threshold bin spread over many chunks, lists short of the bin."""
    wl = make_workload(SHAPE_MAIN, [80000, 30001], seed=7, device=DEV, name="seldec-coarse")
    g = torch.Generator(device=DEV).manual_seed(7)
    wl.keys.copy_(torch.randint(-1, 2, wl.keys.shape, generator=g, device=DEV, dtype=torch.int8))
    a, b = _pair(wl, 4)
    check_layer(wl, a)
    _same(a, b)


@pytest.mark.parametrize("L", [131072, 131080])
def test_select_decode_coarse_ties_either_side_of_the_key_count_switch(L):
    """Rows of up to 131,072 tokens (32 chunks, 16 threads per chunk) take
    lists of 2 x the threads per chunk and 4 keys per thread in the fused
    selection's first round; one more block (33 chunks, 8 threads per chunk)
    switches to lists of 3 x and 6 keys.  Coarse ties put many blocks in each
    list's last bin, so on both sides lists overflow the first round and
    chunks go to the score fallback."""
    wl = make_workload(SHAPE_MAIN, [L, 40001, 5], seed=22, device=DEV, name=f"seldec-switch-{L}")
    g = torch.Generator(device=DEV).manual_seed(22)
    wl.keys.copy_(torch.randint(-1, 2, wl.keys.shape, generator=g, device=DEV, dtype=torch.int8))
    say(f"[gpu] coarse ties at the key-count switch, L={L}")
    a, b = _pair(wl, 4, launches=1)
    check_layer(wl, a)
    _same(a, b)


@pytest.mark.parametrize("L", [100003, 200003])
def test_select_decode_recent_blocks_cluster(L):
    """Request 0's most recent 6,000 tokens get keys aligned with its query
    (random magnitudes, so the scores differ): the top-512 of that row falls
    in the last one or two chunks, each holding far more selected blocks than
    its list, so those chunks take the score fallback while the rest of the
    row has none selected.  Both sides of the key-count switch (25 and 49
    chunks)."""
    wl = make_workload(SHAPE_MAIN, [L, 40001, 777], seed=23, device=DEV, name=f"seldec-cluster-{L}")
    b0 = int(wl.sel_req[0])
    lo, hi = int(wl.key_off[b0]) + L - 6000, int(wl.key_off[b0]) + L
    sign = torch.sign(wl.q_index[0].to(torch.int32))
    g = torch.Generator(device=DEV).manual_seed(23)
    mag = torch.randint(40, 128, (hi - lo, wl.shape.index_dim), generator=g, device=DEV, dtype=torch.int32)
    wl.keys[lo:hi] = (sign[None, :] * mag).to(torch.int8)
    say(f"[gpu] clustered recent blocks, L={L}")
    a, b = _pair(wl, 4, launches=1)
    top = a.topk.cpu().numpy()[0]
    assert (top >= (L - 6000) // 4 - 1).all(), "the row's selection should sit in its recent blocks"
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_repeat_leaves_workspace_clean():
    """Repeated steps give the same results (the histogram and the row
    counters are left clear), and a selecting index call on the same workspace
    afterwards still agrees with the oracle."""
    wl = named_workload(3, device=DEV, scale_ctx=1 / 16)
    layer = QSALayer(wl, 16)
    layer.prefill()
    layer.step()
    torch.cuda.synchronize()
    first = [t.clone() for t in (layer.topk, layer.o_part, layer.lse_part, layer.out, layer.lse)]
    for _ in range(3):
        layer.step()
    torch.cuda.synchronize()
    for x, y in zip(first, (layer.topk, layer.o_part, layer.lse_part, layer.out, layer.lse)):
        assert torch.equal(x, y)
    layer.topk.fill_(-7)
    layer.index()          # selecting call: needs a clean histogram
    torch.cuda.synchronize()
    assert torch.equal(layer.topk, first[0])
    check_layer(wl, layer)


def test_select_decode_prefill_rows():
    """Chunked-prefill rows (one selecting row per query row, own causal lengths)."""
    wl = make_prefill_workload(SHAPE_MAIN, [9000, 4100], 24, seed=12, device=DEV, name="seldec-prefill")
    a, b = _pair(wl, 2, cls=QSAPrefill)
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_named_decode_batch():
    """The 32-request decode batch (scaled): 32 rows x 2 heads x 4 splits = 256 workgroups, one launch."""
    wl = named_workload(2, device=DEV, scale_ctx=1 / 8)
    a, b = _pair(wl, 4, launches=1)
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_rows_beyond_the_lds_bitmap():
    """max_seq_len above 1,048,576 tokens: the selection keeps its bitmap in the
    workspace (rows of up to 4M blocks), and the call takes the two-launch path."""
    wl = make_workload(SHAPE_MAIN, [70001, 9000, 13], seed=44, device=DEV, name="seldec-bigrows")
    a = QSALayer(wl, 2, poison=True, max_seq_len=1_200_000)
    b = QSALayer(wl, 2, poison=True, max_seq_len=1_200_000, select_decode=False)
    assert api.qsa_select_sparse_decode_launches(a.cfg, wl.num_sel, 1, 2, 1_200_000) == 2
    for layer in (a, b):
        layer.prefill()
        layer.step()
        layer.step()          # twice: the workspace protocol across calls
    torch.cuda.synchronize()
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_bf16_out():
    """bf16 merged output: the fp32 merge rounded to nearest even (torch's cast)."""
    wl = make_workload(SHAPE_MAIN, [50000, 8191, 600], seed=413, device=DEV, name="seldec-bf16")
    a, b = _pair(wl, 8, out_dtype=torch.bfloat16)
    f = QSALayer(wl, 8, poison=True)
    f.prefill()
    f.step()
    torch.cuda.synchronize()
    check_layer(wl, f)
    _same(a, b)
    assert torch.equal(a.out, f.out.to(torch.bfloat16)) and torch.equal(a.lse, f.lse)
