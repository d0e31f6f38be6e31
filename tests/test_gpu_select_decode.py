"""GPU parity of qsa_select_sparse_decode (the selection step and the attention
in one call).

Its contract is the selection half of qsa_index_topk followed by
qsa_sparse_decode.  Every case checks the selection bit for bit and the
partials / outputs within the bars against the oracle, and compares with the
two separate calls on the same inputs: the selection and the partials must
be identical (same kernels' arithmetic), bit for bit.  Shapes cover the one-
launch kernel (few workgroups, head groups up to 16, d = 64 and 128, bf16 and
fp8, selecting rows whose query rows are spread over several workgroups) and
the two-launch fallback (large grids, 16 heads per KV head at d = 128), rows
with fewer than k blocks, rows with nothing scored, and rows whose threshold
bin holds more candidates than the LDS (massive ties).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd.pipeline import QSALayer, QSAPrefill
from block_sparse_attention_qsa_amd.workloads import (SHAPE_FP8, SHAPE_MAIN, SHAPE_TINY, QSAShape, make_prefill_workload,
                                                      make_workload, named_workload)
from tests.harness import check_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(wl, P, cls=QSALayer, **kw):
    a = cls(wl, P, poison=True, **kw)
    b = cls(wl, P, poison=True, select_decode=False, **kw)
    assert a.select_decode and not b.select_decode
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
        # order over the tiles): both are checked against the oracle instead
        check_layer(b.wl, b)
        return
    assert torch.equal(a.o_part, b.o_part), "o_part differs from the separate calls"
    assert torch.equal(a.lse_part, b.lse_part), "lse_part differs from the separate calls"
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


CASES = [
    # (name, shape, lengths, q_per_sel, P, seed)
    ("main-mixed", SHAPE_MAIN, [70001, 9000, 2049, 13, 4, 3, 600, 40000], 1, 4, 401),
    ("main-p16", SHAPE_MAIN, [65536, 30000], 1, 16, 402),
    ("main-qps2", SHAPE_MAIN, [20001, 5000, 3], 2, 2, 403),   # 16 heads x d=128: two row groups
    ("g16-fallback", QSAShape(16, 1, 128, 64, 512, 64), [20001, 5000, 3], 1, 2, 418),  # 16 heads per KV head: two launches
    ("tiny-qps4", SHAPE_TINY, [3001, 100, 17, 2], 4, 3, 404),           # 4 heads x 4 rows, d=64
    ("d64-g8-qps2", QSAShape(16, 2, 64, 128, 64, 32), [12000, 777], 2, 5, 405),
    ("fp8", SHAPE_FP8, [50000, 1234, 9], 1, 8, 406),
    ("k7-short", QSAShape(8, 2, 64, 32, 7, 16), [3, 17, 27, 28, 29, 100, 1000], 1, 2, 407),
    ("fp8-d64-qps2", QSAShape(16, 2, 64, 64, 512, 64, kv_dtype="fp8"), [30000, 4099, 2], 2, 4, 408),
    ("page128", QSAShape(16, 2, 128, 64, 512, 128), [50001, 777, 12345], 1, 8, 409),
    ("k2048", QSAShape(16, 2, 128, 64, 2048, 64), [20000, 9003, 5000], 1, 4, 410),   # the largest k
    ("p1", SHAPE_MAIN, [40000, 3001, 2], 1, 1, 411),          # one split
    ("p32", SHAPE_MAIN, [90001, 20000, 7, 64], 1, 32, 412),   # 32 splits (two rounds of the merge's loads)
    # 4 query rows x 8 heads = 32 heads per selecting row, more than one fused workgroup holds:
    # two or four workgroups per KV head, each with its own query rows
    ("fp8-qps4-rowgroups", SHAPE_FP8, [70003, 9001, 4], 4, 4, 415),
    ("bf16-qps2-rowgroups", SHAPE_MAIN, [30001, 6002], 2, 8, 416),
    ("d64-qps4-rowgroups", QSAShape(16, 2, 64, 64, 512, 64), [40003, 5001], 4, 3, 417),
    # 16-token pages: row 0 spans 5,001 pages, more than the LDS page-table copy (looked up in global memory)
    ("page16-long", QSAShape(16, 2, 128, 64, 512, 16), [80001, 5000, 65536], 1, 4, 414),
]


@pytest.mark.parametrize("name,shape,lens,qps,P,seed", CASES, ids=[c[0] for c in CASES])
def test_select_decode_matches_oracle_and_separate_calls(name, shape, lens, qps, P, seed):
    wl = make_workload(shape, lens, q_per_sel=qps, seed=seed, device=DEV, name=f"seldec-{name}")
    say(f"[gpu] select+decode {name} S={wl.num_sel} R={wl.num_rows} P={P}")
    a, b = _pair(wl, P)
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_large_grid_uses_two_launches():
    """64 selecting rows x 2 KV heads x 4 splits = 512 workgroups: the fallback path."""
    lens = [3000 + 97 * i for i in range(64)]
    wl = make_workload(SHAPE_MAIN, lens, seed=31, device=DEV, name="seldec-grid512")
    a, b = _pair(wl, 4)
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
    a, b = _pair(wl, 4)
    check_layer(wl, a)
    _same(a, b)


def test_select_decode_rows_beyond_the_lds_bitmap():
    """max_seq_len above 1,048,576 tokens: the selection keeps its bitmap in the
    workspace (rows of up to 4M blocks), and the call takes the two-launch path."""
    wl = make_workload(SHAPE_MAIN, [70001, 9000, 13], seed=44, device=DEV, name="seldec-bigrows")
    a = QSALayer(wl, 4, poison=True, max_seq_len=1_200_000)
    b = QSALayer(wl, 4, poison=True, max_seq_len=1_200_000, select_decode=False)
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
