"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same split counts), against the CPU oracle.

Every selecting row's top-k is checked bit for bit and every row's partials,
output and LSE against the oracle, in all five workloads; in the 128-request
mixed batch the short rows (<= 2,051 tokens) are also checked against dense
attention over their whole context.
"""
import numpy as np
import pytest
import torch

from bench import BENCH_SPLITS
from block_sparse_attention_qsa_amd.pipeline import QSALayer
from block_sparse_attention_qsa_amd.workloads import mixed_lengths, named_workload
from oracle import qsa_oracle as O
from tests.harness import OUT_TOL, check_lse, check_out, host_copy, oracle_topk, say
from tests.test_gpu_parity import check_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _full(cfg, splits, rows=None):
    wl = named_workload(cfg, device=DEV)
    say(f"[gpu-full] {wl.name}: B={wl.num_reqs} rows={wl.num_rows} Lmax={int(wl.final_len.max())} splits={splits}")
    h = host_copy(wl)
    sel_rows = None if rows is None else sorted({int(h.row_sel[r]) for r in rows})
    ref_topk = oracle_topk(wl, h, sel_rows)
    out = None
    for P in splits:
        layer = QSALayer(wl, num_splits=P)
        layer.prefill()
        layer.step()
        torch.cuda.synchronize()
        check_layer(wl, layer, h, rows=rows, topk_ref=ref_topk)
        out = (layer.out.cpu().numpy(), layer.lse.cpu().numpy())
        del layer
        torch.cuda.empty_cache()
    return wl, h, out


def test_full_cfg1_tiny():
    _full(1, sorted({1, 2, BENCH_SPLITS[1]}))


def test_full_cfg2_decode_32k():
    _full(2, sorted({1, BENCH_SPLITS[2]}))


def test_full_cfg3_long_256k():
    _full(3, sorted({1, 2, 8, BENCH_SPLITS[3]}))


def test_full_cfg4_mixed():
    """128 mixed-length requests; the short ones (<= 2,051 tokens) must equal dense attention."""
    L = np.array(mixed_lengths(3))
    short = [int(r) for r in np.nonzero(L <= 2051)[0]]
    assert len(short) >= 10
    wl, h, (out, lse) = _full(4, [BENCH_SPLITS[4]])
    for r in short:
        toks = np.arange(int(L[r]))
        K = O.decode_kv(O.paged_rows(h.k_cache, h.block_table[r], 64, toks), "bf16")
        V = O.decode_kv(O.paged_rows(h.v_cache, h.block_table[r], 64, toks), "bf16")
        o, l = O.attend(O.bf16_bits_to_f64(h.q[r]), K, V, wl.shape.softmax_scale)
        check_out(out[r], o, OUT_TOL["bf16"], f"dense row {r} L={int(L[r])}")
        check_lse(lse[r], l, f"dense row {r}")


def test_full_cfg5_fp8_1m():
    _full(5, sorted({1, BENCH_SPLITS[5]}))
