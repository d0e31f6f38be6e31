"""GPU parity at the interface's limits, against the CPU oracle: the longest row
the library accepts (QSA_MAX_SEQ_LEN = 8,388,608 tokens, 2^21 micro-blocks:
2,048 chunks per row, more than the LDS bitmap holds, so the two-launch path
with four classification rounds of 512 chunks), the largest split count (64,
most splits of a short row empty), and the smallest top-k (k = 1).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import _lib, api
from block_sparse_attention_qsa_amd.pipeline import QSALayer
from block_sparse_attention_qsa_amd.workloads import QSAShape, make_workload
from tests.harness import check_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(wl, P):
    say(f"[gpu] {wl.name}: B={wl.num_reqs} Lmax={int(wl.final_len.max())} k={wl.shape.topk_blocks} P={P}")
    layer = QSALayer(wl, num_splits=P, poison=True)
    layer.prefill()
    layer.step()
    torch.cuda.synchronize()
    return layer


def test_longest_row_the_library_accepts():
    L = _lib.QSA_MAX_SEQ_LEN
    shape = QSAShape(4, 1, 64, 64, 512, 64)
    wl = make_workload(shape, [L, 4099, 9], seed=61, device=DEV, name="max-seq-len")
    layer = _run(wl, 64)
    assert api.qsa_select_sparse_decode_launches(layer.cfg, wl.num_sel, 1, 64, layer.max_seq_len) == 2
    check_layer(wl, layer)
    del layer
    torch.cuda.empty_cache()


def test_sixty_four_splits_mostly_empty():
    """64 splits over rows of 1 to 300 closed blocks: most splits own nothing
    and must give (0, -inf); the merge still gives the row's attention."""
    shape = QSAShape(16, 2, 128, 64, 512, 64)
    wl = make_workload(shape, [5, 64, 259, 1203, 40000], seed=62, device=DEV, name="p64")
    layer = _run(wl, 64)
    check_layer(wl, layer)
    lse_part = layer.lse_part.cpu().numpy()
    assert np.isneginf(lse_part[:, 0]).sum() >= 60 * lse_part.shape[2]   # row 0 has one closed block


@pytest.mark.parametrize("P", [1, 2])
def test_top_one_block(P):
    shape = QSAShape(8, 2, 64, 32, 1, 16)
    wl = make_workload(shape, [3, 4, 5, 8, 100, 5000, 70001], seed=63, device=DEV, name="k1")
    layer = _run(wl, P)
    check_layer(wl, layer)
