"""qsa_index_topk_noalloc (the library's own scratch, no workspace, no
allocation) against qsa_index_topk with a caller workspace, through the C ABI:
two calls in a row on one GPU, the second with a smaller input, then the
first again; every selection bit for bit, and against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import _lib, api
from block_sparse_attention_qsa_amd.pipeline import QSALayer
from block_sparse_attention_qsa_amd.workloads import SHAPE_MAIN, make_workload, named_workload
from tests.harness import host_copy, oracle_topk, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ready(wl):
    layer = QSALayer(wl, 1)
    layer.prefill()
    layer.compress()          # the step's tokens too: the cache holds every token
    torch.cuda.synchronize()
    return layer


def _noalloc(layer):
    wl, lib = layer.wl, _lib.load()
    out = torch.full((wl.num_sel, wl.shape.topk_blocks), -7, dtype=torch.int32, device=DEV)
    c = layer.cfg.to_c()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.qsa_index_topk_noalloc(ctypes.byref(c), wl.num_sel, layer.max_seq_len, p(wl.q_index), p(wl.sel_req),
                                    p(wl.sel_seq_len), p(wl.block_table), p(layer.ckey), p(out),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.qsa_last_error().decode()
    return out


def _with_workspace(layer):
    layer.topk.fill_(-7)
    layer.index()
    return layer.topk


def test_noalloc_matches_the_workspace_call_twice_then_smaller():
    big = _ready(named_workload(3, device=DEV, scale_ctx=1 / 4))                   # 8 rows of 65,536 tokens
    small = _ready(make_workload(SHAPE_MAIN, [20001, 513, 3], seed=77, device=DEV, name="noalloc-small"))
    runs = [big, small, big]
    for i, layer in enumerate(runs):
        wl = layer.wl
        say(f"[gpu] noalloc call {i}: {wl.name} S={wl.num_sel} Lmax={layer.max_seq_len}")
        got = _noalloc(layer)
        ref = _with_workspace(layer)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: the scratch call differs from the workspace call"
        h = host_copy(wl)
        assert np.array_equal(got.cpu().numpy(), oracle_topk(wl, h)), f"call {i}: differs from the oracle"
