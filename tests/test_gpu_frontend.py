"""GPU parity of the indexer front end (qsa_indexer_project, and
qsa_indexer_project_mrope with three position components) against the
front-end oracle, and of the chain front end -> compress -> selection.

The int8 outputs must equal the oracle's, except by one where the oracle's
value before rounding lies within 2e-3 of a rounding boundary (fp32 sums of
bf16 products vs float64; the header states this).  Expected values come only
from the oracle.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import api
from block_sparse_attention_qsa_amd.pipeline import QSALayer
from block_sparse_attention_qsa_amd.workloads import QSAShape, make_workload
from oracle import qsa_frontend_oracle as F
from oracle import qsa_oracle as O
from tests.harness import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BOUNDARY = 2e-3


def inputs(T, H, D, seed, max_pos=1 << 23):
    g = torch.Generator(device="cpu").manual_seed(seed)
    hidden = torch.randn((T, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((2 * D, H), generator=g) / np.sqrt(H)).to(torch.bfloat16)
    gq = (0.1 * torch.randn(D, generator=g)).float()
    gk = (0.1 * torch.randn(D, generator=g)).float()
    pos = torch.randint(0, max_pos, (T,), generator=g, dtype=torch.int32)
    pos[: min(T, 3)] = torch.tensor([0, 1, max_pos - 1][: min(T, 3)], dtype=torch.int32)
    return hidden, w, gq, gk, pos


def oracle(hidden, w, gq, gk, pos, D, base, qs, ks):
    h = F.bf16_bits_to_f64(hidden.view(torch.int16).numpy())
    wf = F.bf16_bits_to_f64(w.view(torch.int16).numpy())
    return F.indexer_frontend(h, pos.numpy(), wf, gq.numpy().astype(np.float64), gk.numpy().astype(np.float64),
                              base, qs, ks, D, prequant=True)


def check_int8(got, ref, pre, what):
    got = got.astype(np.int32)
    ref = ref.astype(np.int32)
    frac = np.abs(np.abs(pre - np.floor(pre)) - 0.5)
    near = (frac < BOUNDARY) | (np.abs(np.abs(pre) - 127.5) < BOUNDARY)
    diff = np.abs(got - ref)
    assert diff.max() <= 1, f"{what}: off by {diff.max()}"
    assert not np.any((diff > 0) & ~near), f"{what}: {int(((diff > 0) & ~near).sum())} values differ away from a boundary"
    return int((diff > 0).sum()), int(near.sum())


@pytest.mark.parametrize("T,H,D", [(1, 64, 64), (5, 96, 32), (16, 2048, 64), (37, 1024, 128), (300, 4096, 64)])
def test_indexer_project_matches_oracle(T, H, D):
    base, qs, ks = 10000.0, 32.0, 24.0
    hidden, w, gq, gk, pos = inputs(T, H, D, seed=T * 7 + H + D)
    say(f"[gpu] indexer front end T={T} H={H} D={D}")
    q = torch.full((T, D), 99, dtype=torch.int8, device=DEV)
    k = torch.full((T, D), 99, dtype=torch.int8, device=DEV)
    api.qsa_indexer_project(hidden.to(DEV), pos.to(DEV), w.to(DEV), gq.to(DEV), gk.to(DEV), q, k,
                            rope_base=base, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    rq, rk, pq, pk = oracle(hidden, w, gq, gk, pos, D, base, qs, ks)
    nq = check_int8(q.cpu().numpy(), rq, pq, "q")
    nk = check_int8(k.cpu().numpy(), rk, pk, "k")
    say(f"[gpu]   boundary differences q {nq}, k {nk}")


def test_front_end_feeds_compress_and_selection():
    """hidden states -> keys and query (GPU) -> compress -> index_topk, against the
    oracle's own chain on the same hidden states.  A seed whose int8 values differ
    at a rounding boundary (allowed above) is not compared further; at least one
    of the seeds must be."""
    shape = QSAShape(16, 2, 128, 64, 16, 64)
    B, L, H = 2, 256, 512
    compared = 0
    for seed in (123, 124, 125, 126):
        wl = make_workload(shape, [L] * B, seed=5, device=DEV, name="frontend-chain")
        layer = QSALayer(wl, 1, poison=True, max_seq_len=L)
        hidden, w, gq, gk, _ = inputs(B * (L + 1), H, 64, seed=seed)
        pos = torch.as_tensor(np.concatenate([np.arange(L + 1)] * B).astype(np.int32))
        keys = torch.empty((B * (L + 1), 64), dtype=torch.int8, device=DEV)
        qidx = torch.empty_like(keys)
        api.qsa_indexer_project(hidden.to(DEV), pos.to(DEV), w.to(DEV), gq.to(DEV), gk.to(DEV), qidx, keys,
                                q_scale=32.0, k_scale=32.0)
        torch.cuda.synchronize()
        rq, rk, pq, pk = oracle(hidden, w, gq, gk, pos, 64, 10000.0, 32.0, 32.0)
        check_int8(keys.cpu().numpy(), rk, pk, "keys")
        check_int8(qidx.cpu().numpy(), rq, pq, "q")
        if not (np.array_equal(keys.cpu().numpy(), rk) and np.array_equal(qidx.cpu().numpy(), rq)):
            say(f"[gpu]   seed {seed}: a rounding-boundary value differs; selection not compared")
            continue
        # tokens 0..L-1 of request b are its keys; token L's query selects (sel_seq_len = L)
        kv = keys.view(B, L + 1, 64)
        new_keys = kv[:, :L].reshape(B * L, 64).contiguous()
        api.qsa_compress(layer.cfg, new_keys, torch.arange(0, B * L + 1, L, dtype=torch.int32, device=DEV),
                         torch.zeros(B, dtype=torch.int32, device=DEV), wl.block_table, layer.ring, layer.ckey, L)
        q_sel = qidx.view(B, L + 1, 64)[:, L].contiguous()
        sel_len = torch.full((B,), L, dtype=torch.int32, device=DEV)
        api.qsa_index_topk(layer.cfg, q_sel, wl.sel_req, sel_len, wl.block_table, layer.ckey, layer.topk,
                           layer.workspace, L)
        torch.cuda.synchronize()
        got = layer.topk.cpu().numpy()
        rkv = rk.reshape(B, L + 1, 64)
        rqs = rq.reshape(B, L + 1, 64)[:, L]
        for b in range(B):
            assert np.array_equal(got[b], O.index_topk_row(rqs[b], rkv[b, :L], L, shape.topk_blocks)), \
                f"seed {seed} request {b}"
        compared += 1
    assert compared >= 1, "every seed hit a rounding boundary"


def _pos3(T, seed, max_pos=1 << 23):
    """Three position components per token: independent random components, and
    for about 30 % of the tokens three equal ones (text); extremes included."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    p = torch.randint(0, max_pos, (3, T), generator=g, dtype=torch.int32)
    text = torch.rand(T, generator=g) < 0.3
    p[1][text] = p[0][text]
    p[2][text] = p[0][text]
    if T >= 3:
        p[:, 0] = torch.tensor([0, 0, 0], dtype=torch.int32)
        p[:, 1] = torch.tensor([5, max_pos - 1, 0], dtype=torch.int32)
        p[:, 2] = torch.tensor([max_pos - 1, 7, max_pos - 1], dtype=torch.int32)
    return p.contiguous()


@pytest.mark.parametrize("T,H,D,sec", [(1, 64, 64, (8, 12, 12)), (37, 1024, 128, (16, 24, 24)),
                                       (300, 4096, 64, (32, 0, 0)), (64, 512, 32, (0, 8, 8))])
def test_indexer_project_mrope_matches_oracle(T, H, D, sec):
    base, qs, ks = 10000.0, 32.0, 24.0
    hidden, w, gq, gk, _ = inputs(T, H, D, seed=T * 5 + H + D)
    pos3 = _pos3(T, seed=T + D)
    say(f"[gpu] indexer front end (MRoPE {sec}) T={T} H={H} D={D}")
    q = torch.full((T, D), 99, dtype=torch.int8, device=DEV)
    k = torch.full((T, D), 99, dtype=torch.int8, device=DEV)
    api.qsa_indexer_project_mrope(hidden.to(DEV), pos3.to(DEV), sec, w.to(DEV), gq.to(DEV), gk.to(DEV), q, k,
                                  rope_base=base, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    h = F.bf16_bits_to_f64(hidden.view(torch.int16).numpy())
    wf = F.bf16_bits_to_f64(w.view(torch.int16).numpy())
    rq, rk, pq, pk = F.indexer_frontend(h, pos3.numpy(), wf, gq.numpy().astype(np.float64),
                                        gk.numpy().astype(np.float64), base, qs, ks, D, prequant=True,
                                        mrope_sections=sec)
    nq = check_int8(q.cpu().numpy(), rq, pq, "q")
    nk = check_int8(k.cpu().numpy(), rk, pk, "k")
    say(f"[gpu]   boundary differences q {nq}, k {nk}")


def test_mrope_with_equal_components_is_the_1d_call_bit_for_bit():
    T, H, D = 129, 1024, 64
    hidden, w, gq, gk, pos = inputs(T, H, D, seed=77)
    pos3 = torch.stack([pos, pos, pos]).contiguous()
    outs = []
    for mrope in (False, True):
        q = torch.full((T, D), 99, dtype=torch.int8, device=DEV)
        k = torch.full((T, D), 99, dtype=torch.int8, device=DEV)
        if mrope:
            api.qsa_indexer_project_mrope(hidden.to(DEV), pos3.to(DEV), (8, 12, 12), w.to(DEV), gq.to(DEV),
                                          gk.to(DEV), q, k)
        else:
            api.qsa_indexer_project(hidden.to(DEV), pos.to(DEV), w.to(DEV), gq.to(DEV), gk.to(DEV), q, k)
        torch.cuda.synchronize()
        outs.append((q.cpu(), k.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
