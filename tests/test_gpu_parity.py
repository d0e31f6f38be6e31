"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: selected block ids bit-exact; outputs (partials and merged) within
5e-3 max-abs for bf16 K/V and 2e-2 for fp8 K/V; LSE within 1e-4 relative
(|dlse| <= 1e-4 * max(1, |lse|)).  Expected values come only from the oracle.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_qsa_amd import api
from block_sparse_attention_qsa_amd.pipeline import QSALayer
from block_sparse_attention_qsa_amd.workloads import (SHAPE_MAIN, SHAPE_TINY, SHAPE_FP8, QSAShape,
                                                      make_workload, named_workload)
from oracle import qsa_oracle as O
from tests.harness import (OUT_TOL, check_layer, check_lse, check_out, ckey_blocks_from_cache, host_copy,
                           oracle_decode, oracle_topk, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(wl, P=1, poison=False, prefill_chunk=None):
    say(f"[gpu] {wl.name} seed={wl.seed} B={wl.num_reqs} S={wl.num_sel} R={wl.num_rows} "
        f"Lmax={int(wl.final_len.max())} P={P} poison={poison}")
    layer = QSALayer(wl, num_splits=P, poison=poison)
    layer.prefill(prefill_chunk)
    layer.step()
    torch.cuda.synchronize()
    return layer


# ------------------------------------------------------------------ compress

def test_compress_bulk_matches_oracle():
    wl = named_workload(2, device=DEV, scale_ctx=1 / 64)
    layer = QSALayer(wl, 1)
    layer.prefill()
    layer.compress()
    torch.cuda.synchronize()
    ck = layer.ckey.cpu().numpy()
    keys = wl.keys.cpu().numpy()
    for b in range(wl.num_reqs):
        L = int(wl.final_len[b])
        got = ckey_blocks_from_cache(wl, ck, b, L // 4)
        ref = O.compress_keys(keys[wl.key_off[b]:wl.key_off[b] + L], L)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("chunk", [1, 3, 7])
def test_compress_incremental_equals_bulk(chunk):
    shape = QSAShape(16, 2, 128, 64, 512, 64)
    wl = make_workload(shape, [301, 64, 5, 130], seed=11, device=DEV)
    bulk = QSALayer(wl, 1)
    bulk.prefill()
    inc = QSALayer(wl, 1, poison=True)
    inc.prefill(chunk)
    torch.cuda.synchronize()
    keys = wl.keys.cpu().numpy()
    for layer in (bulk, inc):
        ck = layer.ckey.cpu().numpy()
        for b in range(wl.num_reqs):
            L = int(wl.prefix_len[b])
            got = ckey_blocks_from_cache(wl, ck, b, L // 4)
            assert np.array_equal(got, O.compress_keys(keys[wl.key_off[b]:wl.key_off[b] + L], L))
    # the open block's keys sit in the ring, identically
    rb, ri = bulk.ring.cpu().numpy(), inc.ring.cpu().numpy()
    for b in range(wl.num_reqs):
        L = int(wl.prefix_len[b])
        for t in range(4 * (L // 4), L):
            assert np.array_equal(rb[b, t % 8], keys[wl.key_off[b] + t])
            assert np.array_equal(ri[b, t % 8], keys[wl.key_off[b] + t])


def test_compress_skips_dummy_requests():
    shape = QSAShape(16, 2, 128, 64, 512, 64)
    wl = make_workload(shape, [64, 64], seed=12, device=DEV)
    layer = QSALayer(wl, 1, poison=True)
    before = layer.ckey.clone()
    keys = wl.keys[:8].contiguous()
    api.qsa_compress(layer.cfg, keys, torch.tensor([0, 8, 8], dtype=torch.int32, device=DEV),
                     torch.tensor([-1, 0], dtype=torch.int32, device=DEV), wl.block_table, layer.ring,
                     layer.ckey, 8)
    torch.cuda.synchronize()
    assert torch.equal(before, layer.ckey)


# ------------------------------------------------------------------ scan alone

@pytest.mark.parametrize("D,page", [(32, 16), (64, 64), (128, 256), (128, 16)])
def test_scores_only_match_oracle_scores(D, page):
    """qsa_index_topk(topk=NULL): every exact int32 score against the oracle's q.C_j,
    across index widths, page sizes and ragged lengths (one row per length)."""
    shape = QSAShape(16, 2, 128, D, 512, page)
    lens = [3, 4, 257, 1023, 1024, 1027, 4096 + 64 * 5 + 7, 9001]
    wl = make_workload(shape, lens, seed=40 + D + page, device=DEV, name=f"scan-D{D}-p{page}")
    say(f"[gpu] scores-only D={D} page={page}")
    layer = QSALayer(wl, 1, poison=True)
    layer.prefill()
    layer.compress()
    api.qsa_index_topk(layer.cfg, wl.q_index, wl.sel_req, wl.sel_seq_len, wl.block_table, layer.ckey,
                       None, layer.workspace, layer.max_seq_len)
    torch.cuda.synchronize()
    h = host_copy(wl)
    nb_stride = -(-(layer.max_seq_len // 4) // 1024) * 1024
    sc = layer.workspace.view(torch.int32)[: wl.num_sel * nb_stride].cpu().numpy().reshape(wl.num_sel, nb_stride)
    for s_ in range(wl.num_sel):
        b = int(h.sel_req[s_])
        L = int(h.sel_seq_len[s_])
        nb = L // 4
        ref = O.score_blocks(h.q_index[s_], O.compress_keys(h.keys[h.key_off[b]:h.key_off[b] + L], L))
        got = sc[s_, :nb].astype(np.int64)
        assert np.array_equal(got, ref), f"row {s_} (L={L}): first diff at {np.nonzero(got != ref)[0][:5]}"


@pytest.mark.parametrize("D,page,P", [(32, 16, 3), (128, 64, 2), (128, 256, 5), (64, 16, 8)])
def test_index_dims_and_page_sizes(D, page, P):
    """Selection and attention for every built index width and several page sizes."""
    shape = QSAShape(16, 2, 128, D, 512, page)
    wl = make_workload(shape, [4097, 2052, 30000, 511, 12345], seed=60 + D + page, device=DEV,
                       name=f"dims-D{D}-p{page}")
    check_layer(wl, run(wl, P=P))


# ------------------------------------------------------------------ small configs

@pytest.mark.parametrize("cfg,scale", [(1, 1.0), (2, 1 / 16), (3, 1 / 64), (4, 1 / 64), (5, 1 / 200)])
@pytest.mark.parametrize("P", [1, 2, 8])
def test_small_parity(cfg, scale, P):
    wl = named_workload(cfg, device=DEV, scale_ctx=scale)
    layer = run(wl, P)
    check_layer(wl, layer)


# ------------------------------------------------------------------ edge cases

EDGE_LENS = [0, 1, 3, 4, 5, 8, 2047, 2048, 2051, 2052, 2053, 6001]


@pytest.mark.parametrize("P", [1, 3])
def test_edge_lengths_and_dense_equivalence(P):
    wl = make_workload(SHAPE_MAIN, EDGE_LENS, seed=21, device=DEV, name="edge")
    layer = run(wl, P)
    h = host_copy(wl)
    ref = check_layer(wl, layer, h)
    # rows with <= 512 closed blocks attend everything: compare with plain dense attention
    for r, L in enumerate(EDGE_LENS):
        if L == 0:
            assert (layer.out[r].float() == 0).all() and torch.isneginf(layer.lse[r]).all()
            continue
        if L // 4 > 512:
            continue
        toks = np.arange(L)
        K = O.decode_kv(O.paged_rows(h.k_cache, h.block_table[r], 64, toks), "bf16")
        V = O.decode_kv(O.paged_rows(h.v_cache, h.block_table[r], 64, toks), "bf16")
        o, l = O.attend(O.bf16_bits_to_f64(h.q[r]), K, V, wl.shape.softmax_scale)
        check_out(layer.out[r].float().cpu().numpy(), o, OUT_TOL["bf16"], f"dense L={L}")
        check_lse(layer.lse[r].cpu().numpy(), l, f"dense L={L}")


@pytest.mark.parametrize("hq,hkv,d,kv,qps,P", [
    (8, 2, 64, "fp8", 1, 3),      # d = 64 fp8: 4-byte V slices per lane
    (16, 1, 64, "bf16", 1, 2),    # 16 heads per KV head: 8 waves, d = 64
    (16, 2, 128, "fp8", 4, 3),    # 32 head rows (4 rows x 8 heads): 4 waves
    (32, 2, 64, "bf16", 4, 5),    # 64 head rows: 4 waves, d = 64
    (8, 8, 128, "bf16", 1, 1),    # one head per KV head
])
def test_head_dims_dtypes_and_group_sizes(hq, hkv, d, kv, qps, P):
    """The attention kernel's variants: head dim 64/128, bf16/fp8, head rows
    per workgroup from 1 to 64 (8 or 4 waves), reuse rows, uneven splits; rows
    shorter than k blocks and rows with the full k."""
    shape = QSAShape(hq, hkv, d, 64, 128, 64 if d == 128 else 16, kv_dtype=kv)
    lens = [1, 3, 4, 67, 300, 1031, 5003]
    wl = make_workload(shape, lens, step_tokens=qps, q_per_sel=qps, seed=90 + hq + d + qps, device=DEV,
                       name=f"heads-{hq}/{hkv}-d{d}-{kv}-q{qps}")
    check_layer(wl, run(wl, P))


def test_k_larger_than_blocks_and_small_k():
    shape = QSAShape(8, 2, 64, 32, 7, 16)
    wl = make_workload(shape, [3, 17, 27, 28, 29, 100, 1000], seed=5, device=DEV, name="k7")
    layer = run(wl, 2)
    check_layer(wl, layer)


def test_all_tied_scores_take_lowest_blocks():
    wl = make_workload(SHAPE_MAIN, [20000, 9000], seed=6, device=DEV, name="ties")
    wl.keys.fill_(3)
    layer = run(wl, 2)
    got = layer.topk.cpu().numpy()
    assert np.array_equal(got[0], np.arange(512))
    assert np.array_equal(got[1], np.arange(512))
    check_layer(wl, layer)


def test_partial_ties_at_threshold():
    """Few distinct key values -> many equal scores around the k-th: lowest index wins."""
    wl = make_workload(SHAPE_MAIN, [40000, 30001], seed=7, device=DEV, name="coarse-ties")
    g = torch.Generator(device=DEV).manual_seed(7)
    wl.keys.copy_(torch.randint(-1, 2, wl.keys.shape, generator=g, device=DEV, dtype=torch.int8))
    layer = run(wl, 4)
    check_layer(wl, layer)


def test_poisoned_buffers_do_not_change_results():
    wl = named_workload(3, device=DEV, scale_ctx=1 / 32)
    clean = run(wl, 2)
    dirty = run(wl, 2, poison=True)
    for a, b in [(clean.topk, dirty.topk), (clean.o_part, dirty.o_part), (clean.lse, dirty.lse),
                 (clean.out, dirty.out)]:
        assert torch.equal(a, b)


def test_deterministic_repeat():
    wl = named_workload(2, device=DEV, scale_ctx=1 / 8)
    layer = run(wl, 4)
    first = [t.clone() for t in (layer.topk, layer.o_part, layer.lse_part, layer.out, layer.lse)]
    for _ in range(3):
        layer.step()
    torch.cuda.synchronize()
    for a, b in zip(first, (layer.topk, layer.o_part, layer.lse_part, layer.out, layer.lse)):
        assert torch.equal(a, b)


def test_identity_page_table():
    wl = make_workload(SHAPE_MAIN, [5000, 7777, 3000], seed=8, device=DEV, shuffle_pages=False, name="identity")
    layer = run(wl, 2)
    check_layer(wl, layer)


def test_split_counts_agree():
    wl = named_workload(3, device=DEV, scale_ctx=1 / 16)
    outs = []
    for P in (1, 2, 8, 16):
        layer = run(wl, P)
        outs.append((layer.out.float().cpu().numpy(), layer.lse.cpu().numpy()))
    for o, l in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= OUT_TOL["bf16"]
        check_lse(l, outs[0][1].astype(np.float64), "split agreement")


def test_multi_step_appends():
    """Each step appends one token per request (closing blocks on the way); every
    step's selection and output match the oracle at that step's context."""
    shape = SHAPE_MAIN
    final = [9000, 4103, 2049, 700]
    wl = make_workload(shape, final, seed=9, device=DEV, name="multistep")
    B = len(final)
    n_steps = 6
    layer = QSALayer(wl, 2)
    start = np.array(final) - n_steps
    layer.wl.prefix_len = start.copy()
    layer.prefill()
    h = host_copy(wl)
    for i in range(n_steps):
        L = start + i + 1
        before = torch.as_tensor((L - 1).astype(np.int32), device=DEV)
        keys = torch.cat([wl.keys[int(wl.key_off[b] + L[b] - 1)][None] for b in range(B)]).contiguous()
        api.qsa_compress(layer.cfg, keys, torch.arange(B + 1, dtype=torch.int32, device=DEV), before,
                         wl.block_table, layer.ring, layer.ckey, 1)
        wl.sel_seq_len.copy_(torch.as_tensor(L.astype(np.int32)))
        wl.row_seq_len.copy_(torch.as_tensor(L.astype(np.int32)))
        layer.index(); layer.decode(); layer.merge()
        torch.cuda.synchronize()
        h.sel_seq_len = L.astype(np.int32)
        h.row_seq_len = L.astype(np.int32)
        check_layer(wl, layer, h)


def test_fp8_all_codes_through_decode():
    """Every E4M3 code reaches the output exactly: rows with one token (L=1)
    return V itself; heads with one-hot q return scale * K[d] * k_scale as lse."""
    shape = QSAShape(num_q_heads=16, num_kv_heads=1, head_dim=128, index_dim=32, topk_blocks=4,
                     page_size=16, kv_dtype="fp8")
    wl = make_workload(shape, [1] * 16, seed=13, device=DEV, name="fp8-codes")
    codes = torch.arange(256, dtype=torch.uint8, device=DEV)
    nan_codes = {0x7F, 0xFF}
    # K rows carry the finite codes only: a NaN anywhere in K poisons q.K even
    # where q is 0, so the two NaN codes are checked through V alone.
    kcodes = codes.clone()
    kcodes[0x7F] = 0
    kcodes[0xFF] = 0
    for b in range(16):
        pg = int(wl.block_table[b, 0])
        half = codes[(b % 2) * 128:(b % 2) * 128 + 128]
        wl.v_cache[pg, 0, 0, :] = half
        wl.k_cache[pg, 0, 0, :] = kcodes[(b % 2) * 128:(b % 2) * 128 + 128]
        wl.k_scale[pg, 0] = 1.0
        wl.v_scale[pg, 0] = 1.0
    q = torch.zeros((16, 16, 128), dtype=torch.bfloat16, device=DEV)
    for b in range(16):
        for hh in range(16):
            q[b, hh, (b // 2) * 16 + hh] = 1.0
    wl.q.copy_(q)
    layer = run(wl, 1)
    out = layer.out.float().cpu().numpy()
    lse = layer.lse.cpu().numpy()
    ref = O.fp8_e4m3_to_f64(np.arange(256))
    for b in range(16):
        base = (b % 2) * 128
        want = ref[base:base + 128]
        got = out[b, 0]
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])
        for hh in range(16):
            d = (b // 2) * 16 + hh
            c = base + d
            kval = 0.0 if c in nan_codes else ref[c]
            assert abs(lse[b, hh] - wl.shape.softmax_scale * kval) <= 1e-6 * max(1, abs(kval))


def test_bf16_output_is_rounded_fp32_output():
    wl = named_workload(3, device=DEV, scale_ctx=1 / 64)
    layer = run(wl, 4)
    out_bf = torch.empty(layer.out.shape, dtype=torch.bfloat16, device=DEV)
    lse2 = torch.empty_like(layer.lse)
    api.qsa_merge_partials(layer.o_part, layer.lse_part, out_bf, lse2)
    torch.cuda.synchronize()
    assert torch.equal(lse2, layer.lse)
    assert torch.equal(out_bf, layer.out.to(torch.bfloat16))  # torch's cast is round-to-nearest-even


def test_graph_replay_matches_eager():
    """The step captured in a HIP graph gives the eager result on every replay,
    with eager work and synchronisations between replays."""
    wl = named_workload(3, device=DEV, scale_ctx=1 / 32)
    layer = run(wl, 4)
    ref = [t.clone() for t in (layer.topk, layer.o_part, layer.out, layer.lse)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.step(s)
    torch.cuda.synchronize()
    for i in range(4):
        for t in (layer.topk, layer.o_part, layer.out, layer.lse):
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (layer.topk, layer.o_part, layer.out, layer.lse)):
            assert torch.equal(a, b), f"replay {i}"
        layer.step()  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ merge at scale

@pytest.mark.parametrize("P,R,H,d", [(5, 300, 16, 128), (4, 2048, 16, 64), (3, 7, 16, 128)])
def test_merge_matches_oracle_small_and_many_pairs(P, R, H, d):
    """Random partials (with empty splits and rows whose splits are all empty)
    merged on the GPU against the oracle's merge; the first two shapes have
    4,800 and 32,768 (row, head) pairs (8 waves per workgroup), the last one
    112 (one wave per workgroup).  fp32 and bf16 outputs."""
    g = torch.Generator(device="cpu").manual_seed(P * 1000 + R + d)
    o = torch.randn((P, R, H, d), generator=g)
    l = torch.randn((P, R, H), generator=g) * 4.0
    l[torch.rand((P, R, H), generator=g) < 0.3] = -math.inf   # empty splits
    l[:, 1] = -math.inf                                       # a row with nothing at all
    o[torch.isinf(l)] = 0.0
    say(f"[gpu] merge P={P} R={R} H={H} d={d}")
    ref_o, ref_l = O.merge_partials(o.numpy(), l.numpy())
    od, ld = o.to(DEV), l.to(DEV)
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((R, H, d), 7.0, dtype=dt, device=DEV)
        lse = torch.full((R, H), 7.0, dtype=torch.float32, device=DEV)
        api.qsa_merge_partials(od, ld, out, lse)
        torch.cuda.synchronize()
        check_lse(lse.cpu().numpy(), ref_l, f"merge {dt}")
        assert torch.isneginf(lse[1]).all() and (out[1].float() == 0).all()
        outs[dt] = out
    check_out(outs[torch.float32].cpu().numpy(), ref_o, 1e-5, "merge fp32")
    # bf16 output: the fp32 merge rounded to nearest even (torch's cast)
    assert torch.equal(outs[torch.bfloat16], outs[torch.float32].to(torch.bfloat16))
