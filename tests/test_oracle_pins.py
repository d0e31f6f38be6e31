"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- closed forms, brute force, an independent library routine, or an
invariant the method must satisfy -- so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import qsa_oracle as O


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- formats

def test_fp8_anchor_values():
    # OCP E4M3: bias 7, max normal 448 = 1.75 * 2^8, min normal 2^-6, min subnormal 2^-9
    v = O.fp8_e4m3_to_f64(np.array([0x7E, 0x08, 0x01, 0x07, 0x38, 0xB8, 0x00, 0x80, 0x77, 0xFE]))
    assert v[0] == 448.0
    assert v[1] == 2.0 ** -6
    assert v[2] == 2.0 ** -9
    assert v[3] == 7 * 2.0 ** -9
    assert v[4] == 1.0 and v[5] == -1.0
    assert v[6] == 0.0 and v[7] == 0.0 and math.copysign(1, v[7]) == -1
    assert v[8] == 240.0  # E=14, M=7: 1.875 * 2^7
    assert v[9] == -448.0
    assert np.isnan(O.fp8_e4m3_to_f64(np.array([0x7F, 0xFF]))).all()


def test_fp8_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert (both_nan | (ours == ref)).all()
    assert both_nan.sum() == 2


def test_bf16_decode_matches_torch():
    x = torch.randn(10000, dtype=torch.float32, generator=torch.Generator().manual_seed(0)) * 100
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy()
    assert np.array_equal(O.bf16_bits_to_f64(bits), xb.to(torch.float64).numpy())


# ---------------------------------------------------------------- compress + score

def test_compress_then_score_equals_token_level_sum():
    """score(C_j) must equal sum over the block's 4 tokens of q . k_t (plain loops)."""
    r = rng(1)
    D, L = 8, 37
    keys = r.integers(-127, 128, (L, D)).astype(np.int8)
    q = r.integers(-127, 128, D).astype(np.int8)
    s = O.score_blocks(q, O.compress_keys(keys, L))
    assert s.shape == (L // 4,)
    for j in range(L // 4):
        tot = 0
        for t in range(4 * j, 4 * j + 4):
            for i in range(D):
                tot += int(q[i]) * int(keys[t][i])
        assert tot == int(s[j])


def test_compress_only_closed_blocks():
    keys = np.ones((11, 4), dtype=np.int8)
    c = O.compress_keys(keys, 11)
    assert c.shape == (2, 4) and (c == 4).all()
    assert O.compress_keys(keys, 3).shape == (0, 4)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_score_extremes_fit_int32(D):
    keys = np.full((8, D), 127, dtype=np.int8)
    q = np.full(D, 127, dtype=np.int8)
    s = O.score_blocks(q, O.compress_keys(keys, 8))
    assert (s == D * 127 * 508).all()
    assert D * 127 * 508 < 2 ** 31
    s2 = O.score_blocks(-q, O.compress_keys(keys, 8))
    assert (s2 == -D * 127 * 508).all()


# ---------------------------------------------------------------- select

@pytest.mark.parametrize("seed", range(6))
def test_select_matches_bruteforce_with_ties(seed):
    r = rng(100 + seed)
    for nb in [0, 1, 5, 31, 32, 33, 200]:
        for k in [1, 7, 32, 64]:
            scores = r.integers(-3, 4, nb)  # tiny range => many ties
            got = O.select_blocks(scores, k).tolist()
            assert got == O.select_blocks_bruteforce(scores.tolist(), k)


def test_select_all_tied_takes_lowest_indices():
    keys = np.full((400, 16), 5, dtype=np.int8)
    q = np.full(16, 3, dtype=np.int8)
    got = O.index_topk_row(q, keys, 400, 32)
    assert got.tolist() == list(range(32))


def test_select_planted_set():
    r = rng(7)
    D, L, k = 16, 4 * 300, 20
    keys = r.integers(-5, 6, (L, D)).astype(np.int8)
    planted = np.sort(r.choice(300, k, replace=False))
    for j in planted:
        keys[4 * j:4 * j + 4, 0] = 100
    q = np.zeros(D, dtype=np.int8)
    q[0] = 127
    got = O.index_topk_row(q, keys, L, k)
    assert np.array_equal(got, planted)


def test_select_short_rows_pad():
    keys = np.ones((3, 8), dtype=np.int8)
    assert (O.index_topk_row(np.ones(8, np.int8), keys, 3, 4) == -1).all()
    keys = np.ones((9, 8), dtype=np.int8)
    assert O.index_topk_row(np.ones(8, np.int8), keys, 9, 4).tolist() == [0, 1, -1, -1]


# ---------------------------------------------------------------- attention

def _dense_case(L, hq=4, hkv=2, d=32, seed=0, k=512):
    r = rng(seed)
    D = 16
    keys = r.integers(-127, 128, (L, D)).astype(np.int8)
    qi = r.integers(-127, 128, D).astype(np.int8)
    q = torch.randn(1, hq, d, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    K = torch.randn(L, hkv, d, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    V = torch.randn(L, hkv, d, generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16)
    # one contiguous page holding the whole context: cache [1, H_kv, page, d]
    kc = K.permute(1, 0, 2).unsqueeze(0).contiguous().view(torch.int16).numpy()
    vc = V.permute(1, 0, 2).unsqueeze(0).contiguous().view(torch.int16).numpy()
    topk = O.index_topk_row(qi, keys, L, k)[None]
    res = O.decode_rows(q=q.view(torch.int16).numpy(), row_sel=np.array([0]), sel_req=np.array([0]),
                        sel_seq_len=np.array([L]), row_seq_len=np.array([L]), topk=topk,
                        block_table=np.array([[0]]), page_size=max(L, 1), k_cache=kc, v_cache=vc,
                        kv_dtype="bf16", scale=1 / math.sqrt(d), num_splits=1)
    return q, K, V, res


@pytest.mark.parametrize("L", [1, 3, 4, 5, 100, 2047, 2048, 2051])
def test_dense_equivalence_short_context(L):
    """With <= 512 closed blocks everything is selected: QSA == dense attention."""
    hq, hkv, d = 4, 2, 32
    q, K, V, res = _dense_case(L, hq, hkv, d, seed=L)
    qq = q.to(torch.float64).reshape(1, hq, 1, d)
    KK = K.to(torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    VV = V.to(torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, KK, VV, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(res["out"][0], ref[0, :, 0].numpy(), atol=1e-12, rtol=0)
    logits = (qq @ KK.transpose(-1, -2))[0, :, 0] / math.sqrt(d)
    np.testing.assert_allclose(res["lse"][0], torch.logsumexp(logits, dim=-1).numpy(), atol=1e-12)


def test_dense_breaks_when_context_exceeds_budget():
    """Above 4k+3 tokens the selection drops blocks: out differs from dense."""
    L, hq, hkv, d = 4 * 40 + 2, 2, 1, 16
    q, K, V, res = _dense_case(L, hq, hkv, d, seed=3, k=8)
    qq = q.to(torch.float64).reshape(1, hq, 1, d)
    KK = K.to(torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    VV = V.to(torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, KK, VV, scale=1 / math.sqrt(d))
    assert np.abs(res["out"][0] - ref[0, :, 0].numpy()).max() > 1e-3


def test_closed_forms():
    r = rng(5)
    T, hq, hkv, d = 50, 4, 2, 8
    q = r.standard_normal((hq, d))
    V = r.standard_normal((T, hkv, d))
    out, lse = O.attend(q, np.zeros((T, hkv, d)), V, 0.3)
    np.testing.assert_allclose(lse, np.log(T), atol=1e-14)
    for h in range(hq):
        np.testing.assert_allclose(out[h], V[:, h // 2].mean(axis=0), atol=1e-14)
    K = r.standard_normal((T, hkv, d))
    out, _ = O.attend(q, K, np.full((T, hkv, d), 2.5), 0.3)
    np.testing.assert_allclose(out, 2.5, atol=1e-13)
    out, lse = O.attend(q, K[:0], V[:0], 0.3)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_gqa_grouping_contiguous():
    """Head h must read KV head h // G: give each KV head a distinct constant V."""
    T, hq, hkv, d = 6, 8, 4, 4
    r = rng(9)
    V = np.zeros((T, hkv, d))
    for g in range(hkv):
        V[:, g, :] = g + 1
    out, _ = O.attend(r.standard_normal((hq, d)), r.standard_normal((T, hkv, d)), V, 1.0)
    np.testing.assert_allclose(out[:, 0], [1, 1, 2, 2, 3, 3, 4, 4], atol=1e-13)


# ---------------------------------------------------------------- splits + merge

def _row_inputs(L=700, k=64, seed=11):
    r = rng(seed)
    hq, hkv, d = 4, 2, 16
    keys = r.integers(-127, 128, (L, 8)).astype(np.int8)
    qi = r.integers(-127, 128, 8).astype(np.int8)
    topk = O.index_topk_row(qi, keys, L, k)
    q = r.standard_normal((hq, d))
    K = r.standard_normal((L, hkv, d))
    V = r.standard_normal((L, hkv, d))
    return topk, q, K, V


@pytest.mark.parametrize("L", [700, 701, 702, 703])
def test_split_partition_covers_token_set(L):
    topk, *_ = _row_inputs(L)
    full = O.token_positions(topk, L, L)
    for P in [1, 2, 3, 8, 64, 100]:
        parts = O.split_token_positions(topk, L, L, P)
        assert len(parts) == P
        cat = np.concatenate(parts)
        assert np.array_equal(cat, full)
        for p in parts[:-1]:
            assert p.shape[0] % 4 == 0  # block boundaries


def test_split_worked_example_runs_of_the_selection():
    """Split p owns a near-equal run of the ascending selection: 5 selected blocks
    1, 2, 5, 7, 9 over 3 splits are the runs [0, 1), [1, 3), [3, 5) of the list,
    i.e. {1}, {2, 5}, {7, 9}; the last split also takes the row's tail 40, 41 (and
    42, 43 for a reuse row of length 44)."""
    blocks = np.array([1, 2, 5, 7, 9, -1, -1], dtype=np.int32)
    parts = O.split_token_positions(blocks, 42, 44, 3)
    assert [p.tolist() for p in parts] == [[4, 5, 6, 7], [8, 9, 10, 11, 20, 21, 22, 23],
                                           [28, 29, 30, 31, 36, 37, 38, 39, 40, 41, 42, 43]]
    # more splits than blocks: the empty runs yield empty parts
    parts = O.split_token_positions(np.array([0, 1], dtype=np.int32), 9, 9, 4)
    assert [p.tolist() for p in parts] == [[], [0, 1, 2, 3], [], [4, 5, 6, 7, 8]]


@pytest.mark.parametrize("L", [700, 703])
def test_split_parts_are_balanced_contiguous_runs(L):
    """Every part covers a contiguous stretch of the context (its tokens lie
    between its first and last block and no other part's tokens do), the parts
    come in context order, and their block counts differ by at most one."""
    topk, *_ = _row_inputs(L)
    for P in [1, 2, 3, 8, 64, 100]:
        parts = O.split_token_positions(topk, L, L, P)
        sizes = [p.shape[0] // 4 for p in parts[:-1]] + [(parts[-1] < 4 * (L // 4)).sum() // 4]
        assert max(sizes) - min(sizes) <= 1
        prev_hi = -1
        for toks in parts:
            if toks.shape[0]:
                assert toks.min() > prev_hi
                prev_hi = toks.max()


@pytest.mark.parametrize("L", [700, 703])
def test_merge_invariant_to_partition(L):
    topk, q, K, V = _row_inputs(L)
    ref_o, ref_l = O.attend(q, K[O.token_positions(topk, L, L)], V[O.token_positions(topk, L, L)], 0.25)
    for P in [1, 2, 8, 100]:
        parts = O.split_token_positions(topk, L, L, P)
        res = [O.attend(q, K[t], V[t], 0.25) for t in parts]
        o, l = O.merge_partials(np.stack([x[0] for x in res]), np.stack([x[1] for x in res]))
        np.testing.assert_allclose(o, ref_o, atol=1e-12)
        np.testing.assert_allclose(l, ref_l, atol=1e-12)
    # position-owned partitions (how context-parallel ranks own slices), incl. empty ones
    toks = O.token_positions(topk, L, L)
    bounds = [0, 0, L // 3, L // 3, L // 2, L, L]
    parts = [toks[(toks >= a) & (toks < b)] for a, b in zip(bounds[:-1], bounds[1:])]
    assert any(p.shape[0] == 0 for p in parts)
    res = [O.attend(q, K[t], V[t], 0.25) for t in parts]
    o, l = O.merge_partials(np.stack([x[0] for x in res]), np.stack([x[1] for x in res]))
    np.testing.assert_allclose(o, ref_o, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, atol=1e-12)


def test_merge_all_empty():
    o, l = O.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def test_merge_two_halves_closed_form():
    """Two partials with equal lse average their outputs; lse grows by ln 2."""
    o = np.stack([np.full((1, 3), 1.0), np.full((1, 3), 3.0)])
    l = np.array([[0.7], [0.7]])
    out, lse = O.merge_partials(o, l)
    np.testing.assert_allclose(out, 2.0)
    np.testing.assert_allclose(lse, 0.7 + math.log(2))


# ---------------------------------------------------------------- reuse rows

def test_reuse_rows_attend_selection_plus_own_tail():
    sel_L, rows = 1000, [1000, 1001, 1002, 1003]
    topk = np.arange(0, 64, dtype=np.int32) * 3
    for L in rows:
        t = O.token_positions(topk, sel_L, L)
        assert t.shape[0] == 64 * 4 + (L - 1000)
        assert (t[64 * 4:] == np.arange(1000, L)).all()


# ---------------------------------------------------------------- paged storage

def _scatter_to_pages(logical, table, page):
    """Place logical rows [L, ...] into pages by explicit loops: token t goes to
    page table[t // page], slot t % page (cache [num_pages, H, page, d] layout)."""
    L, hkv, d = logical.shape
    num_pages = int(np.max(table)) + 1
    cache = np.zeros((num_pages, hkv, page, d), dtype=logical.dtype)
    for t in range(L):
        for g in range(hkv):
            cache[table[t // page], g, t % page, :] = logical[t, g, :]
    return cache


def test_paged_rows_follow_a_shuffled_block_table():
    """A gather through a shuffled multi-page table returns the logical rows:
    token t sits at page table[t // page], slot t % page."""
    r = rng(21)
    L, hkv, d, page = 200, 2, 8, 16
    npg = (L + page - 1) // page
    logical = r.integers(-1000, 1000, (L, hkv, d)).astype(np.int16)
    table = r.permutation(3 * npg)[:npg]            # scattered over a larger pool
    cache = _scatter_to_pages(logical, table, page)
    toks = np.array([0, 1, 15, 16, 17, 63, 64, 100, 150, 199, 5, 5])
    got = O.paged_rows(cache, table, page, toks)
    assert np.array_equal(got, logical[toks])
    # the same content as one contiguous page gives the same rows
    contig = logical.transpose(1, 0, 2)[None]       # [1, H, L, d]
    assert np.array_equal(O.paged_rows(contig, np.array([0]), L, toks), logical[toks])


def test_paged_scales_follow_a_shuffled_block_table():
    r = rng(22)
    L, page = 130, 16
    npg = (L + page - 1) // page
    logical = r.standard_normal(L)
    table = r.permutation(2 * npg)[:npg]
    scales = np.full((2 * npg, page), np.nan)
    for t in range(L):
        scales[table[t // page], t % page] = logical[t]
    toks = np.arange(L)[::-1]
    assert np.array_equal(O.paged_scales(scales, table, page, toks), logical[toks])


# ---------------------------------------------------------------- fp8 with scales

def test_decode_kv_fp8_applies_the_token_scale():
    """Closed form: E4M3 codes 0x38 = 1, 0x40 = 2, 0xB8 = -1, 0x7E = 448 times
    each token's own scale (scale != 1 everywhere)."""
    raw = np.array([0x38, 0x40, 0xB8, 0x7E], dtype=np.uint8).reshape(4, 1, 1)
    raw = np.broadcast_to(raw, (4, 2, 3)).copy()
    scales = np.array([0.5, 3.0, 10.0, 0.25])
    got = O.decode_kv(raw, "fp8", scales)
    want = np.array([0.5, 6.0, -10.0, 112.0])
    assert np.array_equal(got, np.broadcast_to(want[:, None, None], (4, 2, 3)))


def test_decode_kv_fp8_inverts_per_token_quantisation():
    """N(0,1) rows quantised per token (scale = amax / 448, torch's E4M3 cast,
    an independent routine) decode back within half an E4M3 step: 2^-4 of the
    value for normal codes, 2^-10 of the scale for subnormal ones."""
    g = torch.Generator().manual_seed(23)
    x = torch.randn(64, 2, 16, generator=g, dtype=torch.float64) * torch.exp(torch.randn(64, 1, 1, generator=g,
                                                                                        dtype=torch.float64))
    amax = x.abs().amax(dim=(1, 2))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (x / scale[:, None, None]).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    dec = O.decode_kv(codes, "fp8", scale.numpy())
    xs = x.numpy()
    bound = np.maximum(2.0 ** -4 * np.abs(xs), 2.0 ** -10 * scale.numpy()[:, None, None])
    assert (np.abs(dec - xs) <= bound * (1 + 1e-12)).all()
    assert np.abs(dec - xs).max() > 0                 # the test can see an error at all


# ---------------------------------------------------------------- rows -> selecting rows

def _sdpa_ref(qbits, Kl, Vl, toks, hq, hkv, scale):
    """Dense attention of one row over the given logical tokens, by torch's
    scaled_dot_product_attention in float64 (a library routine, not the oracle)."""
    q = torch.from_numpy(O.bf16_bits_to_f64(qbits)).reshape(1, hq, 1, -1)
    if len(toks) == 0:
        return np.zeros((hq, q.shape[-1])), np.full(hq, -np.inf)
    K = torch.from_numpy(Kl[toks]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    V = torch.from_numpy(Vl[toks]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=scale)[0, :, 0].numpy()
    lse = torch.logsumexp((q @ K.transpose(-1, -2))[0, :, 0] * scale, dim=-1).numpy()
    return out, lse


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_rows_follow_row_sel_with_their_own_tails(kv_dtype):
    """Rows map to selecting rows unevenly (two rows share one, three share
    another, one row is padding), selecting rows map to requests out of order,
    and the caches are paged through shuffled tables.  Each row must equal
    dense attention (torch) over the token set written out here: its selecting
    row's blocks plus its own tail [4 floor(L_sel/4), L_row)."""
    r = rng(31)
    hq, hkv, d, D, k, page = 4, 2, 16, 8, 6, 16
    lens = [203, 150, 97]                    # requests' cached tokens
    sel_req = np.array([2, 0, 1])            # selecting row -> request
    sel_len = np.array([93, 150, 141])       # within each request's tokens
    row_sel = np.array([1, 0, 2, 1, -1, 2, 2, 0])
    row_len = np.array([150, 95, 141, 150, 50, 143, 144, 97])
    keys = [r.integers(-127, 128, (L, D)).astype(np.int8) for L in lens]
    qidx = r.integers(-127, 128, (3, D)).astype(np.int8)
    topk = np.stack([O.index_topk_row(qidx[s], keys[sel_req[s]], int(sel_len[s]), k) for s in range(3)])
    g = torch.Generator().manual_seed(32)
    logical_K, logical_V, kraw, vraw, ksc, vsc = [], [], [], [], [], []
    pool = 3 * sum((L + page - 1) // page for L in lens)
    perm = r.permutation(pool)
    tables, off = np.zeros((3, 13), dtype=np.int64), 0
    for b, L in enumerate(lens):
        n = (L + page - 1) // page
        tables[b, :n] = perm[off:off + n]
        off += n
    for L in lens:
        for store, logical, scl in ((kraw, logical_K, ksc), (vraw, logical_V, vsc)):
            x = torch.randn(L, hkv, d, generator=g, dtype=torch.float64)
            if kv_dtype == "bf16":
                xb = x.to(torch.bfloat16)
                store.append(xb.view(torch.int16).numpy())
                logical.append(xb.to(torch.float64).numpy())
            else:
                sc = x.abs().amax(dim=(1, 2)) / 448.0
                c8 = (x / sc[:, None, None]).to(torch.float32).to(torch.float8_e4m3fn)
                store.append(c8.view(torch.uint8).numpy())
                logical.append((c8.to(torch.float64) * sc[:, None, None]).numpy())
                scl.append(sc.numpy())
    dt = np.int16 if kv_dtype == "bf16" else np.uint8
    k_cache = np.zeros((pool, hkv, page, d), dtype=dt)
    v_cache = np.zeros((pool, hkv, page, d), dtype=dt)
    k_scale = np.zeros((pool, page))
    v_scale = np.zeros((pool, page))
    for b, L in enumerate(lens):
        for t in range(L):
            pg, sl = tables[b][t // page], t % page
            k_cache[pg, :, sl, :] = kraw[b][t]
            v_cache[pg, :, sl, :] = vraw[b][t]
            if kv_dtype == "fp8":
                k_scale[pg, sl], v_scale[pg, sl] = ksc[b][t], vsc[b][t]
    q = torch.randn(len(row_sel), hq, d, generator=g).to(torch.bfloat16).view(torch.int16).numpy()
    scale = 1 / math.sqrt(d)
    res = O.decode_rows(q=q, row_sel=row_sel, sel_req=sel_req, sel_seq_len=sel_len, row_seq_len=row_len,
                        topk=topk, block_table=tables, page_size=page, k_cache=k_cache, v_cache=v_cache,
                        kv_dtype=kv_dtype, scale=scale, num_splits=3,
                        k_scale=k_scale if kv_dtype == "fp8" else None,
                        v_scale=v_scale if kv_dtype == "fp8" else None)
    for rr, s in enumerate(row_sel):
        if s < 0:
            assert (res["out"][rr] == 0).all() and np.isneginf(res["lse"][rr]).all()
            continue
        b = sel_req[s]
        toks = []
        for j in topk[s]:
            if j >= 0:
                toks += [4 * j, 4 * j + 1, 4 * j + 2, 4 * j + 3]
        toks += list(range(4 * (sel_len[s] // 4), row_len[rr]))
        ref_o, ref_l = _sdpa_ref(q[rr], logical_K[b], logical_V[b], np.array(toks), hq, hkv, scale)
        np.testing.assert_allclose(res["out"][rr], ref_o, atol=1e-12)
        np.testing.assert_allclose(res["lse"][rr], ref_l, atol=1e-12)
