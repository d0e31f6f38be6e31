"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong variant (on the CPU,
inside this process only) and checks that at least one pin then fails.  This
shows the pins constrain the parts they are meant to constrain.
"""
import math

import numpy as np
import pytest

from oracle import qsa_oracle as O
import oracle.qsa_frontend_oracle as F
import tests.test_oracle_frontend_pins as FP
import tests.test_oracle_pins as P


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_reversed_tie_break_is_caught(monkeypatch):
    def bad(scores, k):
        s = np.asarray(scores, dtype=np.int64)
        idx = np.arange(s.shape[0])
        order = np.lexsort((-idx, -s))
        keep = np.sort(order[: min(k, s.shape[0])])
        out = np.full(k, -1, dtype=np.int32)
        out[: keep.shape[0]] = keep
        return out
    monkeypatch.setattr(O, "select_blocks", bad)
    assert _fails(P.test_select_matches_bruteforce_with_ties, 0)
    assert _fails(P.test_select_all_tied_takes_lowest_indices)


def test_dropped_tail_is_caught(monkeypatch):
    orig = O.token_positions
    monkeypatch.setattr(O, "tail_start", lambda L: L)  # tail becomes empty
    assert _fails(P.test_dense_equivalence_short_context, 2051)
    monkeypatch.setattr(O, "tail_start", lambda L: 4 * (L // 4))
    assert orig is O.token_positions


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    def bad(q, K, V, scale):
        hq, d = q.shape
        hkv = K.shape[1]
        out, lse = np.zeros((hq, d)), np.zeros(hq)
        if K.shape[0] == 0:
            return out, np.full(hq, -np.inf)
        for h in range(hq):
            z = scale * (K[:, h % hkv] @ q[h])
            m = z.max()
            lse[h] = m + math.log(np.exp(z - m).sum())
            out[h] = np.exp(z - lse[h]) @ V[:, h % hkv]
        return out, lse
    monkeypatch.setattr(O, "attend", bad)
    assert _fails(P.test_gqa_grouping_contiguous)
    assert _fails(P.test_dense_equivalence_short_context, 100)


def test_missing_softmax_scale_is_caught(monkeypatch):
    orig = O.attend
    monkeypatch.setattr(O, "attend", lambda q, K, V, scale: orig(q, K, V, 1.0))
    assert _fails(P.test_dense_equivalence_short_context, 100)


def test_compress_dropping_a_token_is_caught(monkeypatch):
    def bad(keys, seq_len):
        nb = seq_len // 4
        k = np.asarray(keys[: nb * 4]).astype(np.int64)
        return k[0::4] + k[1::4] + k[2::4]
    monkeypatch.setattr(O, "compress_keys", bad)
    assert _fails(P.test_compress_then_score_equals_token_level_sum)


def test_merge_sign_error_is_caught(monkeypatch):
    def bad(o_part, lse_part):
        o = np.asarray(o_part, dtype=np.float64)
        l = np.asarray(lse_part, dtype=np.float64)
        M = l.max(axis=0)
        w = np.where(np.isfinite(l), np.exp(M[None] - l), 0.0)
        s = w.sum(axis=0)
        return (w / s)[..., None].__mul__(o).sum(axis=0), M + np.log(s)
    monkeypatch.setattr(O, "merge_partials", bad)
    assert _fails(P.test_merge_invariant_to_partition, 700)


def test_tail_in_first_split_is_caught(monkeypatch):
    def bad(blocks, sel_seq_len, row_seq_len, num_splits):
        parts = P.O.__dict__["_orig_split"](blocks, sel_seq_len, row_seq_len, num_splits)
        if num_splits > 1:
            tail = np.arange(O.tail_start(sel_seq_len), row_seq_len)
            parts[-1] = parts[-1][: parts[-1].shape[0] - tail.shape[0]]
            parts[0] = np.concatenate([parts[0], tail])
        return parts
    monkeypatch.setitem(O.__dict__, "_orig_split", O.split_token_positions)
    monkeypatch.setattr(O, "split_token_positions", bad)
    assert _fails(P.test_split_partition_covers_token_set, 703)


def test_fp8_wrong_bias_is_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes).astype(np.uint8).astype(np.int64)
        sign = np.where((c >> 7) & 1, -1.0, 1.0)
        e, m = (c >> 3) & 0xF, c & 7
        val = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1 + m / 8.0) * np.exp2(e - 8.0))
        return sign * np.where((e == 15) & (m == 7), np.nan, val)
    monkeypatch.setattr(O, "fp8_e4m3_to_f64", bad)
    assert _fails(P.test_fp8_anchor_values)
    assert _fails(P.test_fp8_decode_matches_torch_all_codes)


def test_gather_ignoring_the_block_table_is_caught(monkeypatch):
    def bad_rows(cache, block_table_row, page_size, tokens):
        t = np.asarray(tokens, dtype=np.int64)
        return cache[t // page_size, :, t % page_size, :]        # identity table
    def bad_scales(scale, block_table_row, page_size, tokens):
        t = np.asarray(tokens, dtype=np.int64)
        return np.asarray(scale, dtype=np.float64)[t // page_size, t % page_size]
    monkeypatch.setattr(O, "paged_rows", bad_rows)
    monkeypatch.setattr(O, "paged_scales", bad_scales)
    assert _fails(P.test_paged_rows_follow_a_shuffled_block_table)
    assert _fails(P.test_paged_scales_follow_a_shuffled_block_table)


def test_fp8_scale_divided_instead_of_multiplied_is_caught(monkeypatch):
    orig = O.decode_kv
    def bad(raw, kv_dtype, scales=None):
        if kv_dtype == "fp8":
            return O.fp8_e4m3_to_f64(raw) / np.asarray(scales, dtype=np.float64)[:, None, None]
        return orig(raw, kv_dtype, scales)
    monkeypatch.setattr(O, "decode_kv", bad)
    assert _fails(P.test_decode_kv_fp8_applies_the_token_scale)
    assert _fails(P.test_decode_kv_fp8_inverts_per_token_quantisation)


def test_front_end_rotation_before_norm_is_caught(monkeypatch):
    import oracle.qsa_frontend_oracle as F
    import tests.test_oracle_frontend_pins as FP
    def bad(hidden, positions, w_qk, g_q, g_k, base, q_scale, k_scale, D, prequant=False):
        q, k = F.project(hidden, w_qk, D)
        q = F.rmsnorm(F.rope(q, positions, base), g_q)
        k = F.rmsnorm(F.rope(k, positions, base), g_k)
        if prequant:
            return F.quantize(q, q_scale), F.quantize(k, k_scale), q * q_scale, k * k_scale
        return F.quantize(q, q_scale), F.quantize(k, k_scale)
    monkeypatch.setattr(F, "indexer_frontend", bad)
    assert _fails(FP.test_composed_front_end_at_position_p)


def test_front_end_swapped_scales_is_caught(monkeypatch):
    import oracle.qsa_frontend_oracle as F
    import tests.test_oracle_frontend_pins as FP
    orig = F.indexer_frontend
    def bad(hidden, positions, w_qk, g_q, g_k, base, q_scale, k_scale, D, prequant=False):
        return orig(hidden, positions, w_qk, g_q, g_k, base, k_scale, q_scale, D, prequant)
    monkeypatch.setattr(F, "indexer_frontend", bad)
    assert _fails(FP.test_composed_front_end_at_position_zero)
    assert _fails(FP.test_composed_front_end_at_position_p)


def test_front_end_swapped_gains_is_caught(monkeypatch):
    import oracle.qsa_frontend_oracle as F
    import tests.test_oracle_frontend_pins as FP
    orig = F.indexer_frontend
    def bad(hidden, positions, w_qk, g_q, g_k, base, q_scale, k_scale, D, prequant=False):
        return orig(hidden, positions, w_qk, g_k, g_q, base, q_scale, k_scale, D, prequant)
    monkeypatch.setattr(F, "indexer_frontend", bad)
    assert _fails(FP.test_composed_front_end_at_position_zero)


def test_split_by_fixed_context_slices_is_caught(monkeypatch):
    """The rule of fixed slices of the context (not runs of the selection)."""
    def bad(blocks, sel_seq_len, row_seq_len, num_splits):
        b = np.asarray(blocks, dtype=np.int64)
        b = np.sort(b[b >= 0])
        nb, parts = sel_seq_len // 4, []
        for p in range(num_splits):
            lo, hi = (p * nb) // num_splits, ((p + 1) * nb) // num_splits
            mine = b[(b >= lo) & (b < hi)]
            toks = (mine[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
            if p == num_splits - 1:
                toks = np.concatenate([toks, np.arange(O.tail_start(sel_seq_len), row_seq_len)])
            parts.append(toks)
        return parts
    monkeypatch.setattr(O, "split_token_positions", bad)
    assert _fails(P.test_split_worked_example_runs_of_the_selection)
    assert _fails(P.test_split_parts_are_balanced_contiguous_runs, 700)


def test_rows_ignoring_row_sel_is_caught(monkeypatch):
    orig = O.decode_rows
    def bad(**kw):
        rs = np.asarray(kw["row_sel"])
        kw["row_sel"] = np.where(rs >= 0, np.minimum(np.arange(rs.shape[0]), len(kw["sel_req"]) - 1), -1)
        return orig(**kw)
    monkeypatch.setattr(O, "decode_rows", bad)
    assert _fails(P.test_rows_follow_row_sel_with_their_own_tails, "bf16")


def test_rows_ignoring_sel_req_is_caught(monkeypatch):
    orig = O.decode_rows
    def bad(**kw):
        kw["sel_req"] = np.arange(len(kw["sel_req"]))
        return orig(**kw)
    monkeypatch.setattr(O, "decode_rows", bad)
    assert _fails(P.test_rows_follow_row_sel_with_their_own_tails, "fp8")


def test_tail_of_the_selecting_row_instead_of_the_own_row_is_caught(monkeypatch):
    orig = O.split_token_positions
    monkeypatch.setattr(O, "split_token_positions",
                        lambda blocks, sel_seq_len, row_seq_len, P_: orig(blocks, sel_seq_len, sel_seq_len, P_))
    assert _fails(P.test_rows_follow_row_sel_with_their_own_tails, "bf16")


def _mrope_variant(assign):
    """An MRoPE whose frequency -> component assignment is assign(i, sections)."""
    def bad(x, pos3, base, sections):
        D = x.shape[-1]
        h = D // 2
        comp = np.array([assign(i, sections) for i in range(h)])
        pos3 = np.asarray(pos3, dtype=np.float64)
        i = np.arange(h, dtype=np.float64)
        ang = pos3[comp, :].T * base ** (-2.0 * i / D)[None, :]
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[:, :h], x[:, h:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return bad


def _contig(i, sec):
    return 0 if i < sec[0] else (1 if i < sec[0] + sec[1] else 2)


def test_mrope_interleaved_sections_are_caught(monkeypatch):
    monkeypatch.setattr(F, "mrope", _mrope_variant(lambda i, sec: i % 3))
    assert _fails(FP.test_mrope_each_section_turns_with_its_own_component_only)
    assert _fails(FP.test_mrope_first_pair_of_each_section_closed_form)


def test_mrope_swapped_height_and_width_is_caught(monkeypatch):
    monkeypatch.setattr(F, "mrope", _mrope_variant(lambda i, sec: [0, 2, 1][_contig(i, sec)]))
    assert _fails(FP.test_mrope_each_section_turns_with_its_own_component_only)
    assert _fails(FP.test_composed_front_end_with_mrope) or _fails(FP.test_mrope_first_pair_of_each_section_closed_form)


def test_mrope_sections_off_by_one_are_caught(monkeypatch):
    monkeypatch.setattr(F, "mrope", _mrope_variant(lambda i, sec: _contig(i + 1, sec) if i + 1 < sum(sec) else 2))
    assert _fails(FP.test_mrope_each_section_turns_with_its_own_component_only)
