"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong variant (on the CPU,
inside this process only) and checks that at least one pin then fails.  This
shows the pins constrain the parts they are meant to constrain.
"""
import math

import numpy as np
import pytest

from oracle import qsa_oracle as O
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
