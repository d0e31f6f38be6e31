"""The oracle and the library's documented contracts against the numbers the
pages print about the method (tests/golden/qsa_pages_facts.json, each with its
citation)."""
import json
import os
import re

import numpy as np

from oracle import qsa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "qsa_pages_facts.json")))
HEADER = open(os.path.join(os.path.dirname(HERE), "include", "qsa.h")).read()


def test_kept_blocks_are_about_2048_token_positions():
    ratio, k = FACTS["compress_ratio"]["value"], FACTS["topk_blocks"]["value"]
    about = FACTS["token_positions_about"]["value"]
    assert O.COMPRESS_RATIO == ratio and k * ratio == about
    rng = np.random.default_rng(0)
    for L in (262144, 262145, 262147, 100003):
        keys = rng.integers(-127, 128, size=(L, 8)).astype(np.int8)
        q = rng.integers(-127, 128, size=8).astype(np.int8)
        sel = O.index_topk_row(q, keys, L, k)
        assert (sel >= 0).sum() == k
        toks = O.token_positions(sel, L, L)
        # the kept blocks' tokens plus the open tail (0..3 tokens): "about 2,048"
        assert about <= len(toks) <= about + ratio - 1


def test_short_rows_are_padded_with_the_pages_value():
    pad = FACTS["output_padding"]["value"]
    sel = O.index_topk_row(np.ones(8, np.int8), np.ones((40, 8), np.int8), 40, FACTS["topk_blocks"]["value"])
    assert (sel[:10] >= 0).all() and (sel[10:] == pad).all()


def test_ring_rollback_covers_the_pages_speculative_depth():
    """The header's rollback contract (up to 8 - L%4 dropped tokens) covers the
    pages' MTP depth: num_speculative_tokens drafts plus the verified token."""
    m = re.search(r"up to (\d+) - L%4", HEADER)
    assert m, "rollback contract not found in include/qsa.h"
    ring = int(m.group(1))
    depth = FACTS["num_speculative_tokens"]["value"] + 1
    assert all(ring - r >= depth for r in range(FACTS["compress_ratio"]["value"]))
