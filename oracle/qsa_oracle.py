"""Plain CPU oracle for the QSA (Qwen Sparse Attention) decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module: only the tests, the graft smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code, headers, tables or constants with the HIP
library; it is written to be read against the method's description, not to be
fast.  Integers are computed in int64, floating point in float64.

Sources (web pages), cited below by the short tags:

  [QSA-DCP]  "Qwen 4 QSA 迎来解码上下文并行：深入解读 vLLM 针对 Qwen3.8-Flash-Next
             的草稿 PR" (orcarouter.ai blog, zh-CN; ru/ko translations carry the same
             text).  Section "拉取请求实际改变了什么" (what the pull request actually
             changes) defines QSA: a lightweight indexer compresses keys into
             micro-blocks at ratio 4, scores them, keeps the best 512 blocks (about
             2,048 token positions), and runs the final softmax and value aggregation
             over the uncompressed K and V.  The same section describes decode
             context parallelism: each rank reads its own slice of the main KV
             cache and the attention results are merged across ranks at the end.
  [PR53896]  "PR #53896 完整报告" (prhub.com.cn report on vLLM PR #53896).  Section
             "实现拆解" (implementation breakdown): the indexer writes token keys into
             a raw-key ring cache, pools them by the compress ratio into a
             compressed key cache and does a weight-free top-k over the compressed
             keys.  Section "关键源码片段" (key source snippets), QSAIndexer.forward:
             the selection is returned as a fixed-width int32 buffer padded with -1,
             and a later MTP step may reuse the first step's selection.

Where the pages leave a step open, the oracle takes these readings (each is
listed with its reason in the design notes of the repository):

  R1  indexer query/keys are int8 vectors of dimension D; one indexer head per
      request, shared by all attention heads;
  R2  the pooled micro-block key is the exact integer SUM of its 4 token keys
      (4 x the mean, hence the same ranking); no normalisation is applied;
  R3  the block score is the plain integer dot product q . C_j;
  R4  ties in score are broken towards the lower block index;
  R5  the open (partial) micro-block at the end of the context -- tokens
      [4*floor(L/4), L) -- is always attended;
  R6  fewer than k closed blocks: all are selected, the rest of the row is -1;
  R7  seq_len counts every cached token including the row's own token;
  R8  a row that reuses another row's selection attends that selection plus its
      own tail [4*floor(L_sel/4), L_row);
  R9  GQA heads are grouped contiguously: query head h reads KV head h // G;
  R10 scores are scaled by softmax_scale; LSE is the natural log of the sum of
      exp(scaled logit);
  R11 a decode split ("partition") p of P owns a contiguous slice of the
      context, as a context-parallel rank does; the slice boundaries are the
      selection's quantiles, so that the splits hold near-equal shares: split p
      owns the selected blocks [floor(p*n/P), floor((p+1)*n/P)) of the n
      ascending selected blocks, and the last split also owns the tail; an
      empty split yields (0, -inf);
  R12 FP8 K/V is OCP E4M3 (bias 7, no infinities, S.1111.111 = NaN) times one
      fp32 scale per token per tensor.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

COMPRESS_RATIO = 4  # [QSA-DCP]: four tokens per micro-block


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16 / int16) exactly.

    bfloat16 is the upper half of an IEEE-754 binary32: widening the 16 bits
    to the top of a 32-bit word gives the same value as a float32.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 ("e4m3fn") bytes from their bit fields (reading R12).

    Layout S.EEEE.MMM, exponent bias 7.  E = 0 is subnormal: (M/8) * 2^-6.
    E = 15 with M = 7 is NaN; there is no infinity, so E = 15, M < 7 are normal
    numbers (the largest is 1.75 * 2^8 = 448).
    """
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


# ---------------------------------------------------------------------------
# Indexer: compress, score, select
# ---------------------------------------------------------------------------

def compress_keys(keys: np.ndarray, seq_len: int) -> np.ndarray:
    """Micro-block keys of one request: C[j] = sum_{t=4j}^{4j+3} k_t (R2).

    [QSA-DCP] keys are compressed into micro-blocks at ratio 4; [PR53896]
    "实现拆解": the raw keys are pooled by the compress ratio into the compressed
    key cache.  Only closed blocks (all four tokens present, j < floor(L/4))
    exist.  keys: int8 [>= seq_len, D].  Returns int64 [floor(L/4), D].
    """
    nb = seq_len // COMPRESS_RATIO
    k = np.asarray(keys[: nb * COMPRESS_RATIO]).astype(np.int64)
    out = np.zeros((nb, k.shape[1]), dtype=np.int64)
    for t in range(COMPRESS_RATIO):
        out += k[t::COMPRESS_RATIO]
    return out


def score_blocks(q_index: np.ndarray, ckeys: np.ndarray) -> np.ndarray:
    """score_j = q . C_j in exact integer arithmetic (R1, R3).

    [QSA-DCP] the indexer scores the compressed micro-blocks; [PR53896] the
    selection is weight-free, made on the compressed keys alone.
    q_index: int8 [D]; ckeys: int64 [nb, D].  Returns int64 [nb].
    """
    q = np.asarray(q_index).astype(np.int64)
    return np.asarray(ckeys, dtype=np.int64) @ q


def select_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """Keep the best k blocks; ascending block ids, padded with -1 to width k.

    [QSA-DCP] keeps the best 512 blocks; [PR53896] "关键源码片段": the result is
    a fixed-width int32 buffer padded with -1.  Order: score descending, then
    block index ascending (R4).  With fewer than k blocks, all are kept (R6).
    """
    s = np.asarray(scores, dtype=np.int64)
    nb = s.shape[0]
    idx = np.arange(nb, dtype=np.int64)
    order = np.lexsort((idx, -s))  # primary key -s (i.e. score desc), then idx asc
    keep = np.sort(order[: min(k, nb)])
    out = np.full(k, -1, dtype=np.int32)
    out[: keep.shape[0]] = keep.astype(np.int32)
    return out


def select_blocks_bruteforce(scores: Sequence[int], k: int) -> List[int]:
    """Pure-Python selection by explicit sort, for tiny inputs (same rule)."""
    nb = len(scores)
    best = sorted(range(nb), key=lambda j: (-int(scores[j]), j))[: min(k, nb)]
    best.sort()
    return best + [-1] * (k - len(best))


def index_topk_row(q_index: np.ndarray, keys: np.ndarray, sel_seq_len: int, k: int) -> np.ndarray:
    """Compress the request's keys, score the closed blocks, select top-k."""
    if sel_seq_len < COMPRESS_RATIO:
        return np.full(k, -1, dtype=np.int32)
    ck = compress_keys(keys, sel_seq_len)
    return select_blocks(score_blocks(q_index, ck), k)


# ---------------------------------------------------------------------------
# Token set, splits, attention, merge
# ---------------------------------------------------------------------------

def tail_start(sel_seq_len: int) -> int:
    """First token of the open block that the selecting row could not score (R5)."""
    return COMPRESS_RATIO * (sel_seq_len // COMPRESS_RATIO)


def token_positions(blocks: np.ndarray, sel_seq_len: int, row_seq_len: int) -> np.ndarray:
    """Ascending token positions a row attends (R5, R8).

    [QSA-DCP] the softmax and value aggregation run over the uncompressed K and
    V at the positions of the kept blocks: block j stands for tokens 4j..4j+3.
    The row also attends its own tail [4*floor(L_sel/4), L_row).
    """
    b = np.asarray(blocks, dtype=np.int64)
    b = b[b >= 0]
    toks = (b[:, None] * COMPRESS_RATIO + np.arange(COMPRESS_RATIO)[None, :]).reshape(-1)
    tail = np.arange(tail_start(sel_seq_len), row_seq_len, dtype=np.int64)
    return np.concatenate([np.sort(toks), tail])


def split_token_positions(blocks: np.ndarray, sel_seq_len: int, row_seq_len: int,
                          num_splits: int) -> List[np.ndarray]:
    """Partition of a row's tokens into num_splits contiguous runs (R11).

    The one-GPU stand-in for decode context parallelism in [QSA-DCP]: each
    partition covers a contiguous stretch of the context, is attended
    separately, and the partial results are merged later.  Part p holds the
    selected blocks [floor(p*n/P), floor((p+1)*n/P)) of the n ascending ones;
    the last part also holds the row's tail (R5, R8).
    """
    b = np.asarray(blocks, dtype=np.int64)
    b = np.sort(b[b >= 0])
    n = b.shape[0]
    parts = []
    for p in range(num_splits):
        lo, hi = (p * n) // num_splits, ((p + 1) * n) // num_splits
        toks = (b[lo:hi, None] * COMPRESS_RATIO + np.arange(COMPRESS_RATIO)[None, :]).reshape(-1)
        if p == num_splits - 1:
            toks = np.concatenate([toks, np.arange(tail_start(sel_seq_len), row_seq_len, dtype=np.int64)])
        parts.append(toks)
    return parts


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of H_q query heads over T tokens, in float64.

    q: [H_q, d]; K, V: [T, H_kv, d] (already decoded to float64).  Head h reads
    KV head h // G with G = H_q / H_kv (R9).  For each head:
      z_t = scale * q_h . K_t,  lse = log sum_t exp(z_t),  out = sum_t exp(z_t - lse) V_t.
    With T = 0 the result is (0, -inf), the identity of the merge below.
    Returns out [H_q, d] and lse [H_q] (natural log, R10).
    """
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    T = K.shape[0]
    if T == 0:
        return np.zeros((hq, d)), np.full(hq, -np.inf)
    hkv = K.shape[1]
    g = hq // hkv
    out = np.zeros((hq, d))
    lse = np.zeros(hq)
    for h in range(hq):
        kh = K[:, h // g, :]
        vh = V[:, h // g, :]
        z = scale * (kh @ q[h])
        m = z.max()
        s = np.exp(z - m).sum()
        lse[h] = m + math.log(s)
        w = np.exp(z - lse[h])
        out[h] = w @ vh
    return out, lse


def merge_partials(o_part: np.ndarray, lse_part: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Log-sum-exp merge of P partial results (the DCP merge of [QSA-DCP]).

    o_part: [P, ..., d] normalised partial outputs; lse_part: [P, ...].
      lse = M + log sum_p exp(lse_p - M),  M = max_p lse_p
      out = sum_p exp(lse_p - lse) * o_p
    All partials empty (lse = -inf everywhere) gives out = 0, lse = -inf.
    """
    o = np.asarray(o_part, dtype=np.float64)
    l = np.asarray(lse_part, dtype=np.float64)
    M = l.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(l), np.exp(l - Ms[None]), 0.0)
    s = w.sum(axis=0)
    lse = np.where(finite, Ms + np.log(np.where(finite, s, 1.0)), -np.inf)
    ww = np.where(finite[None], w / np.where(finite, s, 1.0)[None], 0.0)
    out = (ww[..., None] * o).sum(axis=0)
    return out, lse


# ---------------------------------------------------------------------------
# Paged cache access (the caller-owned storage the GPU path reads)
# ---------------------------------------------------------------------------

def paged_rows(cache: np.ndarray, block_table_row: np.ndarray, page_size: int,
               tokens: np.ndarray) -> np.ndarray:
    """Logical rows of one request from a paged cache [num_pages, H_kv, page, d].

    Token t of the request lives in physical page block_table_row[t // page]
    at slot t % page (one page table serves the main KV cache and the
    compressed key cache, so the two cannot drift -- [QSA-DCP]).
    Returns [T, H_kv, d] in the cache's own dtype.
    """
    t = np.asarray(tokens, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    return cache[pages, :, t % page_size, :]


def paged_scales(scale: np.ndarray, block_table_row: np.ndarray, page_size: int,
                 tokens: np.ndarray) -> np.ndarray:
    """Per-token fp32 scales [num_pages, page] -> [T] for the given tokens."""
    t = np.asarray(tokens, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    return np.asarray(scale, dtype=np.float64)[pages, t % page_size]


def decode_kv(raw: np.ndarray, kv_dtype: str, scales: np.ndarray = None) -> np.ndarray:
    """Decode stored K or V rows [T, H_kv, d] to float64 (bf16 bits or fp8 codes)."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        return fp8_e4m3_to_f64(raw) * np.asarray(scales, dtype=np.float64)[:, None, None]
    raise ValueError(kv_dtype)


# ---------------------------------------------------------------------------
# One decode step for a batch of rows
# ---------------------------------------------------------------------------

def decode_rows(*, q: np.ndarray, row_sel: np.ndarray, sel_req: np.ndarray, sel_seq_len: np.ndarray,
                row_seq_len: np.ndarray, topk: np.ndarray, block_table: np.ndarray, page_size: int,
                k_cache: np.ndarray, v_cache: np.ndarray, kv_dtype: str, scale: float,
                num_splits: int, k_scale: np.ndarray = None, v_scale: np.ndarray = None,
                rows: Sequence[int] = None):
    """Sparse attention for query rows, with num_splits partials and their merge.

    q: bf16 bits [R, H_q, d].  Row r uses the selection of selecting row
    s = row_sel[r] (several rows may share one: the MTP reuse of [PR53896]
    "关键源码片段", where later draft tokens keep the first token's top-k), of
    request sel_req[s]; a row with row_sel[r] < 0 attends nothing and gets the
    empty result (0, -inf).  topk: [S, k] ascending block ids (-1 padded).
    Returns dict with o_part [P, R', H_q, d], lse_part [P, R', H_q],
    out [R', H_q, d], lse [R', H_q] for the requested rows R'.
    """
    R = q.shape[0]
    rows = list(range(R)) if rows is None else list(rows)
    hq, d = q.shape[1], q.shape[2]
    P = num_splits
    o_part = np.zeros((P, len(rows), hq, d))
    lse_part = np.full((P, len(rows), hq), -np.inf)
    for i, r in enumerate(rows):
        s = int(row_sel[r])
        if s < 0:
            continue
        b = int(sel_req[s])
        qr = bf16_bits_to_f64(q[r])
        parts = split_token_positions(topk[s], int(sel_seq_len[s]), int(row_seq_len[r]), P)
        for p, toks in enumerate(parts):
            if toks.shape[0] == 0:
                continue
            kraw = paged_rows(k_cache, block_table[b], page_size, toks)
            vraw = paged_rows(v_cache, block_table[b], page_size, toks)
            ks = paged_scales(k_scale, block_table[b], page_size, toks) if kv_dtype == "fp8" else None
            vs = paged_scales(v_scale, block_table[b], page_size, toks) if kv_dtype == "fp8" else None
            K = decode_kv(kraw, kv_dtype, ks)
            V = decode_kv(vraw, kv_dtype, vs)
            o_part[p, i], lse_part[p, i] = attend(qr, K, V, scale)
    out, lse = merge_partials(o_part, lse_part)
    return {"o_part": o_part, "lse_part": lse_part, "out": out, "lse": lse}
