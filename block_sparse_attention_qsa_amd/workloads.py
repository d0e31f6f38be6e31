"""Seeded synthetic workloads for the QSA decode step.

This module only draws random inputs and lays them out in the caller-owned
buffers the library reads (paged K/V, page tables, raw indexer keys).  It holds
none of the method's arithmetic: no compression, scoring, selection or
attention happens here.  Both the CPU oracle (through the tests) and the HIP
path consume what it produces.

Inputs are drawn with torch's generator on the requested device (CPU and GPU
streams differ, so a workload is identified by (config, seed, device)):

* indexer keys and indexer queries: int8, uniform integers in [-127, 127];
* attention q, K, V: float32 N(0, 1) rounded to bfloat16 (round-to-nearest-even);
* fp8 K/V: per token and tensor, scale = amax / 448 over the token's
  H_kv x d values (amax = 0 gives scale 1), values divided by the scale,
  clamped to +-448 and rounded to OCP E4M3 by torch's float8_e4m3fn cast;
* page tables: a seeded permutation of the page pool, split across requests.

The five named workloads mirror the shapes of the QSA decode path on the pages
(micro-blocks of 4 tokens, top-512 blocks, 256k / 1M contexts, 16 query heads
over 2 KV heads for the 256k model, decode context parallel splits); they stand
in for the pages' serving trace, which is not available.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


@dataclass
class QSAShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    topk_blocks: int
    page_size: int
    kv_dtype: str = "bf16"  # "bf16" or "fp8"
    compress_ratio: int = 4

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass
class Workload:
    """One layer's decode-step inputs.  All tensors live on `device`.

    Request b holds tokens [0, final_len[b]).  Before the step the compressed
    cache covers [0, prefix_len[b]); the step appends tokens
    [prefix_len[b], final_len[b]) through qsa_compress.  Selecting row s
    (request sel_req[s], context sel_seq_len[s]) picks the blocks that the
    query rows r with row_sel[r] == s attend (at most q_per_sel of them).
    """
    name: str
    shape: QSAShape
    seed: int
    device: str
    final_len: np.ndarray          # int64 [B]
    prefix_len: np.ndarray         # int64 [B]
    keys: torch.Tensor             # int8 [sum(final_len), D] (request-major)
    key_off: np.ndarray            # int64 [B+1]
    block_table: torch.Tensor      # int32 [B, max_pages]
    num_pages: int
    k_cache: torch.Tensor          # bf16 or uint8 [num_pages, H_kv, page, d]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]  # fp32 [num_pages, page] (fp8 only)
    v_scale: Optional[torch.Tensor]
    q_per_sel: int                 # most query rows sharing one selecting row
    sel_req: torch.Tensor          # int32 [S]
    sel_seq_len: torch.Tensor      # int32 [S]
    q_index: torch.Tensor          # int8 [S, D]
    row_seq_len: torch.Tensor      # int32 [R]
    q: torch.Tensor                # bf16 [R, H_q, d]
    row_sel: Optional[torch.Tensor] = None  # int32 [R]: selecting row of each query row
    extra: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.row_sel is None:  # rows grouped contiguously, q_per_sel per selecting row
            self.row_sel = torch.arange(self.num_rows, dtype=torch.int32, device=self.q.device) // self.q_per_sel

    @property
    def num_reqs(self) -> int:
        return int(self.final_len.shape[0])

    @property
    def num_sel(self) -> int:
        return int(self.sel_req.shape[0])

    @property
    def num_rows(self) -> int:
        return int(self.q.shape[0])


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _quant_fp8(x: torch.Tensor):
    """Per-token fp8 E4M3 quantisation of x [P, H_kv, page, d] -> (codes u8, scale [P, page])."""
    amax = x.abs().amax(dim=(1, 3))  # [P, page]
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / scale[:, None, :, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def make_workload(shape: QSAShape, final_len: List[int], *, step_tokens: int = 1,
                  q_per_sel: int = 1, seed: int = 0, device: str = "cpu",
                  name: str = "custom", spare_pages: int = 0,
                  shuffle_pages: bool = True, rows_per_req: Optional[List[int]] = None) -> Workload:
    """Draw a workload with the given per-request final lengths.

    step_tokens: tokens each request appends in the step (prefix = final - step).
    q_per_sel:   query rows per selecting row; row j of a request has context
                 final - step_tokens + 1 + j ... when q_per_sel == step_tokens
                 (each appended token is one query row), else every row has
                 context final_len.
    rows_per_req: uneven draft counts instead: request b appends rows_per_req[b]
                 tokens (its prefix is final - rows_per_req[b]), each a query row
                 of context prefix + 1 + j, all sharing the selection of the
                 first one (row_sel maps them); 0 rows leaves the request idle.
    """
    if rows_per_req is not None:
        return _make_uneven(shape, final_len, rows_per_req, seed=seed, device=device, name=name,
                            shuffle_pages=shuffle_pages)
    g = _gen(seed, device)
    D, hkv, d, page = shape.index_dim, shape.num_kv_heads, shape.head_dim, shape.page_size
    fl = np.asarray(final_len, dtype=np.int64)
    B = fl.shape[0]
    prefix = np.maximum(fl - step_tokens, 0)
    pages_per_req = np.maximum((fl + page - 1) // page, 1)
    max_pages = int(pages_per_req.max())
    num_pages = int(pages_per_req.sum()) + spare_pages
    perm = torch.randperm(num_pages, generator=g, device=device) if shuffle_pages else \
        torch.arange(num_pages, device=device)
    bt = torch.zeros((B, max_pages), dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        n = int(pages_per_req[b])
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    key_off = np.zeros(B + 1, dtype=np.int64)
    key_off[1:] = np.cumsum(fl)
    keys = torch.randint(-127, 128, (int(key_off[-1]), D), generator=g, device=device, dtype=torch.int8)

    kv_shape = (num_pages, hkv, page, d)
    if shape.kv_dtype == "bf16":
        k_cache = torch.randn(kv_shape, generator=g, device=device).to(torch.bfloat16)
        v_cache = torch.randn(kv_shape, generator=g, device=device).to(torch.bfloat16)
        k_scale = v_scale = None
    elif shape.kv_dtype == "fp8":
        k_cache, k_scale = _quant_fp8(torch.randn(kv_shape, generator=g, device=device))
        v_cache, v_scale = _quant_fp8(torch.randn(kv_shape, generator=g, device=device))
    else:
        raise ValueError(shape.kv_dtype)

    S = B
    R = B * q_per_sel
    sel_req = torch.arange(B, dtype=torch.int32, device=device)
    if q_per_sel == step_tokens and step_tokens > 1:
        # each appended token is a query row; the first one selects
        row_len = np.concatenate([prefix[b] + 1 + np.arange(q_per_sel) for b in range(B)])
        sel_len = prefix + 1
    else:
        row_len = np.repeat(fl, q_per_sel)
        sel_len = fl.copy()
    q_index = torch.randint(-127, 128, (S, D), generator=g, device=device, dtype=torch.int8)
    q = torch.randn((R, shape.num_q_heads, d), generator=g, device=device).to(torch.bfloat16)
    return Workload(
        name=name, shape=shape, seed=seed, device=device, final_len=fl, prefix_len=prefix,
        keys=keys, key_off=key_off, block_table=bt, num_pages=num_pages,
        k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
        q_per_sel=q_per_sel, sel_req=sel_req,
        sel_seq_len=torch.as_tensor(sel_len.astype(np.int32), device=device),
        q_index=q_index,
        row_seq_len=torch.as_tensor(row_len.astype(np.int32), device=device), q=q)


def _make_uneven(shape: QSAShape, final_len: List[int], rows_per_req: List[int], *, seed: int, device: str,
                 name: str, shuffle_pages: bool) -> Workload:
    n = np.asarray(rows_per_req, dtype=np.int64)
    base = make_workload(shape, final_len, step_tokens=int(max(n.max(), 1)), q_per_sel=1, seed=seed, device=device,
                         name=name, shuffle_pages=shuffle_pages)
    fl = base.final_len
    prefix = np.maximum(fl - n, 0)
    active = np.nonzero(n > 0)[0]
    S = active.shape[0]
    row_len = np.concatenate([prefix[b] + 1 + np.arange(n[b]) for b in active]).astype(np.int64)
    row_sel = np.repeat(np.arange(S), n[active])
    g = _gen(seed + 104729, device)
    q_index = torch.randint(-127, 128, (S, shape.index_dim), generator=g, device=device, dtype=torch.int8)
    q = torch.randn((row_len.shape[0], shape.num_q_heads, shape.head_dim), generator=g,
                    device=device).to(torch.bfloat16)
    return Workload(
        name=name, shape=shape, seed=seed, device=device, final_len=fl, prefix_len=prefix,
        keys=base.keys, key_off=base.key_off, block_table=base.block_table, num_pages=base.num_pages,
        k_cache=base.k_cache, v_cache=base.v_cache, k_scale=base.k_scale, v_scale=base.v_scale,
        q_per_sel=int(n.max()), sel_req=torch.as_tensor(active.astype(np.int32), device=device),
        sel_seq_len=torch.as_tensor((prefix[active] + 1).astype(np.int32), device=device), q_index=q_index,
        row_seq_len=torch.as_tensor(row_len.astype(np.int32), device=device), q=q,
        row_sel=torch.as_tensor(row_sel.astype(np.int32), device=device))


def make_prefill_workload(shape: QSAShape, final_len: List[int], chunk, *, seed: int = 0,
                          device: str = "cpu", name: str = "prefill", shuffle_pages: bool = True) -> Workload:
    """Chunked prefill: request b appends its last chunk[b] tokens (an int applies to
    all), and every appended token is a query row with its own selection: row t of
    request b has context prefix_b + 1 + t (causal).  S = R = sum(chunk);
    sel_req[r] is the row's request; extra["row_cu"] (int32 [B+1]) delimits the
    requests' rows; the K/V and compressed caches hold every token up to final_len."""
    fl = np.asarray(final_len, dtype=np.int64)
    B = fl.shape[0]
    ch = np.broadcast_to(np.asarray(chunk, dtype=np.int64), (B,)).copy()
    base = make_workload(shape, list(fl), step_tokens=int(ch.max()), q_per_sel=1, seed=seed, device=device,
                         name=name, shuffle_pages=shuffle_pages)
    prefix = np.maximum(fl - ch, 0)
    rows = np.concatenate([prefix[b] + 1 + np.arange(fl[b] - prefix[b]) for b in range(B)]).astype(np.int64)
    counts = fl - prefix
    row_cu = np.zeros(B + 1, dtype=np.int64)
    row_cu[1:] = np.cumsum(counts)
    R = int(row_cu[-1])
    g = _gen(seed + 7919, device)
    sel_req = np.repeat(np.arange(B), counts)
    q_index = torch.randint(-127, 128, (R, shape.index_dim), generator=g, device=device, dtype=torch.int8)
    q = torch.randn((R, shape.num_q_heads, shape.head_dim), generator=g, device=device).to(torch.bfloat16)
    lens = torch.as_tensor(rows.astype(np.int32), device=device)
    return Workload(
        name=name, shape=shape, seed=seed, device=device, final_len=fl, prefix_len=prefix,
        keys=base.keys, key_off=base.key_off, block_table=base.block_table, num_pages=base.num_pages,
        k_cache=base.k_cache, v_cache=base.v_cache, k_scale=base.k_scale, v_scale=base.v_scale,
        q_per_sel=1, sel_req=torch.as_tensor(sel_req.astype(np.int32), device=device),
        sel_seq_len=lens, q_index=q_index, row_seq_len=lens.clone(), q=q,
        extra={"row_cu": torch.as_tensor(row_cu.astype(np.int32), device=device),
               "max_rows_per_req": int(counts.max()) if B else 0})


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

SHAPE_TINY = QSAShape(num_q_heads=4, num_kv_heads=1, head_dim=64, index_dim=32,
                      topk_blocks=32, page_size=1024)
SHAPE_MAIN = QSAShape(num_q_heads=16, num_kv_heads=2, head_dim=128, index_dim=64,
                      topk_blocks=512, page_size=64)
SHAPE_FP8 = QSAShape(num_q_heads=16, num_kv_heads=2, head_dim=128, index_dim=64,
                     topk_blocks=512, page_size=64, kv_dtype="fp8")

WORKLOADS = {
    1: "tiny: B=1, 4/1 heads, d=64, L=1,024, top-32, D=32, contiguous",
    2: "decode: B=32, 16/2 heads, d=128, L=32,768, top-512, D=64, 64-token pages",
    3: "long: B=8, 16/2 heads, d=128, L=262,144, top-512, D=64, 64-token pages",
    4: "mixed: 128 requests, L log-uniform in [512, 262,144], 64-token pages",
    5: "fp8: B=4, L=1,000,000, 4 query rows per request, fp8 K/V",
}


def mixed_lengths(seed: int, n: int = 128, n_short: int = 13) -> List[int]:
    """Context lengths of the mixed batch: n_short log-uniform in [512, 2048],
    the rest log-uniform in [2049, 262144], in random order (floor to int)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    short = np.exp(rng.uniform(math.log(512), math.log(2048), n_short))
    long = np.exp(rng.uniform(math.log(2049), math.log(262144), n - n_short))
    L = np.floor(np.concatenate([short, long])).astype(np.int64)
    L = np.clip(L, 512, 262144)
    return [int(x) for x in L[rng.permutation(n)]]


def named_workload(cfg: int, *, device: str = "cpu", seed: Optional[int] = None,
                   scale_ctx: float = 1.0) -> Workload:
    """Workload `cfg` (1..5).  scale_ctx < 1 shrinks the contexts for quick runs."""
    if cfg == 1:
        return make_workload(SHAPE_TINY, [1024], seed=0 if seed is None else seed,
                             device=device, name="cfg1-tiny", shuffle_pages=False)
    if cfg == 2:
        L = max(8, int(32768 * scale_ctx))
        return make_workload(SHAPE_MAIN, [L] * 32, seed=1 if seed is None else seed,
                             device=device, name="cfg2-decode-32k")
    if cfg == 3:
        L = max(8, int(262144 * scale_ctx))
        return make_workload(SHAPE_MAIN, [L] * 8, seed=2 if seed is None else seed,
                             device=device, name="cfg3-long-256k")
    if cfg == 4:
        s = 3 if seed is None else seed
        L = [max(8, int(x * scale_ctx)) for x in mixed_lengths(s)]
        return make_workload(SHAPE_MAIN, L, seed=s, device=device, name="cfg4-mixed-128")
    if cfg == 5:
        L0 = max(8, int(1_000_000 * scale_ctx))
        # rows of request b have contexts L0 .. L0+3; the step appends 4 tokens
        return make_workload(SHAPE_FP8, [L0 + 3] * 4, step_tokens=4, q_per_sel=4,
                             seed=4 if seed is None else seed, device=device,
                             name="cfg5-fp8-1m-mtp4")
    raise ValueError(cfg)
