"""Benchmark of the QSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config 3] [--splits P] [--layers 12]

A step is one decode step of every layer in a stack of `--layers` independent
QSA layers (default 12, the number of QSA layers in the 48-layer model the
pages describe), each layer running the whole hot path on its own caches:

    qsa_compress_index_topk (scan only) -> qsa_select_sparse_decode -> qsa_merge_partials

(--no-fuse: qsa_compress, then the scan of qsa_index_topk; --no-select-fuse:
the selection in qsa_compress_index_topk / qsa_index_topk, then
qsa_sparse_decode)

The per-layer caches (about 84 MB touched per layer at 256k context) rotate so
that one step touches about 1 GB, far beyond the 256 MB Infinity Cache.  The
step is captured once in a HIP graph and replayed; timing uses HIP events on
the capture stream.  Inputs are seeded synthetic data resident in HBM.

Printed: one JSON line with the throughput in query rows per second, the
roofline of each of the step's three kernels (scan, selection + attention,
merge: algorithmic bytes over the average launch time, HIP events on the
launch stream) with the slowest of them as `roofline`, and the CPU oracle's
rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QSA decode query-rows/s at 256k ctx; achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0
BENCH_SPLITS = {1: 1, 2: 4, 3: 16, 4: 1, 5: 8}
DESCR = {
    1: "tiny: B=1, H 4/1, d=64, L=1,024, top-32 blocks, D=32, contiguous cache, bf16 K/V",
    2: "decode-32k: B=32, H 16/2, d=128, L=32,768, top-512 blocks, D=64, 64-token pages, bf16 K/V",
    3: "long-256k: B=8, H 16/2, d=128, L=262,144 (65,536 micro-blocks), top-512 blocks, D=64, "
       "64-token shuffled pages, bf16 K/V",
    4: "mixed-128: 128 requests, L log-uniform in [512, 262,144], H 16/2, d=128, top-512, bf16 K/V",
    5: "fp8-1m: B=4, L=1,000,000, 4 query rows per request sharing one selection, fp8 E4M3 K/V",
}


def algorithmic_parts(wl, num_splits: int):
    """Bytes the step must move, per layer, by part.

    scan: every closed micro-block of every selecting row at its stored width
    (10 bits per index dim: D + D/4 bytes), its page-table entries and the
    indexer query;
    kv: the selected and tail K/V rows of each selecting row's request, read
    once per KV head for all rows sharing the selection (+ fp8 scales);
    q: the attention queries; out: the fp32 output and LSE;
    part: the split partials (fp32 o_part + lse_part), written by the attention
    and read by the merge (an intermediate: not in the step's bytes).
    """
    s = wl.shape
    D, page, d, hkv, hq = s.index_dim, s.page_size, s.head_dim, s.num_kv_heads, s.num_q_heads
    esz = 1 if s.kv_dtype == "fp8" else 2
    sel_len = wl.sel_seq_len.cpu().numpy().astype(np.int64)
    row_len = wl.row_seq_len.cpu().numpy().astype(np.int64)
    row_sel = wl.row_sel.cpu().numpy()
    nb = sel_len // 4
    scan = int((nb * (D + D // 4)).sum() + (((sel_len + page - 1) // page) * 4).sum() + len(sel_len) * D)
    kv = 0
    for si in range(wl.num_sel):
        rows = row_len[row_sel == si]
        if rows.size == 0:
            continue
        ntok = 4 * min(s.topk_blocks, int(nb[si])) + max(0, int(rows.max()) - 4 * int(nb[si]))
        kv += ntok * hkv * d * esz * 2 + (ntok * 4 * 2 if s.kv_dtype == "fp8" else 0)
    R = wl.num_rows
    return {"scan": scan, "kv": kv, "q": R * hq * d * 2, "out": R * hq * d * 4 + R * hq * 4,
            "part": num_splits * R * hq * (d + 1) * 4}


def kernel_times(layers, stream, iters: int):
    """Average launch time (ms) of the step's scan, attention and merge calls,
    from graphs of those calls over all layers, replayed `iters` times and timed
    with HIP events on the launch stream."""
    import torch

    from block_sparse_attention_qsa_amd import api

    def first(layer):
        sel = not layer.select_decode
        if layer.fused:
            layer.compress_index(stream, select=sel)
        else:
            layer.compress(stream)
            layer.index(stream, select=sel)

    def second(layer):
        if layer.select_decode:
            layer.select_attend(stream)
        else:
            layer.decode(stream)

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(iters):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / (iters * len(layers))

    both = timed(lambda: [(first(l), second(l)) for l in layers])
    merge = timed(lambda: [l.merge(stream) for l in layers])
    scan = timed(lambda: [first(l) for l in layers])
    for layer in layers:  # scans without a selection leave their histograms summed: start clean
        api.qsa_index_topk_workspace_init(layer.workspace, stream=stream)
    torch.cuda.synchronize()
    return {"scan": scan, "attention": both - scan, "merge": merge}


def append_bytes(wl):
    """Bytes of the step's append, per layer: the new keys, the ring slots of the
    straddling block read, the new tokens' ring slots and the closed blocks written."""
    D = wl.shape.index_dim
    before = wl.prefix_len.astype(np.int64)
    n = wl.final_len.astype(np.int64) - before
    closed = (before + n) // 4 - before // 4
    return int((n * D + (before % 4) * D + np.minimum(n, 8) * D + closed * (D + D // 4)).sum())


# ---- the CPU oracle on the host cores.  The step starts from a prebuilt
# compressed cache (the oracle's compress_keys of every request, computed once,
# untimed); a timed row is: score + select over the full context, then the
# token set's attention and the merge.  Spawned workers (they import numpy and
# the oracle only, never the GPU runtime) read the workload from shared memory.
_POOL = {}


def _pool_init(spec):
    from multiprocessing import shared_memory

    from threadpoolctl import threadpool_limits
    _POOL["limits"] = threadpool_limits(1)
    _POOL["shm"] = []
    arrs = {}
    for name, (shm_name, shape, dtype) in spec["arrays"].items():
        shm = shared_memory.SharedMemory(name=shm_name)  # the parent owns and unlinks it
        _POOL["shm"].append(shm)
        arrs[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)
    _POOL["a"] = arrs
    _POOL["meta"] = spec["meta"]


def _pool_rows(job):
    """Worker: oracle rows (selecting rows start, start+1, ... cyclically) until the deadline."""
    from oracle import qsa_oracle as O
    start, deadline = job
    a, m = _POOL["a"], _POOL["meta"]
    k, S = m["k"], m["num_sel"]
    done, s = 0, start % S
    while time.time() < deadline:
        b = int(a["sel_req"][s])
        nb = int(a["sel_seq_len"][s]) // 4
        off = int(a["ck_off"][b])
        topk = np.full((S, k), -1, dtype=np.int32)
        topk[s] = O.select_blocks(O.score_blocks(a["q_index"][s], a["ckeys"][off:off + nb]), k)
        rows = np.nonzero(a["row_sel"] == s)[0]
        O.decode_rows(q=a["q"], row_sel=a["row_sel"], sel_req=a["sel_req"], sel_seq_len=a["sel_seq_len"],
                      row_seq_len=a["row_seq_len"], topk=topk, block_table=a["block_table"],
                      page_size=m["page_size"], k_cache=a["k_cache"], v_cache=a["v_cache"],
                      kv_dtype=m["kv_dtype"], scale=m["scale"], num_splits=1,
                      k_scale=a.get("k_scale"), v_scale=a.get("v_scale"), rows=rows)
        done += rows.shape[0]
        s = (s + 1) % S
    return done


def cpu_baseline(wl, seconds: float, procs: int):
    """The oracle as written on rows of layer 0, in `procs` single-threaded processes."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    from oracle import qsa_oracle as O
    from tests.harness import host_copy
    h = host_copy(wl)
    sel_len = h.sel_seq_len.astype(np.int64)
    # the prebuilt compressed cache: per request, the closed blocks its longest selecting row scores
    nb_req = np.zeros(wl.num_reqs, dtype=np.int64)
    for s_, b_ in enumerate(h.sel_req):
        nb_req[b_] = max(nb_req[b_], sel_len[s_] // 4)
    ck_off = np.zeros(wl.num_reqs + 1, dtype=np.int64)
    ck_off[1:] = np.cumsum(nb_req)
    ckeys = np.zeros((int(ck_off[-1]), wl.shape.index_dim), dtype=np.int16)  # |C| <= 512: lossless
    for b_ in range(wl.num_reqs):
        kb = h.keys[h.key_off[b_]:h.key_off[b_] + 4 * nb_req[b_]]
        ckeys[ck_off[b_]:ck_off[b_ + 1]] = O.compress_keys(kb, int(4 * nb_req[b_]))
    arrays = {"ckeys": ckeys, "ck_off": ck_off}
    arrays.update({n: getattr(h, n) for n in ("block_table", "k_cache", "v_cache", "k_scale", "v_scale", "q",
                                              "q_index", "sel_req", "sel_seq_len", "row_seq_len", "row_sel")})
    spec = {"arrays": {}, "meta": {"k": wl.shape.topk_blocks, "num_sel": wl.num_sel,
                                    "page_size": wl.shape.page_size, "kv_dtype": wl.shape.kv_dtype,
                                    "scale": wl.shape.softmax_scale}}
    owned = []
    try:
        for n, arr in arrays.items():
            if arr is None:
                continue
            arr = np.ascontiguousarray(arr)
            shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
            owned.append(shm)
            np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
            spec["arrays"][n] = (shm.name, arr.shape, arr.dtype.str)
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs, initializer=_pool_init, initargs=(spec,)) as pool:
            pool.map(_pool_rows, [(i, 0.0) for i in range(procs)])  # start-up and first touch, untimed
            t0 = time.time()
            counts = pool.map(_pool_rows, [(i, t0 + seconds) for i in range(procs)])
            el = time.time() - t0
    finally:
        for shm in owned:
            shm.close()
            shm.unlink()
    done = int(sum(counts))
    return {"value": done / el, "unit": "query-rows/s", "cores": procs, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{done} query rows of layer 0 ({wl.name}) in {procs} single-threaded processes "
                      f"(the host has {os.cpu_count()} cores), {el:.1f} s; each row: score + select over "
                      f"the full context from the prebuilt compressed cache, then attention + merge, "
                      f"numpy int64/float64"}


def stream_ceiling(stream, reps: int = 10):
    """Read rate of a plain streaming kernel (libqsa_ceiling.so) over 1 GiB, HIP events."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_qsa_amd", "libqsa_ceiling.so"))
    lib.qsa_stream_granule.restype = ctypes.c_size_t
    lib.qsa_stream_sink_bytes.restype = ctypes.c_size_t
    lib.qsa_stream_read.restype = ctypes.c_int
    lib.qsa_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    g = lib.qsa_stream_granule()
    nbytes = max(1, (1 << 30) // g) * g
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(lib.qsa_stream_sink_bytes(), dtype=torch.uint8, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    for _ in range(2):
        assert lib.qsa_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), sp) == 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        lib.qsa_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), sp)
    b.record(stream)
    torch.cuda.synchronize()
    gbs = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    return {"kernel": "qsa_stream_ceiling (2048 workgroups x 256 threads, 8 x 16 B non-temporal loads in flight)",
            "bytes": nbytes, "GBps": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


def stream_at_size(stream, nbytes: int, nbuf: int, iters: int):
    """The same streaming loads over a transfer of `nbytes` (rounded down to the kernel's tile):
    `nbuf` buffers read one after another by single-pass launches captured in a graph (so each
    launch reads cold data, as the scan's rotating layers do), replayed `iters` times, HIP events."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_qsa_amd", "libqsa_ceiling.so"))
    lib.qsa_stream_tile.restype = ctypes.c_size_t
    lib.qsa_stream_granule.restype = ctypes.c_size_t
    lib.qsa_stream_sink_bytes.restype = ctypes.c_size_t
    lib.qsa_stream_read_once.restype = ctypes.c_int
    lib.qsa_stream_read_once.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    tile = lib.qsa_stream_tile()
    n = min(max(1, nbytes // tile) * tile, lib.qsa_stream_granule())
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.empty(lib.qsa_stream_sink_bytes(), dtype=torch.uint8, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for b in bufs:
            assert lib.qsa_stream_read_once(ctypes.c_void_p(b.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), sp) == 0
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record(stream)
        for _ in range(iters):
            g.replay()
        e.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(e) * 1e3 / (iters * nbuf)
    del g, bufs
    return {"kernel": f"the same loads, one pass over {n} bytes ({n // tile} workgroups), "
                      f"{nbuf} buffers in rotation, graph-replayed",
            "bytes": n, "avg_launch_us": us, "GBps": n / (us * 1e-6) / 1e9, "frac_of_peak": n / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


COUNTER_FILES = {"scan": "score_kernel_long256k_hbm_counters.md",
                 "attention": "select_decode_kernel_long256k_hbm_counters.md"}


def measured_traffic(name: str, fused: bool, select_fused: bool, cfg: int):
    """HBM bytes per launch of kernel `name` from its committed rocprofv3
    counter summary (workload 3 only), or None when there is none, when the
    kernel source has changed since the counters were taken, or when they were
    taken for another variant of the step."""
    import hashlib
    if cfg != 3 or name not in COUNTER_FILES:
        return None
    path = os.path.join(ROOT, "profiles", COUNTER_FILES[name])
    want = {"scan": "fused" if fused else "separate",
            "attention": "fused" if select_fused else "separate"}[name]
    try:
        kv = dict(line.split(" = ", 1) for line in open(path).read().splitlines() if " = " in line)
        if kv.get("variant", "separate").strip() != want:
            return None
        h = hashlib.sha256()
        for src in kv["kernel_sources"].split(","):  # the kernel's file and the headers it includes
            h.update(open(os.path.join(ROOT, src.strip()), "rb").read())
        if h.hexdigest() != kv["kernel_sources_sha256"].strip():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    """A plain device copy of known size (for scaling rocprofv3 byte counters)."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


PREFILL_DESCR = ("chunked prefill: B=4 requests, the last 512-token chunk of a 65,536-token prompt "
                 "(2,048 query rows, each with its own causal length), H 16/2, d=128, top-512 blocks, D=64, "
                 "64-token shuffled pages, bf16 K/V")


def prefill_bench(args):
    """Chunked-prefill step (compress the chunk, per-row selection with the int8-GEMM scan,
    attention, merge) over `--layers` independent layers; one JSON line."""
    import torch

    from block_sparse_attention_qsa_amd import api
    from block_sparse_attention_qsa_amd.pipeline import QSAPrefill
    from block_sparse_attention_qsa_amd.workloads import SHAPE_MAIN, make_prefill_workload
    P = args.splits or 1  # 2,048 rows fill the chip without splits (1 split: 3.6M rows/s, 4: 3.2M)
    nl = min(args.layers, 4)
    layers = []
    for li in range(nl):
        wl = make_prefill_workload(SHAPE_MAIN, [65536] * 4, 512, seed=7000 + li, device="cuda",
                                   name="prefill-64k-chunk512")
        layer = QSAPrefill(wl, num_splits=P, select_decode=not args.no_select_fuse)
        layer.prefill()
        layers.append(layer)
        print(f"[bench] prefill layer {li} ready (rows={wl.num_rows})", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def timed(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for layer in layers:
                layer.step(stream)
    torch.cuda.synchronize()
    ms = timed(lambda: [layer.step(stream) for layer in layers], args.steps)
    # the per-row selection alone (compress, then the GEMM scan + filter + finalize)
    ms_index = timed(lambda: [(layer.compress(stream), layer.index(stream)) for layer in layers], args.steps)
    # the scan kernel alone (scores only); it leaves the histograms set, so it runs last
    def scan_only():
        for layer in layers:
            wl = layer.wl
            api.qsa_prefill_index_topk(layer.cfg, wl.q_index, layer.row_cu, wl.row_seq_len, wl.block_table,
                                       layer.ckey, None, layer.workspace, layer.max_seq_len, layer.max_rows,
                                       stream=stream)
    ms_scan = timed(scan_only, args.steps)
    wl0 = layers[0].wl
    lens = wl0.row_seq_len.cpu().numpy().astype(np.int64)
    D = wl0.shape.index_dim
    ops = 2.0 * float((lens // 4).sum()) * D                      # int8 multiply-adds of the scan, x2
    scan_bytes = float(4 * (65536 // 4) * (D + D // 4) + wl0.num_rows * D)
    rows = sum(l.wl.num_rows for l in layers)
    per_launch_s = ms_scan * 1e-3 / nl
    res = {"metric": "QSA chunked-prefill query-rows/s (per-row top-k + attention)",
           "value": rows / (ms * 1e-3), "unit": "query-rows/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": PREFILL_DESCR, "layers_per_step": nl, "query_rows_per_layer": wl0.num_rows,
                      "splits": P, "hip_graph": True},
           "selection_ms_per_step": ms_index, "scan_us_per_launch": per_launch_s * 1e6,
           "roofline": {"kernel": "qsa::prefill_score_kernel (int8 MFMA scan, 16 rows x 16 blocks per instruction)",
                        "bound": "mfma", "achieved": ops / per_launch_s / 1e12, "peak": 5000.0,
                        "unit": "TOP/s", "frac": ops / per_launch_s / 1e12 / 5000.0, "traffic": None,
                        "ops_per_launch": ops, "compressed_key_bytes_per_launch": scan_bytes,
                        "hbm_GBps_of_those_bytes": scan_bytes / per_launch_s / 1e9}}
    print(json.dumps(res))


def frontend_bench(args):
    """The indexer front end (qsa_indexer_project) at a decode step (8 tokens) and a
    prefill chunk (2,048 tokens), hidden size 4,096, D = 64; one JSON line."""
    import torch

    from block_sparse_attention_qsa_amd import api
    H, D = 4096, 64
    stream = torch.cuda.Stream()
    out = {}
    for T in (8, 2048):
        g = torch.Generator(device="cuda").manual_seed(11 + T)
        nl = 8  # rotate over independent inputs so each launch reads cold data
        hs = [torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16) for _ in range(nl)]
        ws = [(torch.randn((2 * D, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16) for _ in range(nl)]
        gq = torch.zeros(D, device="cuda")
        gk = torch.zeros(D, device="cuda")
        pos = torch.arange(T, dtype=torch.int32, device="cuda")
        q = torch.empty((T, D), dtype=torch.int8, device="cuda")
        k = torch.empty((T, D), dtype=torch.int8, device="cuda")
        scratch = torch.empty(max(api.qsa_indexer_project_workspace_size(T, H, D), 16), dtype=torch.uint8,
                              device="cuda")

        def run():
            for i in range(nl):
                api.qsa_indexer_project(hs[i], pos, ws[i], gq, gk, q, k, workspace=scratch, stream=stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(args.steps):
                graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (args.steps * nl)
        nbytes = T * H * 2 + 2 * D * H * 2 + T * 4 + 2 * T * D
        flops = 2.0 * T * H * 2 * D
        out[f"T{T}"] = {"us_per_launch": us, "tokens_per_s": T / (us * 1e-6),
                        "hbm_GBps": nbytes / (us * 1e-6) / 1e9, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                        "bf16_TFLOPs": flops / (us * 1e-6) / 1e12, "bytes": nbytes}
    big = out["T2048"]
    res = {"metric": "QSA indexer front end tokens/s (projection + RMSNorm + rotary + int8)",
           "value": big["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "hidden 4,096 -> D=64 query and key, bf16 weights [128, 4,096]; "
                                  "2,048 tokens (prefill chunk) and 8 tokens (decode step)"},
           "roofline": {"kernel": "qsa::project_kernel<64> (bf16 MFMA projection + fused epilogue)", "bound": "hbm",
                        "achieved": big["hbm_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": big["hbm_frac"], "traffic": None, "bytes_per_launch": big["bytes"],
                        "avg_launch_us": big["us_per_launch"]},
           "sizes": out}
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-fuse", action="store_true",
                    help="append with qsa_compress, then qsa_index_topk (two scans' worth of launches)")
    ap.add_argument("--no-select-fuse", action="store_true",
                    help="select in the index call, then qsa_sparse_decode (instead of qsa_select_sparse_decode)")
    ap.add_argument("--kernel-iters", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--prefill", action="store_true",
                    help="measure the chunked-prefill path instead (its own JSON line)")
    ap.add_argument("--frontend", action="store_true",
                    help="measure the indexer front end instead (its own JSON line)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the one-GPU path only: the library has no multi-GPU mode "
              "(context-parallel sharding is described in the design notes, not built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_attention_qsa_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.prefill:
        prefill_bench(args)
        return
    if args.frontend:
        frontend_bench(args)
        return
    from block_sparse_attention_qsa_amd import api
    from block_sparse_attention_qsa_amd.pipeline import QSALayer
    from block_sparse_attention_qsa_amd.workloads import named_workload

    cfg = args.config
    P = args.splits or BENCH_SPLITS[cfg]
    dev = "cuda"
    layers = []
    for li in range(args.layers):
        wl = named_workload(cfg, device=dev, seed=None if li == 0 else 1000 * cfg + li)
        layer = QSALayer(wl, num_splits=P, fuse_append=not args.no_fuse, select_decode=not args.no_select_fuse)
        layer.prefill()
        layers.append(layer)
        print(f"[bench] layer {li} ready ({wl.name}, rows={wl.num_rows})", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wl0 = layers[0].wl
    rows_per_step = sum(l.wl.num_rows for l in layers)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def step():
        for layer in layers:
            layer.step(stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            if graph is not None:
                graph.replay()
            else:
                step()
            if i < args.steps - 1:
                evs[i].record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    marks = [e0] + evs + [e1]
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))

    # Per-kernel timing, in the step's own launch sequence: each layer's step is
    # three launches (scan, selection + attention, merge).  Graphs of (a) every
    # layer's scan + attention call, (b) every layer's merge and (c) every
    # layer's scan alone are replayed and timed with HIP events on the launch
    # stream; the attention call's time is (a) - (c).  The layers rotate, so each
    # launch reads its own cold data.  (c) runs last: scans without a selection
    # in between add into the same histogram, so the workspaces are reset after it.
    kt = kernel_times(layers, stream, args.kernel_iters) if args.kernel_iters > 0 else None

    parts = [algorithmic_parts(l.wl, P) for l in layers]
    app_b = [append_bytes(l.wl) for l in layers]
    fused = layers[0].fused
    per = {k: float(np.mean([x[k] for x in parts])) for k in parts[0]}
    step_bytes = float(sum(x["scan"] + x["kv"] + x["q"] + x["out"] for x in parts) + sum(app_b))
    rows_s = rows_per_step / (ms * 1e-3)
    sel_fused = layers[0].select_decode
    kernels = {
        "scan": {"kernel": ("qsa::score_kernel<D, true> (qsa_compress_index_topk: append + compressed-key scan)"
                            if fused else "qsa::score_kernel<D, false> (qsa_index_topk compressed-key scan)")
                 + ("" if sel_fused else " + qsa::finalize_kernel"),
                 "bytes_per_launch": per["scan"] + (float(np.mean(app_b)) if fused else 0.0),
                 "bytes": "compressed keys of every closed block at 10 bits per dim, page-table entries, "
                          "indexer query" + (", the append" if fused else "")},
        "attention": {"kernel": ("qsa::select_decode_kernel (selection + sparse attention)" if sel_fused
                                 else "qsa::decode_kernel (sparse attention)"),
                      "bytes_per_launch": per["kv"] + per["q"] + per["part"],
                      "bytes": "selected + tail K/V rows once per KV head (+ fp8 scales), q, "
                               "the split partials written"},
        "merge": {"kernel": "qsa::merge_kernel", "bytes_per_launch": per["part"] + per["out"],
                  "bytes": "split partials read, fp32 output and LSE written"},
    }
    for name, kd in kernels.items():
        us = kt[name] * 1e3 if kt else float("nan")
        ach = kd["bytes_per_launch"] / (us * 1e-6) / 1e9
        kd.update({"bound": "hbm", "avg_launch_us": us, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(name, fused, sel_fused, cfg)})
    dom = max(kernels, key=lambda n: kernels[n]["avg_launch_us"] if kt else 0.0)

    res = {
        "metric": METRIC,
        "value": rows_s,
        "unit": "query-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step[len(per_step) // 2],
        "ms_per_step_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl0.shape.kv_dtype == "bf16" else "fp8",
        "data": "synthetic",
        "config": {"workload": f"cfg{cfg} {DESCR[cfg]}", "layers_per_step": args.layers,
                   "query_rows_per_layer": wl0.num_rows, "splits": P, "hip_graph": graph is not None,
                   "append": "fused into the scan" if fused else "separate qsa_compress launch",
                   "selection": ("with the attention (qsa_select_sparse_decode)" if sel_fused
                                 else "separate finalize launch"),
                   "index_arith": "int8 dot4 -> int32 (exact)", "attention_arith": "bf16 MFMA / fp32 softmax"},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved_GBps": step_bytes / (ms * 1e-3) / 1e9,
                     "frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "wall_s": t_wall},
        # the kernel with the longest average launch of the step's three
        "roofline": dict(kernels[dom], name=dom, launches_timed=args.kernel_iters * len(layers)),
        "kernels": kernels,
    }
    if kt:
        res["kernels_sum_us_per_layer"] = sum(kt.values()) * 1e3
    res["stream_ceiling"] = stream_ceiling(stream)
    if args.kernel_iters > 0:
        # a bare stream of the scan's size: the rate a transfer this short reaches at all
        same = stream_at_size(stream, int(kernels["scan"]["bytes_per_launch"]), len(layers), args.kernel_iters)
        same["scan_frac_of_it"] = kernels["scan"]["achieved"] / same["GBps"]
        res["stream_ceiling"]["at_scan_size"] = same
    if not args.no_cpu_baseline:
        procs = max(1, os.cpu_count() or 1)
        print(f"[bench] cpu baseline (oracle), one core then {procs} processes ...", file=sys.stderr, flush=True)
        one = cpu_baseline(wl0, args.cpu_seconds, 1)
        many = cpu_baseline(wl0, args.cpu_seconds, procs) if procs > 1 else one
        many["single_core"] = {"value": one["value"], "cores": 1, "sample": one["sample"]}
        res["cpu_baseline"] = many
    print(json.dumps(res))


if __name__ == "__main__":
    main()
