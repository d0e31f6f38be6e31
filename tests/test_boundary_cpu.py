"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before enqueueing anything."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_qsa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


def cfg(**kw):
    base = dict(num_q_heads=16, num_kv_heads=2, head_dim=128, index_dim=64, compress_ratio=4,
                topk_blocks=512, page_size=64, max_pages_per_req=4096, ring_size=8, kv_dtype=0, softmax_scale=0.088)
    base.update(kw)
    return _lib.qsa_config(**base)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"qsa_compress", "qsa_index_topk", "qsa_sparse_decode", "qsa_merge_partials"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(qsa_[a-z0-9_]+)\b", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.qsa_version().startswith(b"qsa-mi355x")
    assert lib.qsa_status_string(0) == b"QSA_OK"
    assert lib.qsa_status_string(3) == b"QSA_ERR_WORKSPACE"
    assert lib.qsa_status_string(99) == b"QSA_ERR_UNKNOWN"


def compress(lib, c, nreq=1, **kw):
    a = dict(new_keys=FAKE, new_cu=FAKE, before=FAKE, bt=FAKE, ring=FAKE, ckey=FAKE)
    a.update(kw)
    return lib.qsa_compress(ctypes.byref(c), nreq, 4, a["new_keys"], a["new_cu"], a["before"], a["bt"],
                            a["ring"], a["ckey"], None)


@pytest.mark.parametrize("bad,code", [
    (dict(compress_ratio=3), 1), (dict(compress_ratio=8), 1), (dict(page_size=48), 1),
    (dict(page_size=8), 1), (dict(topk_blocks=0), 1), (dict(topk_blocks=4096), 1),
    (dict(max_pages_per_req=0), 1), (dict(index_dim=48), 2), (dict(index_dim=0), 1),
    (dict(ring_size=4), 1), (dict(ring_size=0), 1), (dict(ring_size=16), 1),
])
def test_compress_rejects_bad_config(lib, bad, code):
    assert compress(lib, cfg(**bad)) == code
    assert lib.qsa_last_error() != b""


def test_compress_rejects_null_and_misaligned(lib):
    assert compress(lib, cfg(), ckey=None) == 1
    assert compress(lib, cfg(), ring=None) == 1
    assert compress(lib, cfg(), ckey=ctypes.c_void_p(0x10004)) == 1
    assert compress(lib, cfg(), nreq=-1) == 1
    assert compress(lib, cfg(), nreq=0) == 0  # nothing to do, nothing enqueued
    assert lib.qsa_ckey_cache_bytes(ctypes.byref(cfg()), 10) == 10 * 64 // 4 * (64 + 64 // 4)
    assert lib.qsa_ckey_cache_bytes(ctypes.byref(cfg(compress_ratio=2)), 10) == 0


def test_workspace_size_and_checks(lib):
    c = cfg()
    n8 = lib.qsa_index_topk_workspace_size(ctypes.byref(c), 8, 262144)
    n16 = lib.qsa_index_topk_workspace_size(ctypes.byref(c), 16, 262144)
    assert 0 < n8 < n16
    assert lib.qsa_index_topk_workspace_size(ctypes.byref(c), 8, _lib.QSA_MAX_SEQ_LEN + 1) == 0
    assert lib.qsa_index_topk_workspace_size(ctypes.byref(c), -1, 100) == 0

    def topk(ws=FAKE, nbytes=n8, S=8, L=262144, **kw):
        return lib.qsa_index_topk(ctypes.byref(kw.get("c", c)), S, L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  ws, nbytes, None)
    assert topk(nbytes=n8 - 1) == 3
    assert topk(ws=None) == 3
    assert topk(ws=ctypes.c_void_p(0x10010)) == 3  # not 256-aligned
    assert topk(L=_lib.QSA_MAX_SEQ_LEN + 4) == 1
    assert topk(S=-2) == 1
    assert topk(c=cfg(index_dim=96)) == 2
    assert topk(S=0) == 0
    assert lib.qsa_index_topk_workspace_init(None, 100, None) == 3


def test_index_topk_noalloc_rejects(lib):
    c = cfg()

    def na(S=8, L=65536, q=FAKE, topk=FAKE, **kw):
        return lib.qsa_index_topk_noalloc(ctypes.byref(kw.get("c", c)), S, L, q, FAKE, FAKE, FAKE, FAKE, topk, None)
    assert na(topk=None) == 1                      # the selection is required
    assert na(q=None) == 1
    assert na(S=-1) == 1
    assert na(L=_lib.QSA_MAX_SEQ_LEN + 4) == 1
    assert na(c=cfg(index_dim=96)) == 2
    assert na(S=64, L=262144) == 3                 # more than the library's scratch
    assert lib.qsa_index_topk_workspace_size(ctypes.byref(c), 12, 262144) <= 16 << 20   # the documented fit
    assert na(S=0) == 0


def test_prefill_index_topk_rejects(lib):
    c = cfg()
    n = lib.qsa_index_topk_workspace_size(ctypes.byref(c), 64, 65536)

    def pf(ws=FAKE, nbytes=n, B=2, R=64, M=32, L=65536, q=FAKE, cu=FAKE, **kw):
        return lib.qsa_prefill_index_topk(ctypes.byref(kw.get("c", c)), B, R, M, L, q, cu, FAKE, FAKE, FAKE,
                                          FAKE, ws, nbytes, None)
    assert pf(nbytes=n - 1) == 3
    assert pf(ws=None) == 3
    assert pf(ws=ctypes.c_void_p(0x10010)) == 3
    assert pf(L=_lib.QSA_MAX_SEQ_LEN + 4) == 1
    assert pf(B=-1) == 1
    assert pf(R=-1) == 1
    assert pf(R=70000) == 1
    assert pf(M=65) == 1                            # more rows per request than rows
    assert pf(q=None) == 1
    assert pf(cu=None) == 1
    assert pf(q=ctypes.c_void_p(0x10004)) == 1       # q_index not 16-byte aligned
    assert pf(c=cfg(index_dim=96)) == 2
    assert pf(c=cfg(compress_ratio=2)) == 1
    assert pf(R=0, M=0) == 0
    assert pf(B=0) == 0


def decode(lib, c, P=2, mr=1, S=4, R=None, rs=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, o=FAKE, l=FAKE)
    a.update(kw)
    R = S if R is None else R
    return lib.qsa_sparse_decode(ctypes.byref(c), R, S, mr, P, a["q"], rs, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 a["k"], a["v"], a["ks"], a["vs"], a["o"], a["l"], None)


def test_decode_rejects(lib):
    assert decode(lib, cfg(num_q_heads=15)) == 1
    assert decode(lib, cfg(head_dim=96)) == 2
    assert decode(lib, cfg(kv_dtype=7)) == 2
    assert decode(lib, cfg(softmax_scale=0.0)) == 1
    assert decode(lib, cfg(), P=0) == 1
    assert decode(lib, cfg(), P=65) == 1
    assert decode(lib, cfg(), mr=0) == 1
    assert decode(lib, cfg(), mr=9) == 2          # 8 heads x 9 rows > 64
    assert decode(lib, cfg(), R=-1) == 1
    assert decode(lib, cfg(), rs=None, R=5) == 1  # no row map: one row per selecting row
    assert decode(lib, cfg(), rs=None, mr=2) == 1
    assert decode(lib, cfg(kv_dtype=1)) == 1       # fp8 without scales
    assert decode(lib, cfg(), q=None) == 1
    assert decode(lib, cfg(), k=ctypes.c_void_p(0x10008)) == 1
    assert decode(lib, cfg(), S=0) == 0
    assert decode(lib, cfg(), R=0) == 0


def test_select_sparse_decode_rejects(lib):
    c = cfg()
    n = lib.qsa_index_topk_workspace_size(ctypes.byref(c), 4, 65536)

    def sd(c=c, S=4, R=4, mr=1, P=2, L=65536, ws=FAKE, nbytes=n, topk=FAKE, q=FAKE, ks=None, vs=None, rs=FAKE):
        return lib.qsa_select_sparse_decode(ctypes.byref(c), R, S, mr, P, L, q, rs, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, ks, vs, topk, FAKE, FAKE, ws, nbytes, None)
    assert sd(c=cfg(index_dim=96)) == 2             # the selection's config check
    assert sd(c=cfg(head_dim=96)) == 2              # the attention's
    assert sd(c=cfg(num_q_heads=15)) == 1
    assert sd(L=_lib.QSA_MAX_SEQ_LEN + 4) == 1
    assert sd(P=0) == 1
    assert sd(mr=9) == 2
    assert sd(topk=None) == 1                       # the selection is an output here
    assert sd(topk=None, R=0) == 1
    assert sd(q=None) == 1
    assert sd(c=cfg(kv_dtype=1)) == 1               # fp8 without scales
    assert sd(nbytes=n - 1) == 3
    assert sd(ws=None) == 3
    assert sd(ws=ctypes.c_void_p(0x10010)) == 3
    assert sd(S=0) == 0


def test_select_sparse_decode_reports_its_launches(lib):
    """One kernel while the grid stays under two workgroups per CU, the rows'
    selection bitmaps fit the LDS and a row's heads fit a workgroup (8 at
    head_dim 128, 16 at 64); else the finalize and the attention."""
    c = cfg()   # 16 query heads over 2 KV heads: 8 heads per row
    f = lambda S, mr, P, L, c=c: lib.qsa_select_sparse_decode_launches(ctypes.byref(c), S, mr, P, L)
    assert f(8, 1, 16, 262144) == 1                 # 16 x 2 x 8 = 256 workgroups
    assert f(8, 1, 32, 262144) == 2                 # 512 workgroups
    assert f(128, 1, 1, 262144) == 1                # the mixed batch: 256
    assert f(4, 4, 8, 1000003) == 1                 # 4 rows x 8 heads: 4 row groups, 256 workgroups
    assert f(4, 4, 16, 1000003) == 2                # 512 workgroups
    assert f(4, 1, 2, 1200000) == 2                 # rows past 262,144 blocks: the bitmap is in the workspace
    assert f(4, 1, 2, 100, cfg(num_q_heads=16, num_kv_heads=1)) == 2   # 16 heads of one row at d = 128
    assert f(4, 1, 2, 100, cfg(num_q_heads=16, num_kv_heads=1, head_dim=64)) == 1
    assert f(0, 1, 2, 100) == 0 and f(4, 9, 2, 100) == 0


def test_merge_rejects(lib):
    assert lib.qsa_merge_partials(0, 4, 16, 128, FAKE, FAKE, FAKE, 0, FAKE, None) == 1
    assert lib.qsa_merge_partials(65, 4, 16, 128, FAKE, FAKE, FAKE, 0, FAKE, None) == 1
    assert lib.qsa_merge_partials(2, 4, 16, 96, FAKE, FAKE, FAKE, 0, FAKE, None) == 2
    assert lib.qsa_merge_partials(2, 4, 16, 128, None, FAKE, FAKE, 0, FAKE, None) == 1
    assert lib.qsa_merge_partials(2, 4, 16, 128, FAKE, FAKE, FAKE, 2, FAKE, None) == 1
    assert lib.qsa_merge_partials(2, 0, 16, 128, None, None, None, 1, None, None) == 0


def test_python_binding_raises_with_message():
    from block_sparse_attention_qsa_amd import api
    bad = api.QSAConfig(16, 2, 128, 64, 512, 48, 10)
    with pytest.raises(api.QSAError, match="page_size"):
        api._check(_lib.load().qsa_compress(ctypes.byref(bad.to_c()), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, None))


def test_indexer_project_rejects(lib):
    n = lib.qsa_indexer_project_workspace_size(8, 256, 64)
    assert n > 0 and lib.qsa_indexer_project_workspace_size(8, 48, 64) == 0
    assert lib.qsa_indexer_project_workspace_size(8, 256, 96) == 0

    def fe(T=8, H=256, D=64, h=FAKE, w=FAKE, base=10000.0, qs=32.0, ks=32.0, q=FAKE, k=FAKE, ws=FAKE, nbytes=n):
        return lib.qsa_indexer_project(T, H, D, h, FAKE, w, FAKE, FAKE, base, qs, ks, q, k, ws, nbytes, None)
    assert fe(ws=None) == 3
    assert fe(nbytes=n - 1) == 3
    assert fe(ws=ctypes.c_void_p(0x10004)) == 3
    assert fe(T=-1) == 1
    assert fe(H=48) == 1              # not a multiple of 32
    assert fe(H=0) == 1
    assert fe(D=48) == 2
    assert fe(base=1.0) == 1
    assert fe(qs=0.0) == 1
    assert fe(ks=float("nan")) == 1
    assert fe(h=None) == 1
    assert fe(w=ctypes.c_void_p(0x10008)) == 1   # weights not 16-byte aligned
    assert fe(q=ctypes.c_void_p(0x10002)) == 1
    assert fe(T=0) == 0


def test_indexer_project_mrope_rejects(lib):
    n = lib.qsa_indexer_project_workspace_size(8, 256, 64)

    def fe(T=8, D=64, sec=(8, 12, 12), ws=FAKE, nbytes=n, base=10000.0):
        return lib.qsa_indexer_project_mrope(T, 256, D, FAKE, FAKE, sec[0], sec[1], sec[2], FAKE, FAKE, FAKE, base,
                                             32.0, 32.0, FAKE, FAKE, ws, nbytes, None)
    assert fe(sec=(8, 12, 11)) == 1       # sections must sum to D/2
    assert fe(sec=(-1, 17, 16)) == 1
    assert fe(D=128) == 1                 # 8 + 12 + 12 != 64
    assert fe(D=128, sec=(16, 24, 24), nbytes=n) == 3    # a D=128 workspace is larger
    assert fe(ws=None) == 3
    assert fe(base=0.5) == 1
    assert fe(T=-1) == 1
    assert fe(T=0) == 0



def test_compress_index_topk_rejects(lib):
    c = cfg()
    n = lib.qsa_index_topk_workspace_size(ctypes.byref(c), 8, 65536)

    def ci(B=4, mx=1, S=8, L=65536, keys=FAKE, ring=FAKE, q=FAKE, ws=FAKE, nbytes=n, **kw):
        return lib.qsa_compress_index_topk(ctypes.byref(kw.get("c", c)), B, mx, keys, FAKE, FAKE, ring, S, L, q,
                                           FAKE, FAKE, FAKE, FAKE, FAKE, ws, nbytes, None)
    assert ci(mx=6) == 1                              # longer appends: the two separate calls
    assert ci(mx=-1) == 1
    assert ci(B=-1) == 1
    assert ci(S=-1) == 1
    assert ci(L=_lib.QSA_MAX_SEQ_LEN + 4) == 1
    assert ci(keys=None) == 1
    assert ci(ring=ctypes.c_void_p(0x10002)) == 1     # ring not 4-byte aligned
    assert ci(keys=ctypes.c_void_p(0x10001)) == 1
    assert ci(q=None) == 1
    assert ci(nbytes=n - 1) == 3
    assert ci(ws=None) == 3
    assert ci(c=cfg(index_dim=96)) == 2
    assert ci(B=0, S=0) == 0
