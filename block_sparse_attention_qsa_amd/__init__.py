"""QSA (Qwen Sparse Attention) decode path for MI355X (gfx950).

libqsa.so (hand-written HIP kernels behind a C ABI, include/qsa.h) does the
work; this package is its thin binding (api), a per-layer driver (pipeline)
and seeded synthetic workloads (workloads).  Importing the package does not
load the library; the first call does, and fails loudly if it is not built.
"""
from .api import (QSAConfig, QSAError, ckey_cache_bytes, qsa_compress, qsa_compress_index_topk, qsa_index_topk,
                  qsa_index_topk_workspace_init, qsa_index_topk_workspace_size,
                  qsa_indexer_project, qsa_indexer_project_workspace_size, qsa_merge_partials, qsa_prefill_index_topk,
                  qsa_select_sparse_decode, qsa_sparse_decode)

__all__ = ["QSAConfig", "QSAError", "ckey_cache_bytes", "qsa_compress", "qsa_compress_index_topk", "qsa_index_topk",
           "qsa_index_topk_workspace_init", "qsa_index_topk_workspace_size", "qsa_merge_partials",
           "qsa_indexer_project", "qsa_indexer_project_workspace_size", "qsa_prefill_index_topk",
           "qsa_select_sparse_decode", "qsa_sparse_decode"]
