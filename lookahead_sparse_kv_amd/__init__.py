"""Lookahead Sparse Attention hot path for MI355X (gfx950).

The compute lives in liblsa.so (HIP kernels behind a C ABI, include/lsa.h);
`binding` marshals torch tensors into it, `pipeline` chains the four calls,
`inputs` draws seeded synthetic workloads.
"""
from .binding import (LSAError, load_library, lsa_index_score, lsa_select_compact,  # noqa: F401
                      lsa_sparse_attend, lsa_topk, lsa_version, lsa_workspace_bytes)

__all__ = ["LSAError", "load_library", "lsa_index_score", "lsa_select_compact", "lsa_topk",
           "lsa_sparse_attend", "lsa_workspace_bytes", "lsa_version"]
