"""ctypes binding of liblsa.so: same names as the C entry points, torch tensors in.

Argument marshalling only: every step runs in the HIP kernels of liblsa.so.
Tensors must live on the current HIP device; work is enqueued on the current
torch stream unless `stream` (a torch.cuda.Stream) is given.  There is no
fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsa.so")

LSA_OK = 0
LSA_ERR_INVALID_ARG = -1
LSA_ERR_UNSUPPORTED = -2
LSA_ERR_WORKSPACE = -3
LSA_ERR_HIP = -4
LSA_DTYPE_F32 = 0
LSA_DTYPE_BF16 = 1
LSA_OP_SELECT = 1
LSA_OP_TOPK = 2
LSA_OP_ATTEND = 3

EXPORTED = ["lsa_query_encode", "lsa_index_score", "lsa_index_score_union", "lsa_index_rescore",
            "lsa_select_compact", "lsa_select_compact_noalloc", "lsa_topk", "lsa_fetch_rows",
            "lsa_sparse_attend", "lsa_sparse_attend_hca", "lsa_sparse_attend_selected",
            "lsa_workspace_bytes", "lsa_status_string", "lsa_last_error", "lsa_version"]


class LSAError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str):
        super().__init__(f"{call} failed with status {status}: {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load liblsa.so (built by lookahead_sparse_kv_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m lookahead_sparse_kv_amd.build`"
                           " (the HIP library has no fallback)")
    lib = ctypes.CDLL(path)
    P, I, L, F, Z = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                     ctypes.c_size_t)
    lib.lsa_index_score.argtypes = [P, I, P, P, P, I, I, I, I, L, P, P, F, I, P, P, P, F, P]
    lib.lsa_index_score_union.argtypes = [I, P, I, P, P, P, I, I, I, I, L, P, P, P, P, P, P, F, P]
    lib.lsa_index_rescore.argtypes = [P, I, P, P, P, P, P, I, I, I, L, P, P, P, P]
    lib.lsa_select_compact.argtypes = [P, P, P, P, I, L, F, P, P, P, Z, P]
    lib.lsa_select_compact_noalloc.argtypes = [P, P, P, I, L, F, P, P, P]
    lib.lsa_topk.argtypes = [P, P, P, I, L, P, P, I, P, P, I, P, Z, P]
    lib.lsa_fetch_rows.argtypes = [P, L, P, P, P, P, I, L, P, P, P]
    lib.lsa_query_encode.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P, P]
    lib.lsa_sparse_attend.argtypes = [P, I, I, I, I, I, P, P, P, P, I, P, P, P, L, F, P, P, P, Z, P]
    lib.lsa_sparse_attend_selected.argtypes = lib.lsa_sparse_attend.argtypes
    lib.lsa_sparse_attend_hca.argtypes = [P, I, I, I, I, I, I, P, P, P, L, F, P, Z, P]
    lib.lsa_workspace_bytes.argtypes = [I, I, I, I, I, L, I, L]
    lib.lsa_workspace_bytes.restype = Z
    lib.lsa_status_string.argtypes = [I]
    lib.lsa_status_string.restype = ctypes.c_char_p
    lib.lsa_last_error.argtypes = []
    lib.lsa_last_error.restype = ctypes.c_char_p
    lib.lsa_version.argtypes = []
    lib.lsa_version.restype = I
    for name in ("lsa_index_score", "lsa_index_rescore", "lsa_select_compact",
                 "lsa_select_compact_noalloc", "lsa_topk",
                 "lsa_fetch_rows", "lsa_query_encode",
                 "lsa_sparse_attend", "lsa_sparse_attend_hca", "lsa_sparse_attend_selected"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _check(call: str, rc: int):
    if rc != LSA_OK:
        lib = load_library()
        raise LSAError(call, rc, lib.lsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LSA_DTYPE_BF16
    if t.dtype == torch.float32:
        return LSA_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def lsa_workspace_bytes(op: int, B: int, T: int = 0, Hq: int = 0, Dl: int = 0, max_len: int = 0,
                        k: int = 0, max_hca: int = 0) -> int:
    return int(load_library().lsa_workspace_bytes(op, B, T, Hq, Dl, max_len, k, max_hca))


def lsa_version() -> int:
    return int(load_library().lsa_version())


def lsa_gate_words(max_len: int) -> int:
    """uint16 words per sequence row of the gate bits (include/lsa.h)."""
    return (int(max_len) + 127) // 128 * 8


def _gate_buf(gate_bits, B: int, max_len: int):
    if gate_bits is None:
        return None
    _dev(gate_bits, "gate_bits", torch.int16)
    if gate_bits.numel() < B * lsa_gate_words(max_len):
        raise ValueError(f"gate_bits needs {B} x {lsa_gate_words(max_len)} int16 words")
    return gate_bits


def lsa_index_score(keys, key_row_start, seq_len, entry_start, max_len: int, q, w, bias: float,
                    reduce_max=False, z_out=None, prob_out=None, gate_bits=None,
                    gate_threshold: float = 0.0, stream=None):
    """Score every entry (see include/lsa.h).  q: [B, T, H, D], w: [B, T, H].

    reduce_max: False/0 per position, True/1 max over positions, 2 OR-union
    with the indexers already in z_out.  gate_bits: int16 [B, lsa_gate_words(
    max_len)] (the words are bit sets), filled with the gate against
    gate_threshold in the same launch."""
    lib = load_library()
    B, T, H, D = q.shape
    _dev(keys, "keys")
    _dev(q, "q", keys.dtype)
    _dev(w, "w", torch.float32)
    _dev(key_row_start, "key_row_start", torch.int64)
    _dev(seq_len, "seq_len", torch.int32)
    _dev(entry_start, "entry_start", torch.int64)
    if z_out is None:
        raise ValueError("z_out must be preallocated (its size depends on entry_start)")
    _dev(z_out, "z_out", torch.float32)
    if prob_out is not None:
        _dev(prob_out, "prob_out", torch.float32)
    gate_bits = _gate_buf(gate_bits, B, max_len)
    rc = lib.lsa_index_score(_ptr(keys), _dtype_code(keys), _ptr(key_row_start), _ptr(seq_len),
                             _ptr(entry_start), B, T, H, D, int(max_len), _ptr(q), _ptr(w),
                             float(bias), int(reduce_max), _ptr(z_out), _ptr(prob_out),
                             _ptr(gate_bits), float(gate_threshold), _stream(stream))
    _check("lsa_index_score", rc)
    return z_out, prob_out


def lsa_index_score_union(keys, key_row_start, seq_len, entry_start, max_len: int, qs, ws,
                          biases, z_out, prob_out=None, gate_bits=None,
                          gate_threshold: float = 0.0, stream=None):
    """OR-union over indexers (see include/lsa.h): keys, qs, ws and biases are
    sequences with one entry per indexer; q: [B, T, H, D], w: [B, T, H]."""
    lib = load_library()
    n = len(keys)
    if not (len(qs) == len(ws) == len(biases) == n):
        raise ValueError("keys, qs, ws and biases need one entry per indexer")
    B, T, H, D = qs[0].shape
    for k, q, w in zip(keys, qs, ws):
        _dev(k, "keys", keys[0].dtype)
        _dev(q, "q", keys[0].dtype)
        _dev(w, "w", torch.float32)
        if tuple(q.shape) != (B, T, H, D) or tuple(w.shape) != (B, T, H):
            raise ValueError("every indexer needs q [B, T, H, D] and w [B, T, H] of one shape")
        if k.dim() != 2 or k.shape[1] != D:
            raise ValueError("keys must be [rows, D]")
    _dev(key_row_start, "key_row_start", torch.int64)
    _dev(seq_len, "seq_len", torch.int32)
    _dev(entry_start, "entry_start", torch.int64)
    _dev(z_out, "z_out", torch.float32)
    if prob_out is not None:
        _dev(prob_out, "prob_out", torch.float32)
    arr = ctypes.c_void_p * n
    kp = arr(*(k.data_ptr() for k in keys))
    qp = arr(*(q.data_ptr() for q in qs))
    wp = arr(*(w.data_ptr() for w in ws))
    bp = (ctypes.c_float * n)(*(float(b) for b in biases))
    gate_bits = _gate_buf(gate_bits, B, max_len)
    rc = lib.lsa_index_score_union(n, kp, _dtype_code(keys[0]), _ptr(key_row_start),
                                   _ptr(seq_len), _ptr(entry_start), B, T, H, D, int(max_len), qp,
                                   wp, bp, _ptr(z_out), _ptr(prob_out), _ptr(gate_bits),
                                   float(gate_threshold), _stream(stream))
    _check("lsa_index_score_union", rc)
    return z_out, prob_out


def lsa_index_rescore(keys, key_row_start, seq_len, entry_start, cand_idx, cand_count,
                      max_cand: int, q, w, r_out, stream=None):
    """Native re-score of each sequence's candidates (see include/lsa.h).
    q: [B, H, D], w: [B, H]; r_out is entry-indexed fp32."""
    lib = load_library()
    B, H, D = q.shape
    _dev(keys, "keys")
    _dev(q, "q", keys.dtype)
    _dev(w, "w", torch.float32)
    _dev(key_row_start, "key_row_start", torch.int64)
    _dev(seq_len, "seq_len", torch.int32)
    _dev(entry_start, "entry_start", torch.int64)
    _dev(cand_idx, "cand_idx", torch.int32)
    _dev(cand_count, "cand_count", torch.int32)
    _dev(r_out, "r_out", torch.float32)
    rc = lib.lsa_index_rescore(_ptr(keys), _dtype_code(keys), _ptr(key_row_start), _ptr(seq_len),
                               _ptr(entry_start), _ptr(cand_idx), _ptr(cand_count), B, H, D,
                               int(max_cand), _ptr(q), _ptr(w), _ptr(r_out), _stream(stream))
    _check("lsa_index_rescore", rc)
    return r_out


def lsa_select_compact(z, entry_start, seq_len, max_len: int, cand_idx, cand_count, workspace,
                       threshold: float = 0.0, stream=None, gate_bits=None):
    """Ascending list of kept entries (see include/lsa.h): from the logits z, or,
    with gate_bits (written by lsa_index_score), from the bits alone (z, the
    threshold and the workspace are then unused and may be None)."""
    lib = load_library()
    B = seq_len.numel()
    if gate_bits is None:
        _dev(z, "z", torch.float32)
    else:
        gate_bits = _gate_buf(gate_bits, B, max_len)
        if z is not None:
            _dev(z, "z", torch.float32)
    _dev(cand_idx, "cand_idx", torch.int32)
    _dev(cand_count, "cand_count", torch.int32)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.lsa_select_compact(_ptr(z), _ptr(gate_bits), _ptr(entry_start), _ptr(seq_len), B,
                                int(max_len), float(threshold), _ptr(cand_idx), _ptr(cand_count),
                                _ptr(workspace), ws_bytes, _stream(stream))
    _check("lsa_select_compact", rc)
    return cand_idx, cand_count


def lsa_select_compact_noalloc(z, entry_start, seq_len, max_len: int, cand_idx, cand_count,
                               threshold: float = 0.0, stream=None):
    """lsa_select_compact with the library's built-in scratch instead of a workspace."""
    lib = load_library()
    _dev(z, "z", torch.float32)
    _dev(cand_idx, "cand_idx", torch.int32)
    _dev(cand_count, "cand_count", torch.int32)
    B = seq_len.numel()
    rc = lib.lsa_select_compact_noalloc(_ptr(z), _ptr(entry_start), _ptr(seq_len), B,
                                        int(max_len), float(threshold), _ptr(cand_idx),
                                        _ptr(cand_count), _stream(stream))
    _check("lsa_select_compact_noalloc", rc)
    return cand_idx, cand_count


def lsa_topk(rank_key, entry_start, seq_len, max_len: int, cand_idx, cand_count, k: int,
             topk_idx, topk_count, workspace=None, stream=None, out_positions: bool = False):
    """Top-k of each candidate list (see include/lsa.h); entry indices, or with
    out_positions the positions in the candidate list."""
    lib = load_library()
    _dev(rank_key, "rank_key", torch.float32)
    _dev(topk_idx, "topk_idx", torch.int32)
    _dev(topk_count, "topk_count", torch.int32)
    B = seq_len.numel()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.lsa_topk(_ptr(rank_key), _ptr(entry_start), _ptr(seq_len), B, int(max_len),
                      _ptr(cand_idx), _ptr(cand_count), int(k), _ptr(topk_idx), _ptr(topk_count),
                      1 if out_positions else 0, _ptr(workspace), ws_bytes, _stream(stream))
    _check("lsa_topk", rc)
    return topk_idx, topk_count


def lsa_query_encode(h, w_down, w_up, w_gate, H: int, D: int, c_buf, q_out, w_out, stream=None):
    """Memory-Indexer query encoder (see include/lsa.h): h [M, d_model] bf16 to the
    score's q [M, H, D] bf16 and w [M, H] fp32, through the rank-r latent c_buf."""
    lib = load_library()
    for t, n in ((h, "h"), (w_down, "w_down"), (w_up, "w_up"), (w_gate, "w_gate"),
                 (c_buf, "c_buf"), (q_out, "q_out")):
        _dev(t, n, torch.bfloat16)
    _dev(w_out, "w_out", torch.float32)
    M, d_model = h.shape
    rank = w_down.shape[0]
    if (w_down.shape != (rank, d_model) or w_up.shape != (H * D, rank)
            or w_gate.shape != (H, d_model)):
        raise ValueError("lsa_query_encode: weight shapes do not match h, H and D")
    if c_buf.numel() < M * rank or q_out.numel() < M * H * D or w_out.numel() < M * H:
        raise ValueError("lsa_query_encode: an output buffer is too small")
    rc = lib.lsa_query_encode(_ptr(h), M, d_model, rank, int(H), int(D), _ptr(w_down), _ptr(w_up),
                              _ptr(w_gate), _ptr(c_buf), _ptr(q_out), _ptr(w_out), _stream(stream))
    _check("lsa_query_encode", rc)
    return q_out, w_out


def lsa_fetch_rows(src, src_row_start, idx, idx_start, count, max_count: int, dst, dst_row_start,
                   stream=None):
    """Copy rows src[src_row_start[b] + idx[idx_start[b] + j]] to dst[dst_row_start[b] + j]
    (see include/lsa.h).  src: a pinned host tensor or a device tensor; dst: device."""
    lib = load_library()
    if not (src.is_cuda or src.is_pinned()):
        raise ValueError("src must be a device tensor or pinned host memory")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _dev(dst, "dst", src.dtype)
    for t, n in ((src_row_start, "src_row_start"), (idx_start, "idx_start"),
                 (dst_row_start, "dst_row_start")):
        _dev(t, n, torch.int64)
    _dev(idx, "idx", torch.int32)
    _dev(count, "count", torch.int32)
    row_bytes = src.shape[-1] * src.element_size()
    if dst.shape[-1] * dst.element_size() != row_bytes:
        raise ValueError("src and dst rows differ in size")
    B = count.numel()
    rc = lib.lsa_fetch_rows(_ptr(src), int(row_bytes), _ptr(src_row_start), _ptr(idx),
                            _ptr(idx_start), _ptr(count), B, int(max_count), _ptr(dst),
                            _ptr(dst_row_start), _stream(stream))
    _check("lsa_fetch_rows", rc)
    return dst


def lsa_sparse_attend(qa, latent, latent_row_start, topk_idx, topk_count, k: int, out,
                      hca=None, hca_row_start=None, hca_count=None, max_hca: int = 0,
                      scale: Optional[float] = None, lse=None, workspace=None, stream=None,
                      _entry: str = "lsa_sparse_attend"):
    lib = load_library()
    B, T, Hq, Dl = qa.shape
    _dev(qa, "qa")
    _dev(latent, "latent", qa.dtype)
    _dev(out, "out", qa.dtype)
    if hca is not None:
        _dev(hca, "hca", qa.dtype)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if scale is None:
        scale = Dl ** -0.5
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = getattr(lib, _entry)(_ptr(qa), _dtype_code(qa), B, T, Hq, Dl, _ptr(latent),
                              _ptr(latent_row_start), _ptr(topk_idx), _ptr(topk_count), int(k),
                              _ptr(hca), _ptr(hca_row_start), _ptr(hca_count), int(max_hca),
                              float(scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                              _stream(stream))
    _check(_entry, rc)
    return out, lse


def lsa_sparse_attend_hca(qa, k: int, hca, hca_row_start, hca_count, max_hca: int,
                          scale: Optional[float] = None, workspace=None, stream=None):
    """First phase of lsa_sparse_attend: the HCA rows' split partials into workspace."""
    lib = load_library()
    B, T, Hq, Dl = qa.shape
    _dev(qa, "qa")
    if hca is not None:
        _dev(hca, "hca", qa.dtype)
    if scale is None:
        scale = Dl ** -0.5
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.lsa_sparse_attend_hca(_ptr(qa), _dtype_code(qa), B, T, Hq, Dl, int(k), _ptr(hca),
                                   _ptr(hca_row_start), _ptr(hca_count), int(max_hca),
                                   float(scale), _ptr(workspace), ws_bytes, _stream(stream))
    _check("lsa_sparse_attend_hca", rc)


def lsa_sparse_attend_selected(qa, latent, latent_row_start, topk_idx, topk_count, k: int, out,
                               hca=None, hca_row_start=None, hca_count=None, max_hca: int = 0,
                               scale: Optional[float] = None, lse=None, workspace=None,
                               stream=None):
    """Second phase: the top-k rows and the merge (after lsa_sparse_attend_hca)."""
    return lsa_sparse_attend(qa, latent, latent_row_start, topk_idx, topk_count, k, out, hca,
                             hca_row_start, hca_count, max_hca, scale, lse, workspace, stream,
                             _entry="lsa_sparse_attend_selected")
