"""ctypes front end of the plain CPU reference (liblsa_oracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of bench.py, never by the product package.  Every function
widens its inputs exactly and computes in IEEE double precision (see
lsa_oracle.c for the definitions and their citations).

Arrays are numpy; bf16 tensors are carried as their raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblsa_oracle.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1


_LIB_MT_PATH = os.path.join(_HERE, "liblsa_oracle_omp.so")
_CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra"]


def _stale(lib: str) -> bool:
    return not os.path.exists(lib) or os.path.getmtime(lib) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "lsa_oracle.h")))


# LSA_ORACLE_SANITIZE=1 swaps the single-threaded build for one instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (the process must preload the
# ASan runtime); the sanitizer test runs the pins against it in a subprocess.
_SANITIZE = os.environ.get("LSA_ORACLE_SANITIZE") == "1"
if _SANITIZE:
    _LIB_PATH = os.path.join(_HERE, "liblsa_oracle_asan.so")


def build(force: bool = False) -> str:
    """Compile the oracle with plain gcc (no fast-math, no FMA contraction), twice:
    single-threaded (the OpenMP pragmas ignored) and with -fopenmp.  Both builds
    run the same scalar operations per output element; the second only shares
    out independent iterations among threads."""
    single = ["-Wno-unknown-pragmas"]
    if _SANITIZE:
        single += ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   "-fno-omit-frame-pointer", "-g"]
    for lib, extra in ((_LIB_PATH, single), (_LIB_MT_PATH, ["-fopenmp"])):
        if force or _stale(lib):
            tmp = lib + ".tmp"
            subprocess.check_call(["gcc"] + _CFLAGS + extra + ["-o", tmp, _SRC, "-lm"])
            os.replace(tmp, lib)
    return _LIB_PATH


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.lsa_ref_index_score.argtypes = [P, I, P, P, P, I, I, I, I, P, P, D, I, P, P]
    lib.lsa_ref_select.argtypes = [P, P, P, I, D, P, P]
    lib.lsa_ref_topk.argtypes = [P, P, P, I, P, P, I, I, P, P]
    lib.lsa_ref_fetch_rows.argtypes = [P, ctypes.c_int64, P, P, P, P, I, P, P]
    lib.lsa_ref_query_encode.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P]
    lib.lsa_ref_sparse_attend.argtypes = [P, I, I, I, I, I, P, P, P, P, I, P, P, P, D, P, P]
    lib.lsa_ref_index_rescore.argtypes = [P, I, P, P, P, P, I, I, I, P, P, P]
    lib.lsa_ref_max_threads.argtypes = []
    lib.lsa_ref_max_threads.restype = ctypes.c_int
    for f in (lib.lsa_ref_index_score, lib.lsa_ref_select, lib.lsa_ref_topk,
              lib.lsa_ref_sparse_attend, lib.lsa_ref_index_rescore, lib.lsa_ref_fetch_rows,
              lib.lsa_ref_query_encode):
        f.restype = ctypes.c_int
    return lib


_default_lib = None
_mt_lib = None
_lib_override = None
_threaded = False


def _load():
    """The compiled reference: the single-threaded build, or the OpenMP build inside
    `with threads():`; tests may point it at another build with use_library()."""
    global _default_lib, _mt_lib
    if _lib_override is not None:
        return _lib_override
    if _threaded:
        if _mt_lib is None:
            build()
            _mt_lib = _bind(_LIB_MT_PATH)
        return _mt_lib
    if _default_lib is None:
        build()
        _default_lib = _bind(_LIB_PATH)
    return _default_lib


class threads:
    """Context manager: calls inside it run on the OpenMP build (all cores, or
    OMP_NUM_THREADS).  Results are bit-identical to the single-threaded build."""

    def __enter__(self):
        global _threaded
        self._prev = _threaded
        _threaded = True
        return self

    def __exit__(self, *exc):
        global _threaded
        _threaded = self._prev
        return False


def max_threads() -> int:
    """Threads the currently selected build may use (1 for the single-threaded one)."""
    return int(_load().lsa_ref_max_threads())


def use_library(path):
    """Route every call below to the library at `path` (None restores the default).

    Used by the mutation tests, which compile altered copies of lsa_oracle.c and
    check that the pins reject them."""
    global _lib_override
    _lib_override = None if path is None else _bind(path)


def compile_variant(src_text: str, out_dir: str, name: str) -> str:
    """Compile C source text (an altered copy of lsa_oracle.c) next to the header."""
    import shutil
    src = os.path.join(out_dir, name + ".c")
    with open(src, "w") as f:
        f.write(src_text)
    shutil.copy(os.path.join(_HERE, "lsa_oracle.h"), os.path.join(out_dir, "lsa_oracle.h"))
    so = os.path.join(out_dir, "lib" + name + ".so")
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-w", "-o", so, src, "-lm"])
    return so


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _dtype_code(a) -> int:
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected the arguments (rc={rc})")


def index_score(keys, key_row_start, seq_len, entry_start, q, w, bias, reduce_max=False,
                want_prob=True, union_with=None):
    """O1: z (and sigmoid) per (b,t,s), or the max over t when reduce_max.

    union_with (implies reduce_max): the union logits of other indexers; the
    result is their elementwise max with this indexer's max over t (OR-mode)."""
    lib = _load()
    keys = np.ascontiguousarray(keys)
    q = np.ascontiguousarray(q)
    dt = _dtype_code(keys)
    assert _dtype_code(q) == dt, "q and keys must share a dtype"
    B, T, H, D = q.shape
    assert keys.shape[1] == D
    key_row_start = _c(key_row_start, np.int64)
    seq_len = _c(seq_len, np.int32)
    entry_start = _c(entry_start, np.int64)
    w = _c(w, np.float32)
    assert w.shape == (B, T, H)
    mode = 2 if union_with is not None else (1 if reduce_max else 0)
    n_out = int(max(int(entry_start[b]) + int(seq_len[b]) for b in range(B)))
    n_out = n_out * (1 if mode else T)
    if union_with is not None:
        z = np.array(union_with, dtype=np.float64, copy=True)
        assert z.shape == (n_out,)
    else:
        z = np.full(n_out, np.nan, dtype=np.float64)
    prob = np.full(n_out, np.nan, dtype=np.float64) if want_prob else None
    rc = lib.lsa_ref_index_score(_ptr(keys), dt, _ptr(key_row_start), _ptr(seq_len),
                                 _ptr(entry_start), B, T, H, D, _ptr(q), _ptr(w), float(bias),
                                 mode, _ptr(z), _ptr(prob))
    _check(rc, "index_score")
    return z, prob


def index_rescore(keys, key_row_start, entry_start, cand_idx, cand_count, q, w, r_init=None):
    """O1b: native re-score of each sequence's candidates (no bias, no sigmoid),
    scattered to r[entry_start[b] + s]; other elements keep r_init (NaN by default)."""
    lib = _load()
    keys = np.ascontiguousarray(keys)
    q = np.ascontiguousarray(q)
    dt = _dtype_code(keys)
    assert _dtype_code(q) == dt, "q and keys must share a dtype"
    B, H, D = q.shape
    assert keys.shape[1] == D
    key_row_start = _c(key_row_start, np.int64)
    entry_start = _c(entry_start, np.int64)
    cand_idx = _c(cand_idx, np.int32)
    cand_count = _c(cand_count, np.int32)
    w = _c(w, np.float32)
    assert w.shape == (B, H)
    n = len(cand_idx)
    r = np.full(n, np.nan, np.float64) if r_init is None else np.array(r_init, np.float64)
    rc = lib.lsa_ref_index_rescore(_ptr(keys), dt, _ptr(key_row_start), _ptr(entry_start),
                                   _ptr(cand_idx), _ptr(cand_count), B, H, D, _ptr(q), _ptr(w),
                                   _ptr(r))
    _check(rc, "index_rescore")
    return r


def select(z, entry_start, seq_len, threshold=0.0):
    """O2: ascending candidate lists of entries with z >= threshold."""
    lib = _load()
    z = _c(z, np.float64)
    entry_start = _c(entry_start, np.int64)
    seq_len = _c(seq_len, np.int32)
    B = len(seq_len)
    cand_idx = np.full(len(z), -1, dtype=np.int32)
    cand_count = np.zeros(B, dtype=np.int32)
    rc = lib.lsa_ref_select(_ptr(z), _ptr(entry_start), _ptr(seq_len), B, float(threshold),
                            _ptr(cand_idx), _ptr(cand_count))
    _check(rc, "select")
    return cand_idx, cand_count


def topk(r, entry_start, seq_len, cand_idx, cand_count, k, positions=False):
    """O3: top-k (rank key descending, ties to the smaller index), ascending; entry
    indices, or with positions the positions in the candidate list."""
    lib = _load()
    r = _c(r, np.float64)
    entry_start = _c(entry_start, np.int64)
    seq_len = _c(seq_len, np.int32)
    cand_idx = _c(cand_idx, np.int32)
    cand_count = _c(cand_count, np.int32)
    B = len(seq_len)
    guard = 64                     # a write past B*k entries lands here and is reported
    buf = np.full(B * k + guard, -1, dtype=np.int32)
    topk_count = np.zeros(B, dtype=np.int32)
    rc = lib.lsa_ref_topk(_ptr(r), _ptr(entry_start), _ptr(seq_len), B, _ptr(cand_idx),
                          _ptr(cand_count), int(k), 1 if positions else 0, _ptr(buf),
                          _ptr(topk_count))
    _check(rc, "topk")
    if np.any(buf[B * k:] != -1):
        raise ValueError("topk wrote past its B*k outputs")
    return buf[:B * k].reshape(B, k), topk_count


def sparse_attend(qa, latent, latent_row_start, topk_idx, topk_count, k, hca=None,
                  hca_row_start=None, hca_count=None, scale=None):
    """O4: attention over the top-k latent rows followed by every HCA row."""
    lib = _load()
    qa = np.ascontiguousarray(qa)
    latent = np.ascontiguousarray(latent)
    dt = _dtype_code(qa)
    assert _dtype_code(latent) == dt
    B, T, Hq, Dl = qa.shape
    if scale is None:
        scale = 1.0 / np.sqrt(Dl)
    latent_row_start = _c(latent_row_start, np.int64)
    topk_idx = _c(topk_idx, np.int32).reshape(-1)
    topk_count = _c(topk_count, np.int32)
    assert topk_idx.size == B * k
    if hca is not None:
        hca = np.ascontiguousarray(hca)
        assert _dtype_code(hca) == dt
        hca_row_start = _c(hca_row_start, np.int64)
        hca_count = _c(hca_count, np.int32)
    out = np.zeros((B, T, Hq, Dl), dtype=np.float64)
    lse = np.zeros((B, T, Hq), dtype=np.float64)
    rc = lib.lsa_ref_sparse_attend(_ptr(qa), dt, B, T, Hq, Dl, _ptr(latent),
                                   _ptr(latent_row_start), _ptr(topk_idx), _ptr(topk_count),
                                   int(k), _ptr(hca), _ptr(hca_row_start), _ptr(hca_count),
                                   float(scale), _ptr(out), _ptr(lse))
    _check(rc, "sparse_attend")
    return out, lse


def query_encode(h, w_down, w_up, w_gate, H, D):
    """O0: c = W_down h, q[h] = W_up[h] c, w[h] = W_gate[h] . h per token (fp64).
    h [M, d_model]; returns c [M, r], q [M, H, D], w [M, H]."""
    lib = _load()
    h = np.ascontiguousarray(h)
    w_down, w_up, w_gate = (np.ascontiguousarray(a) for a in (w_down, w_up, w_gate))
    dt = _dtype_code(h)
    assert all(_dtype_code(a) == dt for a in (w_down, w_up, w_gate))
    M, dm = h.shape
    r = w_down.shape[0]
    assert w_down.shape == (r, dm) and w_up.shape == (H * D, r) and w_gate.shape == (H, dm)
    c = np.zeros((M, r))
    q = np.zeros((M, H, D))
    w = np.zeros((M, H))
    rc = lib.lsa_ref_query_encode(_ptr(h), dt, M, dm, r, H, D, _ptr(w_down), _ptr(w_up),
                                  _ptr(w_gate), _ptr(c), _ptr(q), _ptr(w))
    _check(rc, "query_encode")
    return c, q, w


def fetch_rows(src, src_row_start, idx, idx_start, count, dst_rows, dst_row_start, dst_init=None):
    """O5: rows src[src_row_start[b] + idx[idx_start[b] + j]] copied to
    dst[dst_row_start[b] + j]; dst has dst_rows rows (dst_init, else zeros)."""
    lib = _load()
    src = np.ascontiguousarray(src)
    row_shape = src.shape[1:]
    dst = (np.zeros((dst_rows,) + row_shape, src.dtype) if dst_init is None
           else np.array(dst_init, dtype=src.dtype, copy=True))
    assert dst.shape == (dst_rows,) + row_shape
    row_bytes = int(src.itemsize * int(np.prod(row_shape)))
    count = _c(count, np.int32)
    rc = lib.lsa_ref_fetch_rows(_ptr(src), row_bytes, _ptr(_c(src_row_start, np.int64)),
                                _ptr(_c(idx, np.int32)), _ptr(_c(idx_start, np.int64)),
                                _ptr(count), len(count), _ptr(dst),
                                _ptr(_c(dst_row_start, np.int64)))
    _check(rc, "fetch_rows")
    return dst


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)
