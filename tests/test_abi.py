"""The C-ABI library loads, exports what include/lsa.h declares, and rejects bad arguments on
the host before touching a GPU (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

from lookahead_sparse_kv_amd import binding

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "lsa.h")

FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"static inline[^{]*\{[^}]*\}", "", text)    # header-only helpers
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("liblsa.so is not built; run python -m lookahead_sparse_kv_amd.build")
    return binding.load_library()


def test_header_declares_the_calls():
    syms = declared_symbols()
    for s in ("lsa_query_encode", "lsa_index_score", "lsa_index_score_union", "lsa_index_rescore", "lsa_select_compact",
              "lsa_topk", "lsa_fetch_rows", "lsa_sparse_attend", "lsa_workspace_bytes",
              "lsa_status_string", "lsa_last_error", "lsa_version"):
        assert s in syms
    assert sorted(binding.EXPORTED) == syms


def test_header_compiles_as_c99_and_cpp17(tmp_path):
    """The boundary header is plain C: it builds warning-free as C99 and as C++17,
    and its header-only helper gives the documented gate row length."""
    src = tmp_path / "use.c"
    src.write_text('#include "lsa.h"\n'
                   "int main(void) {\n"
                   "    return lsa_gate_words(0) == 0 && lsa_gate_words(1) == 8 &&\n"
                   "           lsa_gate_words(128) == 8 && lsa_gate_words(129) == 16 ? 0 : 1;\n"
                   "}\n")
    inc = os.path.dirname(HEADER)
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror"],
                ["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-x", "c++"]):
        exe = tmp_path / ("use_" + cmd[0].replace("+", "p"))
        subprocess.run(cmd + ["-I", inc, str(src), "-o", str(exe)], check=True)
        assert subprocess.run([str(exe)]).returncode == 0


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lsa_[a-z_]+)\b", out))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(lib, s)


def test_library_is_built_for_gfx950_only():
    """The embedded device code objects name the gfx950 target and no other."""
    data = open(binding.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx[0-9a-f]+)", data))
    assert targets == {b"gfx950"}, targets


def test_status_strings_and_version(lib):
    assert lib.lsa_version() >= 100
    for code in (0, -1, -2, -3, -4):
        assert lib.lsa_status_string(code)
    assert lib.lsa_status_string(-99) == b"unknown status"


def test_index_score_validation(lib):
    P = FAKE
    f = lib.lsa_index_score
    assert f(None, 1, P, P, P, 1, 1, 64, 128, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -1
    assert b"NULL" in lib.lsa_last_error()
    assert f(P, 1, P, P, P, 0, 1, 64, 128, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -1   # B = 0
    assert f(P, 1, P, P, P, 1, 1, 64, -5, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -1   # D < 0
    assert f(P, 7, P, P, P, 1, 1, 64, 128, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -1  # dtype
    assert f(MISALIGNED, 1, P, P, P, 1, 1, 64, 128, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -1
    assert b"aligned" in lib.lsa_last_error()
    # vector path envelope
    assert f(P, 0, P, P, P, 1, 64, 64, 128, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -2
    assert f(P, 1, P, P, P, 70000, 1, 64, 128, 10, P, P, 0.0, 0, P, None, None, 0.0, None) == -2
    # gate bits: one logit per entry (T = 1 or a reduction), 16-byte aligned rows
    assert f(P, 1, P, P, P, 1, 4, 64, 128, 10, P, P, 0.0, 0, P, None, P, 0.0, None) == -1
    assert b"gate" in lib.lsa_last_error()
    assert f(P, 1, P, P, P, 1, 1, 64, 128, 10, P, P, 0.0, 0, P, None, MISALIGNED, 0.0, None) == -1
    assert b"gate_bits" in lib.lsa_last_error()


def test_select_validation(lib):
    P = FAKE
    f = lib.lsa_select_compact
    assert f(None, None, P, P, 1, 10, 0.0, P, P, P, 1 << 20, None) == -1
    assert f(P, None, P, P, 0, 10, 0.0, P, P, P, 1 << 20, None) == -1
    need = lib.lsa_workspace_bytes(1, 4, 0, 0, 0, 100000, 0, 0)
    assert need >= 4 * 4
    assert f(P, None, P, P, 4, 100000, 0.0, P, P, P, need - 1, None) == -3
    assert f(P, None, P, P, 4, 100000, 0.0, P, P, None, need, None) == -3
    # the bit form: z and the workspace unused, the rows 16-byte aligned
    assert f(None, MISALIGNED, P, P, 4, 100000, 0.0, P, P, None, 0, None) == -1
    assert b"aligned" in lib.lsa_last_error()
    assert f(None, P, None, P, 4, 100000, 0.0, P, P, None, 0, None) == -1
    assert f(None, P, P, P, 0, 100000, 0.0, P, P, None, 0, None) == -1
    assert f(None, P, P, P, 70000, 100000, 0.0, P, P, None, 0, None) == -2


def test_select_noalloc_validation(lib):
    P = FAKE
    f = lib.lsa_select_compact_noalloc
    assert f(None, P, P, 1, 10, 0.0, P, P, None) == -1
    assert f(P, P, P, 0, 10, 0.0, P, P, None) == -1
    assert f(P, P, P, 1, -1, 0.0, P, P, None) == -1
    # the built-in scratch holds 2^18 tile counts (2048 entries each): 5 sequences of
    # 2^27 entries need 5 x 2^16 of them
    assert f(P, P, P, 70000, 10, 0.0, P, P, None) == -2                      # B too large
    assert f(P, P, P, 5, 1 << 27, 0.0, P, P, None) == -2
    assert b"scratch" in lib.lsa_last_error()


def test_topk_validation(lib):
    P = FAKE
    f = lib.lsa_topk
    assert f(P, P, P, 1, 10, P, P, 0, P, P, 0, None, 0, None) == -1        # k = 0
    assert f(P, P, P, 1, 10, P, P, -3, P, P, 0, None, 0, None) == -1
    assert f(P, P, P, 1, 10, P, P, 70000, P, P, 1, None, 0, None) == -2    # k too large
    assert f(None, P, P, 1, 10, P, P, 4, P, P, 0, None, 0, None) == -1
    need = lib.lsa_workspace_bytes(2, 2, 0, 0, 0, 200000, 2048, 0)
    assert need > 0
    assert f(P, P, P, 2, 200000, P, P, 2048, P, P, 0, P, need - 4, None) == -3


def test_encode_validation(lib):
    P = FAKE
    f = lib.lsa_query_encode
    args = [P, 8, 7168, 1536, 64, 128, P, P, P, P, P, P, None]
    for i in (0, 6, 7, 8, 9, 10, 11):                 # every required pointer
        a = list(args); a[i] = None
        assert f(*a) == -1, i
    for i in (1, 2, 3, 4, 5):                          # M, d_model, rank, H, D
        a = list(args); a[i] = 0
        assert f(*a) == -1, i
    a = list(args); a[0] = MISALIGNED                  # h not 16-byte aligned
    assert f(*a) == -1
    a = list(args); a[2] = 7168 + 32                   # d_model not a multiple of 64
    assert f(*a) == -2
    a = list(args); a[3] = 1000                        # rank not a multiple of 64
    assert f(*a) == -2


def test_fetch_validation(lib):
    P = FAKE
    f = lib.lsa_fetch_rows
    args = [P, 1024, P, P, P, P, 8, 20000, P, P, None]
    for i in (0, 2, 3, 4, 5, 8, 9):                  # every required pointer
        a = list(args); a[i] = None
        assert f(*a) == -1, i
    for i, v in ((1, 0), (1, 1000), (6, 0), (7, -1)):  # row_bytes, B, max_count
        a = list(args); a[i] = v
        assert f(*a) == -1, (i, v)
    a = list(args); a[0] = MISALIGNED
    assert f(*a) == -1
    a = list(args); a[8] = MISALIGNED
    assert f(*a) == -1
    a = list(args); a[6] = 70000
    assert f(*a) == -2
    a = list(args); a[1] = 1 << 40
    assert f(*a) == -2


def test_attend_validation(lib):
    P = FAKE
    f = lib.lsa_sparse_attend
    args = [P, 1, 8, 1, 64, 512, P, P, P, P, 2048, P, P, P, 3907, 0.04, P, None, P, 1 << 30, None]
    a = list(args); a[0] = None
    assert f(*a) == -1
    a = list(args); a[12] = None                 # hca without row starts
    assert f(*a) == -1
    a = list(args); a[10] = 0                    # k = 0
    assert f(*a) == -1
    a = list(args); a[0] = MISALIGNED
    assert f(*a) == -1
    a = list(args); a[5] = 2048                  # Dl too large
    assert f(*a) == -2
    a = list(args); a[15] = float("nan")
    assert f(*a) == -1
    a = list(args); a[14] = (1 << 20) - 2048 + 1  # k + max_hca above the per-sequence cap
    assert f(*a) == -2
    need = lib.lsa_workspace_bytes(3, 8, 1, 64, 512, 0, 2048, 3907)
    assert need > 0
    a = list(args); a[19] = need - 1
    assert f(*a) == -3


def test_workspace_sizes(lib):
    assert lib.lsa_workspace_bytes(9, 1, 1, 1, 1, 1, 1, 1) == 0
    assert lib.lsa_workspace_bytes(1, 0, 0, 0, 0, 10, 0, 0) == 0
    # top-k needs a global area only when a candidate list can exceed the LDS capacity
    assert lib.lsa_workspace_bytes(2, 8, 0, 0, 0, 32768, 2048, 0) == 0
    assert lib.lsa_workspace_bytes(2, 8, 0, 0, 0, 32769, 2048, 0) == 8 * 32769 * 4
    # one (b, t) pair per CU-sized split plan: B*T large -> no split, no workspace
    assert lib.lsa_workspace_bytes(3, 16, 64, 64, 512, 0, 2048, 0) == 0


def test_score_reduce_mode_validation(lib):
    P = FAKE
    f = lib.lsa_index_score
    base = [P, 1, P, P, P, 2, 1, 64, 128, 1000, P, P, 0.0, 1, P, None, None, 0.0, None]
    for mode in (-1, 3):
        a = list(base); a[13] = mode
        assert f(*a) == -1
        assert b"reduce_max" in lib.lsa_last_error()


def test_rescore_validation(lib):
    P = FAKE
    f = lib.lsa_index_rescore
    args = [P, 1, P, P, P, P, P, 8, 64, 128, 20000, P, P, P, None]
    for i in (0, 2, 3, 4, 5, 6, 11, 12, 13):          # every required pointer
        a = list(args); a[i] = None
        assert f(*a) == -1, i
    a = list(args); a[7] = 0                        # B = 0
    assert f(*a) == -1
    a = list(args); a[10] = -1                      # max_cand < 0
    assert f(*a) == -1
    a = list(args); a[1] = 7                        # dtype
    assert f(*a) == -1
    a = list(args); a[0] = MISALIGNED
    assert f(*a) == -1
    a = list(args); a[7] = 70000                    # B too large
    assert f(*a) == -2
    a = list(args); a[1] = 0; a[8] = 200; a[9] = 200  # fp32 vector path too large
    assert f(*a) == -2


def test_score_union_validation(lib):
    P = FAKE
    f = lib.lsa_index_score_union
    arr = ctypes.c_void_p * 4
    ks, qs, ws = arr(P, P, P, P), arr(P, P, P, P), arr(P, P, P, P)
    bs = (ctypes.c_float * 4)(0.0, 0.0, 0.0, 0.0)
    base = [3, ks, 1, P, P, P, 2, 1, 64, 128, 1000, qs, ws, bs, P, None, None, 0.0, None]
    for i in (1, 11, 12, 13):                       # the host arrays
        a = list(base); a[i] = None
        assert f(*a) == -1, i
    for n in (0, 5):                                # n_idx outside 1..4
        a = list(base); a[0] = n
        assert f(*a) == -1
    a = list(base); a[1] = arr(P, None, P, P)       # a NULL device pointer of one indexer
    assert f(*a) == -1
    assert b"indexer 1" in lib.lsa_last_error()
    a = list(base); a[11] = arr(P, P, MISALIGNED, P)
    assert f(*a) == -1
    assert b"aligned" in lib.lsa_last_error()
    a = list(base); a[14] = None                    # z_out
    assert f(*a) == -1
    a = list(base); a[6] = 70000                    # B too large
    assert f(*a) == -2
    a = list(base); a[16] = MISALIGNED              # gate bits
    assert f(*a) == -1
    assert b"gate_bits" in lib.lsa_last_error()
    # shapes outside the fused launch go through lsa_index_score's own checks
    a = list(base); a[2] = 7                        # dtype
    assert f(*a) == -1
    assert b"lsa_index_score" in lib.lsa_last_error()


def test_union_binding_checks_its_lists():
    """The Python wrapper refuses lists of different lengths before any pointer is taken."""
    import torch
    k = torch.zeros((4, 128), dtype=torch.bfloat16)
    q = torch.zeros((1, 1, 2, 128), dtype=torch.bfloat16)
    w = torch.zeros((1, 1, 2))
    z = torch.zeros(4)
    i64, i32 = torch.zeros(1, dtype=torch.int64), torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        binding.lsa_index_score_union([k, k], i64, i32, i64, 4, [q], [w, w], [0.0, 0.0], z)
    with pytest.raises(ValueError):
        binding.lsa_index_score_union([k], i64, i32, i64, 4, [q], [w], [0.0, 1.0], z)


def test_c_host_program_is_built():
    """The plain C++ caller used by the GPU tests links against liblsa.so and runs
    (given no arguments it prints its usage before touching the GPU)."""
    from lookahead_sparse_kv_amd import build
    if not os.path.exists(build.C_HOST_BIN):
        pytest.fail("tests/c_host/decode_step is not built; run python -m lookahead_sparse_kv_amd.build")
    r = subprocess.run([build.C_HOST_BIN], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
