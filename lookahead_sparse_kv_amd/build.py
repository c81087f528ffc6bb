"""Compile the HIP sources under csrc/ into liblsa.so (gfx950 only), and the
benchmark's measurement kernels (csrc/ceiling.hip) into libceiling.so.

Run as `python -m lookahead_sparse_kv_amd.build` or through
__graft_entry__.build().  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblsa.so")
CEILING_LIB = os.path.join(HERE, "libceiling.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["host_common.cpp", "encode.hip", "score.hip", "rescore.hip", "select.hip", "topk.hip",
           "fetch.hip",
           "attend.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in architectural VGPRs (no AGPR round trips in loops)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Per-source additions.  attend.hip: the first 16 dwords of kernel arguments are
# preloaded into scalar registers at wave launch (the code object keeps a
# fallback entry that loads them for firmware without preloading).
EXTRA = {"attend.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


REPO = os.path.dirname(HERE)
C_HOST_SRC = os.path.join(REPO, "tests", "c_host", "decode_step.cpp")
C_HOST_BIN = os.path.join(REPO, "tests", "c_host", "decode_step")


def _build_c_host() -> None:
    """The tests' plain C++ caller of the C ABI (host code only, linked to liblsa.so)."""
    if not os.path.exists(C_HOST_SRC):
        return
    tmp = C_HOST_BIN + ".tmp"
    cmd = [HIPCC, "-std=c++17", "-O2", f"--offload-arch={ARCH}", "-I",
           os.path.join(REPO, "include"), C_HOST_SRC, "-L", HERE, "-llsa",
           "-Wl,-rpath,$ORIGIN/../../lookahead_sparse_kv_amd", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, C_HOST_BIN)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + ["ceiling.hip"]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    _build_c_host()
    if verbose:
        print(f"built {LIB}, {CEILING_LIB} and {C_HOST_BIN}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    build()
