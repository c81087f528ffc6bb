"""The C ABI from a plain C++ host program: tests/c_host/decode_step.cpp (built by
the package build) allocates its own device buffers with the HIP runtime, runs
one decode step -- lsa_index_score with gate bits, lsa_select_compact from the
bits, lsa_topk, lsa_sparse_attend -- and writes the results back.  No Python or
torch runs in that process; the same step through the Python binding on the
same inputs must give bit-identical logits, candidate lists, top-k sets,
attention outputs and log-sum-exps."""
import os
import subprocess

import numpy as np
import pytest
import torch

from gpu_util import announce, host
from lookahead_sparse_kv_amd import build, inputs
from lookahead_sparse_kv_amd.pipeline import DeviceInputs, Pipeline

pytestmark = pytest.mark.gpu


def test_c_host_decode_step_matches_binding(tmp_path):
    assert os.path.exists(build.C_HOST_BIN), "tests/c_host/decode_step is not built"
    lens = [3000, 1700, 0, 513]
    hca_lens = [40, 0, 7, 100]
    wl = inputs.random_small(2024, len(lens), 1, 64, 128, lens, k=256, Hq=64, Dl=512,
                             hca_lens=hca_lens, bias=-1.5)
    B = len(lens)
    # the program packs sequences back to back: check the generator does the same
    total, total_h = int(sum(lens)), int(sum(hca_lens))
    starts = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    for arr in (wl.entry_start, wl.key_row_start, wl.latent_row_start):
        np.testing.assert_array_equal(arr, starts)
    np.testing.assert_array_equal(wl.hca_row_start,
                                  np.concatenate([[0], np.cumsum(hca_lens[:-1])]))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        np.array([B, wl.max_len, wl.H, wl.D, wl.k, wl.Hq, wl.Dl, wl.max_hca], np.int32).tofile(f)
        np.array([wl.bias, wl.scale], np.float32).tofile(f)
        np.asarray(wl.seq_len, np.int32).tofile(f)
        np.asarray(wl.hca_count, np.int32).tofile(f)
        for a in (wl.keys, wl.q, wl.w, wl.qa, wl.latent, wl.hca):
            np.ascontiguousarray(a).tofile(f)
    announce("C host program: one decode step")
    r = subprocess.run([build.C_HOST_BIN, str(fin), str(fout)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(fout, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a
    z = take(np.float32, total)
    ccnt = take(np.int32, B)
    cand = take(np.int32, total)
    tcnt = take(np.int32, B)
    tk = take(np.int32, B * wl.k).reshape(B, wl.k)
    out = take(np.uint16, B * wl.Hq * wl.Dl)
    lse = take(np.float32, B * wl.Hq)
    assert off == len(raw)

    announce("the same step through the binding")
    d = DeviceInputs(wl)
    p = Pipeline(d)
    p.topk_idx.fill_(-1)
    p.step()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z.view(np.uint32), host(p.z).view(np.uint32))
    np.testing.assert_array_equal(ccnt, host(p.cand_count))
    pc = host(p.cand_idx)
    for b in range(B):
        np.testing.assert_array_equal(cand[starts[b]:starts[b] + ccnt[b]],
                                      pc[starts[b]:starts[b] + ccnt[b]])
    np.testing.assert_array_equal(tcnt, host(p.topk_count))
    ptk = host(p.topk_idx)
    for b in range(B):
        np.testing.assert_array_equal(tk[b, :tcnt[b]], ptk[b, :tcnt[b]])
    np.testing.assert_array_equal(out, host(p.out).reshape(-1))
    np.testing.assert_array_equal(lse.view(np.uint32), host(p.lse).reshape(-1).view(np.uint32))
    assert ccnt[2] == 0 and tcnt[2] == 0
