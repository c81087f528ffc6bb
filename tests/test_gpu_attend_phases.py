"""Attention in two phases (HCA rows first, then the chosen rows and the merge)
against the one-call attention and the oracle.

The HCA entries are kept for every query whatever the selection (FlashMemory-
DeepSeek-V4 technical summary, section 2.1 "Architectural Design"), so their
split partials can be formed before the top-k list exists; the log-sum-exp
merge of partials over disjoint row sets is the softmax over their union.  The
pair runs the same kernels on the same split plan as the single call, so the
outputs must agree bit for bit; the oracle check covers the arithmetic.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import announce, bf16_to_f64, check_attention, dev, host
from lookahead_sparse_kv_amd import binding as lsa
from lookahead_sparse_kv_amd import inputs
from test_gpu_ops import _attend_gpu, _attend_ref, _random_indices

pytestmark = pytest.mark.gpu


def _pair(wl, idx, cnt, graph_replays=0):
    """HCA phase on a second stream, the selected phase on the current one after
    an event; the workspace starts as NaN bytes so no stale partial can pass."""
    B, T, Hq, Dl = wl.qa.shape
    use_hca = wl.hca is not None
    nb = max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_ATTEND, B, T, Hq, Dl, k=wl.k,
                                        max_hca=wl.max_hca))
    ws = torch.full((nb,), 255, dtype=torch.uint8, device="cuda")
    qa = dev(wl.qa)
    lat, lrs, d_idx, d_cnt = dev(wl.latent), dev(wl.latent_row_start), dev(idx), dev(cnt)
    hca = dev(wl.hca) if use_hca else None
    hrs = dev(wl.hca_row_start) if use_hca else None
    hcnt = dev(wl.hca_count) if use_hca else None
    out = torch.full(qa.shape, float("nan"), dtype=qa.dtype, device="cuda")
    lse = torch.full((B, T, Hq), float("nan"), device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    def enqueue():
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        if use_hca:
            lsa.lsa_sparse_attend_hca(qa, wl.k, hca, hrs, hcnt, wl.max_hca, scale=wl.scale,
                                      workspace=ws, stream=side)
        join.record(side)
        main.wait_event(join)
        lsa.lsa_sparse_attend_selected(qa, lat, lrs, d_idx, d_cnt, wl.k, out, hca=hca,
                                       hca_row_start=hrs, hca_count=hcnt, max_hca=wl.max_hca,
                                       scale=wl.scale, lse=lse, workspace=ws, stream=main)

    def result():
        torch.cuda.synchronize()
        o = host(out)
        o = bf16_to_f64(o) if o.dtype == np.uint16 else o.astype(np.float64)
        return o, host(lse)

    if graph_replays == 0:
        enqueue()
        return [result()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        enqueue()
    res = []
    for _ in range(graph_replays):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        res.append(result())
    return res


def _same(a, b):
    """Bit-identical outputs (NaN positions included)."""
    for x, y in zip(a, b):
        assert x.shape == y.shape
        np.testing.assert_array_equal(np.isnan(x), np.isnan(y))
        np.testing.assert_array_equal(np.nan_to_num(x, nan=0.0), np.nan_to_num(y, nan=0.0))


@pytest.mark.parametrize("B,T,Hq,Dl,lens,counts,hca,k,seed", [
    # decode shape: 8 sequences, ragged top-k and HCA counts, split plan
    (8, 1, 64, 512, [5000] * 8, [2048, 0, 1, 700, 2048, 1500, 33, 2047],
     [3907, 0, 3907, 100, 1, 2000, 3907, 64], 2048, 1),
    (2, 4, 64, 512, [3000, 2500], [700, 2048], [200, 50], 2048, 2),   # 4 query groups
    (2, 1, 64, 128, [300, 40], [200, 40], [64, 0], 200, 3),           # Dl = 128
    (2, 3, 16, 256, [400, 400], [77, 128], [33, 5], 128, 4),           # Dl = 256
    (1, 1, 64, 512, [5000], [1024], None, 1024, 5),                    # no HCA pool
    (4, 1, 8, 96, [80] * 4, [10, 0, 80, 1], [3, 0, 0, 2], 80, 6),      # vector path
    (1, 1, 64, 512, [3000], [2048], [200000], 2048, 7),                # ~100 HCA splits
])
def test_attend_phases_match_single_call(ref, B, T, Hq, Dl, lens, counts, hca, k, seed):
    wl = inputs.random_small(9000 + seed, B, 1, 4, 32, lens, k=k, Hq=Hq, Dl=Dl, hca_lens=hca)
    if T > 1:
        wl.qa = inputs.to_bf16_bits(
            np.random.default_rng(seed).standard_normal((B, T, Hq, Dl)).astype(np.float32))
    idx, cnt = _random_indices(np.random.default_rng(seed), wl.seq_len, k, counts)
    announce(f"attend phases B={B} T={T} Hq={Hq} Dl={Dl} counts={counts} hca={hca}")
    (pair,) = _pair(wl, idx, cnt)
    single = _attend_gpu(wl, idx, cnt)
    _same(pair, single)
    if hca is None or max(hca) <= 5000:
        orf, lr = _attend_ref(ref, wl, idx, cnt)
        check_attention(pair[0], orf, pair[1], lr)


def test_attend_phases_in_graph():
    """The two-stream pair captured in one HIP graph: every replay equals the
    eager single call."""
    lens, counts, hca = [5000] * 8, [2048, 5, 2048, 0, 900, 2048, 1, 2048], [3907] * 7 + [0]
    wl = inputs.random_small(9100, 8, 1, 4, 32, lens, k=2048, Hq=64, Dl=512, hca_lens=hca)
    idx, cnt = _random_indices(np.random.default_rng(11), wl.seq_len, 2048, counts)
    announce("attend phases in a graph, 3 replays")
    single = _attend_gpu(wl, idx, cnt)
    with torch.cuda.stream(torch.cuda.Stream()):   # graphs are captured off the default stream
        replays = _pair(wl, idx, cnt, graph_replays=3)
    for res in replays:
        _same(res, single)


def test_attend_hca_phase_rejects_missing_pool():
    qa = torch.zeros((1, 1, 64, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lsa.LSAError):
        lsa.lsa_sparse_attend_hca(qa, 16, None, None, None, 0)
