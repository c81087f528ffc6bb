"""The four calls, and the union of several indexers, capture into a HIP graph and every
replay matches the eager run."""
import numpy as np
import pytest
import torch

from gpu_util import announce, host
from lookahead_sparse_kv_amd import inputs
from lookahead_sparse_kv_amd.pipeline import DeviceInputs, Pipeline

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    wl = inputs.random_small(31, 3, 1, 64, 128, [5000, 3100, 700], k=256, Hq=64, Dl=512,
                             hca_lens=[70, 0, 33], bias=-10.0)
    announce("graph capture of the pipeline step")
    d = DeviceInputs(wl)
    p = Pipeline(d)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        p.step()
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in (p.z, p.cand_idx, p.cand_count, p.topk_idx, p.topk_count,
                                      p.out, p.lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        p.step()
    for rep in range(4):
        # eager work and a sync between replays; outputs cleared before each replay
        for t in (p.z, p.out, p.lse):
            t.zero_()
        p.topk_idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in (p.z, p.cand_idx, p.cand_count, p.topk_idx, p.topk_count, p.out,
                                 p.lse)]
        for a, b in zip(eager, got):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}")


def test_graph_replays_of_the_union_match_eager():
    """The single-launch union of three indexers (three key replicas) and the
    per-indexer combining launches, each captured and replayed several times."""
    wl = inputs.random_small(37, 2, 1, 64, 128, [9000, 4100], bias=-1.0)
    d = DeviceInputs(wl, key_replicas=3)
    # three different key sets: rotate the rows of the second and third replicas
    for i in (1, 2):
        d.keys[i].copy_(torch.roll(d.keys[0], 5 * i, dims=0))
    p = Pipeline(d)
    stream = torch.cuda.Stream()
    for fused in (True, False):
        announce(f"graph capture of the union of three indexers, fused={fused}")
        with torch.cuda.stream(stream):
            p.score_union(3, 0, fused=fused)
        torch.cuda.synchronize()
        eager = host(p.z).copy()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            p.score_union(3, 0, fused=fused)
        for rep in range(3):
            p.z.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(p.z).view(np.uint32), eager.view(np.uint32),
                                          err_msg=f"replay {rep}")
        if fused:
            first = eager
        else:
            np.testing.assert_array_equal(first.view(np.uint32), eager.view(np.uint32))
