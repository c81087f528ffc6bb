"""The four calls capture into a HIP graph and every replay matches the eager run."""
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
