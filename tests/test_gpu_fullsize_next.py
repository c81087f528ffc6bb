"""The widened rows at the full decode_500k size, in the launch configuration the
benchmark times (the Pipeline object bench.py drives): the native re-score of
the kept entries and its top-k, the just-in-time fetch from a pinned host pool,
attention over the fetched rows, and the OR-union of three indexers.

The reference re-scores sampled kept entries one by one; the top-k is checked
through properties that hold at any size; fetched rows are compared byte for
byte on a sample; attention over the hot buffer (by position) must be
bit-identical to attention over the pool (by entry index).
"""
import numpy as np
import pytest
import torch

from gpu_util import announce, check_scores, check_topk_properties, host
from lookahead_sparse_kv_amd import binding as lsa
from lookahead_sparse_kv_amd import inputs
from lookahead_sparse_kv_amd.pipeline import DeviceInputs, Pipeline

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    wl = inputs.make_workload("decode_500k")
    d = DeviceInputs(wl)
    p = Pipeline(d)
    announce("full size decode_500k: score, select, re-score, native top-k")
    p.score(0)
    p.select()
    p.rescore(0)
    p.topk_native()
    torch.cuda.synchronize()
    return wl, d, p


def test_rescore_and_native_topk_full_size(ref, run):
    wl, d, p = run
    cand, cnt, r = host(p.cand_idx), host(p.cand_count), host(p.r)
    tk, tc = host(p.topk_idx), host(p.topk_count)
    q2, w2 = (host(t) for t in (d.q_native, d.w_native))
    rng = np.random.default_rng(11)
    for b in range(wl.B):
        es, S = int(wl.entry_start[b]), int(wl.seq_len[b])
        c = cand[es:es + cnt[b]]
        # reference re-score of 400 sampled kept entries of this sequence
        s = np.sort(rng.choice(c, size=min(400, len(c)), replace=False)).astype(np.int32)
        rr = ref.index_rescore(wl.keys, wl.key_row_start[b:b + 1], np.zeros(1, np.int64), s,
                               np.array([len(s)], np.int32), q2[b:b + 1], w2[b:b + 1],
                               r_init=np.zeros(S))
        check_scores(r[es + s].astype(np.float64), rr[s])
        # the native top-k over the GPU's own rank keys
        check_topk_properties(tk[b, :tc[b]], c, r[es:es + S], wl.k)


def test_fetch_and_attend_full_size(ref, run):
    wl, d, p = run
    announce("full size decode_500k: fetch from a pinned pool, attend by position")
    pool = torch.empty(d.latent[0].shape, dtype=d.latent[0].dtype, pin_memory=True)
    pool.copy_(d.latent[0])
    hot = torch.zeros_like(d.latent[0])
    torch.cuda.synchronize()
    p.fetch(pool, hot)
    # top-k by position in the candidate list, and by entry index, on the Memory-Indexer logit
    pos_i = torch.full_like(p.topk_idx, -1)
    pos_c = torch.empty_like(p.topk_count)
    lsa.lsa_topk(p.z, d.entry_start, d.seq_len, d.max_len, p.cand_idx, p.cand_count, d.k, pos_i,
                 pos_c, p.ws_topk, out_positions=True)
    p.topk()
    torch.cuda.synchronize()
    cand, cnt = host(p.cand_idx), host(p.cand_count)
    lat, hot_h = host(d.latent[0]), host(hot)
    rng = np.random.default_rng(12)
    for b in range(wl.B):
        es, lrs = int(wl.entry_start[b]), int(wl.latent_row_start[b])
        j = np.sort(rng.choice(cnt[b], size=min(300, cnt[b]), replace=False))
        # fetched row j of sequence b is the pool row of its j-th kept entry
        want = ref.fetch_rows(lat, np.array([lrs], np.int64), cand[es + j].astype(np.int32),
                              np.zeros(1, np.int64), np.array([len(j)], np.int32), len(j),
                              np.zeros(1, np.int64))
        np.testing.assert_array_equal(hot_h[lrs + j], want)
    pi, pc, ti_h, tc_h = host(pos_i), host(pos_c), host(p.topk_idx), host(p.topk_count)
    np.testing.assert_array_equal(pc, tc_h)
    for b in range(wl.B):
        es = int(wl.entry_start[b])
        np.testing.assert_array_equal(cand[es + pi[b, :pc[b]]], ti_h[b, :tc_h[b]])
    outs = []
    for latent, ti in ((d.latent[0], p.topk_idx), (hot, pos_i)):
        out = torch.empty_like(p.out)
        lse = torch.empty_like(p.lse)
        lsa.lsa_sparse_attend(d.qa, latent, d.latent_row_start, ti, p.topk_count, d.k, out,
                              hca=d.hca[0], hca_row_start=d.hca_row_start, hca_count=d.hca_count,
                              max_hca=d.max_hca, scale=d.scale, lse=lse, workspace=p.ws_attend)
        torch.cuda.synchronize()
        outs.append((host(out), host(lse)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_union_of_three_indexers_full_size(ref, run):
    """Three indexers (the key pool and two row-rotated copies of it, so every
    indexer scores different keys) united in one lsa_index_score_union launch:
    bit-identical to the three combining launches, and the reference union on
    sampled entries."""
    wl, d, p = run
    announce("full size decode_500k: union of three indexers, one launch and three")
    keys = [d.keys[0]] + [torch.roll(d.keys[0], 7 * i + 1, dims=0) for i in (1, 2)]
    args = (d.key_row_start, d.seq_len, d.entry_start, d.max_len)
    z3 = torch.full_like(p.z, float("nan"))
    for i, kk in enumerate(keys):
        lsa.lsa_index_score(kk, *args, d.q, d.w, d.bias, 1 if i == 0 else 2, z3)
    z1 = torch.full_like(p.z, float("nan"))
    lsa.lsa_index_score_union(keys, *args, [d.q] * 3, [d.w] * 3, [d.bias] * 3, z1)
    torch.cuda.synchronize()
    z1, z3 = host(z1), host(z3)
    np.testing.assert_array_equal(z1.view(np.uint32), z3.view(np.uint32))
    keys_h = [host(kk) for kk in keys]
    q, w = host(d.q), host(d.w)
    rng = np.random.default_rng(13)
    for b in range(wl.B):
        S, es, krs = int(wl.seq_len[b]), int(wl.entry_start[b]), int(wl.key_row_start[b])
        s = np.sort(rng.choice(S, size=300, replace=False))
        zr = None
        for kk in keys_h:
            zr, _ = ref.index_score(kk[krs + s], np.zeros(1, np.int64),
                                    np.array([len(s)], np.int32), np.zeros(1, np.int64),
                                    q[b:b + 1], w[b:b + 1], d.bias, reduce_max=True,
                                    want_prob=False, union_with=zr)
        check_scores(z1[es + s].astype(np.float64), zr)
