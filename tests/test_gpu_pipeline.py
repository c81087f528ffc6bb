"""End-to-end parity of the four-call pipeline on the workloads the benchmark times.

Small workloads are compared in full.  At the full 500K / burst / ragged sizes
the reference scores a sample of entries one by one, the gate and top-k are
checked through properties that hold at any size, and attention is compared
on sampled (sequence, position) pairs with indices both sides receive.
"""
import numpy as np
import pytest
import torch

from gpu_util import (announce, bf16_to_f64, check_attention, check_scores, check_selection,
                      check_topk, check_topk_properties, host)
from lookahead_sparse_kv_amd import binding as lsa
from lookahead_sparse_kv_amd import inputs
from lookahead_sparse_kv_amd.pipeline import DeviceInputs, Pipeline

pytestmark = pytest.mark.gpu


def _run(wl):
    d = DeviceInputs(wl)
    p = Pipeline(d, with_prob=True)
    p.step()
    torch.cuda.synchronize()
    res = dict(z=host(p.z), prob=host(p.prob), cand=host(p.cand_idx), cnt=host(p.cand_count),
               topk=host(p.topk_idx), tcnt=host(p.topk_count), out=host(p.out), lse=host(p.lse))
    return d, p, res


def _out64(o):
    return bf16_to_f64(o) if o.dtype == np.uint16 else o.astype(np.float64)


@pytest.mark.parametrize("name", ["tiny", "decode_128k"])
def test_pipeline_full_parity(ref, name):
    wl = inputs.make_workload(name)
    announce(f"pipeline {name} full")
    d, p, g = _run(wl)
    zr, pr = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                             wl.bias, reduce_max=True)
    check_scores(g["z"], zr, g["prob"])
    cr, ccr = ref.select(zr, wl.entry_start, wl.seq_len)
    tr, tcr = ref.topk(zr, wl.entry_start, wl.seq_len, cr, ccr, wl.k)
    for b in range(wl.B):
        es, S = int(wl.entry_start[b]), int(wl.seq_len[b])
        check_selection(g["cand"][es:es + g["cnt"][b]], cr[es:es + ccr[b]], zr[es:es + S])
        check_topk(g["topk"][b, :g["tcnt"][b]], tr[b, :tcr[b]], zr[es:es + S], wl.k, g["cnt"][b])
    # attention of the GPU pipeline compared where both top-k sets agree
    same = all(np.array_equal(g["topk"][b, :g["tcnt"][b]], tr[b, :tcr[b]]) for b in range(wl.B))
    if same:
        orf, lr = ref.sparse_attend(wl.qa, wl.latent, wl.latent_row_start, tr, tcr, wl.k, wl.hca,
                                    wl.hca_row_start, wl.hca_count, wl.scale)
        check_attention(_out64(g["out"]), orf, g["lse"], lr)
    # and on the reference's own top-k as input (always comparable)
    announce(f"attend {name} on reference top-k")
    out = torch.empty_like(p.out)
    lse = torch.empty_like(p.lse)
    lsa.lsa_sparse_attend(d.qa, d.latent[0], d.latent_row_start,
                          torch.from_numpy(tr).cuda(), torch.from_numpy(tcr).cuda(), wl.k, out,
                          hca=d.hca[0], hca_row_start=d.hca_row_start, hca_count=d.hca_count,
                          max_hca=d.max_hca, scale=wl.scale, lse=lse, workspace=p.ws_attend)
    torch.cuda.synchronize()
    orf, lr = ref.sparse_attend(wl.qa, wl.latent, wl.latent_row_start, tr, tcr, wl.k, wl.hca,
                                wl.hca_row_start, wl.hca_count, wl.scale)
    check_attention(_out64(host(out)), orf, host(lse), lr)


def _sampled_scores(ref, wl, g, rng, per_seq):
    """Reference scores of per_seq sampled entries of every sequence (max over positions)."""
    for b in range(wl.B):
        S = int(wl.seq_len[b])
        s = np.sort(rng.choice(S, size=min(per_seq, S), replace=False))
        rows = wl.keys[int(wl.key_row_start[b]) + s]
        zr, _ = ref.index_score(rows, np.zeros(1, np.int64), np.array([len(s)], np.int32),
                                np.zeros(1, np.int64), wl.q[b:b + 1], wl.w[b:b + 1], wl.bias,
                                reduce_max=True, want_prob=False)
        es = int(wl.entry_start[b])
        check_scores(g["z"][es + s], zr, g["prob"][es + s])


def _gate_and_topk_properties(wl, g):
    for b in range(wl.B):
        es, S = int(wl.entry_start[b]), int(wl.seq_len[b])
        zb = g["z"][es:es + S]
        want = np.flatnonzero(zb >= 0)
        assert g["cnt"][b] == len(want)
        np.testing.assert_array_equal(g["cand"][es:es + g["cnt"][b]], want)
        check_topk_properties(g["topk"][b, :g["tcnt"][b]], want, zb, wl.k)


def _attention_on_given_indices(ref, wl, d, p, rng, pairs):
    """Run the benchmark's attention launch on indices both sides receive; compare sampled (b,t)."""
    B, k = wl.B, wl.k
    idx = np.full((B, k), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        S = int(wl.seq_len[b])
        pool = np.flatnonzero(wl.planted[int(wl.key_row_start[b]):int(wl.key_row_start[b]) + S])
        if len(pool) < k:
            pool = np.arange(S)
        c = min(k, len(pool))
        idx[b, :c] = np.sort(rng.choice(pool, size=c, replace=False))
        cnt[b] = c
    out = torch.empty_like(p.out)
    lse = torch.empty_like(p.lse)
    lsa.lsa_sparse_attend(d.qa, d.latent[0], d.latent_row_start, torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), k, out, hca=d.hca[0],
                          hca_row_start=d.hca_row_start, hca_count=d.hca_count,
                          max_hca=d.max_hca, scale=wl.scale, lse=lse, workspace=p.ws_attend)
    torch.cuda.synchronize()
    og, lg = _out64(host(out)), host(lse)
    for b, t in pairs:
        qa = wl.qa[b:b + 1, t:t + 1]
        hca = wl.hca
        orf, lr = ref.sparse_attend(qa, wl.latent, wl.latent_row_start[b:b + 1], idx[b:b + 1],
                                    cnt[b:b + 1], k, hca,
                                    None if hca is None else wl.hca_row_start[b:b + 1],
                                    None if hca is None else wl.hca_count[b:b + 1], wl.scale)
        check_attention(og[b:b + 1, t:t + 1], orf, lg[b:b + 1, t:t + 1], lr)


def test_pipeline_decode_500k(ref):
    wl = inputs.make_workload("decode_500k")
    announce("pipeline decode_500k full size")
    d, p, g = _run(wl)
    rng = np.random.default_rng(1)
    # sequence 0 in full against the reference, all sequences sampled
    S0 = int(wl.seq_len[0])
    z0, _ = ref.index_score(wl.keys[:S0], np.zeros(1, np.int64), wl.seq_len[:1],
                            np.zeros(1, np.int64), wl.q[:1], wl.w[:1], wl.bias, reduce_max=True,
                            want_prob=False)
    check_scores(g["z"][:S0], z0)
    c0, n0 = ref.select(z0, np.zeros(1, np.int64), wl.seq_len[:1])
    t0, tn0 = ref.topk(z0, np.zeros(1, np.int64), wl.seq_len[:1], c0, n0, wl.k)
    check_selection(g["cand"][:g["cnt"][0]], c0[:n0[0]], z0)
    check_topk(g["topk"][0, :g["tcnt"][0]], t0[0, :tn0[0]], z0, wl.k, g["cnt"][0])
    _sampled_scores(ref, wl, g, rng, 4000)
    _gate_and_topk_properties(wl, g)
    assert np.all(g["tcnt"] == wl.k)
    announce("attend decode_500k on given indices")
    _attention_on_given_indices(ref, wl, d, p, rng, [(0, 0), (5, 0), (7, 0)])


def test_pipeline_burst(ref):
    wl = inputs.make_workload("burst_tau64")
    announce("pipeline burst_tau64 full size")
    d, p, g = _run(wl)
    rng = np.random.default_rng(2)
    # sampled entries: the reference max over 64 positions of the shared keys
    s = np.sort(rng.choice(65536, size=192, replace=False))
    rows = wl.keys[s]
    n = len(s)
    m, _ = ref.index_score(rows, np.zeros(wl.B, np.int64), np.full(wl.B, n, np.int32),
                           np.arange(wl.B, dtype=np.int64) * n, wl.q, wl.w, wl.bias,
                           reduce_max=True, want_prob=False)
    for b in range(wl.B):
        check_scores(g["z"][int(wl.entry_start[b]) + s], m[b * n:(b + 1) * n])
    _gate_and_topk_properties(wl, g)
    frac = g["cnt"] / 65536.0
    assert np.all((frac > 0.05) & (frac < 0.3)), frac
    announce("attend burst on given indices")
    _attention_on_given_indices(ref, wl, d, p, rng, [(0, 0), (0, 63), (9, 17), (15, 40)])


def test_pipeline_ragged(ref):
    wl = inputs.make_workload("ragged_mix")
    announce("pipeline ragged_mix full size")
    d, p, g = _run(wl)
    rng = np.random.default_rng(3)
    _sampled_scores(ref, wl, g, rng, 1500)
    _gate_and_topk_properties(wl, g)
    announce("attend ragged on given indices")
    _attention_on_given_indices(ref, wl, d, p, rng, [(0, 0), (13, 0), (31, 0)])


def test_pipeline_is_deterministic():
    """Repeated runs give bit-identical index lists and outputs."""
    wl = inputs.make_workload("decode_128k")
    announce("pipeline determinism decode_128k")
    d = DeviceInputs(wl)
    p = Pipeline(d)
    outs = []
    for _ in range(3):
        p.step()
        torch.cuda.synchronize()
        outs.append((host(p.cand_idx).copy(), host(p.topk_idx).copy(), host(p.out).copy(),
                     host(p.z).copy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            np.testing.assert_array_equal(a, b)
