"""GPU parity of the widened rows against the CPU reference on identical inputs:
the native re-score of the kept subset (lsa_index_rescore), the OR-mode union
over several indexers (lsa_index_score with reduce_max = 2, and
lsa_index_score_union in one call), and the
just-in-time fetch of the kept rows into a hot buffer (lsa_fetch_rows, with
lsa_topk naming positions in the candidate list)."""
import numpy as np
import pytest
import torch

from gpu_util import (announce, bf16_to_f64, check_attention, check_scores, check_selection,
                      check_topk, check_topk_properties, dev, host)
from lookahead_sparse_kv_amd import binding as lsa
from lookahead_sparse_kv_amd import inputs

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lsa.load_library()


def _native_queries(seed, B, H, D, dtype):
    """Per-step native indexer queries and weights (drawn like the Memory Indexer's)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 104729])))
    q = (rng.standard_normal((B, H, D)) / np.sqrt(D)).astype(np.float32)
    w = rng.uniform(-0.25, 1.0, (B, H)).astype(np.float32)
    return (inputs.to_bf16_bits(q) if dtype == "bf16" else q), w


def _candidates(seed, lens, frac):
    rng = np.random.default_rng(seed)
    es = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    cand = np.full(max(1, int(np.sum(lens))), -1, np.int32)
    cnt = np.zeros(len(lens), np.int32)
    for b, S in enumerate(lens):
        c = np.flatnonzero(rng.random(S) < frac).astype(np.int32)
        cand[es[b]:es[b] + len(c)] = c
        cnt[b] = len(c)
    return es, cand, cnt


def _rescore_gpu(wl, cand, cnt, q2, w2):
    n = max(1, wl.total_entries)
    r = torch.full((n,), SENTINEL, device="cuda")
    lsa.lsa_index_rescore(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len), dev(wl.entry_start),
                          dev(cand), dev(cnt), int(wl.max_len), dev(q2), dev(w2), r)
    torch.cuda.synchronize()
    return host(r).astype(np.float64)


def _check_rescore(wl, cand, cnt, r_gpu, r_ref):
    mask = np.zeros(len(r_gpu), bool)
    for b in range(wl.B):
        es = int(wl.entry_start[b])
        mask[es + cand[es:es + cnt[b]]] = True
    assert np.all(r_gpu[~mask] == SENTINEL), "entries outside the candidate list were written"
    if mask.any():
        check_scores(r_gpu[mask], r_ref[mask])


@pytest.mark.parametrize("H,D,lens,frac,dtype", [
    (64, 128, [5000, 37, 0, 2100], 0.3, "bf16"),   # several waves, ragged, an empty sequence
    (64, 128, [20000], 1.0, "bf16"),               # every entry a candidate
    (20, 64, [700, 129], 0.5, "bf16"),             # padded heads, 64-dim keys
    (48, 128, [300], 0.02, "bf16"),                # a handful of candidates
    (5, 24, [333, 90], 0.4, "bf16"),               # vector path
    (4, 32, [1024], 0.2, "f32"),                   # vector path, fp32 keys
])
def test_rescore_parity(ref, H, D, lens, frac, dtype):
    wl = inputs.random_small(17 * H + D, len(lens), 1, H, D, lens, dtype=dtype, bias=0.0)
    es, cand, cnt = _candidates(H + D, np.asarray(lens), frac)
    q2, w2 = _native_queries(H * D, len(lens), H, D, dtype)
    announce(f"rescore H={H} D={D} lens={lens} frac={frac} dtype={dtype}")
    r = _rescore_gpu(wl, cand, cnt, q2, w2)
    rr = ref.index_rescore(wl.keys, wl.key_row_start, wl.entry_start, cand, cnt, q2, w2)
    _check_rescore(wl, cand, cnt, r, rr)


def test_rescore_exact_integer_inputs(ref):
    """Integer keys and queries, w' in {0, 0.5, 1}: every partial sum is exact."""
    wl = inputs.random_small(91, 2, 1, 64, 128, [900, 400], bias=0.0, int_valued=True)
    es, cand, cnt = _candidates(5, np.array([900, 400]), 0.5)
    rng = np.random.default_rng(6)
    q2 = inputs.to_bf16_bits(rng.integers(-2, 3, (2, 64, 128)).astype(np.float32))
    w2 = rng.choice(np.array([0.0, 0.5, 1.0], np.float32), size=(2, 64))
    announce("rescore exact integer inputs")
    r = _rescore_gpu(wl, cand, cnt, q2, w2)
    rr = ref.index_rescore(wl.keys, wl.key_row_start, wl.entry_start, cand, cnt, q2, w2)
    for b in range(2):
        s = int(wl.entry_start[b]) + cand[int(wl.entry_start[b]):int(wl.entry_start[b]) + cnt[b]]
        np.testing.assert_array_equal(r[s], rr[s])


def test_rescore_feeds_topk(ref):
    """Per-step tiered selection: gate on the Memory-Indexer score, re-score the kept
    entries with the native indexer, take the top-k by the re-score."""
    wl = inputs.random_small(23, 3, 1, 64, 128, [6000, 2500, 40], bias=-1.0, k=256)
    B = wl.B
    z = torch.empty(wl.total_entries, device="cuda")
    lsa.lsa_index_score(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len), dev(wl.entry_start),
                        wl.max_len, dev(wl.q), dev(wl.w), wl.bias, 1, z)
    cand = torch.empty(wl.total_entries, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_SELECT, B, max_len=wl.max_len)),
                     dtype=torch.uint8, device="cuda")
    lsa.lsa_select_compact(z, dev(wl.entry_start), dev(wl.seq_len), wl.max_len, cand, cnt, ws)
    q2, w2 = _native_queries(77, B, 64, 128, "bf16")
    r = torch.full((wl.total_entries,), SENTINEL, device="cuda")
    announce("rescore -> topk pipeline")
    lsa.lsa_index_rescore(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len), dev(wl.entry_start),
                          cand, cnt, wl.max_len, dev(q2), dev(w2), r)
    tk = torch.full((B, wl.k), -7, dtype=torch.int32, device="cuda")
    tc = torch.empty(B, dtype=torch.int32, device="cuda")
    wst = torch.empty(max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_TOPK, B, max_len=wl.max_len,
                                                     k=wl.k)), dtype=torch.uint8, device="cuda")
    lsa.lsa_topk(r, dev(wl.entry_start), dev(wl.seq_len), wl.max_len, cand, cnt, wl.k, tk, tc, wst)
    torch.cuda.synchronize()
    cand_h, cnt_h, r_h = host(cand), host(cnt), host(r).astype(np.float64)
    tk_h, tc_h = host(tk), host(tc)
    # reference on the GPU's own candidate lists (their gate is checked by the select tests)
    zr, _ = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                            wl.bias, reduce_max=True, want_prob=False)
    cr, ccr = ref.select(zr, wl.entry_start, wl.seq_len)
    rr = ref.index_rescore(wl.keys, wl.key_row_start, wl.entry_start, cand_h, cnt_h, q2, w2)
    tr, tcr = ref.topk(rr, wl.entry_start, wl.seq_len, cand_h, cnt_h, wl.k)
    for b in range(B):
        es = int(wl.entry_start[b])
        check_selection(cand_h[es:es + cnt_h[b]], cr[es:es + ccr[b]], zr[es:es + wl.seq_len[b]])
        check_topk(tk_h[b, :tc_h[b]], tr[b, :tcr[b]], rr[es:es + wl.seq_len[b]], wl.k, cnt_h[b])
        check_topk_properties(tk_h[b, :tc_h[b]], cand_h[es:es + cnt_h[b]],
                              r_h[es:es + wl.seq_len[b]], wl.k)


def _layers(seed, B, T, H, D, lens, n_layers, dtype="bf16"):
    return [inputs.random_small(seed + 1000 * l, B, T, H, D, lens, dtype=dtype,
                                bias=-2.0 + 0.5 * l) for l in range(n_layers)]


def test_union_over_indexers_long_lists(ref):
    """Sequences long enough that every wave of the decode kernel streams more
    groups than its ring holds (so ring slots and their prefetched union values
    are reused); the reference scores sampled entries of each indexer."""
    layers = _layers(91, 2, 1, 64, 128, [60000, 45000], 3)
    z = torch.full((layers[0].total_entries,), float("nan"), device="cuda")
    for i, wl in enumerate(layers):
        announce(f"union over long lists, layer {i}")
        lsa.lsa_index_score(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len),
                            dev(wl.entry_start), wl.max_len, dev(wl.q), dev(wl.w), wl.bias,
                            1 if i == 0 else 2, z)
    torch.cuda.synchronize()
    zg = host(z).astype(np.float64)
    rng = np.random.default_rng(92)
    wl0 = layers[0]
    for b in range(wl0.B):
        S, es = int(wl0.seq_len[b]), int(wl0.entry_start[b])
        s = np.sort(rng.choice(S, size=1500, replace=False))
        zr = None
        for wl in layers:
            rows = wl.keys[int(wl.key_row_start[b]) + s]
            zl, _ = ref.index_score(rows, np.zeros(1, np.int64), np.array([len(s)], np.int32),
                                    np.zeros(1, np.int64), wl.q[b:b + 1], wl.w[b:b + 1], wl.bias,
                                    reduce_max=True, want_prob=False)
            zr = zl if zr is None else np.maximum(zr, zl)
        check_scores(zg[es + s], zr)


@pytest.mark.parametrize("T,H,D,lens,dtype", [
    (1, 64, 128, [3000, 1, 777], "bf16"),     # decode kernel
    (4, 64, 128, [513, 300], "bf16"),          # burst kernel
    (2, 5, 24, [200, 90], "bf16"),             # vector path
    (1, 4, 32, [1024], "f32"),                 # vector path, fp32
])
def test_union_over_indexers(ref, T, H, D, lens, dtype):
    layers = _layers(40 + T, len(lens), T, H, D, lens, 3, dtype)
    n = layers[0].total_entries
    z = torch.full((n,), float("nan"), device="cuda")
    p = torch.full((n,), float("nan"), device="cuda")
    zr = None
    for i, wl in enumerate(layers):
        mode = 1 if i == 0 else 2
        announce(f"union layer {i} T={T} H={H} D={D} lens={lens} dtype={dtype}")
        lsa.lsa_index_score(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len),
                            dev(wl.entry_start), wl.max_len, dev(wl.q), dev(wl.w), wl.bias, mode, z,
                            p)
        zr, _ = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                                wl.bias, reduce_max=True, want_prob=False, union_with=zr)
    torch.cuda.synchronize()
    check_scores(host(z), zr, host(p))


def _union_calls(layers, fused):
    """The union of `layers` on the GPU: one lsa_index_score_union call, or one
    lsa_index_score call per indexer (the first writing, the rest combining)."""
    wl0 = layers[0]
    n = wl0.total_entries
    z = torch.full((n,), float("nan"), device="cuda")
    p = torch.full((n,), float("nan"), device="cuda")
    krs, sl, es = dev(wl0.key_row_start), dev(wl0.seq_len), dev(wl0.entry_start)
    keys = [dev(wl.keys) for wl in layers]
    qs = [dev(wl.q) for wl in layers]
    ws = [dev(wl.w) for wl in layers]
    if fused:
        lsa.lsa_index_score_union(keys, krs, sl, es, wl0.max_len, qs, ws,
                                  [wl.bias for wl in layers], z, p)
    else:
        for i, wl in enumerate(layers):
            lsa.lsa_index_score(keys[i], krs, sl, es, wl0.max_len, qs[i], ws[i], wl.bias,
                                1 if i == 0 else 2, z, p if i == len(layers) - 1 else None)
    torch.cuda.synchronize()
    return host(z), host(p)


@pytest.mark.parametrize("T,H,D,lens,n_layers,dtype", [
    (1, 64, 128, [3000, 1, 777], 3, "bf16"),        # one launch: a few groups per wave
    (1, 16, 64, [0, 2000, 33, 16, 17], 2, "bf16"),  # empty and ragged sequences, D = 64
    (1, 40, 128, [5000, 4099], 4, "bf16"),          # padded head tile, four indexers
    (1, 64, 128, [130000, 70000], 3, "bf16"),       # many groups per wave: ring crosses indexers
    (1, 8, 128, [700], 1, "bf16"),                  # one indexer
    (4, 64, 128, [513, 300], 3, "bf16"),            # several positions: one call per indexer
    (1, 4, 32, [1024], 2, "f32"),                   # vector path
])
def test_union_single_call(ref, T, H, D, lens, n_layers, dtype):
    """lsa_index_score_union equals, bit for bit, the per-indexer calls, and the
    reference union of every indexer's gated score."""
    layers = _layers(70 + T + H, len(lens), T, H, D, lens, n_layers, dtype)
    announce(f"union single call T={T} H={H} D={D} lens={lens} n={n_layers} {dtype}")
    zf, pf = _union_calls(layers, fused=True)
    zs, ps = _union_calls(layers, fused=False)
    np.testing.assert_array_equal(zf.view(np.uint32), zs.view(np.uint32))
    np.testing.assert_array_equal(pf.view(np.uint32), ps.view(np.uint32))
    wl0 = layers[0]
    if wl0.total_entries <= 20000:
        zr = None
        for wl in layers:
            zr, _ = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q,
                                    wl.w, wl.bias, reduce_max=True, want_prob=False, union_with=zr)
        check_scores(zf, zr, pf)
        return
    rng = np.random.default_rng(93)
    for b in range(wl0.B):
        S, es = int(wl0.seq_len[b]), int(wl0.entry_start[b])
        s = np.sort(rng.choice(S, size=1200, replace=False))
        zr = None
        for wl in layers:
            rows = wl.keys[int(wl.key_row_start[b]) + s]
            zr, _ = ref.index_score(rows, np.zeros(1, np.int64), np.array([len(s)], np.int32),
                                    np.zeros(1, np.int64), wl.q[b:b + 1], wl.w[b:b + 1], wl.bias,
                                    reduce_max=True, want_prob=False, union_with=zr)
        check_scores(zf[es + s], zr, pf[es + s])


def test_union_nan_logits_match_per_indexer_calls():
    """NaN logits: the fused launch combines them as the per-indexer calls do.  A NaN
    gate weight makes every logit of that (sequence, indexer) NaN: sequence 0 is NaN
    for indexer 0 only, sequence 1 for every indexer, sequence 2 for the last."""
    layers = _layers(171, 3, 1, 64, 128, [3000, 1000, 777], 3)
    layers[0].w[0, 0, 5] = np.nan
    for wl in layers:
        wl.w[1, 0, 0] = np.nan
    layers[-1].w[2, 0, 63] = np.nan
    announce("union with NaN logits")
    zf, pf = _union_calls(layers, fused=True)
    zs, ps = _union_calls(layers, fused=False)
    for a, b in ((zf, zs), (pf, ps)):
        nan = np.isnan(a)
        np.testing.assert_array_equal(nan, np.isnan(b))
        np.testing.assert_array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32))
    es = layers[0].entry_start
    assert not np.isnan(zf[es[0]:es[0] + 3000]).any()      # the other indexers' max
    assert np.isnan(zf[es[1]:es[1] + 1000]).all()          # NaN from every indexer
    assert not np.isnan(zf[es[2]:es[2] + 777]).any()


# ------------------------------------------------- just-in-time fetch of the kept rows

def _ws(op, B, *args, **kw):
    return torch.empty(max(1, lsa.lsa_workspace_bytes(op, B, *args, **kw)), dtype=torch.uint8,
                       device="cuda")


@pytest.mark.parametrize("lens,k,frac", [
    ([5000, 0, 37, 12000], 64, 0.6),       # register path, ragged, an empty sequence
    ([3000, 3000], 2048, 0.9),
    ([30], 64, 0.5),                       # fewer candidates than k: the whole list
    ([100000, 50000], 1024, 0.5),          # > register capacity: global-key path
])
def test_topk_positions(ref, lens, k, frac):
    """Positions mode: exactly the reference's positions, and cand[pos] is the
    entry-index output of the same call without it."""
    rng = np.random.default_rng(sum(lens) + k)
    lens = np.asarray(lens, np.int32)
    es, cand, cnt = _candidates(k, lens, frac)
    r = rng.integers(-5, 60, size=max(1, int(lens.sum()))).astype(np.float32)   # many ties
    B = len(lens)
    ml = int(lens.max())
    out = {}
    for pos in (False, True):
        ti = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        tc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        announce(f"topk positions={pos} lens={lens.tolist()} k={k}")
        lsa.lsa_topk(dev(r), dev(es), dev(lens), ml, dev(cand), dev(cnt), k, ti, tc,
                     _ws(lsa.LSA_OP_TOPK, B, max_len=ml, k=k), out_positions=pos)
        torch.cuda.synchronize()
        out[pos] = (host(ti), host(tc))
    tr, tcr = ref.topk(r.astype(np.float64), es, lens, cand, cnt, k, positions=True)
    (ti, tc), (pi, pc) = out[False], out[True]
    np.testing.assert_array_equal(pc, tcr)
    np.testing.assert_array_equal(tc, pc)
    for b in range(B):
        np.testing.assert_array_equal(pi[b, :pc[b]], tr[b, :tcr[b]])
        np.testing.assert_array_equal(cand[es[b] + pi[b, :pc[b]]], ti[b, :tc[b]])
        assert np.all(pi[b, pc[b]:] == -7), "entries past the count must be untouched"


def _fetch_case(seed, lens, frac, width, pinned):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    es, cand, cnt = _candidates(seed + 1, lens, frac)
    pool = rng.integers(0, 1 << 16, size=(max(1, int(lens.sum())), width), dtype=np.uint16)
    src = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16)
    src = src.pin_memory() if pinned else src.cuda()
    drs = np.concatenate([[0], np.cumsum(cnt[:-1] + 3)]).astype(np.int64)   # gaps of 3 rows
    n_dst = int(drs[-1] + cnt[-1] + 3)
    init = rng.integers(0, 1 << 16, size=(n_dst, width), dtype=np.uint16)
    return es, cand, cnt, pool, src, drs, init


@pytest.mark.parametrize("pinned", [True, False])
@pytest.mark.parametrize("lens,frac,width", [
    ([5000, 37, 0, 2100], 0.3, 576),       # latent + rope row, ragged, an empty sequence
    ([20000], 1.0, 576),                   # every entry: many tiles per sequence
    ([700, 129], 0.5, 8),                  # one 16-byte segment per row
    ([333, 90, 1], 0.4, 1000),             # 125 segments: a tile spans loop steps
])
def test_fetch_rows_bit_exact(ref, pinned, lens, frac, width):
    es, cand, cnt, pool, src, drs, init = _fetch_case(len(lens) * width, lens, frac, width, pinned)
    dst = dev(init)
    announce(f"fetch pinned={pinned} lens={lens} frac={frac} width={width}")
    lsa.lsa_fetch_rows(src, dev(es), dev(cand), dev(es), dev(cnt), int(cnt.max()), dst, dev(drs))
    torch.cuda.synchronize()
    want = ref.fetch_rows(pool, es, cand, es, cnt, len(init), drs, dst_init=init)
    np.testing.assert_array_equal(host(dst), want)


def test_fetch_refuses_pageable_source():
    src = torch.zeros((64, 576), dtype=torch.bfloat16)           # pageable host memory
    z64 = torch.zeros(1, dtype=torch.int64, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    cnt = torch.ones(1, dtype=torch.int32, device="cuda")
    dst = torch.zeros((1, 576), dtype=torch.bfloat16, device="cuda")
    lib = lsa.load_library()
    announce("fetch from pageable host memory is refused")
    rc = lib.lsa_fetch_rows(src.data_ptr(), 1152, z64.data_ptr(), idx.data_ptr(), z64.data_ptr(),
                            cnt.data_ptr(), 1, 1, dst.data_ptr(), z64.data_ptr(), None)
    assert rc == lsa.LSA_ERR_INVALID_ARG, lib.lsa_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(dst == 0)


@pytest.mark.parametrize("B,Hq,Dl,lens,k,hca", [
    (3, 64, 512, [9000, 2500, 40], 512, [300, 0, 17]),
    (2, 64, 512, [40000, 1500], 2048, [900, 64]),
    (2, 16, 128, [700, 3], 64, None),
])
def test_fetch_then_attend(ref, B, Hq, Dl, lens, k, hca):
    """Gate, fetch every kept row from a pinned host pool into a hot buffer, take the
    top-k as positions in the list and attend over the hot buffer: the output is
    bit-identical to attention over the whole pool by entry index, and within the
    attention tolerance of the reference."""
    wl = inputs.random_small(B * 7 + Dl, B, 1, 64, 128, lens, k=k, Hq=Hq, Dl=Dl, hca_lens=hca,
                             bias=-1.0)
    z = torch.empty(wl.total_entries, device="cuda")
    lsa.lsa_index_score(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len), dev(wl.entry_start),
                        wl.max_len, dev(wl.q), dev(wl.w), wl.bias, 1, z)
    cand = torch.empty(wl.total_entries, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda")
    lsa.lsa_select_compact(z, dev(wl.entry_start), dev(wl.seq_len), wl.max_len, cand, cnt,
                           _ws(lsa.LSA_OP_SELECT, B, max_len=wl.max_len))
    wst = _ws(lsa.LSA_OP_TOPK, B, max_len=wl.max_len, k=k)
    sel = {}
    for pos in (False, True):
        ti = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
        tc = torch.empty(B, dtype=torch.int32, device="cuda")
        lsa.lsa_topk(z, dev(wl.entry_start), dev(wl.seq_len), wl.max_len, cand, cnt, k, ti, tc,
                     wst, out_positions=pos)
        sel[pos] = (ti, tc)
    torch.cuda.synchronize()
    cnt_h = host(cnt)
    # hot buffer: sequence b's kept rows at hot_rs[b] ...
    hot_rs = np.concatenate([[0], np.cumsum(cnt_h[:-1])]).astype(np.int64)
    hot = torch.zeros((max(1, int(cnt_h.sum())), Dl), dtype=torch.bfloat16, device="cuda")
    pool = dev(wl.latent, device="cpu").pin_memory()
    announce(f"fetch->attend B={B} Hq={Hq} Dl={Dl} lens={lens} k={k} counts={cnt_h.tolist()}")
    lsa.lsa_fetch_rows(pool, dev(wl.latent_row_start), cand, dev(wl.entry_start), cnt,
                       int(max(1, cnt_h.max())), hot, dev(hot_rs))
    use_hca = wl.hca is not None
    outs = []
    for latent, lrs, (ti, tc) in ((dev(wl.latent), dev(wl.latent_row_start), sel[False]),
                                  (hot, dev(hot_rs), sel[True])):
        out = torch.full((B, 1, Hq, Dl), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, 1, Hq), float("nan"), device="cuda")
        lsa.lsa_sparse_attend(dev(wl.qa), latent, lrs, ti, tc, k, out,
                              hca=dev(wl.hca) if use_hca else None,
                              hca_row_start=dev(wl.hca_row_start) if use_hca else None,
                              hca_count=dev(wl.hca_count) if use_hca else None,
                              max_hca=wl.max_hca, scale=wl.scale, lse=lse,
                              workspace=_ws(lsa.LSA_OP_ATTEND, B, 1, Hq, Dl, k=k,
                                            max_hca=wl.max_hca))
        torch.cuda.synchronize()
        outs.append((host(out), host(lse)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    ti_h, tc_h = host(sel[False][0]), host(sel[False][1])
    orf, lr = ref.sparse_attend(wl.qa, wl.latent, wl.latent_row_start, ti_h, tc_h, k, wl.hca,
                                wl.hca_row_start, wl.hca_count, wl.scale)
    check_attention(bf16_to_f64(outs[1][0]), orf, outs[1][1], lr)
