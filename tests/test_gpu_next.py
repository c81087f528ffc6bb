"""GPU parity of the two widened rows: the native re-score of the kept subset
(lsa_index_rescore) and the OR-mode union over several indexers (lsa_index_score
with reduce_max = 2), against the CPU reference on identical inputs."""
import numpy as np
import pytest
import torch

from gpu_util import (announce, check_scores, check_selection, check_topk, check_topk_properties,
                      dev, host)
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
