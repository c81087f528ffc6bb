"""Entry-point parity on the GPU: each C-ABI call against the CPU reference on identical inputs.

Sizes span several workgroup tiles with ragged tails, empty sequences and the
degenerate cases of each step.  Gate and top-k decisions are compared bit for
bit when both sides read the same fp32 keys; scores and attention outputs are
compared within the tolerances in gpu_util.
"""
import numpy as np
import pytest
import torch

from gpu_util import (announce, bf16_to_f64, check_attention, check_scores, dev, host)
from lookahead_sparse_kv_amd import binding as lsa
from lookahead_sparse_kv_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lsa.load_library()


def _score_gpu(wl, reduce_max, with_prob=True):
    T = wl.T
    n = wl.total_entries * (1 if reduce_max else T)
    z = torch.full((n,), float("nan"), device="cuda")
    p = torch.full((n,), float("nan"), device="cuda") if with_prob else None
    lsa.lsa_index_score(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len), dev(wl.entry_start),
                        wl.max_len, dev(wl.q), dev(wl.w), wl.bias, reduce_max, z, p)
    torch.cuda.synchronize()
    return host(z), (host(p) if with_prob else None)


def _score_ref(ref, wl, reduce_max):
    return ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                           wl.bias, reduce_max=reduce_max)


# ------------------------------------------------------------------ score

def test_score_tiny_fp32(ref):
    wl = inputs.make_workload("tiny")
    announce("score tiny fp32 vector path")
    z, p = _score_gpu(wl, False)
    zr, _ = _score_ref(ref, wl, False)
    check_scores(z, zr, p)


@pytest.mark.parametrize("H,D,lens", [
    (64, 128, [1000, 37, 0, 2049]),
    (64, 128, [16, 1, 17, 4096 + 5]),
    (16, 64, [300]),
    (48, 128, [5000, 17]),
    (33, 64, [64, 65]),
    (64, 64, [129]),
])
def test_score_decode_matrix_path(ref, H, D, lens):
    wl = inputs.random_small(H * 100 + D, len(lens), 1, H, D, lens, bias=-2.0)
    announce(f"score decode H={H} D={D} lens={lens}")
    z, p = _score_gpu(wl, False)
    zr, _ = _score_ref(ref, wl, False)
    check_scores(z, zr, p)
    zm, _ = _score_gpu(wl, True, with_prob=False)    # T = 1: the max is the score
    np.testing.assert_array_equal(zm, z)


@pytest.mark.parametrize("T,H,D,lens,shared", [
    (1, 64, 128, [777, 1030], False),
    (4, 64, 128, [300, 513], False),
    (3, 5, 24, [100, 7], False),
    (2, 16, 64, [257, 257], True),
])
def test_score_exact_integer_inputs(ref, T, H, D, lens, shared):
    """Integer q and keys, w in {0, 0.5, 1}: every partial sum is exact, so z matches exactly."""
    wl = inputs.random_small(7 + T, len(lens), T, H, D, lens, bias=-7.5, int_valued=True,
                             shared=shared)
    for reduce_max in (False, True):
        announce(f"score exact T={T} H={H} D={D} lens={lens} reduce={reduce_max}")
        z, _ = _score_gpu(wl, reduce_max, with_prob=False)
        zr, _ = _score_ref(ref, wl, reduce_max)
        np.testing.assert_array_equal(z.astype(np.float64), zr)


@pytest.mark.parametrize("T,lens,shared", [
    (2, [700, 300], False),
    (64, [513, 256], False),
    (16, [1024, 1024, 1024], True),
    (5, [1, 0, 255], False),
])
def test_score_burst_matrix_path(ref, T, lens, shared):
    wl = inputs.random_small(100 + T, len(lens), T, 64, 128, lens, bias=-4.0, shared=shared)
    for reduce_max in (False, True):
        announce(f"score burst T={T} lens={lens} shared={shared} reduce={reduce_max}")
        z, p = _score_gpu(wl, reduce_max)
        zr, _ = _score_ref(ref, wl, reduce_max)
        check_scores(z, zr, p)


@pytest.mark.parametrize("T,H,D,lens", [
    (8, 48, 128, [700, 129]),      # padded head rows of the query ring
    (3, 20, 64, [300, 1, 513]),
    (70, 64, 128, [256]),          # more positions than ring slots, one workgroup
])
def test_score_burst_head_shapes(ref, T, H, D, lens):
    wl = inputs.random_small(31 * H + T, len(lens), T, H, D, lens, bias=-3.0)
    for reduce_max in (False, True):
        announce(f"score burst T={T} H={H} D={D} lens={lens} reduce={reduce_max}")
        z, p = _score_gpu(wl, reduce_max)
        zr, _ = _score_ref(ref, wl, reduce_max)
        check_scores(z, zr, p)


def test_score_vector_bf16(ref):
    wl = inputs.random_small(5, 2, 2, 5, 24, [333, 90], bias=-0.5)
    for reduce_max in (False, True):
        announce(f"score vector bf16 reduce={reduce_max}")
        z, p = _score_gpu(wl, reduce_max)
        zr, _ = _score_ref(ref, wl, reduce_max)
        check_scores(z, zr, p)


# ----------------------------------------------------------------- select

def _special_logits(rng, n):
    z = rng.standard_normal(n).astype(np.float32)
    specials = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 1e-38, -1e-38, 1e-45, -1e-45],
                        np.float32)
    pos = rng.choice(n, size=min(n, 64), replace=False)
    z[pos] = specials[rng.integers(0, len(specials), size=len(pos))]
    return z


def _select_gpu(z, lens, es, max_len, thr=0.0):
    B = len(lens)
    ws = torch.empty(max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_SELECT, B, max_len=max_len)),
                     dtype=torch.uint8, device="cuda")
    ci = torch.full((len(z),), -7, dtype=torch.int32, device="cuda")
    cc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    lsa.lsa_select_compact(dev(z), dev(es), dev(lens), max_len, ci, cc, ws, threshold=thr)
    torch.cuda.synchronize()
    return host(ci), host(cc)


@pytest.mark.parametrize("lens", [[0, 1, 2047, 2048, 2049, 5000], [131072, 3, 70001], [10]])
def test_select_bit_exact(ref, lens):
    rng = np.random.default_rng(sum(lens))
    lens = np.array(lens, np.int32)
    es = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    z = _special_logits(rng, int(lens.sum()))
    announce(f"select lens={lens.tolist()}")
    ci, cc = _select_gpu(z, lens, es, int(lens.max()))
    cr, ccr = ref.select(z.astype(np.float64), es, lens)
    np.testing.assert_array_equal(cc, ccr)
    for b in range(len(lens)):
        np.testing.assert_array_equal(ci[es[b]:es[b] + cc[b]], cr[es[b]:es[b] + ccr[b]])


def test_select_none_all_and_threshold(ref):
    lens = np.array([4000, 4000], np.int32)
    es = np.array([0, 4000], np.int64)
    z = np.concatenate([-np.ones(4000, np.float32), np.ones(4000, np.float32)])
    announce("select none/all")
    ci, cc = _select_gpu(z, lens, es, 4000)
    assert cc.tolist() == [0, 4000]
    np.testing.assert_array_equal(ci[4000:], np.arange(4000))
    rng = np.random.default_rng(3)
    z = rng.standard_normal(8000).astype(np.float32)
    announce("select threshold 0.7")
    ci, cc = _select_gpu(z, lens, es, 4000, thr=0.7)
    cr, ccr = ref.select(z.astype(np.float64), es, lens, threshold=float(np.float32(0.7)))
    np.testing.assert_array_equal(cc, ccr)
    for b in range(2):
        np.testing.assert_array_equal(ci[es[b]:es[b] + cc[b]], cr[es[b]:es[b] + ccr[b]])


# ------------------------------------------------------------------ top-k

def _topk_gpu(r, lens, es, cand, cnt, k, max_len):
    B = len(lens)
    ws = torch.empty(max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_TOPK, B, max_len=max_len, k=k)),
                     dtype=torch.uint8, device="cuda")
    ti = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    tc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    lsa.lsa_topk(dev(r), dev(es), dev(lens), max_len, dev(cand), dev(cnt), k, ti, tc, ws)
    torch.cuda.synchronize()
    return host(ti), host(tc)


@pytest.mark.parametrize("lens,k,kind", [
    ([5000, 0, 37, 12000], 64, "ties"),
    ([5000, 0, 37, 12000], 2048, "ties"),
    ([3000, 3000], 1, "normal"),
    ([20000], 4099, "normal"),
    ([9000, 300], 7, "signed_zero_nan"),
    ([40000, 100000], 2048, "ties"),          # > LDS capacity: global-key path
    ([70000], 65536, "normal"),
    ([32768, 32769], 2048, "ties_all"),       # every entry kept: the register path's
    ([32768, 32769], 30000, "normal_all"),    # capacity exactly, and one past it
])
def test_topk_bit_exact(ref, lens, k, kind):
    rng = np.random.default_rng(len(lens) * 1000 + k)
    lens = np.array(lens, np.int32)
    es = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    n = int(lens.sum())
    if kind.startswith("ties"):
        r = rng.integers(-3, 40, size=n).astype(np.float32)
    elif kind.startswith("normal"):
        r = rng.standard_normal(n).astype(np.float32) + 1.0
    else:
        r = rng.integers(-1, 3, size=n).astype(np.float32)
        r[r == 0] = np.where(rng.random((r == 0).sum()) < 0.5, -0.0, 0.0)
        r[rng.choice(n, size=n // 10, replace=False)] = np.nan
    # candidates: a random 60 % of the entries (all of them for kinds *_all), in
    # ascending order, from the reference's gate
    gate = np.where(rng.random(n) < (1.0 if kind.endswith("_all") else 0.6), 1.0, -1.0)
    cand, cnt = ref.select(gate, es, lens)
    announce(f"topk lens={lens.tolist()} k={k} kind={kind}")
    ti, tc = _topk_gpu(r, lens, es, cand, cnt, k, int(lens.max()))
    tr, tcr = ref.topk(r.astype(np.float64), es, lens, cand, cnt, k)
    np.testing.assert_array_equal(tc, tcr)
    for b in range(len(lens)):
        np.testing.assert_array_equal(ti[b, :tc[b]], tr[b, :tcr[b]])
        assert np.all(ti[b, tc[b]:] == -7), "entries past the count must be untouched"


# -------------------------------------------------------------- attention

def _attend_gpu(wl, idx, cnt, scale=None):
    B, T, Hq, Dl = wl.qa.shape
    use_hca = wl.hca is not None
    ws = torch.empty(max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_ATTEND, B, T, Hq, Dl, k=wl.k,
                                                   max_hca=wl.max_hca)),
                     dtype=torch.uint8, device="cuda")
    qa = dev(wl.qa)
    out = torch.full(qa.shape, float("nan"), dtype=qa.dtype, device="cuda")
    lse = torch.full((B, T, Hq), float("nan"), device="cuda")
    lsa.lsa_sparse_attend(qa, dev(wl.latent), dev(wl.latent_row_start), dev(idx), dev(cnt), wl.k,
                          out, hca=dev(wl.hca) if use_hca else None,
                          hca_row_start=dev(wl.hca_row_start) if use_hca else None,
                          hca_count=dev(wl.hca_count) if use_hca else None, max_hca=wl.max_hca,
                          scale=wl.scale if scale is None else scale, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    o = host(out)
    o = bf16_to_f64(o) if o.dtype == np.uint16 else o.astype(np.float64)
    return o, host(lse)


def _attend_ref(ref, wl, idx, cnt, scale=None):
    return ref.sparse_attend(wl.qa, wl.latent, wl.latent_row_start, idx, cnt, wl.k, wl.hca,
                             wl.hca_row_start, wl.hca_count,
                             wl.scale if scale is None else scale)


def _random_indices(rng, lens, k, counts):
    B = len(lens)
    idx = np.full((B, k), -1, np.int32)
    for b in range(B):
        c = counts[b]
        idx[b, :c] = np.sort(rng.choice(lens[b], size=c, replace=False))
    return idx, np.asarray(counts, np.int32)


def test_attend_tiny_fp32(ref):
    wl = inputs.make_workload("tiny")
    rng = np.random.default_rng(0)
    idx, cnt = _random_indices(rng, wl.seq_len, wl.k, [50])
    announce("attend tiny fp32 vector path")
    o, l = _attend_gpu(wl, idx, cnt)
    orf, lr = _attend_ref(ref, wl, idx, cnt)
    check_attention(o, orf, l, lr)


@pytest.mark.parametrize("B,T,Hq,Dl,lens,counts,hca,k", [
    (3, 1, 64, 512, [900, 500, 300], [256, 100, 0], [300, 0, 17], 256),
    (1, 1, 64, 512, [5000], [1024], None, 1024),                 # split over rows
    (2, 3, 16, 256, [400, 400], [77, 128], [33, 5], 128),
    (2, 1, 64, 128, [300, 40], [200, 40], [64, 0], 200),
    (2, 2, 33, 512, [250, 250], [64, 31], None, 64),             # heads not a multiple of 16
    (1, 1, 64, 512, [100], [0], [0], 16),                        # nothing to attend
    (4, 1, 8, 96, [80, 80, 80, 80], [10, 0, 80, 1], [3, 0, 0, 2], 80),  # vector path, bf16
    (2, 4, 64, 512, [3000, 2500], [700, 2048], [200, 50], 2048),  # 4 positions, row splits
    (1, 1, 96, 512, [600], [300], [40], 512),                    # 2 groups of query rows: 64, then 32
    (3, 5, 7, 128, [90, 200, 64], [90, 3, 64], [1, 0, 9], 96),   # 35 query rows per sequence
])
def test_attend_bf16(ref, B, T, Hq, Dl, lens, counts, hca, k):
    wl = inputs.random_small(B * 31 + Dl, B, 1, 4, 32, lens, k=k, Hq=Hq, Dl=Dl, hca_lens=hca)
    if T > 1:
        rng0 = np.random.default_rng(T)
        wl.qa = inputs.to_bf16_bits(rng0.standard_normal((B, T, Hq, Dl)).astype(np.float32))
    rng = np.random.default_rng(B + Dl)
    idx, cnt = _random_indices(rng, wl.seq_len, k, counts)
    announce(f"attend B={B} T={T} Hq={Hq} Dl={Dl} counts={counts} hca={hca}")
    o, l = _attend_gpu(wl, idx, cnt)
    orf, lr = _attend_ref(ref, wl, idx, cnt)
    check_attention(o, orf, l, lr)


def test_attend_many_splits(ref):
    """One sequence with 2048 top-k rows and 200 000 HCA rows: about 250 row
    splits, so the merge of the splits runs over several batches of them."""
    wl = inputs.random_small(4242, 1, 1, 4, 32, [3000], k=2048, Hq=64, Dl=512,
                             hca_lens=[200000])
    rng = np.random.default_rng(42)
    idx, cnt = _random_indices(rng, wl.seq_len, wl.k, [2048])
    announce("attend 2048 + 200000 rows, ~250 row splits")
    o, l = _attend_gpu(wl, idx, cnt)
    with ref.threads():
        orf, lr = _attend_ref(ref, wl, idx, cnt)
    check_attention(o, orf, l, lr)


@pytest.mark.parametrize("growth", [0.0, 6.0, 40.0])
def test_attend_running_max_moves(ref, growth):
    """Logits that grow along the attended list, so the running maximum moves
    in later chunks of every split (and by more than any fixed slack)."""
    S, Hq, Dl = 3000, 64, 512
    wl = inputs.random_small(311, 1, 1, 4, 32, [S], k=2048, Hq=Hq, Dl=Dl, hca_lens=[900])
    # latent row i gets a logit offset rising by ~growth over every 64 rows (the
    # row splits here are 64 rows long, two chunks), along qa's mean direction
    qa = bf16_to_f64(wl.qa)[0, 0]
    u = qa.mean(axis=0)
    u /= np.linalg.norm(u)
    lat = bf16_to_f64(wl.latent)
    ramp = growth * (np.arange(S) % 64) / 64
    wl.latent = inputs.to_bf16_bits((lat + ramp[:, None] * u[None, :] * np.sqrt(Dl)).astype(np.float32))
    hca = bf16_to_f64(wl.hca)
    wl.hca = inputs.to_bf16_bits((hca + growth * u[None, :] * np.sqrt(Dl)).astype(np.float32))
    rng = np.random.default_rng(5)
    idx, cnt = _random_indices(rng, wl.seq_len, wl.k, [2048])
    announce(f"attend running max moves growth={growth}")
    o, l = _attend_gpu(wl, idx, cnt)
    orf, lr = _attend_ref(ref, wl, idx, cnt)
    check_attention(o, orf, l, lr)


@pytest.mark.parametrize("scale_mul", [-3.0, -40.0, 0.0, 8.0])
def test_attend_scale_sign(ref, scale_mul):
    """Negative, zero and large softmax scales on the matrix-core path (full and
    partial chunks, row splits, HCA rows): the slack test of a full chunk takes
    the largest raw product of a lane for a positive scale and the smallest for
    a negative one (at -40 the logits span hundreds of powers of two, so a
    running maximum that missed a growth would overflow the probabilities), and
    a zero scale gives every attended row the same weight."""
    wl = inputs.random_small(733, 2, 1, 4, 32, [2500, 700], k=1024, Hq=64, Dl=512,
                             hca_lens=[300, 45])
    rng = np.random.default_rng(7)
    idx, cnt = _random_indices(rng, wl.seq_len, wl.k, [1024, 333])
    scale = wl.scale * scale_mul
    announce(f"attend scale {scale_mul} x 1/sqrt(Dl)")
    o, l = _attend_gpu(wl, idx, cnt, scale=scale)
    orf, lr = _attend_ref(ref, wl, idx, cnt, scale=scale)
    check_attention(o, orf, l, lr)


def test_attend_all_selected_equals_dense(ref):
    """Every entry kept, k >= S, no HCA: sparse attention is dense attention (torch, fp64)."""
    S, Hq, Dl = 700, 64, 512
    wl = inputs.random_small(77, 1, 1, 4, 32, [S], k=1024, Hq=Hq, Dl=Dl)
    idx = np.full((1, 1024), -1, np.int32)
    idx[0, :S] = np.arange(S)
    cnt = np.array([S], np.int32)
    announce("attend dense equivalence")
    o, l = _attend_gpu(wl, idx, cnt)
    q = torch.from_numpy(bf16_to_f64(wl.qa)[0, 0])[None, :, None, :]
    kv = torch.from_numpy(bf16_to_f64(wl.latent))[None, None].expand(1, Hq, S, Dl)
    dense = torch.nn.functional.scaled_dot_product_attention(q, kv, kv, scale=wl.scale)
    check_attention(o[0, 0], dense[0, :, 0, :].numpy())
