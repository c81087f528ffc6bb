"""GPU parity of the Memory-Indexer query encoder (lsa_query_encode) against the
CPU reference (oracle O0) on identical seeded inputs.

Tolerance, derived from the arithmetic: products of bf16 values are exact in
fp32 and the sums of n of them are within gamma(n) * sum|terms| of the exact
sum (gamma(n) = n u / (1 - n u), u = 2^-24; doubled here to cover any
accumulation order inside the matrix cores).  c is rounded to bf16 (relative
2^-8 at most), then multiplied by W_up, and q is rounded to bf16 again; w stays
fp32.  So, element by element:
    |c_gpu - c|  <= dc = 2 gamma(K) A + 2^-8 (|c| + 2 gamma(K) A),  A = |W_down| |h|
    |q_gpu - q|  <= |W_up| dc + 2 gamma(r) |W_up| (|c| + dc)  (+ 2^-8 of |q| plus all that)
    |w_gpu - w|  <= 2 gamma(K) |W_gate| |h|
and, as the rounding errors are unbiased, the RMS error of q stays below 2^-8 of
the RMS of q.  Integer-valued inputs make every step exact.
"""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev, host
from lookahead_sparse_kv_amd import binding as lsa
from lookahead_sparse_kv_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lsa.load_library()


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1.0 - n * u)


def _f64(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def _encode_gpu(h, wd, wu, wg, H, D):
    M = h.shape[0]
    r = wd.shape[0]
    c = torch.full((M, r), float("nan"), dtype=torch.bfloat16, device="cuda")
    q = torch.full((M, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    w = torch.full((M, H), float("nan"), device="cuda")
    lsa.lsa_query_encode(dev(h), dev(wd), dev(wu), dev(wg), H, D, c, q, w)
    torch.cuda.synchronize()
    return host(c), host(q), host(w)


def _bounds(h, wd, wu, wg, H, D, c_r, q_r):
    """Elementwise error bounds (dc, dq, dw) of the GPU outputs for tokens h."""
    K, r = h.shape[1], wd.shape[0]
    M = h.shape[0]
    ha, wda, wua, wga = (np.abs(_f64(x)) for x in (h, wd, wu, wg))
    A = ha @ wda.T
    dc = 2 * _gamma(K) * A + 2.0 ** -8 * (np.abs(c_r) + 2 * _gamma(K) * A)
    dq = dc @ wua.T + 2 * _gamma(r) * ((np.abs(c_r) + dc) @ wua.T)
    dq = (dq + 2.0 ** -8 * (np.abs(q_r.reshape(M, -1)) + dq)).reshape(M, H, D)
    dw = 2 * _gamma(K) * (ha @ wga.T)
    return dc, dq, dw


def _check(rows, h, wd, wu, wg, H, D, got, ref):
    """Compare GPU outputs of token rows `rows` with the reference on h[rows]."""
    c_g, q_g, w_g = (_f64(got[0][rows]), _f64(got[1][rows]), got[2][rows].astype(np.float64))
    c_r, q_r, w_r = ref
    dc, dq, dw = _bounds(h[rows], wd, wu, wg, H, D, c_r, q_r)
    assert np.all(np.abs(c_g - c_r) <= dc), "latent c outside its bound"
    assert np.all(np.abs(q_g - q_r) <= dq), "queries outside their bound"
    assert np.all(np.abs(w_g - w_r) <= dw), "gate weights outside their bound"
    rms = np.sqrt(np.mean((q_g - q_r) ** 2))
    assert rms <= 2.0 ** -8 * np.sqrt(np.mean(q_r ** 2)), rms


def _sample_rows(M, n=24, seed=0):
    """All rows of a small M; else n rows including both ends and 128-row tile edges."""
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed + M)
    edges = [0, M - 1] + [e for t in range(128, M, 128) for e in (t - 1, t)]
    rows = set(edges[:n // 2]) | set(rng.choice(M, size=n, replace=False).tolist())
    return np.array(sorted(rows)[:n])


@pytest.mark.parametrize("M,d_model,rank,H,D", [
    (1, 256, 64, 2, 32),        # one token
    (1, 4096, 192, 3, 40),      # one token: K split over 8 waves, one row per workgroup (195)
    (1, 4608, 2560, 2, 64),     # one token: more row blocks than CUs (2562 rows, 8 per block)
    (5, 512, 128, 4, 32),       # few tokens: weight-streaming kernel, one 16-row tile
    (17, 256, 192, 3, 40),      # two token tiles, ragged N (H*D = 120), gate past a tile edge
    (32, 4096, 64, 2, 64),      # long K: 16 waves share it
    (3, 4096, 192, 3, 40),      # few tokens, long K: 4-row vector kernel, ragged last block
    (8, 8192, 64, 1, 64),       # eight tokens, long K, the gate row alone in the last block
    (33, 192, 64, 3, 40),       # many tokens, small tiles, ragged everywhere
    (300, 512, 256, 8, 64),     # small tiles, ragged M
    (520, 256, 512, 64, 128),   # up product on large tiles (enough to fill the chip), ragged M
])
def test_encode_parity(ref, M, d_model, rank, H, D):
    wd, wu, wg = inputs.encoder_weights(H, D, d_model, rank, seed=M + rank)
    h = inputs.hidden_states(M, d_model, seed=d_model + H)
    announce(f"encode M={M} d_model={d_model} rank={rank} H={H} D={D}")
    got = _encode_gpu(h, wd, wu, wg, H, D)
    rows = _sample_rows(M)
    _check(rows, h, wd, wu, wg, H, D, got, ref.query_encode(h[rows], wd, wu, wg, H, D))


@pytest.mark.parametrize("M", [1, 8, 1024])
def test_encode_full_size_sampled(ref, M):
    """The benchmark's sizes (d_model 7168, rank 1536, 64 heads of 128): decode
    (1 and 8 tokens) and the tau-burst (1024 tokens), reference on sampled tokens."""
    H, D = 64, 128
    wd, wu, wg = inputs.encoder_weights(H, D)
    h = inputs.hidden_states(M)
    announce(f"encode full size M={M}")
    got = _encode_gpu(h, wd, wu, wg, H, D)
    rows = _sample_rows(M, n=6)
    _check(rows, h, wd, wu, wg, H, D, got, ref.query_encode(h[rows], wd, wu, wg, H, D))


@pytest.mark.parametrize("M,d_model,rank,H,D", [
    (1, 7168, 1536, 64, 128),
    (8, 7168, 1536, 64, 128),
    (200, 1024, 256, 16, 64),
])
def test_encode_exact_integer_inputs(ref, M, d_model, rank, H, D):
    """Entries in {-1, 0, 1}: every sum is an exact integer in fp32 and c fits bf16
    exactly, so c and q equal the reference rounded once to bf16, and w equals it."""
    wd, wu, wg = inputs.encoder_weights(H, D, d_model, rank, seed=3, int_valued=True)
    h = inputs.hidden_states(M, d_model, seed=4, int_valued=True)
    announce(f"encode exact M={M} d_model={d_model}")
    c_g, q_g, w_g = _encode_gpu(h, wd, wu, wg, H, D)
    c_r, q_r, w_r = ref.query_encode(h, wd, wu, wg, H, D)
    assert np.all(np.abs(c_r) <= 256)
    np.testing.assert_array_equal(c_g, inputs.to_bf16_bits(c_r.astype(np.float32)))
    np.testing.assert_array_equal(q_g, inputs.to_bf16_bits(q_r.astype(np.float32)))
    np.testing.assert_array_equal(w_g.astype(np.float64), w_r)


def test_encode_feeds_score(ref):
    """Encoder -> score on the GPU against encoder -> score in the reference: the
    gap is the score's own 1e-3 plus what the encoder bounds allow, carried
    through z = sum_h w_h ReLU(q_h . k) (ReLU is 1-Lipschitz)."""
    H, D, B = 16, 128, 3
    wl = inputs.random_small(5, B, 1, H, D, [700, 90, 2000], bias=-1.0)
    wd, wu, wg = inputs.encoder_weights(H, D, 1024, 256, seed=9)
    h = inputs.hidden_states(B, 1024, seed=10)
    c = torch.empty((B, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((B, 1, H), device="cuda")
    announce("encode -> score")
    lsa.lsa_query_encode(dev(h), dev(wd), dev(wu), dev(wg), H, D, c, q, w)
    z = torch.empty(wl.total_entries, device="cuda")
    lsa.lsa_index_score(dev(wl.keys), dev(wl.key_row_start), dev(wl.seq_len), dev(wl.entry_start),
                        wl.max_len, q, w, wl.bias, 1, z)
    torch.cuda.synchronize()
    z_g = host(z).astype(np.float64)
    c_r, q_r, w_r = ref.query_encode(h, wd, wu, wg, H, D)
    _, dq, dw = _bounds(h, wd, wu, wg, H, D, c_r, q_r)
    # the reference score of the reference encoder's q and w (passed to it in fp32,
    # with the keys widened exactly, so the fp32 rounding joins the bounds)
    q32, w32 = q_r.astype(np.float32), w_r.astype(np.float32)
    dq = dq + np.abs(q32.astype(np.float64) - q_r)
    dw = dw + np.abs(w32.astype(np.float64) - w_r)
    keys32 = inputs.bf16_bits_to_f32(wl.keys)
    z_r, _ = ref.index_score(keys32, wl.key_row_start, wl.seq_len, wl.entry_start, q32[:, None],
                             w32[:, None], wl.bias, reduce_max=True, want_prob=False)
    for b in range(B):
        S, krs, es = int(wl.seq_len[b]), int(wl.key_row_start[b]), int(wl.entry_start[b])
        k = keys32[krs:krs + S].astype(np.float64)
        dots = np.maximum(k @ q_r[b].T, 0.0)                   # ReLU(q_h . k), [S, H]
        err_dot = np.abs(k) @ dq[b].T                          # bound on |delta(q_h . k)|
        tol = 1e-3 + err_dot @ (np.abs(w_r[b]) + dw[b]) + (dots + err_dot) @ dw[b]
        assert np.all(np.abs(z_g[es:es + S] - z_r[es:es + S]) <= tol)
