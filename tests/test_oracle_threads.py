"""The OpenMP build of the CPU reference against its single-threaded build.

The same source is compiled twice; the threaded build only shares out
independent loop iterations, so every output must match bit for bit.  The
full-size GPU parity tests and the CPU baseline use the threaded build.
"""
import numpy as np

from lookahead_sparse_kv_amd import inputs


def _both(ref, fn):
    single = fn()
    with ref.threads():
        assert ref.max_threads() >= 1
        multi = fn()
    return single, multi


def _same(a, b):
    if isinstance(a, tuple):
        for x, y in zip(a, b):
            _same(x, y)
    elif a is None:
        assert b is None
    else:
        assert a.dtype == b.dtype and a.shape == b.shape
        assert a.tobytes() == b.tobytes()


def test_single_build_reports_one_thread(ref):
    assert ref.max_threads() == 1


def test_threaded_matches_single_on_tiny(ref):
    wl = inputs.make_workload("tiny")

    def run():
        z, p = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                               wl.bias, reduce_max=True)
        zt, pt = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q,
                                 wl.w, wl.bias, reduce_max=False)
        c, n = ref.select(z, wl.entry_start, wl.seq_len)
        t, tn = ref.topk(z, wl.entry_start, wl.seq_len, c, n, wl.k)
        tp, tpn = ref.topk(z, wl.entry_start, wl.seq_len, c, n, wl.k, positions=True)
        o, l = ref.sparse_attend(wl.qa, wl.latent, wl.latent_row_start, t, tn, wl.k, wl.hca,
                                 wl.hca_row_start, wl.hca_count, wl.scale)
        return z, p, zt, pt, c, n, t, tn, tp, tpn, o, l

    _same(*_both(ref, run))


def test_threaded_matches_single_ragged_multi_position(ref):
    """Ragged bf16 batch with several positions, HCA rows, an empty sequence,
    the union mode, the re-score and the encoder."""
    wl = inputs.random_small(77, 3, 4, 8, 64, [700, 0, 1234], k=96, Hq=16, Dl=128,
                             hca_lens=[5, 3, 0], bias=-2.0)
    nq, nw = inputs.native_queries(wl)
    h, wd, wu, wg = (inputs.hidden_states(5, d_model=128),) + tuple(
        inputs.encoder_weights(4, 32, d_model=128, rank=64))

    def run():
        z, p = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                               wl.bias, reduce_max=True)
        zu, pu = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q,
                                 wl.w, wl.bias + 0.5, union_with=z)
        c, n = ref.select(zu, wl.entry_start, wl.seq_len)
        r = ref.index_rescore(wl.keys, wl.key_row_start, wl.entry_start, c, n, nq, nw)
        t, tn = ref.topk(r, wl.entry_start, wl.seq_len, c, n, wl.k)
        o, l = ref.sparse_attend(wl.qa, wl.latent, wl.latent_row_start, t, tn, wl.k, wl.hca,
                                 wl.hca_row_start, wl.hca_count, wl.scale)
        enc = ref.query_encode(h, wd, wu, wg, 4, 32)
        return (z, p, zu, pu, c, n, r, t, tn, o, l) + tuple(enc)

    _same(*_both(ref, run))
