"""The synthetic workloads realise the shapes and selection fractions they are meant to have.

Fractions are measured with the CPU reference on the drawn inputs, so these
tests also pin the stored bias table (tests/golden/workload_bias.json) and its copy in
inputs.WORKLOAD_BIAS."""
import numpy as np
import pytest

from lookahead_sparse_kv_amd import inputs


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e38], np.float32)
    bits = inputs.to_bf16_bits(x)
    back = inputs.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert back[1] == 1.0
    assert back[2] == 1.0078125
    assert back[0] == 1.0 and back[3] == 1.0078125 and back[4] == -2.5
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8 + 1e-45)


@pytest.mark.parametrize("name,lo,hi", [("tiny", 0.12, 0.15), ("decode_128k", 0.12, 0.15)])
def test_selected_fraction(ref, name, lo, hi):
    wl = inputs.make_workload(name, with_attention=False)
    z, _ = ref.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                           wl.bias, want_prob=False)
    frac = float((z >= 0).mean())
    assert lo <= frac <= hi, frac
    if wl.planted.any():
        assert (z[wl.planted] >= 0).mean() > 0.99


def test_decode_500k_shape_and_fraction(ref):
    wl = inputs.make_workload("decode_500k", with_attention=False)
    assert wl.B == 8 and np.all(wl.seq_len == 125000) and wl.keys.shape == (1_000_000, 128)
    # score one sequence (125000 entries) with the reference
    S = int(wl.seq_len[0])
    z, _ = ref.index_score(wl.keys[:S], np.zeros(1, np.int64), wl.seq_len[:1], np.zeros(1, np.int64),
                           wl.q[:1], wl.w[:1], wl.bias, want_prob=False)
    frac = float((z >= 0).mean())
    assert 0.085 <= frac <= 0.115, frac


def test_burst_shape_and_union_fraction(ref):
    wl = inputs.make_workload("burst_tau64", with_attention=False)
    assert (wl.B, wl.T) == (16, 64) and wl.keys.shape == (65536, 128)
    assert np.all(wl.key_row_start == 0)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(65536, 512, replace=False))
    n = len(rows)
    m, _ = ref.index_score(wl.keys[rows], np.zeros(wl.B, np.int64), np.full(wl.B, n, np.int32),
                           np.arange(wl.B, dtype=np.int64) * n, wl.q, wl.w, wl.bias,
                           reduce_max=True, want_prob=False)
    frac = float((m >= 0).mean())
    assert 0.10 <= frac <= 0.17, frac


def test_ragged_mix_shapes():
    wl = inputs.make_workload("ragged_mix", with_attention=False)
    assert wl.B == 32
    tokens = wl.seq_len.astype(np.int64) * inputs.TOKENS_PER_ENTRY
    assert np.all(tokens % 128 == 0) and tokens.min() >= 65536 and tokens.max() <= 524288
    assert np.all(np.diff(wl.key_row_start) == wl.seq_len[:-1])
    assert np.all((wl.target_fraction >= 0.05) & (wl.target_fraction <= 0.25))
    planted = np.add.reduceat(wl.planted.astype(np.int64), wl.key_row_start.astype(np.int64))
    pf = planted / wl.seq_len
    assert np.all(np.abs(pf - (wl.target_fraction - inputs.NOISE_PASS)) < 0.01)


def test_tiny_attention_side():
    wl = inputs.make_workload("tiny")
    assert wl.qa.shape == (1, 1, 8, 64) and wl.latent.shape == (1024, 64)
    assert wl.qa.dtype == np.float32 and wl.hca is None and wl.k == 64


def test_embedded_bias_table_equals_the_golden_file():
    """inputs.WORKLOAD_BIAS is the table tests/golden/make_workload_bias.py writes."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "workload_bias.json")
    table = json.load(open(path))
    assert {k: float(v["bias"]) for k, v in table.items()} == inputs.WORKLOAD_BIAS
