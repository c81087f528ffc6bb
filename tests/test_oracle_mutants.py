"""Plant plausible mistakes in copies of the CPU reference and check that the pins catch them.

Each mutant is an altered copy of oracle/lsa_oracle.c compiled into a temporary
directory; the real reference is never modified.  A mutant passes this test
when at least one pin of test_oracle_pins.py fails against it.
"""
import inspect

import pytest

import test_oracle_pins as pins

MUTANTS = {
    "drop_relu_gate": ("dot > 0.0 ? dot : 0.0", "dot"),
    "bias_sign": ("const double z = u + bias;", "const double z = u - bias;"),
    "q_index_transposed": ("const int64_t qrow = (((int64_t)b * T + t) * H + h) * (int64_t)D;",
                           "const int64_t qrow = (((int64_t)b * H + h) * T + t) * (int64_t)D;"),
    "weight_index_dropped": ("u += (double)w[((int64_t)b * T + t) * H + h] * gated;",
                             "u += (double)w[h] * gated;"),
    "sigmoid_sign": ("prob_out[o] = 1.0 / (1.0 + exp(-z));", "prob_out[o] = 1.0 / (1.0 + exp(z));"),
    "union_uses_min": ("} else if (t == 0 || z > m) {", "} else if (t == 0 || z < m) {"),
    "bf16_shift": ("(uint32_t)((const uint16_t*)base)[i] << 16;",
                   "(uint32_t)((const uint16_t*)base)[i] << 15;"),
    "gate_strict": ("if (v >= threshold) {", "if (v > threshold) {"),
    "tie_break_reversed": ("return (a->s > b->s) - (a->s < b->s);",
                           "return (a->s < b->s) - (a->s > b->s);"),
    "nan_ranked_first": ("if (an != bn) return an ? 1 : -1;", "if (an != bn) return an ? -1 : 1;"),
    "topk_keeps_k_plus_one": ("const int32_t keep = n < k ? n : k;",
                              "const int32_t keep = n < k + 1 ? n : k + 1;"),
    "attend_unscaled": ("logit[j] = scale * dot;", "logit[j] = dot;"),
    "attend_unnormalised": ("for (int d = 0; d < Dl; ++d) o[d] /= Z;", ""),
    "lse_missing_max": ("if (lse) lse[lidx] = mu + log(Z);", "if (lse) lse[lidx] = log(Z);"),
    "hca_dropped": ("const int32_t nh = hca ? hca_count[b] : 0;", "const int32_t nh = 0;"),
    "hca_row_offset": ("row_off[nt + i] = (hca_row_start[b] + i) * (int64_t)Dl;",
                       "row_off[nt + i] = (hca_row_start[b]) * (int64_t)Dl;"),
    "rescore_no_relu": ("(dot < 0.0 ? 0.0 : dot)", "dot"),
    "rescore_weight_of_head_only": ("r += (double)w[(int64_t)b * H + h] *", "r += (double)w[h] *"),
    "rescore_row_by_position": ("const int64_t krow = (key_row_start[b] + s) * (int64_t)D;\n            double r",
                                "const int64_t krow = (key_row_start[b] + j) * (int64_t)D;\n            double r"),
    "union_drops_previous": ("if (reduce_max == 2 && (isnan(m) || prev > m)) m = prev;", ""),
    "union_takes_min": ("if (reduce_max == 2 && (isnan(m) || prev > m)) m = prev;",
                        "if (reduce_max == 2 && (isnan(m) || prev < m)) m = prev;"),
    "positions_are_entries": ("out[j] = out_positions ? items[j].j : items[j].s;",
                              "out[j] = items[j].s;"),
    "fetch_dst_offset_dropped": ("const int64_t to = dst_row_start[b] + j;",
                                 "const int64_t to = j;"),
    "fetch_src_offset_dropped": ("const int64_t from = src_row_start[b] + idx[idx_start[b] + j];",
                                 "const int64_t from = idx[idx_start[b] + j];"),
    "encoder_down_transposed": ("acc += load_elem(w_down, dtype, (int64_t)i * d_model + k) *",
                                "acc += load_elem(w_down, dtype, (int64_t)k * r + i) *"),
    "encoder_up_head_offset_dropped": ("const int64_t urow = ((int64_t)hd * D + d) * r;",
                                       "const int64_t urow = ((int64_t)d) * r;"),
    "encoder_gate_reads_down": ("acc += load_elem(w_gate, dtype, (int64_t)hd * d_model + k) *",
                                "acc += load_elem(w_down, dtype, (int64_t)hd * d_model + k) *"),
    "encoder_token_row_dropped": ("const int64_t hrow = (int64_t)m * d_model;",
                                  "const int64_t hrow = 0;"),
    "encoder_latent_of_token0": ("acc += load_elem(w_up, dtype, urow + i) * c_out[(int64_t)m * r + i];",
                                 "acc += load_elem(w_up, dtype, urow + i) * c_out[i];"),
    "fetch_list_offset_dropped": ("const int64_t from = src_row_start[b] + idx[idx_start[b] + j];",
                                  "const int64_t from = src_row_start[b] + idx[j];"),
}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = list(inspect.signature(fn).parameters)
        if params == ["ref"]:
            out.append((name, fn, None))
        elif params == ["ref", "seed"]:
            for seed in range(12):
                out.append((f"{name}[{seed}]", fn, seed))
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_reject_mutant(mutant, tmp_path, ref):
    old, new = MUTANTS[mutant]
    src = ref.source_text()
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = ref.compile_variant(src.replace(old, new), str(tmp_path), "mut_" + mutant)
    ref.use_library(path)
    failed = []
    try:
        for name, fn, seed in _pin_functions():
            try:
                fn(ref) if seed is None else fn(ref, seed)
            except (AssertionError, ValueError):
                failed.append(name)
    finally:
        ref.use_library(None)
    assert failed, f"no pin rejects mutant {mutant}"


def test_unmutated_reference_passes_every_pin(ref):
    for name, fn, seed in _pin_functions():
        fn(ref) if seed is None else fn(ref, seed)
