"""Write tests/golden/workload_bias.json: the indexer bias of each synthetic workload
(the generator lookahead_sparse_kv_amd/inputs.py carries the same values in
WORKLOAD_BIAS; a CPU test checks the two agree).

The bias is an input of the score (a scalar per indexer).  It is chosen so that
each workload keeps about the fraction of entries the pages quote (13.5 % on
average, 10 % at 500K tokens), by scoring the drawn keys with the CPU
reference only (bias 0), then placing the threshold in the widest gap between
neighbouring scores near the wanted rank, which leaves few entries near the
gate.  Run from the repo root:  python tests/golden/make_workload_bias.py
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, REPO)

from lookahead_sparse_kv_amd import inputs  # noqa: E402
from oracle import oracle  # noqa: E402


def widest_gap_threshold(values: np.ndarray, target_count: int, window: float) -> float:
    """Threshold between two neighbours of the sorted (descending) values,
    at the widest gap among ranks within +-window of target_count."""
    v = np.sort(values)[::-1]
    lo = max(1, int(target_count * (1 - window)))
    hi = min(len(v) - 1, int(target_count * (1 + window)))
    gaps = v[lo - 1:hi] - v[lo:hi + 1]          # gap below rank r (r kept)
    i = int(np.argmax(gaps))
    return 0.5 * (v[lo - 1 + i] + v[lo + i])


def bias_for(name: str, seed: int) -> dict:
    wl = inputs.make_workload(name, seed, bias=0.0, with_attention=False)
    t0 = time.time()
    if name == "tiny":
        u, _ = oracle.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                                  0.0, want_prob=False)
        thr = widest_gap_threshold(u, int(round(0.135 * len(u))), 0.05)
        how = "widest gap within 5% of rank 0.135*S over all entries"
    elif name == "burst_tau64":
        rng = np.random.Generator(np.random.PCG64(seed + 1))
        rows = np.sort(rng.choice(wl.keys.shape[0], size=2048, replace=False))
        sub = wl.keys[rows]
        n = len(rows)
        m, _ = oracle.index_score(sub, np.zeros(wl.B, np.int64), np.full(wl.B, n, np.int32),
                                  np.arange(wl.B, dtype=np.int64) * n, wl.q, wl.w, 0.0,
                                  reduce_max=True, want_prob=False)
        thr = widest_gap_threshold(m, int(round(0.135 * len(m))), 0.05)
        how = "union (max over positions) of a 2048-entry sample, widest gap near 13.5%"
    else:
        u, _ = oracle.index_score(wl.keys, wl.key_row_start, wl.seq_len, wl.entry_start, wl.q, wl.w,
                                  0.0, want_prob=False)
        noise = u[~wl.planted]
        thr = widest_gap_threshold(noise, int(round(inputs.NOISE_PASS * len(noise))), 0.10)
        how = "noise entries only: widest gap within 10% of a 2% pass rate"
    bias = float(np.float32(-thr))
    return {"bias": bias, "rule": how, "seconds": round(time.time() - t0, 1)}


TABLE = os.path.join(HERE, "workload_bias.json")


def main(argv):
    names = argv[1:] or list(inputs.CONFIGS)
    table = {}
    if os.path.exists(TABLE):
        with open(TABLE) as f:
            table = json.load(f)
    for name in names:
        seed = inputs.DEFAULT_SEED[name]
        entry = bias_for(name, seed)
        table[f"{name}:{seed}"] = entry
        print(name, seed, entry, flush=True)
        with open(TABLE, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv)
