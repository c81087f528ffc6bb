"""Benchmark of the LSA hot path on one MI355X.

One step = one pass of the whole path over one batch: index score (max over
positions) -> gate + compaction -> top-k -> sparse attention, all enqueued on
one stream.  Also timed, outside the step: the native indexer's per-step
re-score of the kept entries with its top-k, the OR-mode union of three
indexers, the query encoder, the cold-pool fetch, and -- on its own workload
(16 sequences x 64 positions against one shared set of 65536 entries) -- the
tau-burst trigger score on the matrix cores.  The default workload is 8
sequences at 500K tokens (125000 compressed entries each, 3907 HCA rows, top-k
2048, latent 512, 64 heads).

Prints one JSON line.  `value` = indexer scores per second of whole steps
(sum of S_b per step / step time).  The roofline object covers the score
kernel, the dominant one by bytes; attention, re-score, union, encoder and
the tau-burst score get their own.  HBM fractions are given against the
8 TB/s peak and against a 1 GiB read and a 1 GiB copy measured in the same
run.  Inputs are resident in HBM before timing; key and latent pools are
replicated and rotated so each timed launch reads memory the 256 MB on-die
cache does not hold.  Timed work is replayed from HIP graphs captured on one
stream; `latency_us` times single calls from one-launch graphs.  The CPU
baseline is the reference on all host cores, with its one-thread figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

METRIC = "indexer scores/sec + sparse-attn decode tokens/sec at 500K ctx; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, TFLOP/s
ROTATE_BYTES = 1 << 30         # distinct bytes per rotation cycle (>= 4x the on-die cache)
PROFILES = os.path.join(REPO, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_500k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=8, help="sequences the CPU baseline scores")
    ap.add_argument("--kernel-reps", type=int, default=0,
                    help="launches per timing interval (0 = pick for >= 1 ms)")
    ap.add_argument("--fetch-reps", type=int, default=4,
                    help="back-to-back fetches per timed interval")
    ap.add_argument("--profile-launches", type=int, default=0,
                    help="only run N launches of each kernel (for rocprofv3 counter runs)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="with --profile-launches: also run a plain copy of this many bytes")
    return ap.parse_args()


def src_sha(name: str) -> str:
    """Hash of a kernel source and the device header it includes."""
    h = hashlib.sha256()
    for f in (name, "common.hpp"):
        h.update(open(os.path.join(REPO, "lookahead_sparse_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, src: str):
    """HBM bytes per launch measured by rocprofv3 counters, if still valid for this source."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_sha") != src_sha(src):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def capture(torch, stream, fns):
    """One HIP graph holding the launches of `fns` in order (on `stream`)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    return g


def encoder_setup(torch, lsa, inputs, wl, rotate):
    """Encoder inputs for the workload's B*T tokens: weight replicas (enough to
    rotate through ROTATE_BYTES if rotate), hidden states and output buffers."""
    from lookahead_sparse_kv_amd.pipeline import _to_dev
    H, D, rk = wl.H, wl.D, inputs.ENCODER_RANK
    M = wl.B * wl.T
    w0 = [_to_dev(x, "cuda") for x in inputs.encoder_weights(H, D)]
    wbytes = sum(t.numel() * 2 for t in w0)
    nrep = max(1, -(-ROTATE_BYTES // wbytes)) if rotate else 1
    reps = [w0] + [[t.clone() for t in w0] for _ in range(nrep - 1)]
    h = _to_dev(inputs.hidden_states(M), "cuda")
    c = torch.empty((M, rk), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((M, H), dtype=torch.float32, device="cuda")

    def call(i):
        lsa.lsa_query_encode(h, *reps[i % nrep], H, D, c, q, w)
    return call, reps, h, wbytes


def time_encoder(torch, lsa, inputs, stream, wl, reps_for, args):
    """Seconds per lsa_query_encode call for the workload's B*T tokens, and per pair
    of torch.mm products of the same shapes; plus the sizes."""
    H, D, dm, rk = wl.H, wl.D, inputs.ENCODER_D_MODEL, inputs.ENCODER_RANK
    M = wl.B * wl.T
    call, reps, h, wbytes = encoder_setup(torch, lsa, inputs, wl, rotate=True)
    nrep = len(reps)
    calls = [lambda i=i: call(i) for i in range(max(nrep, reps_for(2e-5)))]
    t_enc = timed_graph(torch, stream, capture(torch, stream, calls), len(calls))
    # library reference: [W_down; W_gate] and W_up, transposed once, contiguous
    lib_w = [(torch.cat([r[0], r[2]]).t().contiguous(), r[1].t().contiguous()) for r in reps]
    cw = torch.empty((M, rk + H), dtype=torch.bfloat16, device="cuda")
    qq = torch.empty((M, H * D), dtype=torch.bfloat16, device="cuda")

    def lib_pair(i):
        a, b = lib_w[i % nrep]
        torch.mm(h, a, out=cw)
        torch.mm(cw[:, :rk], b, out=qq)
    lib_pair(0)                   # the library sets itself up outside graph capture
    torch.cuda.synchronize()
    calls = [lambda i=i: lib_pair(i) for i in range(len(calls))]
    t_lib = timed_graph(torch, stream, capture(torch, stream, calls), len(calls))
    flops = 2.0 * M * (dm * (rk + H) + rk * H * D)
    alg_bytes = wbytes + M * dm * 2 + 2 * M * rk * 2 + M * H * D * 2 + M * H * 4
    del reps, lib_w
    return {"t": t_enc, "t_lib": t_lib, "M": M, "flops": flops, "bytes": alg_bytes,
            "d_model": dm, "rank": rk}


def timed_eager(torch, stream, calls, launches, intervals=5, warm=1):
    """Median seconds per launch of `calls` (`launches` launches) issued eagerly on
    `stream`, for long launches whose issue cost is small beside their run time."""
    res = []
    with torch.cuda.stream(stream):
        for it in range(warm + intervals):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for c in calls:
                c()
            e1.record(stream)
            e1.synchronize()
            if it >= warm:
                res.append(e0.elapsed_time(e1) * 1e-3 / launches)
    return statistics.median(res)


def timed_graph(torch, stream, g, launches, intervals=10, warm=3):
    """Median seconds per launch over `intervals` replays of graph `g`, which holds
    `launches` launches; HIP events recorded on `stream`, where the graph runs."""
    res = []
    for it in range(warm + intervals):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        if it >= warm:
            res.append(e0.elapsed_time(e1) * 1e-3 / launches)
    return statistics.median(res)


def cpu_baseline(wl, nseq: int):
    """The CPU reference as it stands on sequences 0..nseq-1 of the workload: score,
    gate, top-k and attention of those sequences, on all host cores (its OpenMP
    build) and on one thread (its single-threaded build; the same arithmetic);
    returned as scores/s."""
    from oracle import oracle
    oracle.build()
    nseq = min(nseq, wl.B)
    hca = wl.hca is not None

    def path():
        z, _ = oracle.index_score(wl.keys, wl.key_row_start[:nseq], wl.seq_len[:nseq],
                                  wl.entry_start[:nseq], wl.q[:nseq], wl.w[:nseq], wl.bias,
                                  reduce_max=True, want_prob=False)
        c, n = oracle.select(z, wl.entry_start[:nseq], wl.seq_len[:nseq])
        t, tn = oracle.topk(z, wl.entry_start[:nseq], wl.seq_len[:nseq], c, n, wl.k)
        oracle.sparse_attend(wl.qa[:nseq], wl.latent, wl.latent_row_start[:nseq], t, tn, wl.k,
                             wl.hca, wl.hca_row_start[:nseq] if hca else None,
                             wl.hca_count[:nseq] if hca else None, wl.scale)

    with oracle.threads():
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        path()
        dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    path()
    dt1 = time.perf_counter() - t0
    scores = int(wl.seq_len[:nseq].sum()) * wl.T
    return {"value": scores / dt, "unit": "scores/s", "cores": threads, "kind": "oracle",
            "sample": f"whole path (score, gate, top-k, attention) of sequences 0..{nseq - 1} of "
                      f"{wl.B}, {scores} scores: {dt:.2f} s on {threads} threads, "
                      f"{dt1:.2f} s on one",
            "nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "value_1_thread": scores / dt1,
            "decode_tokens_per_s": nseq * wl.T / dt,
            "decode_tokens_per_s_1_thread": nseq * wl.T / dt1}


def cpu_burst_prefix(wl, prefix_all: int = 2048, prefix_one: int = 256):
    """The CPU reference's tau-burst score (max over the 64 positions) of every
    sequence against a prefix of the shared key set: `prefix_all` entries on all
    cores, `prefix_one` on one thread; scores/s (a score = one (position, entry)
    pair), labelled as prefix measurements."""
    from oracle import oracle

    def run(n):
        B = wl.B
        return oracle.index_score(wl.keys[:n], np.zeros(B, np.int64), np.full(B, n, np.int32),
                                  np.arange(B, dtype=np.int64) * n, wl.q, wl.w, wl.bias,
                                  reduce_max=True, want_prob=False)

    with oracle.threads():
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        run(prefix_all)
        dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    run(prefix_one)
    dt1 = time.perf_counter() - t0
    per = wl.B * wl.T
    return {"value": per * prefix_all / dt, "unit": "scores/s", "cores": threads,
            "kind": "oracle", "value_1_thread": per * prefix_one / dt1,
            "sample": f"prefix measurement: score + max over {wl.T} positions of {wl.B} "
                      f"sequences against the first {prefix_all} shared entries on {threads} "
                      f"threads ({dt:.2f} s), the first {prefix_one} on one ({dt1:.2f} s)"}


def measured_hbm(torch, stream, gather_rows: int, row_bytes: int, read_bytes: int,
                 nbytes: int = 1 << 30):
    """Ceilings measured in this run by libceiling.so (the best over a few grid sizes):
    a 1 GiB streaming read, a 1 GiB copy (read + write bytes counted), a streaming
    read of `read_bytes` (the score launch's size, so its launch ramp and tail
    weigh as they do in the score; four buffers rotate), and a gather of
    `gather_rows` random rows of `row_bytes` (the attention launch's row count and
    row size) from a 4 GiB pool, rotating over 24 index lists; GB/s."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(REPO, "lookahead_sparse_kv_amd", "libceiling.so"))
    P, L, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ceiling_read.argtypes = [P, L, I, P, P]
    lib.ceiling_copy.argtypes = [P, P, L, I, P]
    lib.ceiling_gather.argtypes = [P, P, L, L, I, P, P]
    st = ctypes.c_void_p(stream.cuda_stream)
    a = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")

    def ok(rc):
        assert rc == 0, f"ceiling kernel launch failed ({rc})"

    def best(fn, launches, grids):
        return min(timed_graph(torch, stream, capture(torch, stream, [lambda g=g: fn(g)] * launches),
                               launches) for g in grids)
    t_read = best(lambda g: ok(lib.ceiling_read(a.data_ptr(), nbytes, g, sink.data_ptr(), st)), 4,
                  (1024, 2048, 4096, 8192))
    t_copy = best(lambda g: ok(lib.ceiling_copy(a.data_ptr(), b.data_ptr(), nbytes, g, st)), 4,
                  (1024, 2048, 4096, 8192))
    del a, b
    rb = read_bytes // 16 * 16
    bufs = [torch.ones(rb // 4, dtype=torch.int32, device="cuda") for _ in range(4)]
    t_read_same = min(timed_graph(torch, stream, capture(torch, stream, [
        lambda i=i, g=g: ok(lib.ceiling_read(bufs[i % 4].data_ptr(), rb, g, sink.data_ptr(), st))
        for i in range(8)]), 8) for g in (1024, 2048, 4096, 8192))
    del bufs
    pool_rows = (4 << 30) // row_bytes
    pool = torch.empty(pool_rows * row_bytes // 4, dtype=torch.int32, device="cuda").fill_(5)
    gen = torch.Generator(device="cuda").manual_seed(1)
    lists = [torch.randperm(pool_rows, device="cuda", generator=gen)[:gather_rows]
             .to(torch.int32).sort().values for _ in range(24)]
    t_gather = min(timed_graph(torch, stream, capture(torch, stream, [
        lambda i=i, g=g: ok(lib.ceiling_gather(pool.data_ptr(), lists[i].data_ptr(), gather_rows,
                                               row_bytes, g, sink.data_ptr(), st))
        for i in range(24)]), 24) for g in (256, 512, 1024, 2048))
    del pool, lists
    return {"read_GBs": round(nbytes / t_read / 1e9, 1),
            "copy_GBs": round(2 * nbytes / t_copy / 1e9, 1),
            "read_GBs_score_size": round(rb / t_read_same / 1e9, 1), "score_size_bytes": rb,
            "gather_GBs": round(gather_rows * row_bytes / t_gather / 1e9, 1),
            "gather": f"{gather_rows} random {row_bytes}-byte rows (sorted indices) per launch",
            "bytes": nbytes}


def measured_row_gather(torch, stream, pools, rows, row_bytes: int):
    """A plain gather (libceiling.so) of the given pool rows, in the given order,
    rotating over `pools` (replicas of one pool, as the kernel it rates reads
    them); the best over a few grid sizes; GB/s."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(REPO, "lookahead_sparse_kv_amd", "libceiling.so"))
    P, L, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ceiling_gather.argtypes = [P, P, L, L, I, P, P]
    st = ctypes.c_void_p(stream.cuda_stream)
    idx = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int32)).cuda()
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    n = len(pools)

    def ok(rc):
        assert rc == 0, f"ceiling kernel launch failed ({rc})"
    t = min(timed_graph(torch, stream, capture(torch, stream, [
        lambda i=i, g=g: ok(lib.ceiling_gather(pools[i % n].data_ptr(), idx.data_ptr(), len(rows),
                                               row_bytes, g, sink.data_ptr(), st))
        for i in range(max(n, 8))]), max(n, 8)) for g in (256, 512, 1024, 2048))
    return len(rows) * row_bytes / t / 1e9


def measured_mfma(torch, stream, n: int = 8192, reps: int = 8):
    """The bf16 matrix rate a library GEMM reaches in this run, as a measured
    ceiling for matrix-core-bound kernels: torch.mm (hipBLASLt) of two n x n bf16
    matrices with fp32 accumulation, timed over `reps` launches after three
    untimed ones; TFLOP/s.  Under sustained matrix load the engine clock settles
    below the 2.4 GHz that the published peak assumes."""
    with torch.cuda.stream(stream):
        gen = torch.Generator(device="cuda").manual_seed(3)
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
        c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.mm(a, b, out=c)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            torch.mm(a, b, out=c)
        e1.record(stream)
        e1.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del a, b, c
    return {"bf16_gemm_TFLOPs": round(2.0 * n ** 3 / t / 1e12, 1),
            "gemm": f"torch.mm {n}x{n}x{n} bf16, fp32 accumulation (hipBLASLt)"}


def single_launch_us(torch, stream, fn, intervals: int = 25):
    """Latency of one call: HIP events around the replay of a one-launch graph
    (includes the graph launch itself, reported beside as graph_launch_floor for a
    one-element add), median over `intervals` replays."""
    g = capture(torch, stream, [fn])
    res = []
    for it in range(intervals + 3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        if it >= 3:
            res.append(e0.elapsed_time(e1) * 1e3)
    return round(statistics.median(res), 2)


def burst_leg(torch, lsa, inputs, stream, args):
    """The tau-burst trigger score on its own workload (16 sequences x 64 positions
    against one shared set of 65536 entries, 64 heads x 128): matrix-core bound,
    1.0995 TFLOP per launch; key and query replicas rotate."""
    from lookahead_sparse_kv_amd.pipeline import DeviceInputs
    wl = inputs.make_workload("burst_tau64")
    nrep = 4
    with torch.cuda.stream(stream):
        d = DeviceInputs(wl, key_replicas=nrep)
        qs = [d.q] + [d.q.clone() for _ in range(nrep - 1)]
        z = torch.empty(d.total_entries, dtype=torch.float32, device="cuda")

        def call(i):
            lsa.lsa_index_score(d.keys[i % nrep], d.key_row_start, d.seq_len, d.entry_start,
                                d.max_len, qs[i % nrep], d.w, d.bias, reduce_max=True, z_out=z)
        call(0)
        torch.cuda.synchronize()
        r = args.kernel_reps or 8
        t = timed_graph(torch, stream, capture(torch, stream, [lambda i=i: call(i)
                                                               for i in range(r)]), r)
    flops = 2.0 * wl.B * wl.T * int(wl.seq_len[0]) * wl.H * wl.D
    del d, qs, z
    return wl, t, flops, measured_mfma(torch, stream)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by "
              f"sequence with no exchange between GPUs, so one GPU's rate is the per-GPU rate",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from lookahead_sparse_kv_amd import binding as lsa
    from lookahead_sparse_kv_amd import inputs
    from lookahead_sparse_kv_amd.pipeline import DeviceInputs, Pipeline

    lsa.load_library()
    t_gen = time.time()
    wl = inputs.make_workload(args.workload)
    key_bytes = wl.keys.nbytes
    rk = max(1, -(-ROTATE_BYTES // key_bytes))
    # an upper bound of the bytes the attention touches per launch (k top-k rows
    # and max_hca HCA rows per sequence): sizes the replica rotation
    rl = max(1, -(-ROTATE_BYTES // (wl.B * (wl.k + wl.max_hca) * wl.Dl * 2)))
    if args.profile_launches:
        # three key sets so the union's indexers read distinct keys, as in the timed runs
        rk, rl = (3 if wl.T == 1 else 1), 1
    stream = torch.cuda.Stream()   # default priority
    with torch.cuda.stream(stream):
        d = DeviceInputs(wl, key_replicas=rk, latent_replicas=rl)
        p = Pipeline(d)
    torch.cuda.synchronize()
    print(f"[bench] workload {args.workload} ready in {time.time() - t_gen:.1f}s; key replicas "
          f"{rk}, latent replicas {rl}", file=sys.stderr, flush=True)

    with torch.cuda.stream(stream):
        if args.profile_launches:
            for i in range(args.profile_launches):
                p.step(i)
            for i in range(args.profile_launches):
                p.rescore(i)
            if wl.T == 1:
                for i in range(args.profile_launches):
                    p.score_union(3, i)
            enc_call = encoder_setup(torch, lsa, inputs, wl, rotate=False)[0]
            for i in range(args.profile_launches):
                enc_call(i)
            if args.copy_bytes:
                a = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
                b = torch.empty_like(a)
                for _ in range(args.profile_launches):
                    b.copy_(a)
            torch.cuda.synchronize()
            print(json.dumps({"profile_launches": args.profile_launches,
                              "copy_bytes": args.copy_bytes}))
            return

        # Steps and per-kernel runs are replayed from HIP graphs (no host work in
        # the timed region); replicas rotate so reads come from HBM, not the cache.
        # The W warm-up steps form one graph and the K timed steps another, as a
        # decode loop captures its steps: every step runs all four calls on its own
        # replica, and no per-step graph launch sits between steps.
        nrot = max(rk, rl)
        p.step(0)
        torch.cuda.synchronize()
        # the rows each attention launch attends: the step's top-k rows plus every
        # HCA row of each sequence (ragged workloads attend fewer than k + max_hca)
        att_topk = int(np.minimum(p.topk_count.cpu().numpy(), wl.k).sum())
        att_hca = int(np.minimum(wl.hca_count, wl.max_hca).sum()) if wl.hca is not None else 0
        att_rows = att_topk + att_hca
        # The step runs on one stream.  Beside it, the same steps with the
        # attention's HCA phase forked onto a second stream after the score (it
        # needs no top-k list) and joined before the selected phase.
        side = torch.cuda.Stream()   # default priority
        step_s_by = {}
        for mode, sd in (("one_stream", None), ("two_stream", side)):
            if args.warmup:
                capture(torch, stream,
                        [lambda i=i: p.step(i, stream, sd) for i in range(args.warmup)]).replay()
            timed = capture(torch, stream, [lambda i=i: p.step((args.warmup + i) % nrot, stream, sd)
                                            for i in range(args.steps)])
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            timed.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            step_s_by[mode] = e0.elapsed_time(e1) * 1e-3 / args.steps
            del timed
        step_s = step_s_by["one_stream"]

        # per-kernel launch durations: graphs of R back-to-back launches of one call
        def reps_for(est_s):
            return args.kernel_reps or max(8, min(400, int(2e-3 / max(est_s, 1e-6)) + 1))
        r = reps_for(step_s / 2)
        t_score = timed_graph(torch, stream, capture(
            torch, stream, [lambda i=i: p.score(i) for i in range(r)]), r)
        r = reps_for(4e-6)
        t_select = timed_graph(torch, stream, capture(torch, stream, [p.select] * r), r)
        t_select_z = timed_graph(torch, stream, capture(torch, stream, [p.select_from_logits] * r),
                                 r)
        # the floor of this timing method: back-to-back launches of a one-element add
        floor_e = torch.zeros(1, device="cuda")
        t_floor = timed_graph(torch, stream, capture(torch, stream, [lambda: floor_e.add_(1)] * r),
                              r)
        t_topk = timed_graph(torch, stream, capture(torch, stream, [p.topk] * r), r)
        # a1 + a2 as the step runs them: the score with its gate bits, then the compaction
        rs = reps_for(step_s / 2)
        t_score_gate = timed_graph(torch, stream, capture(
            torch, stream, [f for i in range(rs) for f in (lambda i=i: p.score(i), p.select)]), rs)
        r = reps_for(step_s / 4)
        t_attend = timed_graph(torch, stream, capture(
            torch, stream, [lambda i=i: p.attend(i) for i in range(r)]), r)
        if wl.hca is not None:
            t_att_hca = timed_graph(torch, stream, capture(
                torch, stream, [lambda i=i: p.attend_hca(i) for i in range(r)]), r)
            t_att_sel = timed_graph(torch, stream, capture(
                torch, stream, [lambda i=i: p.attend_selected(i) for i in range(r)]), r)
        else:
            t_att_hca, t_att_sel = 0.0, t_attend
        # per-step native tiered selection on the current candidates: re-score + top-k
        r = reps_for(1e-5)
        t_rescore = timed_graph(torch, stream, capture(
            torch, stream, [lambda i=i: p.rescore(i) for i in range(r)]), r)
        t_topk_native = timed_graph(torch, stream, capture(torch, stream, [p.topk_native] * r), r)
        # OR-mode union of three indexers: three score launches (the last two
        # combining), and the single streaming launch
        r = max(2, reps_for(step_s) // 3)
        t_union3 = timed_graph(torch, stream, capture(
            torch, stream, [lambda i=i: p.score_union(3, 3 * i, fused=False) for i in range(r)]), r)
        t_union3f = timed_graph(torch, stream, capture(
            torch, stream, [lambda i=i: p.score_union(3, 3 * i) for i in range(r)]), r)
        # Memory-Indexer query encoder: the step's B*T hidden states -> q, w (weight
        # replicas rotate, as a trigger finds them in HBM); beside it, the same two
        # products through torch.mm (hipBLASLt), a library reference point
        enc = time_encoder(torch, lsa, inputs, stream, wl, reps_for, args)
        p.score(0)
        p.select()
        # just-in-time fetch of the kept latent rows into a hot buffer, once per
        # lookahead trigger: from a pinned host cold pool, and from device memory
        fetch = None
        if d.latent[0] is not None:
            pool = torch.empty(d.latent[0].shape, dtype=d.latent[0].dtype, pin_memory=True)
            pool.copy_(d.latent[0])
            hot = torch.empty_like(d.latent[0])
            torch.cuda.synchronize()
            fr = args.fetch_reps
            t_fetch_host = timed_eager(torch, stream, [lambda: p.fetch(pool, hot)] * fr, fr)
            nl = len(d.latent)
            t_fetch_dev = timed_eager(torch, stream, [lambda i=i: p.fetch(d.latent[i % nl], hot)
                                                      for i in range(fr)], fr)
            # the DMA engines' own rate for a plain pinned-host -> device copy of the pool
            t_h2d = timed_eager(torch, stream, [lambda: hot.copy_(pool, non_blocking=True)], 1)
            # overlap: the next window's fetch on a second stream (default priority)
            # while the current window's tau = 64 attention steps run
            win = capture(torch, stream, [lambda i=i: p.attend(i) for i in range(64)])
            t_win = timed_graph(torch, stream, win, 1, intervals=5)
            s2 = torch.cuda.Stream()
            both = []
            for it in range(5):
                e0, e1, ef = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(stream)
                s2.wait_event(e0)
                with torch.cuda.stream(s2):
                    p.fetch(pool, hot)
                ef.record(s2)
                win.replay()
                stream.wait_event(ef)
                e1.record(stream)
                e1.synchronize()
                if it:
                    both.append(e0.elapsed_time(e1) * 1e-3)
            fetch = (t_fetch_host, t_fetch_dev, t_h2d, pool.numel() * pool.element_size(), t_win,
                     statistics.median(both))
            del pool, hot, win

        # single-call latency: one-launch graphs (graph launch included)
        floor_t = torch.zeros(1, device="cuda")
        latency = {"graph_launch_floor": single_launch_us(torch, stream, lambda: floor_t.add_(1)),
                   "index_score": single_launch_us(torch, stream, p.score),
                   "select_compact": single_launch_us(torch, stream, p.select),
                   "topk": single_launch_us(torch, stream, p.topk),
                   "sparse_attend": single_launch_us(torch, stream, p.attend),
                   "step": single_launch_us(torch, stream, p.step)}
        hbm = measured_hbm(torch, stream, att_rows, wl.Dl * wl.latent.itemsize,
                           int(wl.seq_len.sum()) * wl.D * 2 if wl.T == 1 else 1 << 28)
        # the re-score's own rows (every sequence's kept entries, key pool rows in
        # list order) gathered by a plain kernel from the same key replicas
        cc, ci = p.cand_count.cpu().numpy(), p.cand_idx.cpu().numpy()
        rs_rows = np.concatenate([wl.key_row_start[b] + ci[wl.entry_start[b]:wl.entry_start[b] + cc[b]]
                                  for b in range(wl.B)])
        if len(rs_rows):
            hbm["rescore_gather_GBs"] = round(measured_row_gather(
                torch, stream, d.keys, rs_rows, wl.D * wl.keys.itemsize), 1)
            hbm["rescore_gather"] = (f"{len(rs_rows)} kept {wl.D * wl.keys.itemsize}-byte key rows "
                                     f"(the step's lists) per launch")
    burst = None
    if wl.T == 1:
        # the tau-burst trigger score on its own workload, beside the decode step
        burst = burst_leg(torch, lsa, inputs, stream, args)

    torch.cuda.synchronize()
    counts = p.cand_count.cpu().numpy()
    scores_per_step = int(wl.seq_len.sum()) * wl.T
    # algorithmic bytes of one score launch: every key once, the queries and gates, the logits
    if wl.B > 1 and int(wl.key_row_start.max()) == 0:
        score_bytes = int(wl.seq_len[0]) * wl.D * 2          # one key set shared by the batch
    else:
        score_bytes = int(wl.seq_len.sum()) * wl.D * 2
    score_bytes += wl.q.nbytes + wl.w.nbytes + int(wl.seq_len.sum()) * 4
    score_flops = 2.0 * scores_per_step * wl.H * wl.D
    # union of three indexers in one launch: three key sets, queries and gates, one logit write
    union3_bytes = 3 * (score_bytes - int(wl.seq_len.sum()) * 4) + int(wl.seq_len.sum()) * 4
    # attended rows, qa in, out, top-k indices
    att_alg_bytes = att_rows * wl.Dl * 2 + wl.qa.nbytes * 2 + att_topk * 4
    att_flops = 4.0 * wl.T * wl.Hq * att_rows * wl.Dl
    # native re-score: per candidate one key row, its index and its logit; the queries
    rescore_bytes = int(counts.sum()) * (wl.D * 2 + 4 + 4) + wl.B * wl.H * (wl.D * 2 + 4)

    def roof(bound, alg, t, peak, unit, traffic):
        ach = alg / t / (1e9 if unit == "GB/s" else 1e12)
        r = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
             "frac": round(ach / peak, 4), "traffic": traffic}
        if unit == "GB/s":   # against the ceilings measured in this run, too
            r["frac_of_measured_read"] = round(ach / hbm["read_GBs"], 4)
            r["frac_of_measured_copy"] = round(ach / hbm["copy_GBs"], 4)
        return r

    def rescore_roof(r):
        """the re-score gathers key rows: also rate it against a gather of the same rows"""
        if "rescore_gather_GBs" in hbm:
            r["frac_of_measured_gather"] = round(r["achieved"] / hbm["rescore_gather_GBs"], 4)
        return r

    def gather_roof(r):
        """attention reads gathered rows: also rate it against the measured gather"""
        r["frac_of_measured_gather"] = round(r["achieved"] / hbm["gather_GBs"], 4)
        return r

    if wl.T == 1:
        roofline = roof("hbm", score_bytes, t_score, HBM_PEAK_GBS, "GB/s",
                        read_traffic("score_decode", args.workload, "score.hip"))
        # against a plain streaming read of the same size in one launch
        roofline["frac_of_measured_read_same_size"] = round(
            roofline["achieved"] / hbm["read_GBs_score_size"], 4)
    else:
        roofline = roof("mfma", score_flops, t_score, BF16_PEAK_TFLOPS, "TFLOP/s", None)
    ta, tc = (read_traffic("attend", args.workload, "attend.hip"),
              read_traffic("attend_combine", args.workload, "attend.hip"))
    roof_att = roof("hbm", att_alg_bytes, t_attend, HBM_PEAK_GBS, "GB/s",
                    None if ta is None else ta + (tc or 0.0))
    roof_att["mfma_frac"] = round(att_flops / t_attend / 1e12 / BF16_PEAK_TFLOPS, 4)
    gather_roof(roof_att)

    line = {
        "metric": METRIC,
        "value": round(scores_per_step / step_s, 1),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "ms_per_step_two_stream": round(step_s_by["two_stream"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; planted critical chunks among Gaussian noise keys)",
        "config": {"workload": args.workload, "batch": wl.B, "positions": wl.T,
                   "entries_per_seq": int(wl.seq_len.max()), "indexer_heads": wl.H,
                   "d_idx": wl.D, "topk": wl.k, "query_heads": wl.Hq, "latent_dim": wl.Dl,
                   "hca_rows_per_seq": wl.max_hca, "parallelism": "single GPU"},
        "kernels_us": {"index_score": round(t_score * 1e6, 2),
                       "select_compact": round(t_select * 1e6, 2),
                       "index_score_and_gate": round(t_score_gate * 1e6, 2),
                       "select_compact_from_logits": round(t_select_z * 1e6, 2),
                       "one_element_add_floor": round(t_floor * 1e6, 2),
                       "topk": round(t_topk * 1e6, 2),
                       "sparse_attend": round(t_attend * 1e6, 2),
                       "sparse_attend_hca": round(t_att_hca * 1e6, 2),
                       "sparse_attend_selected": round(t_att_sel * 1e6, 2),
                       "index_rescore": round(t_rescore * 1e6, 2),
                       "topk_native": round(t_topk_native * 1e6, 2),
                       "index_score_union3": round(t_union3 * 1e6, 2),
                       "index_score_union3_fused": round(t_union3f * 1e6, 2)},
        "index_scores_per_s": round(scores_per_step / t_score, 1),
        "decode_tokens_per_s": round(wl.B * wl.T / t_attend, 1),
        "decode_tokens_per_s_tau64": round(
            wl.B * wl.T / (t_attend + (t_score + t_select + t_topk) / 64.0), 1),
        "decode_tokens_per_s_native_topk": round(
            wl.B * wl.T / (t_attend + t_rescore + t_topk_native + (t_score + t_select) / 64.0), 1),
        "selected_fraction": round(float(counts.sum()) / float(wl.seq_len.sum()), 4),
        "attended_rows_per_step": att_rows,
        "roofline": roofline,
        "roofline_attend": roof_att,
        "roofline_rescore": rescore_roof(roof("hbm", rescore_bytes, t_rescore, HBM_PEAK_GBS, "GB/s",
                                              read_traffic("rescore", args.workload, "rescore.hip"))),
        "roofline_union3": None if wl.T != 1 else roof(
            "hbm", union3_bytes, t_union3f, HBM_PEAK_GBS, "GB/s",
            read_traffic("score_union", args.workload, "score.hip")),
        "cpu_baseline": None,
        "hbm_measured": hbm,
        "latency_us": latency,
    }
    if burst is not None:
        bwl, t_b, b_flops, mfma_meas = burst
        line["kernels_us"]["index_score_burst_tau64"] = round(t_b * 1e6, 2)
        line["roofline_burst"] = roof("mfma", b_flops, t_b, BF16_PEAK_TFLOPS, "TFLOP/s",
                                      read_traffic("score_burst", "burst_tau64", "score.hip"))
        line["roofline_burst"]["frac_of_measured_gemm"] = round(
            line["roofline_burst"]["achieved"] / mfma_meas["bf16_gemm_TFLOPs"], 4)
        line["mfma_measured"] = mfma_meas
        line["roofline_burst"]["workload"] = (
            f"burst_tau64: {bwl.B} sequences x {bwl.T} positions against one shared set of "
            f"{int(bwl.seq_len[0])} entries, {bwl.H} heads x {bwl.D} bf16")
    t_e = enc["t"]
    line["kernels_us"]["query_encode"] = round(t_e * 1e6, 2)
    line["kernels_us"]["query_encode_torch_mm"] = round(enc["t_lib"] * 1e6, 2)
    line["encoder"] = {"tokens": enc["M"], "d_model": enc["d_model"], "rank": enc["rank"],
                       "heads": wl.H, "head_dim": wl.D}
    enc_traffic = read_traffic("encode", args.workload, "encode.hip")
    if enc["M"] <= 64:   # few tokens: a stream of the weights
        line["roofline_encode"] = roof("hbm", enc["bytes"], t_e, HBM_PEAK_GBS, "GB/s", enc_traffic)
    else:
        line["roofline_encode"] = roof("mfma", enc["flops"], t_e, BF16_PEAK_TFLOPS, "TFLOP/s",
                                       enc_traffic)
    line["decode_tokens_per_s_tau64_with_encoder"] = round(
        wl.B * wl.T / (t_attend + (t_e + t_score + t_select + t_topk) / 64.0), 1)
    if fetch is not None:
        t_fh, t_fd, t_h2d, pool_bytes, t_win, t_both = fetch
        fetched = int(counts.sum()) * wl.Dl * 2
        line["kernels_us"]["fetch_rows_pinned_host"] = round(t_fh * 1e6, 2)
        line["kernels_us"]["fetch_rows_device"] = round(t_fd * 1e6, 2)
        line["fetch"] = {
            "rows": int(counts.sum()), "bytes": fetched,
            "pinned_host_GBs": round(fetched / t_fh / 1e9, 2),
            "device_GBs": round(2 * fetched / t_fd / 1e9, 1),   # read + write
            "h2d_dma_copy_GBs": round(pool_bytes / t_h2d / 1e9, 2),
            "per_step_us_tau64": round(t_fh * 1e6 / 64.0, 2),
            "window_attend64_us": round(t_win * 1e6, 1),
            "fetch_beside_window_us": round(t_both * 1e6, 1),
        }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seqs)
        line["cpu_baseline"]["burst_prefix"] = cpu_burst_prefix(
            burst[0] if burst is not None else wl)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
