"""Device-resident inputs and the four-call decode pipeline over them.

Holds preallocated outputs and workspaces so that one `step()` enqueues
exactly: index score (which also writes the gate bits) -> compaction from the
bits -> top-k -> sparse attention, all in liblsa.so kernels on one stream,
with no host synchronisation.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as lsa
from .inputs import Workload


def _to_dev(a: Optional[np.ndarray], device, bf16: bool = False):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


class DeviceInputs:
    """A Workload copied to HBM.  Replicas (distinct copies of the key pool and
    of the latent/HCA pools) let timing loops rotate through more memory than
    the on-die cache holds; replica 0 is the one parity tests use."""

    def __init__(self, wl: Workload, device: str = "cuda", key_replicas: int = 1,
                 latent_replicas: int = 1):
        self.wl = wl
        self.device = device
        self.B, self.T, self.H, self.D = wl.B, wl.T, wl.H, wl.D
        self.k, self.Hq, self.Dl = wl.k, wl.Hq, wl.Dl
        self.max_len = wl.max_len
        self.total_entries = wl.total_entries
        self.max_hca = wl.max_hca
        self.bias = wl.bias
        self.scale = wl.scale
        keys = _to_dev(wl.keys, device)
        self.keys = [keys] + [keys.clone() for _ in range(key_replicas - 1)]
        self.q = _to_dev(wl.q, device)
        self.w = _to_dev(wl.w, device)
        self.seq_len = _to_dev(wl.seq_len.astype(np.int32), device)
        self.key_row_start = _to_dev(wl.key_row_start.astype(np.int64), device)
        self.entry_start = _to_dev(wl.entry_start.astype(np.int64), device)
        self.qa = _to_dev(wl.qa, device)
        from .inputs import native_queries
        q2, w2 = native_queries(wl)
        self.q_native = _to_dev(q2, device)     # the native indexer's per-step queries
        self.w_native = _to_dev(w2, device)
        if wl.latent is not None:
            lat = _to_dev(wl.latent, device)
            self.latent = [lat] + [lat.clone() for _ in range(latent_replicas - 1)]
            self.latent_row_start = _to_dev(wl.latent_row_start.astype(np.int64), device)
        else:
            self.latent, self.latent_row_start = [None], None
        if wl.hca is not None:
            h = _to_dev(wl.hca, device)
            self.hca = [h] + [h.clone() for _ in range(latent_replicas - 1)]
            self.hca_row_start = _to_dev(wl.hca_row_start.astype(np.int64), device)
            self.hca_count = _to_dev(wl.hca_count.astype(np.int32), device)
        else:
            self.hca, self.hca_row_start, self.hca_count = [None] * max(1, latent_replicas), None, None


class Pipeline:
    """Preallocated buffers for the four calls on one DeviceInputs."""

    def __init__(self, d: DeviceInputs, with_prob: bool = False):
        self.d = d
        dev = d.device
        B, T = d.B, d.T
        n = d.total_entries
        # T > 1: the pipeline keeps the OR-union of positions, i.e. max over t.
        self.z = torch.empty(n, dtype=torch.float32, device=dev)
        self.prob = torch.empty(n, dtype=torch.float32, device=dev) if with_prob else None
        self.cand_idx = torch.empty(n, dtype=torch.int32, device=dev)
        # the gate of z >= 0, one bit per entry, written by the score launch
        self.gate = torch.empty(B * lsa.lsa_gate_words(d.max_len), dtype=torch.int16, device=dev)
        self.cand_count = torch.empty(B, dtype=torch.int32, device=dev)
        self.ws_select = torch.empty(
            max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_SELECT, B, max_len=d.max_len)),
            dtype=torch.uint8, device=dev)
        ws_t = lsa.lsa_workspace_bytes(lsa.LSA_OP_TOPK, B, max_len=d.max_len, k=d.k)
        self.ws_topk = torch.empty(max(1, ws_t), dtype=torch.uint8, device=dev)
        self.topk_idx = torch.full((B, d.k), -1, dtype=torch.int32, device=dev)
        self.topk_count = torch.empty(B, dtype=torch.int32, device=dev)
        self.out = torch.empty((B, T, d.Hq, d.Dl), dtype=d.qa.dtype, device=dev)
        self.lse = torch.empty((B, T, d.Hq), dtype=torch.float32, device=dev)
        ws_a = lsa.lsa_workspace_bytes(lsa.LSA_OP_ATTEND, B, T, d.Hq, d.Dl, k=d.k,
                                       max_hca=d.max_hca)
        self.ws_attend = torch.empty(max(1, ws_a), dtype=torch.uint8, device=dev)
        self.r = torch.zeros(n, dtype=torch.float32, device=dev)   # native re-score (entry-indexed)

    def score(self, replica: int = 0, stream=None):
        d = self.d
        lsa.lsa_index_score(d.keys[replica % len(d.keys)], d.key_row_start, d.seq_len,
                            d.entry_start, d.max_len, d.q, d.w, d.bias, reduce_max=True,
                            z_out=self.z, prob_out=self.prob, gate_bits=self.gate, stream=stream)

    def score_union(self, n_indexers: int, replica: int = 0, fused: bool = True, stream=None):
        """OR-mode union of n indexers (key replicas replica .. replica+n-1 stand in
        for the indexers' key sets), gate logits left in z: one lsa_index_score_union
        call, or (fused=False) one lsa_index_score call per indexer."""
        d = self.d
        keys = [d.keys[(replica + i) % len(d.keys)] for i in range(n_indexers)]
        if fused:
            lsa.lsa_index_score_union(keys, d.key_row_start, d.seq_len, d.entry_start, d.max_len,
                                      [d.q] * n_indexers, [d.w] * n_indexers,
                                      [d.bias] * n_indexers, self.z, gate_bits=self.gate,
                                      stream=stream)
            return
        for i in range(n_indexers):
            lsa.lsa_index_score(keys[i], d.key_row_start, d.seq_len,
                                d.entry_start, d.max_len, d.q, d.w, d.bias,
                                reduce_max=1 if i == 0 else 2, z_out=self.z,
                                gate_bits=self.gate if i == n_indexers - 1 else None,
                                stream=stream)

    def rescore(self, replica: int = 0, stream=None):
        """The native indexer's per-step score of the kept entries, into r."""
        d = self.d
        lsa.lsa_index_rescore(d.keys[replica % len(d.keys)], d.key_row_start, d.seq_len,
                              d.entry_start, self.cand_idx, self.cand_count, d.max_len,
                              d.q_native, d.w_native, self.r, stream=stream)

    def topk_native(self, stream=None):
        """Top-k of the kept entries by the native re-score."""
        d = self.d
        lsa.lsa_topk(self.r, d.entry_start, d.seq_len, d.max_len, self.cand_idx, self.cand_count,
                     d.k, self.topk_idx, self.topk_count, self.ws_topk, stream=stream)

    def fetch(self, src, dst, stream=None):
        """Just-in-time fetch: every kept entry's latent row of sequence b, from the
        cold pool src (pinned host or device memory, laid out like the latent
        pool), packed in list order into dst at latent_row_start[b]."""
        d = self.d
        lsa.lsa_fetch_rows(src, d.latent_row_start, self.cand_idx, d.entry_start, self.cand_count,
                           d.max_len, dst, d.latent_row_start, stream=stream)

    def select(self, stream=None):
        """Compaction from the gate bits the score launch wrote (one launch)."""
        d = self.d
        lsa.lsa_select_compact(None, d.entry_start, d.seq_len, d.max_len, self.cand_idx,
                               self.cand_count, None, gate_bits=self.gate, stream=stream)

    def select_from_logits(self, stream=None):
        """The same compaction taken on z (a count launch and a scatter launch)."""
        d = self.d
        lsa.lsa_select_compact(self.z, d.entry_start, d.seq_len, d.max_len, self.cand_idx,
                               self.cand_count, self.ws_select, stream=stream)

    def topk(self, stream=None):
        d = self.d
        lsa.lsa_topk(self.z, d.entry_start, d.seq_len, d.max_len, self.cand_idx, self.cand_count,
                     d.k, self.topk_idx, self.topk_count, self.ws_topk, stream=stream)

    def attend(self, replica: int = 0, stream=None):
        d = self.d
        r = replica % len(d.latent)
        lsa.lsa_sparse_attend(d.qa, d.latent[r], d.latent_row_start, self.topk_idx,
                              self.topk_count, d.k, self.out, hca=d.hca[r],
                              hca_row_start=d.hca_row_start, hca_count=d.hca_count,
                              max_hca=d.max_hca, scale=d.scale, lse=self.lse,
                              workspace=self.ws_attend, stream=stream)

    def attend_hca(self, replica: int = 0, stream=None):
        d = self.d
        r = replica % len(d.latent)
        lsa.lsa_sparse_attend_hca(d.qa, d.k, d.hca[r], d.hca_row_start, d.hca_count, d.max_hca,
                                  scale=d.scale, workspace=self.ws_attend, stream=stream)

    def attend_selected(self, replica: int = 0, stream=None):
        d = self.d
        r = replica % len(d.latent)
        lsa.lsa_sparse_attend_selected(d.qa, d.latent[r], d.latent_row_start, self.topk_idx,
                                       self.topk_count, d.k, self.out, hca=d.hca[r],
                                       hca_row_start=d.hca_row_start, hca_count=d.hca_count,
                                       max_hca=d.max_hca, scale=d.scale, lse=self.lse,
                                       workspace=self.ws_attend, stream=stream)

    def step(self, replica: int = 0, stream=None, side=None):
        """One decode step.  With a second stream `side`, the attention's HCA
        phase (which needs no top-k list) runs there beside the gate and the
        top-k, forked after the score and joined before the selected phase."""
        self.score(replica, stream)
        if side is None or self.d.hca is None:
            self.select(stream)
            self.topk(stream)
            self.attend(replica, stream)
            return
        main = stream if stream is not None else torch.cuda.current_stream()
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        self.attend_hca(replica, side)
        join.record(side)
        self.select(main)
        self.topk(main)
        main.wait_event(join)
        self.attend_selected(replica, main)
