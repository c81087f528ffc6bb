"""Helpers shared by the GPU parity tests: moving arrays, tolerance checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances, for fp32-accumulated bf16 products (bf16 products are exact in fp32, so
# the error is the fp32 summation's, far below these bounds at the tested sizes):
Z_ABS_TOL = 1e-3        # |z_gpu - z_ref| and |I_gpu - I_ref|
GATE_BAND = 4e-3        # |z_ref| <= band: the 1e-3 band on I = sigmoid(z) around 0.5
RANK_BAND = 1e-3        # top-k keys this close to the k-th key may swap
ATT_REL_TOL = 2e-2      # per (b,t,h) row: ||o_gpu - o_ref|| / ||o_ref||
LSE_ABS_TOL = 5e-3


def announce(msg: str) -> None:
    """Name the case on the real stderr, flushed, before a GPU step."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sigmoid64(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def check_scores(z_gpu, z_ref, prob_gpu=None):
    z_gpu = np.asarray(z_gpu, np.float64)
    err = np.abs(z_gpu - z_ref)
    assert np.all(np.isfinite(z_gpu)), "non-finite score"
    assert err.max() <= Z_ABS_TOL, f"max |dz| = {err.max()}"
    if prob_gpu is not None:
        perr = np.abs(np.asarray(prob_gpu, np.float64) - sigmoid64(z_ref))
        assert perr.max() <= Z_ABS_TOL, f"max |dI| = {perr.max()}"
    return float(err.max())


def check_selection(c_gpu, c_ref, z_ref_seq):
    """Sets equal outside the gate band (|z_ref| <= GATE_BAND may differ)."""
    a, b = set(np.asarray(c_gpu).tolist()), set(np.asarray(c_ref).tolist())
    for s in a ^ b:
        assert abs(z_ref_seq[s]) <= GATE_BAND, f"entry {s} differs outside the band (z={z_ref_seq[s]})"
    assert np.all(np.diff(np.asarray(c_gpu)) > 0), "candidate list not ascending"


def check_topk(t_gpu, t_ref, r_ref_seq, k, n_cand_gpu):
    """|T| = min(k, |C|); sets equal except near the k-th key or the gate."""
    t_gpu = np.asarray(t_gpu)
    assert len(t_gpu) == min(k, n_cand_gpu)
    assert np.all(np.diff(t_gpu) > 0), "top-k not ascending"
    if len(t_ref) == 0:
        return
    kth = np.sort(r_ref_seq[np.asarray(t_ref)])[0]
    for s in set(t_gpu.tolist()) ^ set(np.asarray(t_ref).tolist()):
        near_k = abs(r_ref_seq[s] - kth) <= RANK_BAND
        near_gate = abs(r_ref_seq[s]) <= GATE_BAND
        assert near_k or near_gate, f"entry {s} differs (r={r_ref_seq[s]}, kth={kth})"


def check_topk_properties(t_gpu, cand_gpu, r_gpu_seq, k):
    """Properties of a top-k over the GPU's own keys, valid at any size."""
    t_gpu = np.asarray(t_gpu)
    cand_gpu = np.asarray(cand_gpu)
    assert len(t_gpu) == min(k, len(cand_gpu))
    assert np.all(np.diff(t_gpu) > 0)
    assert set(t_gpu.tolist()) <= set(cand_gpu.tolist())
    rest = np.setdiff1d(cand_gpu, t_gpu)
    if len(rest) and len(t_gpu):
        lo = r_gpu_seq[t_gpu].min()
        hi = r_gpu_seq[rest].max()
        assert lo >= hi
        if lo == hi:  # ties at the boundary go to the smaller index
            assert t_gpu[r_gpu_seq[t_gpu] == lo].max() < rest[r_gpu_seq[rest] == hi].min()


def check_attention(o_gpu, o_ref, lse_gpu=None, lse_ref=None):
    o_gpu = np.asarray(o_gpu, np.float64)
    D = o_ref.shape[-1]
    og = o_gpu.reshape(-1, D)
    orf = o_ref.reshape(-1, D)
    num = np.linalg.norm(og - orf, axis=1)
    den = np.linalg.norm(orf, axis=1)
    empty = den == 0
    assert np.all(num[empty] == 0), "rows with nothing to attend must be 0"
    rel = num[~empty] / den[~empty] if (~empty).any() else np.zeros(1)
    assert rel.max() <= ATT_REL_TOL, f"max row rel err {rel.max()}"
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, np.float64).reshape(-1)
        lr = np.asarray(lse_ref, np.float64).reshape(-1)
        inf = np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), inf)
        if (~inf).any():
            assert np.abs(lg[~inf] - lr[~inf]).max() <= LSE_ABS_TOL, np.abs(lg[~inf] - lr[~inf]).max()
    return float(rel.max())
