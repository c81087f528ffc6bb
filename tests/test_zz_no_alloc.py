"""lsa_select_compact_noalloc (built-in scratch, no workspace) against lsa_select_compact.

Two calls in a row through the C ABI, the second with a smaller batch and
shorter sequences, each compared element by element (bit-exact lists and
counts) with the workspace call on the same logits; then the size limit."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev, host
from lookahead_sparse_kv_amd import binding as lsa

pytestmark = pytest.mark.gpu


def _case(seed, lens):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    es = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    n = int(lens.sum())
    z = rng.normal(-1.2, 1.0, n).astype(np.float32)
    z[rng.random(n) < 0.01] = 0.0                       # exactly on the gate: kept
    z[rng.random(n) < 0.01] = -0.0
    z[rng.random(n) < 0.005] = np.nan                   # never kept
    return z, lens, es


def _both(z, lens, es):
    B, n = len(lens), len(z)
    max_len = int(lens.max())
    zd, ld, ed = dev(z), dev(lens), dev(es)
    ws = torch.empty(max(1, lsa.lsa_workspace_bytes(lsa.LSA_OP_SELECT, B, max_len=max_len)),
                     dtype=torch.uint8, device="cuda")
    ci_a = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    cc_a = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ci_b, cc_b = ci_a.clone(), cc_a.clone()
    lsa.lsa_select_compact(zd, ed, ld, max_len, ci_a, cc_a, ws)
    lsa.lsa_select_compact_noalloc(zd, ed, ld, max_len, ci_b, cc_b)
    torch.cuda.synchronize()
    return host(ci_a), host(cc_a), host(ci_b), host(cc_b)


def test_noalloc_select_matches_workspace_call_twice():
    for seed, lens in ((1, [131072, 4097, 0, 70000, 2048, 1]), (2, [5000, 17, 2049])):
        announce(f"select noalloc vs workspace, lens {lens}")
        z, lens_a, es = _case(seed, lens)
        ia, ca, ib, cb = _both(z, lens_a, es)
        np.testing.assert_array_equal(ca, cb)
        for b in range(len(lens_a)):
            s, c = int(es[b]), int(ca[b])
            want = np.flatnonzero(z[s:s + lens_a[b]] >= 0)
            assert c == len(want)
            np.testing.assert_array_equal(ib[s:s + c], ia[s:s + c])
            np.testing.assert_array_equal(ib[s:s + c], want)


def test_noalloc_select_rejects_batches_beyond_its_scratch():
    z, lens, es = _case(3, [16, 16])
    zd, ld, ed = dev(z), dev(lens), dev(es)
    ci = torch.empty(32, dtype=torch.int32, device="cuda")
    cc = torch.empty(2, dtype=torch.int32, device="cuda")
    # 2 sequences x 2^31 / 2048 tiles = 2^21 tiles > 2^18: refused before any launch
    with pytest.raises(lsa.LSAError) as e:
        lsa.lsa_select_compact_noalloc(zd, ed, ld, 1 << 31, ci, cc)
    assert e.value.status == lsa.LSA_ERR_UNSUPPORTED
    assert "scratch" in str(e.value)
