"""The allocation-free entry point sa_indexer_scores_noalloc against sa_indexer_scores
with a caller workspace, through the C ABI: two calls in a row on the same device (the
static scratch keeps the first call's contents), the second smaller."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


@pytest.fixture(scope="module")
def sa():
    import indexer_routed_sparse_amd as m
    return m


def _noalloc(sa, x, topk, out_idx, out_val, cu=None, max_seqlen=0):
    T, H_I, D_I = x["q_I"].shape
    f = sa.lib.sa_indexer_scores_noalloc
    f.restype = ctypes.c_int
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = f(p(x["q_I"]), p(x["k_I"]), p(x["w"]), 1, T, p(cu), 0 if cu is None else cu.numel() - 1,
           max_seqlen, H_I, D_I, 1, None, 0, topk, 0, p(out_idx), p(out_val),
           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_entry_twice(sa):
    wl = workloads.WORKLOADS["long_dsa"]
    limit = sa.lib.sa_noalloc_scratch_bytes
    limit.restype = ctypes.c_size_t
    assert limit() == 128 << 20
    results = []
    for T, k, lengths in [(5000, 2048, None), (2500, 300, (1200, 1, 1299))]:
        x = {n: t.to(DEV) for n, t in workloads.indexer_inputs(wl, T=T).items()}
        cu = torch.from_numpy(workloads.cu_seqlens(lengths)).to(DEV) if lengths else None
        maxlen = max(lengths) if lengths else 0
        need = sa.sa_indexer_workspace_bytes(torch.bfloat16, T, maxlen or T, 64, 128, 1, k)
        assert 0 < need <= limit()
        i1 = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
        v1 = torch.full((T, k), 7.0, dtype=torch.float32, device=DEV)
        assert _noalloc(sa, x, k, i1, v1, cu, maxlen) == 0
        kw = dict(cu_seqlens=cu, max_seqlen=maxlen) if lengths else {}
        i2, v2 = sa.indexer_topk(x["q_I"], x["k_I"], x["w"], k, with_values=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2), (T, k)
        assert torch.equal(v1.view(torch.int32), v2.view(torch.int32)), (T, k)
        results.append(i1)
    assert len(results) == 2


def test_noalloc_rejects_beyond_scratch(sa):
    wl = workloads.WORKLOADS["long_dsa"]
    T, k = 32768, 2048
    need = sa.sa_indexer_workspace_bytes(torch.bfloat16, T, T, 64, 128, 1, k)
    assert need > 128 << 20
    q = torch.empty((T, 64, 128), dtype=torch.bfloat16, device=DEV)
    x = {"q_I": q, "k_I": torch.empty((T, 128), dtype=torch.bfloat16, device=DEV),
         "w": torch.empty((T, 64), dtype=torch.float32, device=DEV)}
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    assert _noalloc(sa, x, k, idx, None) == 7          # SA_ERR_WORKSPACE, nothing launched
    torch.cuda.synchronize()
