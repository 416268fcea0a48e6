"""GPU parity of the attention variants against the CPU oracle, through the C ABI:
a per-head sink in sparse MLA (forward, backward, teacher), the compressed + window +
sink chain with its indexer loss, complete-pool selection and the k-pool expansion
with the query's incomplete tail pool (width 2048 + 3). Tolerances as in the other GPU
tests (forward: max-abs 2e-2 / relative 1e-2 bf16, 1e-5 fp32; gradients: see
test_gpu_backward); routes bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_backward import grad_close

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
W = workloads.WORKLOADS
BF16_TOL = dict(atol=2e-2, rtol=1e-2)


@pytest.fixture(scope="module")
def sa():
    import indexer_routed_sparse_amd as m
    return m


def close(got, ref, atol, rtol, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finiteness differs"
    err = np.abs(got[fin] - ref[fin])
    bad = err > atol + rtol * np.abs(ref[fin])
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, max err {err.max():.3g}"


@pytest.mark.parametrize("H,k,d_qk,shift", [(16, 65, 512, 0.0), (64, 127, 576, 0.0), (128, 2051, 576, 0.0),
                                            (128, 96, 576, 40.0), (32, 33, 576, -40.0)])
def test_sparse_mla_sink(sa, H, k, d_qk, shift):
    """Forward with a sink: heads 16..128, widths 512/576, k up to 2051, an all-invalid
    row (out = 0, lse = sink), and sinks far above (shift +40: the sink takes almost all
    the mass) or below every logit."""
    T, S = 16, 3000
    g = torch.Generator().manual_seed(H + k + int(shift))
    q = torch.randn((T, H, d_qk), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, d_qk), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < 0.1] = -1
    idx[2] = -1
    sink = (torch.randn(H, generator=g) * 2 + shift).float()
    scale = 1 / math.sqrt(d_qk)
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), scale, sink=sink.to(DEV))
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), scale, sink=sink.numpy())
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, **BF16_TOL, what="lse")
    assert torch.all(out[2] == 0)
    assert torch.equal(lse[2].cpu(), sink)


def test_sparse_mla_sink_fp32(sa):
    wl = W["tiny_fp32"]
    x = workloads.indexer_inputs(wl)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 64)
    m = workloads.mla_inputs(wl)
    sink = torch.linspace(-3, 3, wl.H)
    out, lse = sa.sparse_mla(m["q"].to(DEV), m["kv"].to(DEV), torch.from_numpy(ref_idx).to(DEV), wl.scale,
                             sink=sink.to(DEV))
    ro, rl = oracle.sparse_mla(m["q"], m["kv"], ref_idx, wl.scale, sink=sink.numpy())
    close(out.cpu().numpy(), ro, 1e-5, 1e-5, "out")
    close(lse.cpu().numpy(), rl, 1e-5, 1e-5, "lse")


@pytest.mark.parametrize("H,k", [(16, 127), (128, 300)])
def test_sparse_mla_bwd_sink(sa, H, k):
    T, S, d_qk = 20, 900, 576
    g = torch.Generator().manual_seed(H * 3 + k)
    q = torch.randn((T, H, d_qk), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, d_qk), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < 0.1] = -1
    idx[5] = -1
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g).float()
    scale = 1 / math.sqrt(d_qk)
    qd, kvd, idxd, sd = q.to(DEV), kv.to(DEV), idx.to(DEV), sink.to(DEV)
    _, lse = sa.sparse_mla(qd, kvd, idxd, scale, sink=sd)
    dq, dkv, dsink = sa.sparse_mla_bwd(qd, kvd, idxd, dout.to(DEV), lse, scale, sink=sd)
    rdq, rdkv, rds = oracle.sparse_mla_bwd(q, kv, idx.numpy(), dout, scale, sink=sink.numpy())
    grad_close(dq.float().cpu().numpy(), rdq, "dq")
    grad_close(dkv.cpu().numpy(), rdkv, "dkv")
    close(dsink.cpu().numpy(), rds, 1e-3 * np.abs(rds).max() + 1e-4, 1e-2, "dsink")


def test_compressed_window_sink_chain(sa):
    """Compressed sparse attention as the CSA page describes it (compressed + window +
    sink): each token attends to its selected compressed entries (four tokens each,
    complete ones only) plus a 32-token causal window of raw keys, with a per-head sink;
    the indexer scores compressed entries, and its KL teacher keeps the full denominator
    (window and sink included), so a row's teacher mass is below one. Routes, window
    slots, attention, teacher, loss and indexer gradients against the oracle."""
    T, r, k, win = 1024, 4, 32, 32
    Sc = T // r
    H, d_qk, H_I, D_I = 16, 576, 16, 128
    gen = torch.Generator().manual_seed(90)
    q = torch.randn((T, H, d_qk), generator=gen).to(torch.bfloat16)
    kv_c = torch.randn((Sc, d_qk), generator=gen).to(torch.bfloat16)
    kv_r = torch.randn((T, d_qk), generator=gen).to(torch.bfloat16)
    kv = torch.cat([kv_c, kv_r]).contiguous()
    qI = torch.randn((T, H_I, D_I), generator=gen).to(torch.bfloat16)
    kI = torch.randn((Sc, D_I), generator=gen).to(torch.bfloat16)
    w = (torch.randn((T, H_I), generator=gen) / 8).float()
    sink = torch.randn(H, generator=gen).float()
    # selected compressed entries: random among the complete ones (4c + 3 <= t)
    sel = torch.full((T, k), -1, dtype=torch.int32)
    for t in range(T):
        n = (t + 1) // r
        if n:
            c = torch.randperm(n, generator=gen)[:k].sort().values
            sel[t, :c.numel()] = c.to(torch.int32)
    scale = 1 / math.sqrt(d_qk)
    seld = sel.to(DEV)
    idx = sa.append_window(seld, win, offset=Sc)
    ref_idx = oracle.append_window(sel.numpy(), win, offset=Sc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    qd, kvd, sd = q.to(DEV), kv.to(DEV), sink.to(DEV)
    out, lse = sa.sparse_mla(qd, kvd, idx, scale, sink=sd)
    ro, rl = oracle.sparse_mla(q, kv, ref_idx, scale, sink=sink.numpy())
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, **BF16_TOL, what="lse")
    # teacher over the selected compressed slots under the full denominator
    teacher = sa.attn_teacher(qd, kvd, idx[:, :k].contiguous(), lse, scale)
    rt = oracle.attn_teacher(q, kv, ref_idx[:, :k], scale, sink=sink.numpy())
    # the full-denominator teacher of the selected slots = the oracle's head mean over
    # all slots (selected + window) restricted to the selected ones
    full = oracle.attn_teacher(q, kv, ref_idx, scale, sink=sink.numpy())[:, :k]
    close(teacher.cpu().numpy(), full, 1e-6, 1e-3, "teacher")
    assert np.all(full.sum(1) < 1 + 1e-9)
    loss, dq, dw, dk = sa.indexer_kl_bwd(qI.to(DEV), kI.to(DEV), w.to(DEV), seld, teacher)
    rl2, _, rdq, rdw, rdk = oracle.indexer_kl(qI, kI, w, sel.numpy(), full)
    close(loss.cpu().numpy(), rl2, 1e-4, 1e-3, "loss")
    grad_close(dq.float().cpu().numpy(), rdq, "dq_I")
    grad_close(dw.cpu().numpy(), rdw, "dw")
    grad_close(dk.cpu().numpy(), rdk, "dk_I")
    del rt


def test_kpool_chain_glm_width_2051(sa):
    """GLM-shaped k-pool routing on the integer grid: 4096 tokens, pools of four keys
    scored by the block max of the indexer scores, the top 512 complete pools per query
    (sa_topk_select, complete blocks only), expanded to token slots with the query's
    incomplete tail pool appended (512 * 4 + 3 = 2051), then NoPE (512-wide) sparse
    MLA over them. Pool routes and token slots bit-exact; attention within bf16
    tolerance on sampled rows."""
    wl = W["nope_unaligned"]
    T, P, kp = 4096, 4, 512
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    xd = {n: t.to(DEV) for n, t in x.items()}
    scores = sa.indexer_scores(xd["q_I"], xd["k_I"], xd["w"], block_size=P)
    pools = sa.topk_select(scores, kp, block_size=P, force_own_block=2)
    slots = sa.kpool_expand(pools, P)
    assert slots.shape == (T, 2051)
    rows = np.union1d(np.arange(0, T, 97), [0, 1, 2, 3, 4, 2047, 2048, 2049, 2050, 2051, T - 2, T - 1])
    ref_sc = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"], block_size=P, rows=rows)
    ref_pools, _ = oracle.complete_block_topk(ref_sc, kp, P, rows=rows)
    np.testing.assert_array_equal(pools.cpu().numpy()[rows], ref_pools)
    full_pools = pools.cpu().numpy()
    ref_slots = oracle.kpool_expand(full_pools, P)
    np.testing.assert_array_equal(slots.cpu().numpy(), ref_slots)
    m = workloads.mla_inputs(wl, T=T)
    out, lse = sa.sparse_mla(m["q512"].to(DEV), m["kv512"].to(DEV), slots, wl.scale)
    ro, rl = oracle.sparse_mla(m["q512"], m["kv512"], ref_slots, wl.scale, rows=rows)
    close(out.float().cpu().numpy()[rows], ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy()[rows], rl, **BF16_TOL, what="lse")


def test_kpool_and_window_thd(sa):
    lengths = (10, 1, 7, 13)
    T = sum(lengths)
    cu = torch.from_numpy(workloads.cu_seqlens(lengths)).to(DEV)
    rng = np.random.default_rng(91)
    start, _ = oracle.seq_bounds(T, workloads.cu_seqlens(lengths))
    pools = np.full((T, 3), -1, dtype=np.int32)
    for t in range(T):
        n = (t - start[t] + 1) // 4
        c = np.sort(rng.permutation(n)[:3])
        pools[t, :c.size] = c
    got = sa.kpool_expand(torch.from_numpy(pools).to(DEV), 4, cu_seqlens=cu, max_seqlen=13)
    np.testing.assert_array_equal(got.cpu().numpy(),
                                  oracle.kpool_expand(pools, 4, cu_seqlens=workloads.cu_seqlens(lengths)))
    idx = torch.from_numpy(pools).to(DEV)
    gw = sa.append_window(idx, 5, offset=7, cu_seqlens=cu, max_seqlen=13)
    np.testing.assert_array_equal(gw.cpu().numpy(),
                                  oracle.append_window(pools, 5, offset=7, cu_seqlens=workloads.cu_seqlens(lengths)))
