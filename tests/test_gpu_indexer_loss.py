"""GPU parity of the sparse KL indexer loss (teacher, loss and indexer gradients)
against the CPU oracle, through the C ABI.

Teacher probabilities come from fp32 arithmetic on bf16 inputs (the logits' bf16
products are exact in fp32): |got - ref| <= 1e-6 + 1e-3 |ref|. Losses: 1e-4 + 1e-3
|ref|. Gradients use the backward tests' bar (2e-2 rms_row + 1e-2 |ref| + 1e-4 for
bf16: the per-key factors dI_j w_h enter the matrix cores as bf16; 1e-4 rms_row +
1e-5 |ref| + 1e-5 for fp32). Gradients into k_I are summed with atomics.
"""
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


@pytest.fixture(scope="module")
def sa():
    import indexer_routed_sparse_amd as m
    return m


def close(got, ref, atol, rtol, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance, max err {err.max():.3g}"


@pytest.mark.parametrize("H,k,d_qk", [(16, 127, 512), (8, 64, 576), (128, 300, 576), (80, 33, 576),
                                      (96, 65, 512), (64, 40, 576)])
def test_attn_teacher_shapes(sa, H, k, d_qk):
    T, S = 20, 600
    g = torch.Generator().manual_seed(H + k + d_qk)
    q = torch.randn((T, H, d_qk), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, d_qk), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < 0.1] = -1
    idx[4] = -1
    scale = 1 / math.sqrt(d_qk)
    qd, kvd, idxd = q.to(DEV), kv.to(DEV), idx.to(DEV)
    _, lse = sa.sparse_mla(qd, kvd, idxd, scale)
    got = sa.attn_teacher(qd, kvd, idxd, lse, scale).cpu().numpy()
    ref = oracle.attn_teacher(q, kv, idx.numpy(), scale)
    close(got, ref, 1e-6, 1e-3, "teacher")
    assert np.all(got[4] == 0)


def test_attn_teacher_long_rows_sampled(sa):
    """The bench's teacher launch shape: 128 heads, k = 2048 over the long workload's
    32768-row latent, on its last 64 query rows (2048-wide index rows, 5 % -1 slots)."""
    wl = W["long_dsa"]
    T = 64
    m = workloads.mla_inputs(wl, device=DEV)
    q = m["q"][-T:].contiguous()
    idx = workloads.random_causal_index(wl.T, 2048, wl.seed, device=DEV)[-T:].contiguous()
    _, lse = sa.sparse_mla(q, m["kv"], idx, wl.scale)
    got = sa.attn_teacher(q, m["kv"], idx, lse, wl.scale)
    got2 = sa.attn_teacher(q, m["kv"], idx, lse, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, got2)                          # one plain store per slot: bitwise replay
    ref = oracle.attn_teacher(q.cpu(), m["kv"].cpu(), idx.cpu().numpy(), wl.scale)
    close(got.cpu().numpy(), ref, 1e-6, 1e-3, "teacher")


def test_attn_teacher_fp32_tiny(sa):
    wl = W["tiny_fp32"]
    x = workloads.indexer_inputs(wl)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 64)
    m = workloads.mla_inputs(wl)
    qd, kvd, idxd = m["q"].to(DEV), m["kv"].to(DEV), torch.from_numpy(ref_idx).to(DEV)
    _, lse = sa.sparse_mla(qd, kvd, idxd, wl.scale)
    got = sa.attn_teacher(qd, kvd, idxd, lse, wl.scale).cpu().numpy()
    close(got, oracle.attn_teacher(m["q"], m["kv"], ref_idx, wl.scale), 1e-6, 1e-4, "teacher")


def _random_teacher(idx, seed):
    rng = np.random.default_rng(seed)
    p = rng.random(idx.shape) * (idx >= 0)
    p[rng.random(idx.shape) < 0.05] = 0.0                 # some zero-probability slots
    s = p.sum(1, keepdims=True)
    return np.where(s > 0, p / np.where(s > 0, s, 1), 0.0).astype(np.float32)


@pytest.mark.parametrize("H_I,D_I,k", [(64, 128, 2048), (16, 128, 127), (32, 64, 65), (64, 64, 1)])
def test_indexer_kl_bwd_shapes(sa, H_I, D_I, k):
    """Head counts 16/32/64, head dims 64/128, top-k 1..2048 over a 4096-row key array,
    -1 slots, a row without slots, per-row loss weights; the teacher is an arbitrary
    distribution over each row's slots (so the kernel is checked on its own)."""
    import dataclasses
    wl = dataclasses.replace(W["long_dsa"], H_I=H_I, D_I=D_I)
    T, S = 24, 4096
    x = workloads.indexer_inputs(wl, T=S)
    qI, kI, wv = x["q_I"][-T:].contiguous(), x["k_I"], x["w"][-T:].contiguous()
    idx = workloads.random_causal_index(S, k, 7, frac_invalid=0.05)[-T:].contiguous()
    idx[3] = -1
    teacher = _random_teacher(idx.numpy(), 8)
    grad = (np.random.default_rng(9).random(T) + 0.5).astype(np.float32)
    loss, dq, dw, dk = sa.indexer_kl_bwd(qI.to(DEV), kI.to(DEV), wv.to(DEV), idx.to(DEV),
                                         torch.from_numpy(teacher).to(DEV), torch.from_numpy(grad).to(DEV))
    loss2, dq2, dw2, _ = sa.indexer_kl_bwd(qI.to(DEV), kI.to(DEV), wv.to(DEV), idx.to(DEV),
                                           torch.from_numpy(teacher).to(DEV), torch.from_numpy(grad).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2) and torch.equal(dq, dq2) and torch.equal(dw, dw2)   # no atomics
    rl, _, rdq, rdw, rdk = oracle.indexer_kl(qI, kI, wv, idx.numpy(), teacher, grad)
    close(loss.cpu().numpy(), rl, 1e-4, 1e-3, "loss")
    grad_close(dq.float().cpu().numpy(), rdq, "dq_I")
    grad_close(dw.cpu().numpy(), rdw, "dw")
    grad_close(dk.cpu().numpy(), rdk, "dk_I")
    assert loss[3].item() == 0 and torch.all(dq[3] == 0)


def test_indexer_kl_bwd_long_rows_sampled(sa):
    """The bench's KL launch shape: 64 indexer heads x 128, k = 2048 over the long
    workload's 32768 key rows, on 32 of its query rows (T is the only difference); dk_I
    is complete, since only these rows contribute."""
    wl = W["long_dsa"]
    rows = np.linspace(wl.T // 2, wl.T - 1, 32).astype(np.int64)
    x = workloads.indexer_inputs(wl, device=DEV)
    sel = torch.from_numpy(rows).to(DEV)
    qI, wv, kI = x["q_I"][sel].contiguous(), x["w"][sel].contiguous(), x["k_I"]
    idx = workloads.random_causal_index(wl.T, 2048, wl.seed, device=DEV)[sel].contiguous()
    teacher = _random_teacher(idx.cpu().numpy(), 11)
    loss, dq, dw, dk = sa.indexer_kl_bwd(qI, kI, wv, idx, torch.from_numpy(teacher).to(DEV))
    torch.cuda.synchronize()
    rl, _, rdq, rdw, rdk = oracle.indexer_kl(qI.cpu(), kI.cpu(), wv.cpu(), idx.cpu().numpy(), teacher)
    close(loss.cpu().numpy(), rl, 1e-4, 1e-3, "loss")
    grad_close(dq.float().cpu().numpy(), rdq, "dq_I")
    grad_close(dw.cpu().numpy(), rdw, "dw")
    grad_close(dk.cpu().numpy(), rdk, "dk_I")


def test_indexer_kl_bwd_fp32_tiny(sa):
    wl = W["tiny_fp32"]
    x = workloads.indexer_inputs(wl)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 64)
    teacher = _random_teacher(ref_idx, 10)
    loss, dq, dw, dk = sa.indexer_kl_bwd(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV),
                                         torch.from_numpy(ref_idx).to(DEV), torch.from_numpy(teacher).to(DEV))
    rl, _, rdq, rdw, rdk = oracle.indexer_kl(x["q_I"], x["k_I"], x["w"], ref_idx, teacher)
    close(loss.cpu().numpy(), rl, 1e-5, 1e-5, "loss")
    for got, ref, what in [(dq, rdq, "dq_I"), (dw, rdw, "dw"), (dk, rdk, "dk_I")]:
        grad_close(got.cpu().numpy(), ref, what, a=1e-4, r=1e-5, floor=1e-5)


def test_sparse_kl_chain_nope_workload(sa):
    """The whole chain on the NoPE workload (1024 tokens, 16 indexer heads on the integer
    grid, k = 127, 16 attention heads 512 wide): fused indexer top-k -> sparse MLA ->
    teacher -> KL loss and indexer gradients, every step on the GPU, against the same
    chain in the oracle (indices bit-exact, then the tolerances above)."""
    wl = W["nope_unaligned"]
    k = 127
    x = workloads.indexer_inputs(wl, integer=True)
    m = workloads.mla_inputs(wl)
    xd = {n: t.to(DEV) for n, t in x.items()}
    idx = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], k)
    q, kv = m["q512"].to(DEV), m["kv512"].to(DEV)
    _, lse = sa.sparse_mla(q, kv, idx, wl.scale)
    teacher = sa.attn_teacher(q, kv, idx, lse, wl.scale)
    loss, dq, dw, dk = sa.indexer_kl_bwd(xd["q_I"], xd["k_I"], xd["w"], idx, teacher)
    torch.cuda.synchronize()
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    ref_t = oracle.attn_teacher(m["q512"], m["kv512"], ref_idx, wl.scale)
    close(teacher.cpu().numpy(), ref_t, 1e-6, 1e-3, "teacher")
    rl, _, rdq, rdw, rdk = oracle.indexer_kl(x["q_I"], x["k_I"], x["w"], ref_idx, ref_t)
    close(loss.cpu().numpy(), rl, 1e-4, 1e-3, "loss")
    grad_close(dq.float().cpu().numpy(), rdq, "dq_I")
    grad_close(dw.cpu().numpy(), rdw, "dw")
    grad_close(dk.cpu().numpy(), rdk, "dk_I")
