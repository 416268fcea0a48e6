"""GPU parity of the backward kernels against the CPU oracle's closed-form gradients,
through the C ABI.

The backward accumulates key gradients with floating-point atomics, so it is checked
numerically, not bit for bit. Tolerance for bf16 gradients, per element:
|got - ref| <= 2e-2 * rms_row(ref) + 1e-2 * |ref| + 1e-4, where rms_row is the root mean
square of the element's row (its channels: one query head of dq, one latent or key row
of dkv). Two bf16 roundings set the error, each at most 2^-9 relative: the
probabilities and their gradients ds_j enter the matrix cores as bf16, and the
outputs are stored as bf16. Both stay near 2^-9 * rms_row: the terms' signs vary, so
a sum's error and its size both grow like sqrt(n). (The kernel sums D = sum_j p_j dp_j
itself; D taken from the forward's bf16 output instead would shift every ds_j of a
head together, and on rows whose few keys nearly cancel that error alone exceeds this
bound.) A floor of 1e-4 covers rows that cancel
exactly (one valid slot: p = 1 and dp = D, so the reference is exactly zero while the
device's p is 1 only to within rounding). fp32 inputs: |got - ref| <= 1e-4 * rms_row +
1e-5 * |ref| + 1e-5: the sums dp_j = dout . v_j and D are of order sqrt(d) |dout| |v|
(about 10 here) and keep about 1e-6 of fp32 rounding in dp_j - D, which every ds_j
carries into a gradient summed over the row's keys.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
W = workloads.WORKLOADS


@pytest.fixture(scope="module")
def sa():
    import indexer_routed_sparse_amd as m
    return m


def grad_close(got, ref, what, a=2e-2, r=1e-2, floor=1e-4):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    err = np.abs(got - ref)
    bad = err > a * rms + r * np.abs(ref) + floor
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance; max err {err.max():.3g}"


def _mla_case(T, S, H, k, d_qk, seed, dtype=torch.bfloat16, frac_invalid=0.1):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((T, H, d_qk), generator=g).to(dtype)
    kv = torch.randn((S, d_qk), generator=g).to(dtype)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < frac_invalid] = -1
    dout = torch.randn((T, H, 512), generator=g).to(dtype)
    return q, kv, idx, dout


def _run_mla_bwd(sa, q, kv, idx, dout, scale):
    qd, kvd, idxd, gd = q.to(DEV), kv.to(DEV), idx.to(DEV), dout.to(DEV)
    out, lse = sa.sparse_mla(qd, kvd, idxd, scale)
    dq, dkv = sa.sparse_mla_bwd(qd, kvd, idxd, gd, lse, scale)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dkv.cpu().numpy()


@pytest.mark.parametrize("H,k,d_qk", [(16, 65, 512), (16, 127, 576), (8, 64, 576), (64, 33, 576),
                                      (64, 200, 512), (128, 96, 512), (128, 2051, 576), (80, 1, 576),
                                      (32, 70, 576), (128, 1, 576), (64, 17, 576)])
def test_sparse_mla_bwd_shapes(sa, H, k, d_qk):
    """Head counts 8..128 (partial 16-head groups), widths 512/576, top-k from 1 to the
    GLM width 2051; -1 slots, a repeated index, an all-invalid row."""
    T, S = 24, 700
    q, kv, idx, dout = _mla_case(T, S, H, k, d_qk, seed=H * 7 + k + d_qk)
    idx[3] = -1
    if k >= 3:
        idx[5, :3] = torch.tensor([11, 11, 40], dtype=torch.int32)
    scale = 1 / math.sqrt(d_qk)
    dq, dkv = _run_mla_bwd(sa, q, kv, idx, dout, scale)
    rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx.numpy(), dout, scale)
    grad_close(dq, rdq, "dq")
    grad_close(dkv, rdkv, "dkv")
    assert np.all(dq[3] == 0)


def test_sparse_mla_bwd_nope_unaligned(sa):
    """The NoPE workload: 512-wide q/kv (the kernel's 512 instantiation) equal to the
    zero-padded 576 case, at k = 127 with the all-invalid row 511, against the oracle."""
    wl = W["nope_unaligned"]
    x = workloads.indexer_inputs(wl, integer=True)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 127)
    ref_idx[511] = -1
    m = workloads.mla_inputs(wl)
    g = torch.Generator().manual_seed(77)
    dout = torch.randn((wl.T, wl.H, 512), generator=g).to(torch.bfloat16)
    idx = torch.from_numpy(ref_idx)
    dq5, dkv5 = _run_mla_bwd(sa, m["q512"], m["kv512"], idx, dout, wl.scale)
    dq6, dkv6 = _run_mla_bwd(sa, m["q"], m["kv"], idx, dout, wl.scale)
    rdq, rdkv = oracle.sparse_mla_bwd(m["q512"], m["kv512"], ref_idx, dout, wl.scale)
    grad_close(dq5, rdq, "dq 512")
    grad_close(dkv5, rdkv, "dkv 512")
    grad_close(dq6[:, :, :512], rdq, "dq 576")
    grad_close(dkv6[:, :512], rdkv, "dkv 576")
    assert np.all(dq6[:, :, 512:] == 0)                    # zero RoPE slot of q: no gradient flows
    assert np.all(dq5[511] == 0)


def test_sparse_mla_bwd_tiny_fp32(sa):
    wl = W["tiny_fp32"]
    x = workloads.indexer_inputs(wl)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 64)
    m = workloads.mla_inputs(wl)
    g = torch.Generator().manual_seed(78)
    dout = torch.randn((wl.T, wl.H, 512), generator=g)
    dq, dkv = _run_mla_bwd(sa, m["q"], m["kv"], torch.from_numpy(ref_idx), dout, wl.scale)
    rdq, rdkv = oracle.sparse_mla_bwd(m["q"], m["kv"], ref_idx, dout, wl.scale)
    grad_close(dq, rdq, "dq", a=1e-4, r=1e-5, floor=1e-5)
    grad_close(dkv, rdkv, "dkv", a=1e-4, r=1e-5, floor=1e-5)


def test_sparse_mla_bwd_long_rows_sampled(sa):
    """128 heads, k = 2048 over a 32768-row latent: dq of sampled rows against the
    oracle, and dkv over the whole call (64 rows, so the oracle sums every row)."""
    wl = W["long_dsa"]
    T = 64
    m = workloads.mla_inputs(wl, device=DEV)
    q = m["q"][-T:].contiguous()
    idx = workloads.random_causal_index(wl.T, 2048, wl.seed, device=DEV)[-T:].contiguous()
    g = torch.Generator(device=DEV).manual_seed(79)
    dout = torch.randn((T, wl.H, 512), generator=g, device=DEV).to(torch.bfloat16)
    out, lse = sa.sparse_mla(q, m["kv"], idx, wl.scale)
    dq, dkv = sa.sparse_mla_bwd(q, m["kv"], idx, dout, lse, wl.scale)
    dq2, _ = sa.sparse_mla_bwd(q, m["kv"], idx, dout, lse, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2)                            # dq has no atomics: bitwise replay
    rdq, rdkv = oracle.sparse_mla_bwd(q.cpu(), m["kv"].cpu(), idx.cpu().numpy(), dout.cpu(), wl.scale)
    grad_close(dq.float().cpu().numpy(), rdq, "dq")
    grad_close(dkv.cpu().numpy(), rdkv, "dkv")


# ------------------------------------------------------------------ block-sparse GQA

def _run_gqa_bwd(sa, q, k, v, blk, dout, B, scale, lengths=None):
    d = {n: t.to(DEV) for n, t in dict(q=q, k=k, v=v, blk=blk, dout=dout).items()}
    kw = {}
    if lengths:
        kw = dict(cu_seqlens=torch.from_numpy(workloads.cu_seqlens(lengths)).to(DEV), max_seqlen=max(lengths))
    out, lse = sa.block_sparse_gqa(d["q"], d["k"], d["v"], d["blk"], scale, block_size=B, **kw)
    dq, dk, dv = sa.block_sparse_gqa_bwd(d["q"], d["k"], d["v"], d["blk"], d["dout"], lse, scale,
                                         block_size=B, **kw)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


@pytest.mark.parametrize("Hq,Hkv,D,B,dtype", [(32, 4, 128, 64, "bf16"), (8, 4, 128, 32, "bf16"),
                                              (16, 1, 64, 16, "bf16"), (12, 2, 64, 48, "bf16"),
                                              (8, 2, 64, 32, "f32")])
def test_block_gqa_bwd_shapes_thd(sa, Hq, Hkv, D, B, dtype):
    """Head groups 1..16, D 64/128, block sizes 16..64, packed sequences with one shorter
    than a block, routes with repeated blocks, blocks past the own one and -1 slots."""
    lengths = (300, 7, 213)
    T = sum(lengths)
    gen = torch.Generator().manual_seed(Hq * 131 + D + B + 5)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((T, Hq, D), generator=gen).to(tdt)
    k = torch.randn((T, Hkv, D), generator=gen).to(tdt)
    v = torch.randn((T, Hkv, D), generator=gen).to(tdt)
    dout = torch.randn((T, Hq, D), generator=gen).to(tdt)
    nblk = 6
    blk = workloads.random_block_index(T, nblk, B, 29, lengths=lengths).clone()
    starts = workloads.cu_seqlens(lengths)
    for t in range(0, T, 3):
        c = int(starts[np.searchsorted(starts, t, side="right") - 1])
        own = (t - c) // B
        if blk[t, 0] >= 0:
            blk[t, nblk - 1] = blk[t, 0]                  # repeated block
        blk[t, nblk - 2] = own + 1                        # past the own block
    blk[50] = -1                                          # no key at all
    dq, dk, dv = _run_gqa_bwd(sa, q, k, v, blk, dout, B, 0.3, lengths)
    rdq, rdk, rdv = oracle.block_sparse_gqa_bwd(q, k, v, blk.numpy(), dout, B, 0.3, cu_seqlens=starts)
    kw = dict(a=1e-4, r=1e-5, floor=1e-5) if dtype == "f32" else {}
    grad_close(dq, rdq, "dq", **kw)
    grad_close(dk, rdk, "dk", **kw)
    grad_close(dv, rdv, "dv", **kw)
    assert np.all(dq[50] == 0)


@pytest.mark.parametrize("lengths,Hq,Hkv,D,B", [((1500, 2900, 777), 8, 2, 128, 48),
                                                 ((4100,), 16, 4, 64, 64),
                                                 ((2047, 1, 2049), 4, 4, 128, 32)])
def test_block_gqa_bwd_key_major_chunks(sa, lengths, Hq, Hkv, D, B):
    """dk and dv are summed key-major over chunks of 2048 tokens per 64-key block: packed
    sequences that cross chunk boundaries, block sizes that do not align with the
    64-key blocks, a one-token sequence; every row of dq, dk and dv against the oracle."""
    T = sum(lengths)
    gen = torch.Generator().manual_seed(T + Hq + D + B)
    q = torch.randn((T, Hq, D), generator=gen).to(torch.bfloat16)
    k = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16)
    v = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16)
    dout = torch.randn((T, Hq, D), generator=gen).to(torch.bfloat16)
    blk = workloads.random_block_index(T, 8, B, 31, lengths=lengths)
    dq, dk, dv = _run_gqa_bwd(sa, q, k, v, blk, dout, B, 0.2, lengths)
    rdq, rdk, rdv = oracle.block_sparse_gqa_bwd(q, k, v, blk.numpy(), dout, B, 0.2,
                                                cu_seqlens=workloads.cu_seqlens(lengths))
    grad_close(dq, rdq, "dq")
    grad_close(dk, rdk, "dk")
    grad_close(dv, rdv, "dv")


def test_block_gqa_bwd_long_sequence_per_token_kernel(sa):
    """One 130,003-token sequence at D = 128: the grouped backward's rows, stages and
    set-up tables would exceed the LDS, so the per-(token, kv head) kernel serves it.
    Routes hold only the own block (16 keys), so a block's dk and dv come from its own
    16 rows: the oracle runs on the rows of a few sampled blocks and their gradients
    are compared in full."""
    T, Hq, Hkv, D, B = 130_003, 2, 2, 128, 16
    gen = torch.Generator(device=DEV).manual_seed(78)
    q = torch.randn((T, Hq, D), generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn((T, Hkv, D), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((T, Hkv, D), generator=gen, device=DEV).to(torch.bfloat16)
    dout = torch.randn((T, Hq, D), generator=gen, device=DEV).to(torch.bfloat16)
    blk = (torch.arange(T, device=DEV) // B).to(torch.int32).reshape(T, 1).contiguous()
    scale = 1 / math.sqrt(D)
    out, lse = sa.block_sparse_gqa(q, k, v, blk, scale, block_size=B)
    dq, dk, dv = sa.block_sparse_gqa_bwd(q, k, v, blk, dout, lse, scale, block_size=B)
    torch.cuda.synchronize()
    blocks = [0, 1, 777, 4000, T // B - 1, T // B]           # the last one is partial
    rows = np.concatenate([np.arange(b * B, min(b * B + B, T)) for b in blocks])
    rdq, rdk, rdv = oracle.block_sparse_gqa_bwd(q.cpu(), k.cpu(), v.cpu(), blk.cpu().numpy(), dout.cpu(),
                                                B, scale, rows=rows)
    grad_close(dq.float().cpu().numpy()[rows], rdq, "dq")
    grad_close(dk.cpu().numpy()[rows], rdk[rows], "dk")
    grad_close(dv.cpu().numpy()[rows], rdv[rows], "dv")


def test_block_gqa_bwd_block_routed_workload(sa):
    """The block-routed workload's shapes (32/4 heads x 128, 64-key blocks, 16 blocks
    with the own block) on oracle routes over 2048 tokens: dq of every row, dk and dv."""
    wl = W["block_gqa"]
    T = 2048
    x = workloads.indexer_inputs(wl, T=T)
    blk, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 16, block_size=64, force_own_block=True)
    g = workloads.gqa_inputs(wl, T=T)
    gen = torch.Generator().manual_seed(81)
    dout = torch.randn((T, wl.Hq, wl.Dv), generator=gen).to(torch.bfloat16)
    dq, dk, dv = _run_gqa_bwd(sa, g["q"], g["k"], g["v"], torch.from_numpy(blk), dout, 64, wl.scale)
    rdq, rdk, rdv = oracle.block_sparse_gqa_bwd(g["q"], g["k"], g["v"], blk, dout, 64, wl.scale)
    grad_close(dq, rdq, "dq")
    grad_close(dk, rdk, "dk")
    grad_close(dv, rdv, "dv")
