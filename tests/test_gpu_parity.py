"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Indices are compared bit for bit: top-k selection is fed the oracle's own fp32
scores, and the end-to-end indexer runs use integer-valued inputs whose scores are
exact in fp32. Attention outputs are compared within max-abs 2e-2 + relative 1e-2
(bf16) or 1e-5 (fp32 inputs), always on the same index tensor as the oracle. Small
workloads are checked whole; the two full-size ones on sampled rows.
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


def close(got, ref, atol, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finiteness differs"
    bad = np.abs(got[fin] - ref[fin]) > atol + rtol * np.abs(ref[fin])
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err " \
                          f"{np.abs(got[fin] - ref[fin]).max():.3g}"
    assert np.array_equal(got[~fin], ref[~fin]), f"{what}: infinities differ"


BF16_TOL = dict(atol=2e-2, rtol=1e-2)
F32_TOL = dict(atol=1e-5, rtol=1e-5)


def sample_rows(T, n, seed, lengths=None):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows |= {0, T - 1}
    if lengths:
        cu = workloads.cu_seqlens(lengths)
        rows |= {int(c) for c in cu[:-1]} | {int(c) - 1 for c in cu[1:]}
    return np.array(sorted(rows))


def cu_dev(lengths):
    return torch.from_numpy(workloads.cu_seqlens(lengths)).to(DEV)


# ------------------------------------------------------------------------ top-k select

@pytest.mark.parametrize("name,k,T", [("tiny_fp32", 64, None), ("nope_unaligned", 65, None),
                                      ("nope_unaligned", 127, None), ("nope_unaligned", 2051, None)])
def test_topk_select_on_oracle_scores(sa, name, k, T):
    wl = W[name]
    x = workloads.indexer_inputs(wl, T=T)
    sc = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"])
    ld = (sc.shape[1] + 3) // 4 * 4
    scp = np.full((sc.shape[0], ld), -np.inf, dtype=np.float32)
    scp[:, :sc.shape[1]] = sc
    ref_i, ref_v = oracle.topk_select_dense(scp, k)
    idx, val = sa.topk_select(torch.from_numpy(scp).to(DEV), k, with_values=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(val.cpu().numpy().view(np.uint32), ref_v.view(np.uint32))


def test_topk_select_block_mode_forced_own(sa):
    wl = W["block_gqa"]
    T = 2048
    x = workloads.indexer_inputs(wl, T=T)
    sc = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"], block_size=64)
    ref_i, ref_v = oracle.topk_select_dense(sc, 16, block_size=64, force_own_block=True)
    idx, val = sa.topk_select(torch.from_numpy(sc).to(DEV), 16, block_size=64,
                              force_own_block=True, with_values=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(val.cpu().numpy(), ref_v)


def test_topk_select_thd_and_candidates(sa):
    lengths = (300, 1, 77, 1000, 2)
    T = sum(lengths)
    wl = W["nope_unaligned"]
    x = workloads.indexer_inputs(wl, T=T)
    cu = workloads.cu_seqlens(lengths)
    sc = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"], cu_seqlens=cu, ld=1000)
    ref_i, _ = oracle.topk_select_dense(sc, 65, cu_seqlens=cu)
    idx = sa.topk_select(torch.from_numpy(sc).to(DEV), 65, cu_seqlens=cu_dev(lengths), max_seqlen=1000)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
    # explicit candidate lists with -1 holes: same selection over the remaining ones
    rng = np.random.default_rng(3)
    cand = np.where(np.isfinite(sc), np.arange(1000)[None, :] + cu[:-1].repeat(lengths)[:, None], -1)
    holes = rng.random(cand.shape) < 0.2
    cand = np.where(holes, -1, cand).astype(np.int32)
    ref_c, ref_cv = oracle.topk_select_candidates(np.where(cand >= 0, sc, -np.inf), cand, 65)
    idx_c, val_c = sa.topk_select(torch.from_numpy(np.ascontiguousarray(sc)).to(DEV), 65,
                                  cand_idx=torch.from_numpy(cand).to(DEV), with_values=True)
    np.testing.assert_array_equal(idx_c.cpu().numpy(), ref_c)
    np.testing.assert_array_equal(val_c.cpu().numpy(), ref_cv)


@pytest.mark.parametrize("name", ["long_dsa", "thd_varlen"])
def test_topk_select_full_size_sampled(sa, name):
    wl = W[name]
    T = wl.T
    x = workloads.indexer_inputs(wl, device=DEV)
    lengths = wl.lengths if len(wl.lengths) > 1 else None
    rows = sample_rows(T, 10, 7, lengths)
    cu = workloads.cu_seqlens(wl.lengths)
    maxlen = max(wl.lengths)
    ld = (maxlen + 3) // 4 * 4
    sc = oracle.indexer_scores_dense(x["q_I"].cpu(), x["k_I"].cpu(), x["w"].cpu(),
                                     cu_seqlens=cu if lengths else None, rows=rows, ld=ld)
    vals = torch.full((T, ld), float("-inf"), device=DEV)
    vals[torch.from_numpy(rows).to(DEV)] = torch.from_numpy(sc).to(DEV)
    kw = dict(cu_seqlens=cu_dev(wl.lengths), max_seqlen=maxlen) if lengths else {}
    idx, val = sa.topk_select(vals, 2048, with_values=True, **kw)
    ref_i, ref_v = oracle.topk_select_dense(sc, 2048, cu_seqlens=cu if lengths else None, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i)
    np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v)


@pytest.mark.parametrize("T", [17884, 32768])
def test_topk_select_wide_rows(sa, T):
    """Rows of 16K-32K token positions of one sequence (the widest class of the bench's
    materialised matrix): dense normal scores, with rows of four distinct values (ties at
    the k-th key), constant rows (every pivot fails, so the retry launch takes them) and
    rows that repeat one value over their first 4096 positions; sampled rows against the
    oracle, ids and values bit for bit."""
    gen = torch.Generator(device=DEV).manual_seed(T)
    ld = T
    vals = torch.randn((T, ld), generator=gen, device=DEV)
    lo = 16384
    tied = torch.arange(lo + 1, T, 7, device=DEV)
    vals[tied] = torch.randint(0, 4, (tied.numel(), ld), generator=gen, device=DEV).float()
    const = torch.arange(lo + 3, T, 61, device=DEV)
    vals[const] = 0.5
    front = torch.arange(lo + 5, T, 97, device=DEV)
    vals[front, :4096] = 3.0
    rows = np.unique(np.concatenate([
        np.arange(lo, lo + 12), np.arange(lo + 508, lo + 520), np.arange(lo + 1020, lo + 1030),
        np.arange(T - 8, T), tied.cpu().numpy()[-3:], const.cpu().numpy()[:4], front.cpu().numpy()[:3]]))
    rows = rows[(rows >= lo) & (rows < T)]
    idx, val = sa.topk_select(vals, 2048, with_values=True)
    sc = vals[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    ref_i, ref_v = oracle.topk_select_dense(sc, 2048, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i)
    np.testing.assert_array_equal(val.cpu().numpy()[rows].view(np.uint32), ref_v.view(np.uint32))


def _cand_case(case, rng):
    """(vals [T, ld] fp32, cand [T, ld] int32, topk) for one selection stress case.

    Candidate ids are position + 1000 so that a position reported as an id shows.
    """
    def normal(T, ld):
        return rng.standard_normal((T, ld)).astype(np.float32)
    holes = None
    if case == "normal_64k":
        v, k = normal(3, 65536), 2048
    elif case == "ties_64k":           # one value everywhere: selection is by index alone
        v, k = np.ones((2, 65536), np.float32), 2048
        v[0, 40000] = 2.0
    elif case == "few_values":         # four distinct values: huge ties at the k-th
        v, k = rng.integers(0, 4, (4, 20000)).astype(np.float32), 2048
    elif case == "zeros_infs":         # -0/+0 tie, infinities, denormals
        pool = np.array([-0.0, 0.0, -np.inf, np.inf, 1e-40, -1e-40, 1.0, -1.0], np.float32)
        v, k = pool[rng.integers(0, pool.size, (4, 12288))], 3000
    elif case == "big_topk":           # topk above the candidate buffer
        v, k = normal(2, 40000), 8000
    elif case == "holes":
        v, k = normal(4, 30000), 2048
        holes = rng.random(v.shape) < 0.9
    elif case == "under_cap":          # more valid than k but fewer than the buffer
        v, k = normal(4, 8192), 2048
        holes = rng.random(v.shape) < 0.4
    elif case == "trend":              # scores rising with position
        v = (np.arange(32768)[None, :] * 1e-3 + rng.standard_normal((3, 32768))).astype(np.float32)
        k = 2048
    elif case == "dup_bins":           # quarter steps: each radix bin holds a few repeated values
        v = (1000.0 + 0.25 * rng.integers(0, 3000, (4, 20000))).astype(np.float32)
        k = 2048
    elif case == "clustered":          # one dense cluster around the k-th value
        v = (100.0 + 1e-3 * rng.standard_normal((3, 32768))).astype(np.float32)
        k = 2048
    else:
        raise ValueError(case)
    cand = np.broadcast_to(np.arange(v.shape[1], dtype=np.int32) + 1000, v.shape).copy()
    if holes is not None:
        cand[holes] = -1
    return v, cand, k


@pytest.mark.parametrize("case", ["normal_64k", "ties_64k", "few_values", "zeros_infs", "big_topk",
                                  "holes", "under_cap", "trend", "clustered", "dup_bins"])
def test_topk_select_candidate_stress(sa, case):
    rng = np.random.default_rng(11)
    v, cand, k = _cand_case(case, rng)
    ref_i, ref_v = oracle.topk_select_candidates(np.where(cand >= 0, v, -np.inf), cand, k)
    idx, val = sa.topk_select(torch.from_numpy(v).to(DEV), k, cand_idx=torch.from_numpy(cand).to(DEV),
                              with_values=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(val.cpu().numpy().view(np.uint32), ref_v.view(np.uint32))


@pytest.mark.parametrize("ld", [2044, 2048, 2052, 4096, 6144, 6148, 16388])
def test_topk_select_row_width_edges(sa, ld):
    rng = np.random.default_rng(ld)
    v = rng.standard_normal((3, ld)).astype(np.float32)
    cand = np.broadcast_to(np.arange(ld, dtype=np.int32), v.shape).copy()
    for k in (1, 2048, ld - 1):
        ref_i, ref_v = oracle.topk_select_candidates(v, cand, k)
        idx, val = sa.topk_select(torch.from_numpy(v).to(DEV), k, cand_idx=torch.from_numpy(cand).to(DEV),
                                  with_values=True)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_i, err_msg=f"k={k}")
        np.testing.assert_array_equal(val.cpu().numpy(), ref_v, err_msg=f"k={k}")


def test_topk_select_wide_block_mode_forced_own(sa):
    # block_size 2 over 14000 rows: rows up to 7000 blocks wide, above the candidate buffer
    T, B, k = 14000, 2, 2048
    n_cols = (T - 1) // B + 1
    rng = np.random.default_rng(5)
    vals = torch.from_numpy(rng.standard_normal((T, n_cols)).astype(np.float32)).to(DEV)
    idx, val = sa.topk_select(vals, k, block_size=B, force_own_block=True, with_values=True)
    rows = sample_rows(T, 40, 9)
    rows = np.union1d(rows, [2 * 6144 - 1, 2 * 6144, 2 * 6145, 2 * 2048, 2 * 2049 + 1])
    sc = vals.cpu().numpy()[rows]
    ref_i, ref_v = oracle.topk_select_dense(sc, k, block_size=B, force_own_block=True, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i)
    np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v)


# ---------------------------------------------------------------------- indexer

@pytest.mark.parametrize("name,T,B", [("tiny_fp32", None, 1), ("nope_unaligned", None, 1),
                                      ("block_gqa", 1024, 1), ("block_gqa", 2048, 64)])
def test_indexer_dense_integer_exact(sa, name, T, B):
    wl = W[name]
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    ref = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"], block_size=B)
    got = sa.indexer_scores(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), block_size=B)
    got = got.cpu().numpy()[:, :ref.shape[1]]
    np.testing.assert_array_equal(got, ref)


def test_indexer64_head_dim_64(sa):
    """64 indexer heads of dimension 64 (the 64-head kernel's other instantiation): dense
    scores equal the oracle on the integer grid, and the fused selection equals the
    select over those scores, bit for bit, with a ragged last tile."""
    import dataclasses
    wl = dataclasses.replace(W["long_dsa"], D_I=64)
    T = 1000
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    assert x["q_I"].shape == (T, 64, 64)
    ref = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"])
    xd = {n: t.to(DEV) for n, t in x.items()}
    dense = sa.indexer_scores(xd["q_I"], xd["k_I"], xd["w"])
    np.testing.assert_array_equal(dense.cpu().numpy()[:, :ref.shape[1]], ref)
    for k in (100, 513):
        i1, v1 = sa.topk_select(dense, k, with_values=True)
        i2, v2 = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], k, with_values=True)
        assert torch.equal(i1, i2), f"k={k}"
        assert torch.equal(v1, v2), f"k={k}"


@pytest.mark.parametrize("name,T", [("tiny_fp32", None), ("nope_unaligned", None), ("long_dsa", 1536)])
def test_indexer_dense_normal_within_bound(sa, name, T):
    # fp32 accumulation of bf16 products: |err| <= (D_I + H_I) * 2^-24 * B[t,s] with
    # B[t,s] = sum_h |w| sum_d |q||k|; checked at 2e-5 * B.
    wl = W[name]
    x = workloads.indexer_inputs(wl, T=T)
    ref = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"])
    bound = oracle.indexer_scores_dense(x["q_I"].float().abs(), x["k_I"].float().abs(), x["w"].abs())
    got = sa.indexer_scores(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV)).cpu().numpy()
    got = got[:, :ref.shape[1]]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(np.abs(got[fin] - ref[fin]) <= 2e-5 * bound[fin] + 1e-30)


@pytest.mark.parametrize("B", [2, 4, 8, 16, 32, 128, 256])
def test_indexer_block_sizes_integer_exact(sa, B):
    """Block mode at every other supported block size (the block max runs over a lane
    group of B lanes up to 64, and across key tiles above): dense block scores equal
    the oracle on the integer grid, and the fused top-k with the own block forced equals
    the oracle's, on one sequence and on packed sequences with ragged lengths."""
    wl = W["block_gqa"]
    for lengths in [(1000,), (300, 7, 520, 129)]:
        T = sum(lengths)
        x = workloads.indexer_inputs(wl, integer=True, T=T)
        cu = workloads.cu_seqlens(lengths) if len(lengths) > 1 else None
        kw = dict(cu_seqlens=cu_dev(lengths), max_seqlen=max(lengths)) if cu is not None else {}
        ref = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"], cu_seqlens=cu, block_size=B)
        got = sa.indexer_scores(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), block_size=B,
                                **kw).cpu().numpy()
        np.testing.assert_array_equal(got[:, :ref.shape[1]], ref, err_msg=f"lengths {lengths}")
        k = 5
        ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k, cu_seqlens=cu, block_size=B,
                                           force_own_block=True)
        idx, val = sa.indexer_topk(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), k, block_size=B,
                                   force_own_block=True, with_values=True, **kw)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_i, err_msg=f"lengths {lengths}")
        np.testing.assert_array_equal(val.cpu().numpy(), ref_v, err_msg=f"lengths {lengths}")


def test_indexer_dense_thd(sa):
    lengths = (300, 5, 700, 64, 129)
    T = sum(lengths)
    wl = W["long_dsa"]
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    cu = workloads.cu_seqlens(lengths)
    for B in (1, 64):
        ref = oracle.indexer_scores_dense(x["q_I"], x["k_I"], x["w"], cu_seqlens=cu, block_size=B)
        got = sa.indexer_scores(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), block_size=B,
                                cu_seqlens=cu_dev(lengths), max_seqlen=700).cpu().numpy()
        np.testing.assert_array_equal(got[:, :ref.shape[1]], ref)


@pytest.mark.parametrize("name,k,T,B", [("tiny_fp32", 64, None, 1), ("nope_unaligned", 65, None, 1),
                                        ("nope_unaligned", 127, None, 1), ("long_dsa", 2048, 3000, 1),
                                        ("block_gqa", 16, 2048, 64)])
def test_indexer_topk_fused_integer_exact(sa, name, k, T, B):
    wl = W[name]
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k, block_size=B,
                                       force_own_block=B > 1)
    idx, val = sa.indexer_topk(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), k,
                               block_size=B, force_own_block=B > 1, with_values=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(val.cpu().numpy(), ref_v)


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("lengths", [(8192,), (3000, 64, 5128)])
def test_block_routed_path_full_size_against_oracle(sa, lengths, workspace):
    """The block-routed workload at its stated size (8192 tokens, 16 indexer heads x 128,
    64-key blocks, top 16 blocks with the query's own block forced) on the integer grid:
    the fused block top-k equals the oracle bit for bit (ids and values) on sampled rows,
    among them the last 64 rows, whose candidate blocks (128 on one sequence, 81 in the
    last packed sequence) overflow the 80-entry candidate buffer so that it is cut back
    mid-stream; then sparse GQA over those GPU
    routes equals the oracle's attention on the same rows. With a workspace the key
    range of each group of rows is split over 4 (3) workgroups and their partial
    top-k lists are merged; without one, one workgroup walks it all."""
    wl = W["block_gqa"]
    T = sum(lengths)
    assert T == wl.T
    x = workloads.indexer_inputs(wl, integer=True)
    assert workloads.exact_sum_bound(x["q_I"], x["k_I"], x["w"]) < 2 ** 24
    multi = len(lengths) > 1
    cu = workloads.cu_seqlens(lengths) if multi else None
    kw = dict(cu_seqlens=cu_dev(lengths), max_seqlen=max(lengths)) if multi else {}
    xd = {n: t.to(DEV) for n, t in x.items()}
    blk, val = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], 16, block_size=64,
                               force_own_block=True, with_values=True, workspace=workspace, **kw)
    rows = sample_rows(T, 64, 29, lengths if multi else None)
    rows = np.union1d(rows, np.arange(T - 64, T))
    ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 16, cu_seqlens=cu, block_size=64,
                                       force_own_block=True, rows=rows)
    np.testing.assert_array_equal(blk.cpu().numpy()[rows], ref_i)
    np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v)
    g = workloads.gqa_inputs(wl, device=DEV)
    out, lse = sa.block_sparse_gqa(g["q"], g["k"], g["v"], blk, wl.scale, block_size=64, **kw)
    ro, rl = oracle.block_sparse_gqa(g["q"].cpu(), g["k"].cpu(), g["v"].cpu(), blk.cpu().numpy(), 64,
                                     wl.scale, cu_seqlens=cu, rows=rows)
    close(out.float().cpu().numpy()[rows], ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy()[rows], rl, **BF16_TOL, what="lse")


@pytest.mark.parametrize("B,k,own", [(64, 16, True), (16, 64, True), (128, 8, True), (256, 3, False),
                                      (32, 1, False)])
def test_block_topk_split_key_ranges(sa, B, k, own):
    """Block top-k with a workspace: each group of rows' key tiles split over 2-3
    workgroups (windows of whole blocks: 4 tiles per block at B = 256, 4 blocks per
    tile at B = 16) whose exact partial lists a merge combines. Ids and values equal
    the one-pass kernel bit for bit on every row, and the oracle on sampled rows, for
    one sequence and for packed ones (short sequences whose windows hold no tile)."""
    wl = W["block_gqa"]
    for lengths in [(6000,), (2100, 37, 4000, 1900)]:
        T = sum(lengths)
        multi = len(lengths) > 1
        x = workloads.indexer_inputs(wl, integer=True, T=T)
        xd = {n: t.to(DEV) for n, t in x.items()}
        kw = dict(cu_seqlens=cu_dev(lengths), max_seqlen=max(lengths)) if multi else {}
        ws = sa.indexer_workspace(xd["q_I"], k, max_seqlen=max(lengths), block_size=B)
        assert ws is not None and ws.numel() > 0
        i1, v1 = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], k, block_size=B, force_own_block=own,
                                 with_values=True, workspace=ws, **kw)
        i2, v2 = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], k, block_size=B, force_own_block=own,
                                 with_values=True, workspace=False, **kw)
        assert torch.equal(i1, i2), f"lengths {lengths}"
        assert torch.equal(v1, v2), f"lengths {lengths}"
        rows = np.union1d(sample_rows(T, 16, 41 + B, lengths if multi else None), np.arange(T - 8, T))
        ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k,
                                           cu_seqlens=workloads.cu_seqlens(lengths) if multi else None,
                                           block_size=B, force_own_block=own, rows=rows)
        np.testing.assert_array_equal(i1.cpu().numpy()[rows], ref_i, err_msg=f"lengths {lengths}")
        np.testing.assert_array_equal(v1.cpu().numpy()[rows], ref_v, err_msg=f"lengths {lengths}")


@pytest.mark.parametrize("B,k", [(16, 5), (32, 1), (16, 64)])
def test_block_topk_buffer_cutback_against_oracle(sa, B, k):
    """Block routes with more candidate blocks than the buffer holds (2048 tokens of
    16-key blocks: 128 blocks against a 69-entry buffer at k = 5), so the fused block
    top-k cuts its buffer back mid-stream; every row equals the oracle bit for bit."""
    wl = W["block_gqa"]
    T = 2048
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k, block_size=B,
                                       force_own_block=True)
    idx, val = sa.indexer_topk(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), k, block_size=B,
                               force_own_block=True, with_values=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(val.cpu().numpy(), ref_v)


@pytest.mark.parametrize("B,k,own,T", [(64, 1, True, 8192), (128, 3, False, 12288), (256, 2, True, 20480)])
def test_block_topk_wide_blocks_cutback_against_oracle(sa, B, k, own, T):
    """Blocks of one or more 64-key tiles, one pass (no workspace), on the integer grid:
    each row's block maxima (running over a block's tiles at B = 128 and 256) go to the
    token's buffer, which fills after k + 64 blocks and is cut back mid-stream (twice on
    the last rows at B = 64, k = 1); sampled rows, among them the last 48, equal the
    oracle bit for bit."""
    wl = W["block_gqa"]
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    assert workloads.exact_sum_bound(x["q_I"], x["k_I"], x["w"]) < 2 ** 24
    xd = {n: t.to(DEV) for n, t in x.items()}
    idx, val = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], k, block_size=B, force_own_block=own,
                               with_values=True)
    rows = np.union1d(sample_rows(T, 24, B + k), np.arange(T - 48, T))
    ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k, block_size=B,
                                       force_own_block=own, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i)
    np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v)


@pytest.mark.parametrize("H_I,dtype,B", [(4, "f32", 64), (4, "bf16", 128), (8, "bf16", 64), (32, "bf16", 64),
                                          (64, "bf16", 64), (64, "bf16", 128), (16, "f32", 256)])
def test_block_topk_head_counts_against_oracle(sa, H_I, dtype, B):
    """Block top-k with blocks of one to four key tiles at every indexer head count the
    kernels take (4..64 heads, so 16..1 tokens per wave share a tile's block pass), bf16
    and fp32, packed sequences, one pass and through a workspace: rows past k + 64
    blocks cut their buffers back; sampled rows equal the oracle bit for bit."""
    import dataclasses
    wl = dataclasses.replace(W["block_gqa"], H_I=H_I, dtype=dtype, name=f"block_h{H_I}")
    lengths = (6000, 37, 4500) if B == 64 else (9000, 300, 7000)
    T = sum(lengths)
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    assert workloads.exact_sum_bound(x["q_I"], x["k_I"], x["w"]) < 2 ** 24
    xd = {n: t.to(DEV) for n, t in x.items()}
    cu = workloads.cu_seqlens(lengths)
    rows = np.union1d(sample_rows(T, 24, H_I + B, lengths), np.arange(T - 16, T))
    rows = np.union1d(rows, np.arange(lengths[0] - 16, lengths[0]))
    ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 4, cu_seqlens=cu, block_size=B,
                                       force_own_block=True, rows=rows)
    for workspace in (False, True):
        idx, val = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], 4, block_size=B, force_own_block=True,
                                   with_values=True, workspace=workspace, cu_seqlens=cu_dev(lengths),
                                   max_seqlen=max(lengths))
        np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i, err_msg=f"workspace={workspace}")
        np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v, err_msg=f"workspace={workspace}")


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("k", [1, 100, 777, 2048])
def test_indexer64_fused_small_k_against_oracle(sa, k, workspace):
    """64 indexer heads on the integer grid, one sequence of 4096 tokens and packed
    sequences: the fused selection, in one pass (many buffer cut-backs at small k) and
    in two passes through a workspace (sampled pivot, then the exact select), equals
    the oracle bit for bit on sampled rows, among them each sequence's first and last
    rows and the last 32 rows."""
    wl = W["long_dsa"]
    for lengths in [(4096,), (1000, 3, 2048, 1045)]:
        T = sum(lengths)
        multi = len(lengths) > 1
        x = workloads.indexer_inputs(wl, integer=True, T=T)
        kw = dict(cu_seqlens=cu_dev(lengths), max_seqlen=max(lengths)) if multi else {}
        idx, val = sa.indexer_topk(x["q_I"].to(DEV), x["k_I"].to(DEV), x["w"].to(DEV), k,
                                   with_values=True, workspace=workspace, **kw)
        rows = np.union1d(sample_rows(T, 24, 31 + k, lengths if multi else None),
                          np.arange(T - 32, T))
        ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k,
                                           cu_seqlens=workloads.cu_seqlens(lengths) if multi else None,
                                           rows=rows)
        np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i, err_msg=f"lengths {lengths}")
        np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v, err_msg=f"lengths {lengths}")


@pytest.mark.parametrize("k", [100, 2048])
def test_indexer64_two_pass_redo_rows_against_oracle(sa, k):
    """64 heads with 70 % of the key rows scoring exactly zero (their entries are
    non-positive while every query entry is non-negative): at k = 2048 the k-th score
    of the later rows is a zero shared by thousands of keys, so the sampled pivot keeps
    more keys than a workspace row holds and those rows are marked for the exact
    one-pass kernel. The marks are read back from the workspace's count array, and
    every sampled row equals the oracle bit for bit."""
    import dataclasses
    wl = dataclasses.replace(W["long_dsa"], neg_key_frac=0.7)
    T = 4096
    x = workloads.indexer_inputs(wl, integer=True, T=T)
    xd = {n: t.to(DEV) for n, t in x.items()}
    ws = sa.indexer_workspace(xd["q_I"], k)
    idx, val = sa.indexer_topk(xd["q_I"], xd["k_I"], xd["w"], k, with_values=True, workspace=ws)
    torch.cuda.synchronize()
    cap = (ws.numel() - 4 * T) // (8 * T)
    cnt = ws[8 * T * cap:8 * T * cap + 4 * T].view(torch.int32).cpu().numpy()
    if k == 2048:
        assert (cnt == -1).sum() > 100, "no row was left to the exact kernel"
    assert np.all((cnt == -1) | ((cnt >= np.minimum(k, np.arange(T) + 1)) & (cnt <= cap)))
    rows = np.union1d(sample_rows(T, 40, 37), np.arange(T - 16, T))
    rows = np.union1d(rows, np.nonzero(cnt == -1)[0][:16])
    ref_i, ref_v = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k, rows=rows)
    np.testing.assert_array_equal(idx.cpu().numpy()[rows], ref_i)
    np.testing.assert_array_equal(val.cpu().numpy()[rows], ref_v)


@pytest.mark.parametrize("name", ["nope_unaligned", "block_gqa"])
def test_indexer_fused_matches_dense_then_select(sa, name):
    # On non-integer inputs both GPU paths compute the same fp32 scores, so the fused
    # selection must equal sa_topk_select over the dense scores, bit for bit.
    wl = W[name]
    T = 1024 if name == "nope_unaligned" else 4096
    B = wl.block_size
    k = wl.topk[0]
    x = {n: t.to(DEV) for n, t in workloads.indexer_inputs(wl, T=T).items()}
    dense = sa.indexer_scores(x["q_I"], x["k_I"], x["w"], block_size=B)
    i1, v1 = sa.topk_select(dense, k, block_size=B, force_own_block=B > 1, with_values=True)
    i2, v2 = sa.indexer_topk(x["q_I"], x["k_I"], x["w"], k, block_size=B, force_own_block=B > 1,
                             with_values=True)
    assert torch.equal(i1, i2)
    assert torch.equal(v1, v2)


@pytest.mark.parametrize("k", [1, 100, 777, 2048])
@pytest.mark.parametrize("integer", [False, True])
def test_indexer64_fused_matches_dense_then_select(sa, k, integer):
    """64 indexer heads: the fused selection (many buffer cut-backs at small k, exact
    ties on the integer grid) equals sa_topk_select over the dense scores, bit for bit,
    on one sequence and on packed sequences."""
    wl = W["long_dsa"]
    for lengths in [(4096,), (1000, 3, 2048, 1045)]:
        T = sum(lengths)
        x = {n: t.to(DEV) for n, t in workloads.indexer_inputs(wl, integer=integer, T=T).items()}
        kw = dict(cu_seqlens=cu_dev(lengths), max_seqlen=max(lengths)) if len(lengths) > 1 else {}
        dense = sa.indexer_scores(x["q_I"], x["k_I"], x["w"], **kw)
        i1, v1 = sa.topk_select(dense, k, with_values=True, **kw)
        i2, v2 = sa.indexer_topk(x["q_I"], x["k_I"], x["w"], k, with_values=True, **kw)
        assert torch.equal(i1, i2), f"lengths {lengths}"
        assert torch.equal(v1, v2), f"lengths {lengths}"


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("name", ["long_dsa", "thd_varlen"])
def test_indexer_topk_full_size_integer_sampled(sa, name, workspace):
    wl = W[name]
    T = wl.T
    lengths = wl.lengths if len(wl.lengths) > 1 else None
    x = workloads.indexer_inputs(wl, integer=True, device=DEV)
    assert workloads.exact_sum_bound(x["q_I"][:2048], x["k_I"], x["w"][:2048]) < 2 ** 24
    kw = dict(cu_seqlens=cu_dev(wl.lengths), max_seqlen=max(wl.lengths)) if lengths else {}
    idx = sa.indexer_topk(x["q_I"], x["k_I"], x["w"], 2048, workspace=workspace, **kw).cpu().numpy()
    rows = sample_rows(T, 8, 11, lengths)
    cu = workloads.cu_seqlens(wl.lengths) if lengths else None
    xc = {n: t.cpu() for n, t in x.items()}
    ref_i, _ = oracle.indexer_topk(xc["q_I"], xc["k_I"], xc["w"], 2048, cu_seqlens=cu, rows=rows)
    np.testing.assert_array_equal(idx[rows], ref_i)


# ---------------------------------------------------------------------- sparse MLA

def test_sparse_mla_tiny_fp32(sa):
    wl = W["tiny_fp32"]
    x = workloads.indexer_inputs(wl)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 64)
    m = workloads.mla_inputs(wl)
    out, lse = sa.sparse_mla(m["q"].to(DEV), m["kv"].to(DEV), torch.from_numpy(ref_idx).to(DEV), wl.scale)
    ro, rl = oracle.sparse_mla(m["q"], m["kv"], ref_idx, wl.scale)
    close(out.cpu().numpy(), ro, **F32_TOL, what="out")
    close(lse.cpu().numpy(), rl, **F32_TOL, what="lse")


@pytest.mark.parametrize("H,d_qk,k,with_sink", [(20, 576, 37, False), (40, 512, 300, True),
                                                (1, 576, 16, True), (128, 576, 129, False)])
def test_sparse_mla_fp32_shapes(sa, H, d_qk, k, with_sink):
    """fp32 sparse MLA on its MFMA kernel: head counts that leave a partial 16-head
    group, a slot count with a ragged last sub-tile, -1 slots, an all-invalid row and
    the optional sink, against the oracle at the fp32 bar."""
    T, S = 24, 700
    g = torch.Generator().manual_seed(H * 7 + k)
    q = torch.randn((T, H, d_qk), generator=g)
    kv = torch.randn((S, d_qk), generator=g)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < 0.2] = -1
    idx[3] = -1
    sink = torch.randn(H, generator=g) if with_sink else None
    scale = 1 / math.sqrt(d_qk)
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), scale,
                             sink=sink.to(DEV) if with_sink else None)
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), scale, sink=sink.numpy() if with_sink else None)
    close(out.cpu().numpy(), ro, **F32_TOL, what="out")
    close(lse.cpu().numpy(), rl, **F32_TOL, what="lse")
    assert torch.all(out[3] == 0)


@pytest.mark.parametrize("k", [65, 127])
def test_sparse_mla_nope_unaligned(sa, k):
    wl = W["nope_unaligned"]
    x = workloads.indexer_inputs(wl, integer=True)
    ref_idx, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], k)
    for r in wl.invalid_rows:
        ref_idx[r] = -1
    m = workloads.mla_inputs(wl)
    idx = torch.from_numpy(ref_idx).to(DEV)
    o576, l576 = sa.sparse_mla(m["q"].to(DEV), m["kv"].to(DEV), idx, wl.scale)
    o512, l512 = sa.sparse_mla(m["q512"].to(DEV), m["kv512"].to(DEV), idx, wl.scale)
    # zero padding adds exact zeros to every logit: identical results
    assert torch.equal(o576, o512) and torch.equal(l576, l512)
    ro, rl = oracle.sparse_mla(m["q512"], m["kv512"], ref_idx, wl.scale)
    close(o576.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(l576.cpu().numpy(), rl, **BF16_TOL, what="lse")
    for r in wl.invalid_rows:
        assert torch.all(o576[r] == 0) and torch.all(torch.isneginf(l576[r]))


@pytest.mark.parametrize("H", [8, 16, 32, 64, 80, 128])
@pytest.mark.parametrize("k", [1, 64, 65, 127])
@pytest.mark.parametrize("d_qk", [512, 576])
def test_sparse_mla_shapes(sa, H, k, d_qk):
    T, S = 40, 300
    g = torch.Generator().manual_seed(H * 1000 + k * 10 + d_qk)
    q = torch.randn((T, H, d_qk), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, d_qk), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < 0.1] = -1
    idx[3] = -1                                  # an all-invalid row
    scale = 1 / math.sqrt(d_qk)
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), scale)
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), scale)
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, **BF16_TOL, what="lse")


@pytest.mark.parametrize("H", [16, 64, 128])
@pytest.mark.parametrize("d_qk", [512, 576])
def test_sparse_mla_glm_width_2051(sa, H, d_qk):
    """Top-k width 2048 + 3 (the GLM k-pool width: a query's incomplete tail pool
    appended), 512 and 576 wide: a ragged last 32-slot tile of three slots, -1 slots
    spread through the row, a row that ends inside the tail and an all-invalid row."""
    T, S, k = 24, 5000, 2051
    g = torch.Generator().manual_seed(2051 + H + d_qk)
    q = torch.randn((T, H, d_qk), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, d_qk), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[torch.rand((T, k), generator=g) < 0.05] = -1
    idx[5, 2049:] = -1
    idx[6, 2050] = -1
    idx[7] = -1
    scale = 1 / math.sqrt(d_qk)
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), scale)
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), scale)
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, **BF16_TOL, what="lse")


@pytest.mark.parametrize("H", [32, 128])
def test_sparse_mla_large_logits_restart(sa, H):
    # a later key whose logit exceeds the first tile's max by far: exercises the
    # softmax reference restart (H = 128 runs the four-wave kernel)
    T, S, k = 4, 200, 128
    g = torch.Generator().manual_seed(5)
    q = torch.randn((T, H, 576), generator=g)
    kv = torch.randn((S, 576), generator=g) * 0.01
    kv[150] = q[0, 0] * 0.5                     # one very aligned key for row 0, head 0
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    idx = torch.arange(k, dtype=torch.int32)[None].repeat(T, 1) + 40
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), 1.0)
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), 1.0)
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, atol=2e-2, rtol=1e-3, what="lse")


@pytest.mark.parametrize("H", [16, 64, 128])
def test_sparse_mla_trailing_masked_tiles(sa, H):
    # index rows whose valid slots end early (ragged -1 tails ending inside, at and past
    # the 32-slot tile edges), a whole masked tile between valid ones, and an empty row:
    # trailing all-masked tiles are skipped, inner masked tiles are visited
    T, S, k = 8, 300, 160
    g = torch.Generator().manual_seed(11)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, 576), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    for t, n in enumerate([160, 159, 129, 128, 97, 33, 1, 0]):
        idx[t, n:] = -1
    idx[0, 32:64] = -1
    scale = 576 ** -0.5
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), scale)
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), scale)
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, **BF16_TOL, what="lse")


@pytest.mark.parametrize("H", [16, 128])
def test_sparse_mla_negative_scale(sa, H):
    # the caller's scale is used as given, sign included: with a negative scale the
    # largest logit comes from the smallest raw product (full and masked tiles)
    T, S, k = 6, 400, 96
    g = torch.Generator().manual_seed(5)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((S, 576), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, S, (T, k), generator=g, dtype=torch.int32)
    idx[1, 40:] = -1
    idx[2, 5::3] = -1
    scale = -(576 ** -0.5)
    out, lse = sa.sparse_mla(q.to(DEV), kv.to(DEV), idx.to(DEV), scale)
    ro, rl = oracle.sparse_mla(q, kv, idx.numpy(), scale)
    close(out.float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy(), rl, **BF16_TOL, what="lse")


@pytest.mark.parametrize("name", ["long_dsa", "thd_varlen"])
def test_sparse_mla_full_size_sampled(sa, name):
    wl = W[name]
    T = wl.T
    lengths = wl.lengths if len(wl.lengths) > 1 else None
    m = workloads.mla_inputs(wl, device=DEV)
    idx = workloads.random_causal_index(T, 2048, wl.seed, lengths=wl.lengths, device=DEV)
    out, lse = sa.sparse_mla(m["q"], m["kv"], idx, wl.scale)
    rows = sample_rows(T, 12, 13, lengths)
    rt = torch.from_numpy(rows).to(DEV)
    ro, rl = oracle.sparse_mla(m["q"][rt].cpu(), m["kv"].cpu(), idx[rt].cpu().numpy(), wl.scale)
    close(out[rt].float().cpu().numpy(), ro, **BF16_TOL, what="out")
    close(lse[rt].cpu().numpy(), rl, **BF16_TOL, what="lse")


# ------------------------------------------------------------------ block-sparse GQA

def test_block_gqa_on_oracle_routes(sa):
    wl = W["block_gqa"]
    T = 2048
    x = workloads.indexer_inputs(wl, T=T)
    blk, _ = oracle.indexer_topk(x["q_I"], x["k_I"], x["w"], 16, block_size=64, force_own_block=True)
    g = workloads.gqa_inputs(wl, T=T)
    out, lse = sa.block_sparse_gqa(g["q"].to(DEV), g["k"].to(DEV), g["v"].to(DEV),
                                   torch.from_numpy(blk).to(DEV), wl.scale, block_size=64)
    rows = sample_rows(T, 200, 17)
    ro, rl = oracle.block_sparse_gqa(g["q"], g["k"], g["v"], blk, 64, wl.scale, rows=rows)
    close(out.float().cpu().numpy()[rows], ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy()[rows], rl, **BF16_TOL, what="lse")


def test_block_gqa_full_size_thd_sampled(sa):
    wl = W["block_gqa"]
    lengths = (3000, 64, 5128)
    T = sum(lengths)
    g = workloads.gqa_inputs(wl, device=DEV)
    blk = workloads.random_block_index(T, 16, 64, 9, lengths=lengths, device=DEV)
    blk[100] = -1                                      # a row with no key
    out, lse = sa.block_sparse_gqa(g["q"], g["k"], g["v"], blk, wl.scale, block_size=64,
                                   cu_seqlens=cu_dev(lengths), max_seqlen=5128)
    rows = sample_rows(T, 40, 19, lengths)
    rows = np.union1d(rows, [100])
    ro, rl = oracle.block_sparse_gqa(g["q"].cpu(), g["k"].cpu(), g["v"].cpu(), blk.cpu().numpy(), 64,
                                     wl.scale, cu_seqlens=workloads.cu_seqlens(lengths), rows=rows)
    close(out.float().cpu().numpy()[rows], ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy()[rows], rl, **BF16_TOL, what="lse")


def test_block_gqa_long_sequence_per_token_kernel(sa):
    """One 600,000-token sequence: the grouped kernel's set-up bitmap over the group's
    key range would not fit the LDS, so the per-(token, kv head) kernel serves it.
    Routes of two blocks (a random earlier or equal block, and the own block, possibly
    the same); sampled rows against the oracle."""
    T, Hq, Hkv, D, B = 600_000, 4, 4, 64, 128
    gen = torch.Generator(device=DEV).manual_seed(77)
    q = torch.randn((T, Hq, D), generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn((T, Hkv, D), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((T, Hkv, D), generator=gen, device=DEV).to(torch.bfloat16)
    own = torch.arange(T, device=DEV) // B
    other = (torch.rand(T, generator=gen, device=DEV) * (own + 1).float()).long()
    other = torch.minimum(other, own)
    blk = torch.stack([other, own], 1).to(torch.int32).contiguous()
    out, lse = sa.block_sparse_gqa(q, k, v, blk, 0.125, block_size=B)
    rows = np.array([0, 1, 127, 128, 5000, 123457, 333333, T - 2, T - 1])
    ro, rl = oracle.block_sparse_gqa(q.cpu(), k.cpu(), v.cpu(), blk.cpu().numpy(), B, 0.125, rows=rows)
    close(out.float().cpu().numpy()[rows], ro, **BF16_TOL, what="out")
    close(lse.cpu().numpy()[rows], rl, **BF16_TOL, what="lse")


@pytest.mark.parametrize("Hq,Hkv,D,B,dtype", [(32, 4, 128, 64, "bf16"), (8, 4, 128, 32, "bf16"),
                                              (4, 4, 64, 16, "bf16"), (16, 1, 128, 128, "bf16"),
                                              (12, 2, 64, 48, "bf16"), (8, 2, 64, 32, "f32"),
                                              (32, 4, 128, 64, "f32"), (16, 1, 128, 16, "f32")])
def test_block_gqa_shapes_routes_with_repeats(sa, Hq, Hkv, D, B, dtype):
    """Head-group sizes 1..16, D 64/128, block sizes 16..128, THD with a sequence shorter
    than a block, and routes holding repeated blocks, blocks past the query's own and
    -1 slots at random positions."""
    lengths = (300, 7, 213)
    T = sum(lengths)
    gen = torch.Generator().manual_seed(Hq * 131 + D + B)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((T, Hq, D), generator=gen).to(tdt)
    k = torch.randn((T, Hkv, D), generator=gen).to(tdt)
    v = torch.randn((T, Hkv, D), generator=gen).to(tdt)
    nblk = 6
    blk = workloads.random_block_index(T, nblk, B, 23, lengths=lengths).clone()
    starts = workloads.cu_seqlens(lengths)
    for t in range(T):
        c = int(starts[np.searchsorted(starts, t, side="right") - 1])
        own = (t - c) // B
        r = int(torch.randint(0, 4, (1,), generator=gen))
        if r == 1 and blk[t, 0] >= 0:
            blk[t, nblk - 1] = blk[t, 0]                  # repeated block
        elif r == 2:
            blk[t, nblk - 1] = own + 1                    # past the own block
        elif r == 3:
            blk[t, int(torch.randint(0, nblk, (1,), generator=gen))] = -1
    out, lse = sa.block_sparse_gqa(q.to(DEV), k.to(DEV), v.to(DEV), blk.to(DEV), 0.3, block_size=B,
                                   cu_seqlens=cu_dev(lengths), max_seqlen=max(lengths))
    ro, rl = oracle.block_sparse_gqa(q, k, v, blk.numpy(), B, 0.3, cu_seqlens=starts)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    close(out.float().cpu().numpy(), ro, **tol, what="out")
    close(lse.cpu().numpy(), rl, **tol, what="lse")


# ------------------------------------------------------------ determinism and inputs

def test_replay_bitwise_and_inputs_preserved(sa):
    wl = W["nope_unaligned"]
    x = {n: t.to(DEV) for n, t in workloads.indexer_inputs(wl).items()}
    m = {n: t.to(DEV) for n, t in workloads.mla_inputs(wl).items()}
    gq = {n: t.to(DEV) for n, t in workloads.gqa_inputs(W["block_gqa"], T=1024).items()}
    before = {n: t.clone() for n, t in {**x, **m, **gq}.items()}

    def run():
        idx, val = sa.indexer_topk(x["q_I"], x["k_I"], x["w"], 127, with_values=True)
        dense = sa.indexer_scores(x["q_I"], x["k_I"], x["w"])
        sel = sa.topk_select(dense, 127)
        out, lse = sa.sparse_mla(m["q"], m["kv"], idx, wl.scale)
        blk = sa.indexer_topk(x["q_I"], x["k_I"], x["w"], 16, block_size=64, force_own_block=True)
        go, gl = sa.block_sparse_gqa(gq["q"], gq["k"], gq["v"], blk, 0.1, block_size=64)
        return [idx, val, dense, sel, out, lse, blk, go, gl]

    a = run()
    b = run()
    # third run under contention from another stream
    side = torch.cuda.Stream()
    big = torch.randn((4096, 4096), device=DEV)
    with torch.cuda.stream(side):
        for _ in range(8):
            big = big @ big.T * 1e-3
    c = run()
    torch.cuda.synchronize()
    for u, v, w_ in zip(a, b, c):
        assert torch.equal(u, v) and torch.equal(u, w_)
    for n, t in before.items():
        assert torch.equal(t, {**x, **m, **gq}[n]), n


def test_debug_build_rejects_out_of_range_contents(sa):
    """libsa_debug.so checks device contents: an index outside [-1, S) in sparse MLA and
    malformed sequence offsets return SA_ERR_SHAPE before any launch; valid inputs give
    the release library's results bit for bit."""
    import ctypes
    import os
    dbg = ctypes.CDLL(os.path.join(os.path.dirname(sa.__file__), "libsa_debug.so"))
    dbg.sa_sparse_mla_fwd.argtypes = sa.lib.sa_sparse_mla_fwd.argtypes
    dbg.sa_block_sparse_gqa_fwd.argtypes = sa.lib.sa_block_sparse_gqa_fwd.argtypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    T, S, H, k = 16, 100, 16, 40
    g = torch.Generator().manual_seed(3)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn((S, 576), generator=g).to(torch.bfloat16).to(DEV)
    idx = torch.randint(-1, S, (T, k), generator=g, dtype=torch.int32).to(DEV)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)

    def mla(ix):
        return dbg.sa_sparse_mla_fwd(p(q), p(kv), p(ix), 1, T, S, H, 576, 512, k, 0.05, None, p(out), None, stream)

    assert mla(idx) == 0
    ref = sa.sparse_mla(q, kv, idx, 0.05, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for bad in (S, -2, 1 << 30):
        ix = idx.clone()
        ix[T - 1, k - 1] = bad
        assert mla(ix) == 2, bad
    # sequence offsets: wrong total, a sequence longer than max_seqlen, a negative length
    gq = workloads.gqa_inputs(W["block_gqa"], T=64)
    gq = {n: t.to(DEV) for n, t in gq.items()}
    blk = torch.zeros((64, 2), dtype=torch.int32, device=DEV)
    o = torch.empty((64, 32, 128), dtype=torch.bfloat16, device=DEV)

    def gqa(cu, maxlen):
        c = torch.tensor(cu, dtype=torch.int32, device=DEV)
        return dbg.sa_block_sparse_gqa_fwd(p(gq["q"]), p(gq["k"]), p(gq["v"]), p(blk), 1, 64, p(c),
                                           len(cu) - 1, maxlen, 32, 4, 128, 128, 64, 2, 0.1, p(o),
                                           None, stream)

    assert gqa([0, 30, 64], 34) == 0
    assert gqa([0, 30, 63], 34) == 2
    assert gqa([0, 30, 64], 33) == 2
    assert gqa([0, 40, 30, 64], 34) == 2
    torch.cuda.synchronize()


def test_empty_inputs_are_noops(sa):
    z = torch.empty((0, 16, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((4, 576), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0, 16, 512), dtype=torch.bfloat16, device=DEV)
    sa.sa_sparse_mla_fwd(z, kv, torch.empty((0, 8), dtype=torch.int32, device=DEV), 1.0, out)
    sa.sa_topk_select(torch.empty((0, 4), device=DEV), torch.empty((0, 2), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
