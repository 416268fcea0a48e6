"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks an oracle function against one of: a hand-derived fixture under
tests/golden/, a library routine the definition reduces to in a special case
(torch scaled-dot-product attention in float64, numpy/torch matmul), brute force
over Python tuples on tiny rows, or an invariant the mathematics fixes. The cases
are chosen so that a dropped term, a wrong sign or index, or a transposed operand
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _none_to(x, v):
    return np.array([[v if e is None else e for e in r] for r in x], dtype=np.float32)


# ----------------------------------------------------------------- indexer (O1/O2)

def test_indexer_golden_tokens_and_blocks():
    g = _load("indexer_tiny.json")
    q = np.array(g["q_I"], dtype=np.float32)
    k = np.array(g["k_I"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    got = oracle.indexer_scores_dense(q, k, w)
    np.testing.assert_array_equal(got, _none_to(g["scores"], -np.inf))
    got_b = oracle.indexer_scores_dense(q, k, w, block_size=2)
    np.testing.assert_array_equal(got_b, _none_to(g["block2"], -np.inf))


def test_indexer_single_head_unit_weight_is_relu_matmul():
    # H_I = 1, w = 1: the score is max(Q K^T, 0), a plain library matmul.
    rng = np.random.default_rng(5)
    T, D = 37, 16
    q = rng.standard_normal((T, 1, D)).astype(np.float32)
    k = rng.standard_normal((T, D)).astype(np.float32)
    w = np.ones((T, 1), dtype=np.float32)
    ref = torch.relu(torch.from_numpy(q[:, 0, :]).double() @ torch.from_numpy(k).double().T)
    ref = ref.float().numpy()
    got = oracle.indexer_scores_dense(q, k, w)
    for t in range(T):
        np.testing.assert_array_equal(got[t, :t + 1], np.where(ref[t, :t + 1] == 0, 0, ref[t, :t + 1]))
        assert np.all(np.isneginf(got[t, t + 1:]))


def test_indexer_integer_inputs_exact_and_invariants():
    rng = np.random.default_rng(6)
    T, H, D = 29, 5, 8
    q = rng.integers(-3, 4, (T, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, (T, D)).astype(np.float32)
    w = (rng.integers(-8, 9, (T, H)) / 4).astype(np.float32)
    base = oracle.indexer_scores_dense(q, k, w)
    # exact brute force with Python integers / fractions
    for t in [0, 7, 28]:
        for s in range(t + 1):
            acc = 0.0
            for h in range(H):
                z = int(sum(int(q[t, h, d]) * int(k[s, d]) for d in range(D)))
                acc += float(w[t, h]) * max(z, 0)
            assert base[t, s] == np.float32(acc)
    # permuting heads together with their weights leaves scores unchanged
    perm = rng.permutation(H)
    np.testing.assert_array_equal(oracle.indexer_scores_dense(q[:, perm], k, w[:, perm]), base)
    # positive homogeneity in w and in k (powers of two keep it exact)
    np.testing.assert_array_equal(oracle.indexer_scores_dense(q, k, 2 * w), 2 * base)
    np.testing.assert_array_equal(oracle.indexer_scores_dense(q, 4 * k, w), 4 * base)
    # a negative k flips which heads pass the ReLU: not homogeneous (guards a dropped ReLU)
    neg = oracle.indexer_scores_dense(q, -k, w)
    assert not np.array_equal(neg[np.isfinite(neg)], -base[np.isfinite(base)])


def test_indexer_thd_rows_only_see_their_sequence():
    rng = np.random.default_rng(7)
    lengths = (5, 9, 3)
    cu = workloads.cu_seqlens(lengths)
    T = sum(lengths)
    q = rng.standard_normal((T, 3, 4)).astype(np.float32)
    k = rng.standard_normal((T, 4)).astype(np.float32)
    w = rng.uniform(0, 1, (T, 3)).astype(np.float32)
    got = oracle.indexer_scores_dense(q, k, w, cu_seqlens=cu)
    for j in range(3):
        a, b = cu[j], cu[j + 1]
        alone = oracle.indexer_scores_dense(q[a:b], k[a:b], w[a:b], ld=got.shape[1])
        np.testing.assert_array_equal(got[a:b], alone)


def test_block_scores_are_blockwise_max_of_token_scores():
    rng = np.random.default_rng(8)
    T, B = 70, 8
    q = rng.standard_normal((T, 2, 4)).astype(np.float32)
    k = rng.standard_normal((T, 4)).astype(np.float32)
    w = rng.standard_normal((T, 2)).astype(np.float32)
    tok = oracle.indexer_scores_dense(q, k, w)
    blk = oracle.indexer_scores_dense(q, k, w, block_size=B)
    for t in range(T):
        nb = t // B + 1
        for b in range(nb):
            lo, hi = b * B, min(b * B + B - 1, t)
            assert blk[t, b] == max(tok[t, s] for s in range(lo, hi + 1))
        assert np.all(np.isneginf(blk[t, nb:]))


# ----------------------------------------------------------------------- top-k (O3)

def test_topk_golden_ties():
    g = _load("topk_ties.json")
    row = np.array([-0.0 if v is None else v for v in g["row"]], dtype=np.float32)
    assert np.signbit(row[3])
    for c in g["cases"]:
        idx, val = oracle.topk_select_row(row, c["n_valid"], c["k"], force_last=c["force_last"])
        assert idx.tolist() == c["idx"], c["why"]
        for j, i in enumerate(idx):
            if i < 0:
                assert np.isneginf(val[j])
            else:
                assert val[j] == row[i]
                assert val[j] != 0 or not np.signbit(val[j])      # -0.0 reported as +0.0


def _brute_topk(vals, n, k, base=0):
    keyed = sorted(((-float(vals[c]) + 0.0, c) for c in range(n)))
    pick = sorted(c for _, c in keyed[:k])
    return [c + base for c in pick] + [-1] * (k - len(pick))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_tuple_sort_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        n = int(rng.integers(0, 60))
        k = int(rng.integers(1, 70))
        # few distinct values -> many ties, including signed zeros
        vals = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32), size=64)
        base = int(rng.integers(0, 1000))
        idx, _ = oracle.topk_select_row(vals, n, k, base)
        assert idx.tolist() == _brute_topk(vals, n, k, base)


def test_topk_invariants_random_rows():
    rng = np.random.default_rng(9)
    for _ in range(50):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 200))
        vals = np.round(rng.standard_normal(n) * 2).astype(np.float32)  # heavy ties
        idx, val = oracle.topk_select_row(vals, n, k)
        sel = idx[idx >= 0]
        assert sel.size == min(k, n)
        assert np.all(np.diff(sel) > 0)                       # ascending, no duplicates
        assert np.all(idx[sel.size:] == -1)
        assert sel.min() >= 0 and sel.max() < n
        uns = np.setdiff1d(np.arange(n), sel)
        if uns.size:
            assert vals[sel].min() >= vals[uns].max()
            tau = vals[sel].min()
            if np.any(vals[uns] == tau):                      # boundary tie: smaller wins
                assert sel[vals[sel] == tau].max() < uns[vals[uns] == tau].min()


def test_topk_special_cases():
    z = np.zeros(100, dtype=np.float32)
    idx, _ = oracle.topk_select_row(z, 100, 10)
    assert idx.tolist() == list(range(10))                    # all-equal: k smallest indices
    v = np.arange(50, dtype=np.float32)
    idx, _ = oracle.topk_select_row(v, 50, 64)
    assert idx.tolist() == list(range(50)) + [-1] * 14         # k >= valid: all valid
    idx, _ = oracle.topk_select_row(v, 50, 3)
    assert idx.tolist() == [47, 48, 49]


def test_topk_union_of_tile_topks_equals_global():
    # exactness of a per-tile partial top-k followed by a final top-k
    rng = np.random.default_rng(10)
    for _ in range(20):
        n = int(rng.integers(100, 900))
        k = int(rng.integers(1, 120))
        vals = np.round(rng.standard_normal(n) * 3).astype(np.float32)
        glob, _ = oracle.topk_select_row(vals, n, k)
        tile = int(rng.integers(16, 200))
        cv, ci = [], []
        for a in range(0, n, tile):
            i, v = oracle.topk_select_row(vals[a:], min(tile, n - a), k, index_base=a)
            cv.extend(v[i >= 0].tolist())
            ci.extend(i[i >= 0].tolist())
        cv = np.array(cv, dtype=np.float32)[None]
        ci = np.array(ci, dtype=np.int32)[None]
        merged, _ = oracle.topk_select_candidates(cv, ci, k)
        assert merged[0].tolist() == glob.tolist()


def test_topk_dense_thd_and_block_mode():
    lengths = (3, 5)
    cu = workloads.cu_seqlens(lengths)
    sc = np.full((8, 5), -np.inf, dtype=np.float32)
    sc[0, :1] = [1]
    sc[1, :2] = [0, 1]
    sc[2, :3] = [2, 0, 1]
    sc[3, :1] = [7]
    sc[4, :2] = [1, 1]
    sc[5, :3] = [0, 5, 0]
    sc[6, :4] = [3, 3, 3, 3]
    sc[7, :5] = [0, 1, 2, 3, 4]
    idx, _ = oracle.topk_select_dense(sc, 2, cu_seqlens=cu)
    assert idx.tolist() == [[0, -1], [0, 1], [0, 2], [3, -1], [3, 4], [3, 4], [3, 4], [6, 7]]
    # block mode (B = 2), own block forced, ids local to the sequence
    bs = np.full((8, 3), -np.inf, dtype=np.float32)
    bs[7, :3] = [9, 1, 0]        # row 7 = offset 4 in seq 1 -> own block 2
    idx, _ = oracle.topk_select_dense(bs[[7]], 2, cu_seqlens=cu, block_size=2,
                                      force_own_block=True, rows=[7])
    assert idx.tolist() == [[0, 2]]
    # score row r belongs to query row rows[r]: a different best block must show
    bs[7, :3] = [0, 9, 1]
    idx, _ = oracle.topk_select_dense(bs[[7]], 2, cu_seqlens=cu, block_size=2,
                                      force_own_block=True, rows=[7])
    assert idx.tolist() == [[1, 2]]
    # the full matrix without rows= gives the same row 7
    full, _ = oracle.topk_select_dense(bs, 2, cu_seqlens=cu, block_size=2, force_own_block=True)
    assert full[7].tolist() == [1, 2]


def _brute_indexer_topk(q, k, w, K, lengths, B, force_own, rows):
    """From-scratch top-k of the indexer scores with exact rational arithmetic.

    Scores: Fractions of the stored values, sum over heads of w * max(q.k, 0). Block
    mode takes the max over the block's causal keys. Ranking: a Python sort of
    (-score, id) tuples; the own block first when forced. Returns ids, values, and the
    score lists per row (global key ids in token mode, local block ids in block mode).
    """
    from fractions import Fraction as F
    starts = np.concatenate([[0], np.cumsum(lengths)])
    ids_out, vals_out, score_rows = [], [], []
    for t in rows:
        j = int(np.searchsorted(starts, t, side="right") - 1)
        c = int(starts[j])
        tok = []
        for s in range(c, t + 1):
            acc = F(0)
            for h in range(q.shape[1]):
                z = sum(F(float(q[t, h, d])) * F(float(k[s, d])) for d in range(q.shape[2]))
                acc += F(float(w[t, h])) * max(z, F(0))
            tok.append(acc)
        if B == 1:
            cands = [(sc, c + i) for i, sc in enumerate(tok)]
        else:
            cands = [(max(tok[b * B:(b + 1) * B]), b) for b in range((t - c) // B + 1)]
        score_rows.append(cands)
        chosen = []
        rest = cands
        if force_own:
            chosen = [cands[-1]]
            rest = cands[:-1]
        chosen += sorted(rest, key=lambda e: (-e[0], e[1]))[:K - len(chosen)]
        chosen.sort(key=lambda e: e[1])
        ids_out.append([i for _, i in chosen] + [-1] * (K - len(chosen)))
        vals_out.append([np.float32(float(v)) for v, _ in chosen] + [np.float32(-np.inf)] * (K - len(chosen)))
    return np.array(ids_out), np.array(vals_out, dtype=np.float32), score_rows


@pytest.mark.parametrize("B,K,force_own", [(1, 5, False), (1, 1, False), (4, 3, True),
                                           (4, 3, False), (3, 1, True)])
def test_indexer_topk_and_row_subsets_match_brute_force_thd(B, K, force_own):
    """oracle.indexer_topk (and indexer_scores_dense with rows=) on packed sequences,
    against exact rational scores and a tuple sort; rows given out of order, so a
    wrong row slice, start offset or sequence boundary shows."""
    rng = np.random.default_rng(20 + B * 7 + K)
    lengths = (7, 1, 13, 20)
    T = sum(lengths)
    cu = workloads.cu_seqlens(lengths)
    q = (rng.integers(-4, 5, (T, 3, 4)) * 0.5).astype(np.float32)
    k = (rng.integers(-4, 5, (T, 4)) * 0.5).astype(np.float32)
    w = (rng.integers(-64, 65, (T, 3)) / 64).astype(np.float32)
    rows = np.array([40, 0, 7, 8, 21, 6, 33, 20, 9, 28, 1])
    ref_i, ref_v, ref_rows = _brute_indexer_topk(q, k, w, K, lengths, B, force_own, rows)
    got_i, got_v = oracle.indexer_topk(q, k, w, K, cu_seqlens=cu, block_size=B,
                                       force_own_block=force_own, rows=rows)
    np.testing.assert_array_equal(got_i, ref_i)
    np.testing.assert_array_equal(got_v, ref_v)
    # dense scores of a row subset: same as the brute-force scores, column by column
    sub = oracle.indexer_scores_dense(q, k, w, cu_seqlens=cu, block_size=B, rows=rows)
    full = oracle.indexer_scores_dense(q, k, w, cu_seqlens=cu, block_size=B)
    np.testing.assert_array_equal(sub, full[rows])
    for r, cands in enumerate(ref_rows):
        vals = [np.float32(float(v)) for v, _ in cands]
        np.testing.assert_array_equal(sub[r, :len(vals)], np.array(vals, dtype=np.float32))
        assert np.all(np.isneginf(sub[r, len(vals):]))
    # the oracle's chunking of rows (64 at a time) is invisible: more than 64 rows
    many = np.concatenate([np.arange(T)[::-1], np.arange(T)])
    gi, _ = oracle.indexer_topk(q, k, w, K, cu_seqlens=cu, block_size=B,
                                force_own_block=force_own, rows=many)
    ai, _ = oracle.indexer_topk(q, k, w, K, cu_seqlens=cu, block_size=B,
                                force_own_block=force_own)
    np.testing.assert_array_equal(gi, ai[many])


# ------------------------------------------------------------------ sparse MLA (O4)

def test_mla_golden():
    g = _load("attention_tiny.json")["mla"]
    kv = np.array(g["kv"], dtype=np.float64)
    for c in g["cases"]:
        out, lse = oracle.sparse_mla_row(np.array(c["q"]), kv, np.array(c["idx"]), c["scale"], g["d_v"])
        np.testing.assert_allclose(out, np.array(c["out"]), rtol=0, atol=1e-15)
        if c["lse"][0] is None:
            assert np.isneginf(lse[0])
        else:
            np.testing.assert_allclose(lse, c["lse"], rtol=1e-15)


def _sdpa_masked(q, kv, mask, scale, d_v):
    """torch's scaled-dot-product attention in float64 with a boolean key mask."""
    qt = torch.from_numpy(q).double()[None]                  # [1, H, 1?]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(kv).double()[None, None],
        torch.from_numpy(kv[:, :d_v]).double()[None, None],
        attn_mask=torch.from_numpy(mask)[None, None], scale=scale)[0].numpy()


def test_mla_matches_library_dense_masked_attention():
    rng = np.random.default_rng(11)
    S, H, dqk, dv, k = 40, 4, 24, 16, 9
    kv = rng.standard_normal((S, dqk))
    for t in [0, 5, 39]:
        q = rng.standard_normal((H, dqk))
        idx = np.full(k, -1)
        n = min(k - 2, t + 1)
        idx[rng.permutation(k)[:n]] = rng.permutation(t + 1)[:n]
        out, lse = oracle.sparse_mla_row(q, kv, idx, 0.3, dv)
        mask = np.zeros((1, S), dtype=bool)
        mask[0, idx[idx >= 0]] = True
        ref = _sdpa_masked(q[:, None, :], kv, mask, 0.3, dv)[:, 0, :]
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        logits = 0.3 * q @ kv[idx[idx >= 0]].T
        np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(logits), 1).numpy(), rtol=1e-13)


def test_mla_invariants():
    rng = np.random.default_rng(12)
    S, H = 30, 3
    kv = rng.standard_normal((S, 576))
    q = rng.standard_normal((H, 576))
    idx = rng.permutation(S)[:12]
    out, lse = oracle.sparse_mla_row(q, kv, idx, 1 / 24, 512)
    # slot permutation and -1 insertion
    o2, l2 = oracle.sparse_mla_row(q, kv, np.concatenate([[-1, -1], idx[::-1], [-1]]), 1 / 24, 512)
    np.testing.assert_allclose(o2, out, atol=1e-12)
    np.testing.assert_allclose(l2, lse, atol=1e-12)
    # one valid slot: the output is that row's value channels exactly
    o1, l1 = oracle.sparse_mla_row(q, kv, np.array([-1, 7, -1]), 1 / 24, 512)
    np.testing.assert_array_equal(o1, np.broadcast_to(kv[7, :512], o1.shape))
    np.testing.assert_allclose(l1, (q @ kv[7]) / 24, rtol=1e-13)
    # all invalid
    o0, l0 = oracle.sparse_mla_row(q, kv, np.full(5, -1), 1 / 24, 512)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))
    # the value is the first 512 channels: changing channels 512..575 of kv only
    # moves the logits, so with q's RoPE slot zero the output is unchanged
    qz = q.copy(); qz[:, 512:] = 0
    kv2 = kv.copy(); kv2[:, 512:] = rng.standard_normal((S, 64))
    np.testing.assert_array_equal(oracle.sparse_mla_row(qz, kv, idx, 0.1, 512)[0],
                                  oracle.sparse_mla_row(qz, kv2, idx, 0.1, 512)[0])


def test_mla_nope_512_equals_zero_padded_576():
    rng = np.random.default_rng(13)
    S, H = 50, 4
    q512 = rng.standard_normal((S, H, 512)).astype(np.float32)
    kv512 = rng.standard_normal((S, 512)).astype(np.float32)
    q576 = np.pad(q512, ((0, 0), (0, 0), (0, 64)))
    kv576 = np.pad(kv512, ((0, 0), (0, 64)))
    idx = np.stack([np.where(np.arange(20) <= t, np.arange(20) * 2 % (t + 1), -1) for t in range(S)])
    a, la = oracle.sparse_mla(q512, kv512, idx, 1 / math.sqrt(512), 512)
    b, lb = oracle.sparse_mla(q576, kv576, idx, 1 / math.sqrt(512), 512)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_mla_all_causal_keys_equals_causal_attention():
    rng = np.random.default_rng(14)
    S, H, d = 33, 2, 40
    q = rng.standard_normal((S, H, d))
    kv = rng.standard_normal((S, d))
    idx = np.stack([np.where(np.arange(S) <= t, np.arange(S), -1) for t in range(S)])
    out, _ = oracle.sparse_mla(q, kv, idx, 0.2, 32)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None],
        torch.from_numpy(kv)[None, None].expand(1, H, S, d),
        torch.from_numpy(kv[:, :32])[None, None].expand(1, H, S, 32),
        is_causal=True, scale=0.2)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------- block-sparse GQA (O5)

def test_gqa_golden():
    g = _load("attention_tiny.json")["gqa"]
    k = np.array(g["k"], dtype=np.float64)[:, None, :]
    v = np.array(g["v"], dtype=np.float64)[:, None, :]
    q = np.zeros((g["Hq"], g["D"]))
    for c in g["cases"]:
        out, _ = oracle.block_sparse_gqa_row(q, k, v, np.array(c["blk"]), c["t"], 0,
                                             g["block_size"], 1.0)
        np.testing.assert_allclose(out[:, 0], c["out"], atol=1e-15)


def _gqa_sdpa(q, k, v, mask, scale):
    Hq, Hkv = q.shape[1], k.shape[1]
    rep = Hq // Hkv
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
    qq = torch.from_numpy(q).permute(1, 0, 2)[None]
    return torch.nn.functional.scaled_dot_product_attention(
        qq, kk, vv, attn_mask=torch.from_numpy(mask)[None, None], scale=scale)[0].permute(1, 0, 2).numpy()


def test_gqa_matches_library_with_block_mask_thd():
    rng = np.random.default_rng(15)
    lengths = (13, 20)
    cu = workloads.cu_seqlens(lengths)
    T, Hq, Hkv, D, Dv, B, nb = 33, 6, 2, 8, 5, 4, 3
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, Dv))
    start, _ = oracle.seq_bounds(T, cu)
    blk = np.full((T, nb), -1)
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        own = (t - start[t]) // B
        choice = rng.permutation(own + 1)[:nb - 1].tolist()
        row = sorted(set(choice + [own]))
        blk[t, :len(row)] = row
        for b in row:
            for s in range(start[t] + b * B, min(start[t] + b * B + B - 1, t) + 1):
                mask[t, s] = True
    out, lse = oracle.block_sparse_gqa(q, k, v, blk, B, 0.35, cu_seqlens=cu)
    ref = _gqa_sdpa(q, k, v, mask, 0.35)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_gqa_reductions():
    rng = np.random.default_rng(16)
    T, H, D, B = 24, 3, 6, 4
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, H, D))
    v = rng.standard_normal((T, H, D))
    # Hq = Hkv with every block selected: dense causal attention
    blk = np.stack([np.where(np.arange(T // B) <= t // B, np.arange(T // B), -1) for t in range(T)])
    out, _ = oracle.block_sparse_gqa(q, k, v, blk, B, 0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], is_causal=True, scale=0.5)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # B = 1 is token routing: same as a key mask from the token list
    tok = np.stack([rng.permutation(t + 1)[:5].tolist() + [-1] * max(0, 5 - (t + 1)) for t in range(T)])
    tok = tok[:, :5]
    out1, _ = oracle.block_sparse_gqa(q, k, v, tok, 1, 0.5)
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        mask[t, tok[t][tok[t] >= 0]] = True
    np.testing.assert_allclose(out1, _gqa_sdpa(q, k, v, mask, 0.5), rtol=1e-12, atol=1e-12)


def test_gqa_route_is_a_set():
    """A block listed twice, or a block past the query's own, adds no key: the result
    equals the library's masked attention over the set of routed causal keys."""
    rng = np.random.default_rng(18)
    T, Hq, Hkv, D, B = 40, 4, 2, 8, 8
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    blk = np.full((T, 6), -1, dtype=np.int64)
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        own = t // B
        picks = rng.integers(0, own + 1, size=3)
        blk[t, :3] = picks
        blk[t, 3] = picks[0]                  # repeated block
        blk[t, 4] = own + 1                   # past the own block: no causal key
        for b in set(picks.tolist()):
            mask[t, b * B:min(b * B + B, t + 1)] = True
    out, _ = oracle.block_sparse_gqa(q, k, v, blk, B, 0.7)
    np.testing.assert_allclose(out, _gqa_sdpa(q, k, v, mask, 0.7), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- workloads / recipe

def test_thd_lengths_recipe():
    L = workloads.thd_lengths(4)
    assert sorted(L) == [512, 595, 1171, 1198, 1445, 1699, 1912, 2141, 2667, 5005, 5235,
                         6666, 7411, 8538, 9579, 9762]
    assert sum(L) == 65536


def test_integer_variant_is_exact_in_fp32():
    for name in ["tiny_fp32", "nope_unaligned", "block_gqa"]:
        wl = workloads.WORKLOADS[name]
        x = workloads.indexer_inputs(wl, integer=True, T=min(wl.T, 2048))
        assert workloads.exact_sum_bound(x["q_I"], x["k_I"], x["w"]) < 2 ** 24


def test_generators_are_deterministic():
    wl = workloads.WORKLOADS["nope_unaligned"]
    a = workloads.indexer_inputs(wl, T=64)
    b = workloads.indexer_inputs(wl, T=64)
    for n in a:
        assert torch.equal(a[n], b[n])
    # the forced-negative key rows score exactly zero for every query
    neg = (a["k_I"].float() <= 0).all(dim=1)
    assert 0.15 < neg.float().mean().item() < 0.45
    sc = oracle.indexer_scores_dense(a["q_I"], a["k_I"], a["w"])
    for t in range(64):
        s = np.nonzero(neg[:t + 1].numpy())[0]
        assert np.all(sc[t, s] == 0)


# ------------------------------------------------------- backward of O4 / O5

def _torch_sparse_mla_loss(q, kv, idx, dout, scale, d_v):
    """sum(out * dout) of sparse attention over the slots of idx, written with torch
    gathers (each slot on its own, so repeated indices count per slot); differentiated
    by autograd, it gives the gradients without the oracle's closed form."""
    total = q.new_zeros(())
    for t in range(q.shape[0]):
        sl = [j for j in range(idx.shape[1]) if idx[t, j] >= 0]
        if not sl:
            continue
        rows = kv[torch.as_tensor(idx[t, sl], dtype=torch.long)]
        p = torch.softmax(scale * q[t] @ rows.T, dim=-1)
        total = total + (p @ rows[:, :d_v] * dout[t]).sum()
    return total


@pytest.mark.parametrize("d_qk,d_v", [(24, 16), (20, 20)])
def test_mla_bwd_matches_autograd(d_qk, d_v):
    """Closed-form dq and dkv against torch autograd through a gather-based forward,
    with -1 slots, a repeated index (two slots, two contributions), an all-invalid row
    and a row with one valid slot."""
    rng = np.random.default_rng(40 + d_qk)
    T, S, H, k, scale = 7, 30, 3, 9, 0.37
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S, d_qk))
    dout = rng.standard_normal((T, H, d_v))
    idx = np.full((T, k), -1)
    for t in range(T):
        n = int(rng.integers(2, k + 1))
        idx[t, rng.permutation(k)[:n]] = rng.integers(0, S, n)
    idx[2, :3] = [5, 5, 11]                      # repeated index
    idx[3] = -1                                  # all invalid
    idx[4] = -1
    idx[4, 6] = 17                               # one valid slot
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, dout, scale, d_v)
    qt = torch.from_numpy(q).requires_grad_()
    kvt = torch.from_numpy(kv).requires_grad_()
    _torch_sparse_mla_loss(qt, kvt, idx, torch.from_numpy(dout), scale, d_v).backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv, kvt.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.all(dq[3] == 0) and np.all(dq[4] == 0)         # no key / one key: dq = 0
    only = np.zeros(d_qk)
    only[:d_v] = dout[4].sum(0)                               # one key: its gradient is dout
    _, alone = oracle.sparse_mla_bwd(q[4:5], kv, idx[4:5], dout[4:5], scale, d_v)
    np.testing.assert_allclose(alone[17], only, atol=1e-12)


def test_mla_bwd_matches_library_attention_autograd():
    """Against autograd through torch's scaled-dot-product attention (float64) with a
    boolean key mask, on rows without repeated indices."""
    rng = np.random.default_rng(45)
    T, S, H, d_qk, d_v, k = 5, 40, 4, 32, 16, 12
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S, d_qk))
    dout = rng.standard_normal((T, H, d_v))
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)])
    idx[1, 5:] = -1
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, dout, 0.2, d_v)
    mask = np.zeros((T, S), dtype=bool)
    for t in range(T):
        mask[t, idx[t][idx[t] >= 0]] = True
    qt = torch.from_numpy(q).permute(1, 0, 2)[None].requires_grad_()
    kvt = torch.from_numpy(kv).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kvt[None, None].expand(1, H, S, d_qk), kvt[:, :d_v][None, None].expand(1, H, S, d_v),
        attn_mask=torch.from_numpy(mask)[None, None], scale=0.2)
    (o * torch.from_numpy(dout).permute(1, 0, 2)[None]).sum().backward()
    np.testing.assert_allclose(dq, qt.grad[0].permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv, kvt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_mla_bwd_finite_differences():
    """Central differences of sum(out * dout) through the (separately pinned) forward
    oracle match the backward, for a q entry, a RoPE-slot kv entry and a value entry."""
    rng = np.random.default_rng(46)
    T, S, H, d_qk, d_v, k, scale = 3, 12, 2, 10, 6, 5, 0.5
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S, d_qk))
    dout = rng.standard_normal((T, H, d_v))
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)])
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, dout, scale, d_v)

    def loss(qq, kk):
        o, _ = oracle.sparse_mla(qq, kk, idx, scale, d_v)
        return float((o * dout).sum())

    eps = 1e-6
    for (t, h, c) in [(1, 1, 3), (2, 0, 9)]:
        qp, qm = q.copy(), q.copy()
        qp[t, h, c] += eps
        qm[t, h, c] -= eps
        assert abs((loss(qp, kv) - loss(qm, kv)) / (2 * eps) - dq[t, h, c]) < 1e-7
    for (s, c) in [(int(idx[0, 0]), 8), (int(idx[1, 2]), 2)]:
        kp, km = kv.copy(), kv.copy()
        kp[s, c] += eps
        km[s, c] -= eps
        assert abs((loss(q, kp) - loss(q, km)) / (2 * eps) - dkv[s, c]) < 1e-7


def test_gqa_bwd_matches_library_attention_autograd_thd():
    """Block-routed GQA gradients against autograd through torch's SDPA with the block
    key mask, on packed sequences, with repeated blocks and blocks past the own one."""
    rng = np.random.default_rng(47)
    lengths = (13, 20)
    cu = workloads.cu_seqlens(lengths)
    T, Hq, Hkv, D, Dv, B, nb = 33, 6, 2, 8, 5, 4, 5
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, Dv))
    dout = rng.standard_normal((T, Hq, Dv))
    start, _ = oracle.seq_bounds(T, cu)
    blk = np.full((T, nb), -1)
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        own = (t - start[t]) // B
        row = sorted(set(rng.permutation(own + 1)[:2].tolist() + [own]))
        blk[t, :len(row)] = row                           # at most 3 of the 5 slots
        blk[t, nb - 1] = row[0]                           # repeated block
        if t % 3 == 0:
            blk[t, nb - 2] = own + 1                      # past the own block
        for b in row:
            mask[t, start[t] + b * B:min(start[t] + b * B + B - 1, t) + 1] = True
    dq, dk, dv = oracle.block_sparse_gqa_bwd(q, k, v, blk, dout, B, 0.35, cu_seqlens=cu)
    rep = Hq // Hkv
    qt = torch.from_numpy(q).requires_grad_()
    kt = torch.from_numpy(k).requires_grad_()
    vt = torch.from_numpy(v).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2)[None], kt.permute(1, 0, 2).repeat_interleave(rep, 0)[None],
        vt.permute(1, 0, 2).repeat_interleave(rep, 0)[None],
        attn_mask=torch.from_numpy(mask)[None, None], scale=0.35)[0].permute(1, 0, 2)
    (o * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


# ------------------------------------------- sparse KL indexer loss and backward

def test_attn_teacher_is_head_mean_of_attention_weights():
    """The teacher is the head mean of the probabilities the forward oracle weights
    the values with: sum_j p_j v_j equals the head mean of sparse_mla's outputs, the
    teacher sums to one over valid slots, and matches torch.softmax of masked logits."""
    rng = np.random.default_rng(60)
    T, S, H, d_qk, d_v, k = 6, 40, 5, 24, 16, 9
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S, d_qk))
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)])
    idx[2, 4:] = -1
    idx[3] = -1
    p = oracle.attn_teacher(q, kv, idx, 0.3)
    out, _ = oracle.sparse_mla(q, kv, idx, 0.3, d_v)
    for t in range(T):
        ok = idx[t] >= 0
        if not ok.any():
            assert np.all(p[t] == 0)
            continue
        np.testing.assert_allclose(p[t][ok].sum(), 1.0, rtol=1e-13)
        assert np.all(p[t][~ok] == 0)
        np.testing.assert_allclose(p[t][ok] @ kv[idx[t][ok], :d_v], out[t].mean(0), atol=1e-12)
        lg = torch.from_numpy(0.3 * q[t] @ kv[idx[t][ok]].T)
        np.testing.assert_allclose(p[t][ok], torch.softmax(lg, -1).mean(0).numpy(), rtol=1e-12)


def test_indexer_kl_matches_autograd_through_library_kl():
    """Loss and gradients against torch autograd through the indexer score written
    with torch ops and the library's kl_div, with -1 slots, a zero-probability teacher
    slot, a repeated key, ReLU zeros from integer inputs, and per-row loss weights."""
    rng = np.random.default_rng(61)
    T, S, H, D, k = 5, 30, 4, 6, 8
    q = rng.integers(-2, 3, (T, H, D)).astype(np.float64)
    kk = rng.integers(-2, 3, (S, D)).astype(np.float64)
    w = rng.standard_normal((T, H))
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)])
    idx[1, 6:] = -1
    idx[2, :2] = [7, 7]                               # a key in two slots
    teacher = rng.random((T, k)) * (idx >= 0)
    teacher[0, 3] = 0.0                               # zero teacher probability
    teacher /= teacher.sum(1, keepdims=True)
    teacher[4] *= 0.6                                 # mass outside the slots (a sink)
    grad = rng.random(T) + 0.5
    loss, dI, dq, dw, dk = oracle.indexer_kl(q, kk, w, idx, teacher, grad)
    qt = torch.from_numpy(q).requires_grad_()
    kt = torch.from_numpy(kk).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    total = qt.new_zeros(())
    for t in range(T):
        ok = np.nonzero(idx[t] >= 0)[0]
        K = kt[torch.as_tensor(idx[t][ok])]
        I = (torch.relu(qt[t] @ K.T) * wt[t][:, None]).sum(0)
        pt = torch.from_numpy(teacher[t][ok])
        lt = torch.nn.functional.kl_div(torch.log_softmax(I, -1), pt, reduction="sum")
        np.testing.assert_allclose(loss[t], lt.item(), rtol=1e-12, atol=1e-14)
        total = total + grad[t] * lt
    total.backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    # dI = grad * (student * sum(teacher) - teacher) sums to zero per row
    np.testing.assert_allclose(dI.sum(1), 0.0, atol=1e-13)


def test_indexer_kl_zero_when_student_equals_teacher():
    """KL is zero, with zero gradients, when the teacher is the student's own
    distribution; and positive otherwise."""
    rng = np.random.default_rng(62)
    T, S, H, D, k = 3, 20, 3, 5, 6
    q = rng.standard_normal((T, H, D))
    kk = rng.standard_normal((S, D))
    w = rng.random((T, H))
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)])
    z = np.einsum("thd,tkd->thk", q, kk[idx])          # exact float64 scores of the slots
    sc = (np.maximum(z, 0) * w[:, :, None]).sum(1)
    st = np.exp(sc - sc.max(1, keepdims=True))
    st /= st.sum(1, keepdims=True)
    loss, dI, dq, dw, dk = oracle.indexer_kl(q, kk, w, idx, st)
    np.testing.assert_allclose(loss, 0.0, atol=1e-14)
    np.testing.assert_allclose(dI, 0.0, atol=1e-14)
    flat = np.full_like(st, 1.0 / k)
    l2, *_ = oracle.indexer_kl(q, kk, w, idx, flat)
    assert np.all(l2 > 0)


# ------------------------------------------------- variants: sink, pools, window

def test_mla_sink_is_an_extra_zero_value_key():
    """A sink equals one more key per head with logit sink[h] and value zero: the
    library softmax over the augmented logits weights the values; lse is its log
    denominator; with no valid slot out = 0 and lse = sink."""
    rng = np.random.default_rng(70)
    S, H, d_qk, d_v, k = 30, 4, 20, 12, 7
    kv = rng.standard_normal((S, d_qk))
    q = rng.standard_normal((H, d_qk))
    sink = rng.standard_normal(H) * 2
    idx = rng.permutation(S)[:k]
    idx[2] = -1
    out, lse = oracle.sparse_mla_row(q, kv, idx, 0.4, d_v, sink=sink)
    rows = kv[idx[idx >= 0]]
    aug = torch.cat([torch.from_numpy(0.4 * q @ rows.T), torch.from_numpy(sink)[:, None]], 1)
    p = torch.softmax(aug, 1).numpy()
    vals = np.concatenate([rows[:, :d_v], np.zeros((1, d_v))])
    np.testing.assert_allclose(out, p @ vals, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(aug, 1).numpy(), rtol=1e-13)
    o0, l0 = oracle.sparse_mla_row(q, kv, np.full(3, -1), 0.4, d_v, sink=sink)
    assert np.all(o0 == 0) and np.array_equal(l0, sink)
    # the teacher keeps the sink in its denominator
    pt = oracle.attn_teacher_row(q, kv, idx, 0.4, sink=sink)
    np.testing.assert_allclose(pt[idx >= 0], p[:, :-1].mean(0), rtol=1e-12)
    assert pt.sum() < 1


def test_mla_bwd_with_sink_matches_autograd():
    rng = np.random.default_rng(71)
    T, S, H, d_qk, d_v, k = 4, 25, 3, 16, 8, 6
    q = rng.standard_normal((T, H, d_qk))
    kv = rng.standard_normal((S, d_qk))
    dout = rng.standard_normal((T, H, d_v))
    sink = rng.standard_normal(H)
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)])
    idx[1, 3:] = -1
    idx[2] = -1                                          # only the sink: no gradient but dsink
    dq, dkv, dsink = oracle.sparse_mla_bwd(q, kv, idx, dout, 0.3, d_v, sink=sink)
    qt = torch.from_numpy(q).requires_grad_()
    kvt = torch.from_numpy(kv).requires_grad_()
    st = torch.from_numpy(sink).requires_grad_()
    total = qt.new_zeros(())
    for t in range(T):
        sl = idx[t][idx[t] >= 0]
        rows = kvt[torch.as_tensor(sl, dtype=torch.long)]
        aug = torch.cat([0.3 * qt[t] @ rows.T, st[:, None]], 1)
        p = torch.softmax(aug, 1)[:, :-1]
        total = total + (p @ rows[:, :d_v] * torch.from_numpy(dout[t])).sum()
    total.backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv, kvt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dsink, st.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_complete_block_topk_brute_force():
    """Only blocks whose keys are all causal compete: row offsets o give (o + 1) // B
    candidates; checked against a tuple sort on packed sequences."""
    rng = np.random.default_rng(72)
    lengths = (9, 14, 3)
    cu = workloads.cu_seqlens(lengths)
    T, B, k = sum(lengths), 4, 2
    sc = np.round(rng.standard_normal((T, 4)) * 2).astype(np.float32)
    got, _ = oracle.complete_block_topk(sc, k, B, cu_seqlens=cu)
    start, _ = oracle.seq_bounds(T, cu)
    for t in range(T):
        n = (t - start[t] + 1) // B
        assert got[t].tolist() == _brute_topk(sc[t], n, k)
    # offsets 3 and 7 complete their own block, which then competes
    assert (3 + 1) // B == 1 and (2 + 1) // B == 0
    # a row subset (score row r belongs to query rows[r]) gives the same rows
    sub = np.array([20, 3, 11, 25])
    part, _ = oracle.complete_block_topk(sc[sub], k, B, cu_seqlens=cu, rows=sub)
    np.testing.assert_array_equal(part, got[sub])
    sc2 = np.round(rng.standard_normal((T, 8)) * 2).astype(np.float32)   # one sequence: 26 keys
    one, _ = oracle.complete_block_topk(sc2[[7, 20]], k, B, rows=[7, 20])
    full_one, _ = oracle.complete_block_topk(sc2, k, B)
    np.testing.assert_array_equal(one, full_one[[7, 20]])


def test_kpool_expand_hand_example():
    """Pools of four keys: a row at sequence offset 9 (its pool 2 holds keys 8, 9 so
    far) with pools 0 and 1 selected gets keys 0..7, then the tail 8, 9 and one -1: the
    width is k*4 + 3, as 512 pools give the quoted 2048 + 3 = 2051."""
    pools = np.full((12, 2), -1)
    pools[9] = [0, 1]
    pools[11] = [2, -1]
    out = oracle.kpool_expand(pools, 4)
    assert out.shape == (12, 11)
    assert out[9].tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, -1]
    assert out[11].tolist() == [8, 9, 10, 11] + [-1] * 7        # offset 11: pool complete, no tail
    pools[11] = [-1, 2]                                          # a -1 slot keeps its place
    assert oracle.kpool_expand(pools, 4)[11].tolist() == [-1] * 4 + [8, 9, 10, 11] + [-1] * 3
    assert out[0].tolist() == [-1] * 8 + [0, -1, -1]             # offset 0: tail is the query
    assert oracle.kpool_expand(np.full((1, 512), -1), 4).shape[1] == 2051
    # packed sequences: ids are global rows
    cu = workloads.cu_seqlens((5, 7))
    p2 = np.full((12, 1), -1)
    p2[10] = [1]                                                 # offset 5 in sequence 1
    o2 = oracle.kpool_expand(p2, 4, cu_seqlens=cu)
    assert o2[10].tolist() == [9, 10, 11, 12, 9, 10, -1]


def test_append_window_hand_example():
    idx = np.array([[0, -1], [1, 0], [2, 1], [3, 0], [4, -1]])
    cu = workloads.cu_seqlens((3, 2))
    out = oracle.append_window(idx, 2, offset=100, cu_seqlens=cu)
    assert out.tolist() == [[0, -1, -1, 100], [1, 0, 100, 101], [2, 1, 101, 102],
                            [3, 0, -1, 103], [4, -1, 103, 104]]
