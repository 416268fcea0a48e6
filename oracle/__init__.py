"""CPU oracle for the indexer -> top-k -> sparse-attention forward path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute
this package: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU
baseline leg use it. It shares no code, headers, tables or helpers with the HIP
library, and it imports nothing from it.

Every function is the plain definition of its step, written in numpy with float64
arithmetic, one query row at a time, with no blocking, fusion or reordering beyond
what the definition states. Library primitives (matmul, sort, exp) serve as steps.

Sources (web pages on indexer-routed sparse attention in Megatron-LM):

* [QSA] "Add trainable QSA sparse attention with a TileLang backend"
  (Megatron-LM issue #7060).
* [DSA] "Enable DSA CP/absorbed/THD paths with TileLang fused ops"
  (Megatron-LM PR #3674).
* [NOPE] "Support NoPE shapes and unaligned top-k in TileLang sparse MLA"
  (Megatron-LM PR #7617), including the downstream GLM-5.3-Flash PR body quoted
  on that page.

Readings taken where the pages are silent (each is listed with its reason in the
design notes):

* score I[t,s] = sum_h w[t,h] * max(q[t,h,:].k[s,:], 0); one indexer key row per
  token shared by all indexer heads; any score scaling is folded into w;
* causal: key s is a candidate for query t iff seq_start(t) <= s <= t;
* block score = max of the token scores I over the block's causal keys;
* order: a before b iff val_a > val_b, or val_a == val_b and idx_a < idx_b;
  -0.0 counts as +0.0;
* selected slots are emitted in ascending index order, then -1 padding;
* sparse attention over the slots of an index row: each slot counts once, -1
  slots are skipped, a row with no valid slot gives zeros and lse = -inf;
  natural-log lse;
* block-routed attention attends to a set of keys: the causal keys of every block
  that appears in the route (a block id listed twice contributes its keys once).

Parity status: every function below is pinned by CPU tests against brute force,
library routines, hand-derived fixtures and invariants, except the two points the
pages leave undefined: the indexer's "official score scaling" and the exact block
statistic. For those two, "parity unpinned" holds: the oracle follows the readings
above and nothing on the pages can confirm them.
"""
from __future__ import annotations

import numpy as np

NEG_INF = np.float32(-np.inf)


# ------------------------------------------------------------------------ helpers

def _f64(x) -> np.ndarray:
    """Host float64 copy of a numpy array or a (CPU/GPU, any dtype) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def seq_bounds(T: int, cu_seqlens=None):
    """Per row t: (start, end) of the packed sequence holding t.

    THD packing as used by [DSA] ("What does this PR do ?": packed THD with varlen
    bounds): sequence j spans rows [cu[j], cu[j+1]); no cu_seqlens means one
    sequence [0, T).
    """
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else _i64(cu_seqlens)
    start = np.empty(T, dtype=np.int64)
    end = np.empty(T, dtype=np.int64)
    for j in range(len(cu) - 1):
        start[cu[j]:cu[j + 1]] = cu[j]
        end[cu[j]:cu[j + 1]] = cu[j + 1]
    return start, end


def _canon_zero(x: np.ndarray) -> np.ndarray:
    """-0.0 -> +0.0 (ReLU times a negative weight gives -0.0; it must tie with +0.0)."""
    x = np.array(x, dtype=np.float32, copy=True)
    x[x == 0] = 0.0
    return x


# ------------------------------------------------------------------ O1: indexer

def indexer_scores_row(q_t, k_keys, w_t) -> np.ndarray:
    """Token scores of one query against a run of keys, fp32.

    [QSA] "Describe the solution you'd like": a multi-head indexer whose ReLU scores
    tie at zero; [DSA] file table: fused indexer forward. Definition:
    I[s] = sum_h w[h] * max(sum_d q[h,d] k[s,d], 0), evaluated in float64 from the
    stored values, then rounded once to fp32 (nearest even) with -0 -> +0.

    q_t [H_I, D_I], k_keys [n, D_I], w_t [H_I] -> [n] float32.
    """
    q = _f64(q_t)
    k = _f64(k_keys)
    w = _f64(w_t)
    z = k @ q.T                       # [n, H_I]: z[s,h] = q[h,:] . k[s,:]
    relu = np.maximum(z, 0.0)
    I = relu @ w                      # [n]: sum_h w[h] * relu[s,h]
    return _canon_zero(I.astype(np.float32))


def indexer_scores_dense(q_I, k_I, w, cu_seqlens=None, block_size: int = 1,
                         rows=None, ld: int | None = None) -> np.ndarray:
    """Causal score matrix: token scores (block_size 1) or block scores (block_size B).

    Row t, column c: token mode -> key s = start(t) + c for c <= t - start(t);
    block mode -> block c of t's sequence, the max of the token scores over the
    block's causal keys [start + cB, min(start + cB + B - 1, t)] ([QSA] "Is your
    feature request related to a problem?": exact block TopK over the
    [sequence, sequence / block_size] scores). Columns outside the causal range are
    -inf. Rounding commutes with max (round-to-nearest is monotone), so taking the
    max of fp32 token scores equals rounding the max of the float64 ones.

    ``rows`` restricts to a subset of query rows (returned in that order).
    """
    T = q_I.shape[0]
    start, end = seq_bounds(T, cu_seqlens)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    if ld is None:
        Lmax = int((end - start).max())
        ld = Lmax if block_size == 1 else -(-Lmax // block_size)
    out = np.full((len(rows), ld), NEG_INF, dtype=np.float32)
    kk = _f64(k_I)
    for r, t in enumerate(rows):
        s0 = int(start[t])
        tok = indexer_scores_row(q_I[t], kk[s0:t + 1], w[t])
        if block_size == 1:
            out[r, :tok.size] = tok
        else:
            nb = -(-tok.size // block_size)
            for b in range(nb):
                out[r, b] = tok[b * block_size:(b + 1) * block_size].max()
    return out


# ------------------------------------------------------------------ O3: top-k

def topk_select_row(vals, n_valid: int, k: int, index_base: int = 0,
                    force_last: bool = False):
    """Exact deterministic top-k of one row.

    [QSA] "Describe the solution you'd like": selection keyed lexicographically on
    (score, id) so that ReLU ties at zero resolve the same way every run; [NOPE]
    "What does this PR do?": unused slots carry the -1 sentinel.

    Candidates are columns 0..n_valid-1 of ``vals``. Order: higher score first,
    equal scores -> smaller column first (-0.0 ties +0.0). Take the first min(k, n)
    of a full sort. With ``force_last`` (block routing: the query's own block is
    the last valid column) the last column is taken first and counts toward k; the
    other k-1 come from the sort of the remaining columns. Output: the chosen
    columns + index_base in ascending order, then -1; values in the same slots,
    -inf on pads.
    """
    v = _canon_zero(np.asarray(vals, dtype=np.float32)[:n_valid]).astype(np.float64)
    cols = np.arange(n_valid, dtype=np.int64)
    chosen = []
    if force_last and n_valid > 0 and k > 0:
        chosen.append(n_valid - 1)
        v, cols = v[:-1], cols[:-1]
        k_rest = k - 1
    else:
        k_rest = k
    order = np.lexsort((cols, -v))    # primary: -value ascending; secondary: column
    chosen.extend(cols[order[:max(k_rest, 0)]].tolist())
    chosen = np.sort(np.asarray(chosen, dtype=np.int64))
    idx = np.full(k, -1, dtype=np.int32)
    val = np.full(k, NEG_INF, dtype=np.float32)
    idx[:chosen.size] = chosen + index_base
    val[:chosen.size] = _canon_zero(np.asarray(vals, dtype=np.float32)[chosen])
    return idx, val


def topk_select_dense(scores, k: int, cu_seqlens=None, block_size: int = 1,
                      force_own_block: bool = False, rows=None):
    """Row-wise ``topk_select_row`` over a causal dense score matrix.

    Token mode (block_size 1): row t has t - start + 1 valid columns and the
    output indices are global key rows (column + start). Block mode: row t has
    (t - start) // B + 1 valid blocks, the indices are block ids local to the
    sequence, and ``force_own_block`` keeps the query's own (last) block.
    Score row r belongs to query row ``rows[r]`` (default: r). Without
    ``cu_seqlens`` every row is in one sequence starting at 0.
    """
    scores = np.asarray(scores)
    rows = np.arange(scores.shape[0]) if rows is None else np.asarray(rows)
    if cu_seqlens is None:
        starts = np.zeros(len(rows), dtype=np.int64)
    else:
        cu = _i64(cu_seqlens)
        start, _ = seq_bounds(int(cu[-1]), cu)
        starts = start[rows]
    idx = np.full((len(rows), k), -1, dtype=np.int32)
    val = np.full((len(rows), k), NEG_INF, dtype=np.float32)
    for r, t in enumerate(rows):
        off = int(t - starts[r])
        if block_size == 1:
            n, base = off + 1, int(starts[r])
        else:
            n, base = off // block_size + 1, 0
        idx[r], val[r] = topk_select_row(scores[r], n, k, base,
                                         force_last=(block_size > 1 and force_own_block))
    return idx, val


def topk_select_candidates(cand_val, cand_idx, k: int):
    """Top-k of an explicit candidate list (value, index) per row; -1 entries skipped.

    Same order as ``topk_select_row``, with the candidate's own index in place of
    its column. Output ascending by index, -1 padded.
    """
    cv = np.asarray(cand_val, dtype=np.float32)
    ci = _i64(cand_idx)
    T = cv.shape[0]
    idx = np.full((T, k), -1, dtype=np.int32)
    val = np.full((T, k), NEG_INF, dtype=np.float32)
    for t in range(T):
        keep = ci[t] >= 0
        v = _canon_zero(cv[t][keep]).astype(np.float64)
        ii = ci[t][keep]
        order = np.lexsort((ii, -v))[:k]
        sel = np.sort(ii[order])
        idx[t, :sel.size] = sel
        pos = {int(i): j for j, i in enumerate(ii)}
        val[t, :sel.size] = [_canon_zero(cv[t][keep])[pos[int(i)]] for i in sel]
    return idx, val


# ------------------------------------------------------------- O4: sparse MLA

def sparse_mla_row(q_t, kv, idx_t, scale: float, d_v: int = 512, sink=None):
    """Absorbed-MLA attention of one query row over its selected latent rows.

    [DSA] file table: sparse-MLA forward; [NOPE] "What does this PR do?" and the
    quoted GLM PR body ("Change"): q/k share the latent row, the value is the
    first 512 channels of the same row, -1 slots are masked, the caller's softmax
    scale is used as given. Definition, in float64 over valid slots j:
      l[h,j] = scale * sum_c q[h,c] kv[idx_j, c]; m = max_j l; p = exp(l - m);
      out[h,:] = sum_j p[h,j] kv[idx_j, :d_v] / sum_j p[h,j]; lse[h] = m + ln sum p.
    No valid slot -> out = 0, lse = -inf. Each slot counts once (duplicates count
    per slot).

    ``sink`` [H] (optional; "Add fused SBHD compressed sparse attention", "Scope":
    the compressed + window + sink attention of DeepSeek-V4): a per-head logit that
    joins the softmax's denominator and carries no value, i.e. the attention over the
    slots plus one extra key of logit sink[h] and value 0: Z = sum_j exp(l_j) +
    exp(sink[h]), out = sum_j exp(l_j) v_j / Z, lse = ln Z (so with no valid slot
    out = 0 and lse = sink[h]).

    q_t [H, d_qk], kv [S, d_qk], idx_t [k] -> out [H, d_v] float64, lse [H].
    """
    q = _f64(q_t)
    idx = _i64(idx_t)
    valid = idx[idx >= 0]
    H = q.shape[0]
    sk = None if sink is None else _f64(sink)
    if valid.size == 0:
        return np.zeros((H, d_v)), (np.full(H, -np.inf) if sk is None else sk.copy())
    rows = _f64(kv[valid.tolist()] if hasattr(kv, "detach") else kv[valid])
    logits = scale * (q @ rows.T)                    # [H, n]
    m = logits.max(axis=1, keepdims=True)
    if sk is not None:
        m = np.maximum(m, sk[:, None])
    p = np.exp(logits - m)
    Z = p.sum(axis=1, keepdims=True)
    if sk is not None:
        Z = Z + np.exp(sk[:, None] - m)
    out = (p @ rows[:, :d_v]) / Z
    lse = m[:, 0] + np.log(Z[:, 0])
    return out, lse


def sparse_mla(q, kv, idx, scale: float, d_v: int = 512, rows=None, sink=None):
    """``sparse_mla_row`` for every row (or a subset); returns float64 out, lse."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    kvh = _f64(kv)
    idxh = _i64(idx)
    H = q.shape[1]
    out = np.zeros((len(rows), H, d_v))
    lse = np.zeros((len(rows), H))
    for r, t in enumerate(rows):
        out[r], lse[r] = sparse_mla_row(q[t], kvh, idxh[t], scale, d_v, sink)
    return out, lse


# -------------------------------------------------------- O5: block-sparse GQA

def block_sparse_gqa_row(q_t, k, v, blk_t, t: int, seq_start: int,
                         block_size: int, scale: float):
    """Grouped-query attention of one query over its selected key blocks.

    [QSA] "Describe the solution you'd like": sparse GQA attention over the blocks
    chosen by the block TopK. The attended keys form a set: every s with s <= t whose
    local block (s - seq_start) // B appears among the slots of blk_t (slot -1
    skipped; a block id listed twice contributes its keys once). Head h reads kv
    head g = h // (Hq / Hkv). Per head, float64:
      l[s] = scale * q[h,:].k[s,g,:]; out[h,:] = softmax(l) @ v[:, g, :];
      lse[h] = log sum exp l. No key -> zeros and lse = -inf.

    q_t [Hq, D], k [S, Hkv, D], v [S, Hkv, Dv] -> out [Hq, Dv], lse [Hq].
    """
    q = _f64(q_t)
    Hq = q.shape[0]
    Hkv = k.shape[1]
    Dv = v.shape[2]
    keys = []
    for b in sorted(set(int(x) for x in _i64(blk_t) if x >= 0)):
        lo = seq_start + b * block_size
        hi = min(lo + block_size - 1, t)
        keys.extend(range(lo, hi + 1))
    out = np.zeros((Hq, Dv))
    lse = np.full(Hq, -np.inf)
    if not keys:
        return out, lse
    keys = np.asarray(keys, dtype=np.int64)
    kk = _f64(k[keys])                                # [n, Hkv, D]
    vv = _f64(v[keys])
    group = Hq // Hkv
    for h in range(Hq):
        g = h // group
        l = scale * (kk[:, g, :] @ q[h])
        m = l.max()
        p = np.exp(l - m)
        Z = p.sum()
        out[h] = (p @ vv[:, g, :]) / Z
        lse[h] = m + np.log(Z)
    return out, lse


def block_sparse_gqa(q, k, v, blk, block_size: int, scale: float,
                     cu_seqlens=None, rows=None):
    """``block_sparse_gqa_row`` for every row (or a subset)."""
    T = q.shape[0]
    start, _ = seq_bounds(T, cu_seqlens)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    kh, vh = _f64(k), _f64(v)
    blkh = _i64(blk)
    Hq, Dv = q.shape[1], v.shape[2]
    out = np.zeros((len(rows), Hq, Dv))
    lse = np.zeros((len(rows), Hq))
    for r, t in enumerate(rows):
        out[r], lse[r] = block_sparse_gqa_row(q[t], kh, vh, blkh[t], int(t), int(start[t]),
                                              block_size, scale)
    return out, lse


# ------------------------------------------------------- composed: the path

def indexer_topk(q_I, k_I, w, k: int, cu_seqlens=None, block_size: int = 1,
                 force_own_block: bool = False, rows=None):
    """Scores then selection, row by row (O1/O2 then O3)."""
    T = q_I.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    idx = np.full((len(rows), k), -1, dtype=np.int32)
    val = np.full((len(rows), k), NEG_INF, dtype=np.float32)
    for r0 in range(0, len(rows), 64):
        rr = rows[r0:r0 + 64]
        sc = indexer_scores_dense(q_I, k_I, w, cu_seqlens, block_size, rows=rr)
        i, v = topk_select_dense(sc, k, cu_seqlens, block_size, force_own_block, rows=rr)
        idx[r0:r0 + len(rr)], val[r0:r0 + len(rr)] = i, v
    return idx, val


# ------------------------------------------------------- backward of O4 / O5
#
# "Enable DSA CP/absorbed/THD paths with TileLang fused ops", file table (sparse-MLA
# backward kernels) and "Add trainable QSA sparse attention with a TileLang backend",
# "Is your feature request related to a problem?" (sparse GQA attention forward and
# backward). Gradients of the forward definitions above, in closed form: for one
# query row and head over its attended keys j with logits l_j = scale * q . k_j,
# probabilities p = softmax(l) and output o = sum_j p_j v_j, an upstream gradient g of
# o gives
#     dp_j = g . v_j,   D = sum_j p_j dp_j (= g . o),   dl_j = p_j (dp_j - D),
#     dq   = scale * sum_j dl_j k_j,
#     dk_j = scale * dl_j q,   dv_j = p_j g,
# summed over heads (and, for a key attended by several rows or slots, over those).

def sparse_mla_bwd_row(q_t, kv, idx_t, dout_t, scale: float, d_v: int = 512, sink=None):
    """Gradients of ``sparse_mla_row`` for one query row.

    q_t [H, d_qk], kv [S, d_qk], idx_t [k], dout_t [H, d_v] (upstream gradient of
    out). The latent row is both key (all d_qk channels) and value (first d_v), so a
    slot's gradient row is dk_j on all channels plus dv_j on the first d_v. Returns
    dq [H, d_qk] and dkv_slots [k, d_qk] (one row per slot, zero for -1 slots; a
    repeated index gets one row per slot), float64.

    With ``sink`` (see ``sparse_mla_row``) the probabilities p_j share their
    denominator with the sink's p_sink = exp(sink - lse); the sink holds no value, so
    D = sum_j p_j dp_j still, and the sink logit's gradient is -p_sink D (returned as
    a third value, zeros without a sink).
    """
    q = _f64(q_t)
    g = _f64(dout_t)
    idx = _i64(idx_t)
    H, d_qk = q.shape
    dq = np.zeros((H, d_qk))
    dslots = np.zeros((idx.size, d_qk))
    dsink = np.zeros(H)
    sel = np.nonzero(idx >= 0)[0]
    if sel.size == 0:
        return dq, dslots, dsink
    rows = _f64(kv[idx[sel].tolist()] if hasattr(kv, "detach") else kv[idx[sel]])
    logits = scale * (q @ rows.T)                     # [H, n]
    m = logits.max(axis=1, keepdims=True)
    if sink is not None:
        m = np.maximum(m, _f64(sink)[:, None])
    p = np.exp(logits - m)
    Z = p.sum(axis=1, keepdims=True)
    if sink is not None:
        psink = np.exp(_f64(sink)[:, None] - m)
        Z = Z + psink
    p /= Z
    dp = g @ rows[:, :d_v].T                          # [H, n]
    D = (p * dp).sum(axis=1, keepdims=True)
    dl = p * (dp - D)
    dq = scale * (dl @ rows)
    dk = scale * (dl.T @ q)                           # [n, d_qk], summed over heads
    dk[:, :d_v] += p.T @ g
    dslots[sel] = dk
    if sink is not None:
        dsink = -(psink / Z)[:, 0] * D[:, 0]
    return dq, dslots, dsink


def sparse_mla_bwd(q, kv, idx, dout, scale: float, d_v: int = 512, rows=None, sink=None):
    """``sparse_mla_bwd_row`` over every row (or a subset): dq [len(rows), H, d_qk] and
    dkv [S, d_qk] (the slot gradients of those rows scattered onto their latent rows);
    with ``sink`` also dsink [H] (summed over the rows)."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    kvh = _f64(kv)
    idxh = _i64(idx)
    H, d_qk = q.shape[1], q.shape[2]
    dq = np.zeros((len(rows), H, d_qk))
    dkv = np.zeros(kvh.shape)
    dsink = np.zeros(H)
    for r, t in enumerate(rows):
        dq[r], ds, dsk = sparse_mla_bwd_row(q[t], kvh, idxh[t], dout[t], scale, d_v, sink)
        ok = idxh[t] >= 0
        np.add.at(dkv, idxh[t][ok], ds[ok])
        dsink += dsk
    return (dq, dkv) if sink is None else (dq, dkv, dsink)


def _gqa_keys(blk_t, t: int, seq_start: int, block_size: int) -> np.ndarray:
    keys = []
    for b in sorted(set(int(x) for x in _i64(blk_t) if x >= 0)):
        lo = seq_start + b * block_size
        keys.extend(range(lo, min(lo + block_size - 1, t) + 1))
    return np.asarray(keys, dtype=np.int64)


def block_sparse_gqa_bwd(q, k, v, blk, dout, block_size: int, scale: float,
                         cu_seqlens=None, rows=None):
    """Gradients of ``block_sparse_gqa`` (same key sets: the causal keys of the routed
    blocks, each block once; head h reads kv head h // (Hq / Hkv)). Returns dq
    [len(rows), Hq, D], dk [S, Hkv, D], dv [S, Hkv, Dv], float64; dk and dv collect the
    contributions of the listed rows."""
    T = q.shape[0]
    start, _ = seq_bounds(T, cu_seqlens)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    qh, kh, vh, gh = _f64(q), _f64(k), _f64(v), _f64(dout)
    blkh = _i64(blk)
    Hq, D = qh.shape[1], qh.shape[2]
    Hkv = kh.shape[1]
    group = Hq // Hkv
    dq = np.zeros((len(rows), Hq, D))
    dk = np.zeros(kh.shape)
    dv = np.zeros(vh.shape)
    for r, t in enumerate(rows):
        keys = _gqa_keys(blkh[t], int(t), int(start[t]), block_size)   # distinct keys
        if keys.size == 0:
            continue
        for gi in range(Hkv):
            hs = slice(gi * group, (gi + 1) * group)     # the query heads reading kv head gi
            K = kh[keys, gi, :]
            V = vh[keys, gi, :]
            l = scale * (K @ qh[t, hs].T)                # [n, group]
            p = np.exp(l - l.max(axis=0))
            p /= p.sum(axis=0)
            dp = V @ gh[t, hs].T
            dl = p * (dp - (p * dp).sum(axis=0))
            dq[r, hs] = scale * (dl.T @ K)
            dk[keys, gi, :] += scale * (dl @ qh[t, hs])   # keys are distinct within a row
            dv[keys, gi, :] += p @ gh[t, hs]
    return dq, dk, dv


# ------------------------------------- sparse KL indexer loss and indexer backward
#
# "Add trainable QSA sparse attention with a TileLang backend", sections "Is your
# feature request related to a problem?" and "Describe the solution you'd like"
# (sparse KL supervision of the indexer, a stage-2 teacher/KL loss), and "Enable DSA
# CP/absorbed/THD paths with TileLang fused ops" (streaming sparse-KL for the indexer
# loss; fused indexer backward). The pages do not write the loss out; the reading
# taken here: over the slots a row selected, the teacher is the sparse attention's
# probability of each slot averaged over the attention heads (no gradient flows into
# it), the student is the softmax of the indexer scores of the same slots, and the
# row's loss is KL(teacher || student). Gradients reach the indexer's q_I, k_I and w.

def attn_teacher_row(q_t, kv, idx_t, scale: float, sink=None) -> np.ndarray:
    """Head-averaged sparse attention probability of every slot of one row, float64.

    p[j] = (1/H) sum_h softmax_h(scale q[h] . kv[idx_j])_j over the valid slots (the
    probabilities ``sparse_mla_row`` weights the values with); 0 on -1 slots. With a
    sink the denominator keeps the sink's term ("Add fused SBHD compressed sparse
    attention", "Scope": the teacher keeps the full compressed + window + sink
    denominator), so the slots' probabilities sum to less than one.
    """
    q = _f64(q_t)
    idx = _i64(idx_t)
    p = np.zeros(idx.size)
    sel = np.nonzero(idx >= 0)[0]
    if sel.size == 0:
        return p
    rows = _f64(kv[idx[sel].tolist()] if hasattr(kv, "detach") else kv[idx[sel]])
    logits = scale * (q @ rows.T)                      # [H, n]
    m = logits.max(axis=1, keepdims=True)
    if sink is not None:
        m = np.maximum(m, _f64(sink)[:, None])
    e = np.exp(logits - m)
    Z = e.sum(axis=1, keepdims=True)
    if sink is not None:
        Z = Z + np.exp(_f64(sink)[:, None] - m)
    p[sel] = (e / Z).mean(axis=0)
    return p


def attn_teacher(q, kv, idx, scale: float, rows=None, sink=None) -> np.ndarray:
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    kvh = _f64(kv)
    idxh = _i64(idx)
    return np.stack([attn_teacher_row(q[t], kvh, idxh[t], scale, sink) for t in rows])


def indexer_kl_row(q_I_t, k_I, w_t, idx_t, teacher_t):
    """Sparse KL loss of one row and its gradients, float64.

    Scores of the valid slots I_j = sum_h w_h max(z_hj, 0) with z_hj = q_I[h] . k_I[idx_j]
    (the indexer definition, unrounded); student s = softmax(I) over them; loss =
    sum_j p_j (log p_j - log s_j) with 0 log 0 = 0 (p = teacher_t). With
    dI_j = s_j sum_i p_i - p_j (d loss / d I_j; s_j - p_j when the teacher sums to one,
    less when part of the teacher's mass lies outside the slots, e.g. on a sink):
      dw_h  = sum_j dI_j max(z_hj, 0)
      dq_h  = sum_j dI_j w_h [z_hj > 0] k_I[idx_j]
      dk_j  = sum_h dI_j w_h [z_hj > 0] q_I[h]        (a slot's gradient row)
    Returns loss, dI [k] (0 on -1 slots), dq [H_I, D_I], dw [H_I], dk_slots [k, D_I].
    """
    q = _f64(q_I_t)
    w = _f64(w_t)
    idx = _i64(idx_t)
    p_all = _f64(teacher_t)
    H, D = q.shape
    dI = np.zeros(idx.size)
    dk = np.zeros((idx.size, D))
    sel = np.nonzero(idx >= 0)[0]
    if sel.size == 0:
        return 0.0, dI, np.zeros((H, D)), np.zeros(H), dk
    K = _f64(k_I[idx[sel].tolist()] if hasattr(k_I, "detach") else k_I[idx[sel]])
    z = q @ K.T                                        # [H, n]
    I = np.maximum(z, 0.0).T @ w                       # [n]
    ls = I - I.max()
    ls = ls - np.log(np.exp(ls).sum())                 # log student
    p = p_all[sel]
    nz = p > 0
    loss = float((p[nz] * (np.log(p[nz]) - ls[nz])).sum())
    d = np.exp(ls) * p.sum() - p
    dI[sel] = d
    on = (z > 0).astype(np.float64)                    # [H, n]
    dw = np.maximum(z, 0.0) @ d
    dz = on * w[:, None] * d[None, :]                  # [H, n]
    dq = dz @ K
    dk[sel] = dz.T @ q
    return loss, dI, dq, dw, dk


def indexer_kl(q_I, k_I, w, idx, teacher, grad=None, rows=None):
    """``indexer_kl_row`` over rows; the gradients are those of sum_t grad[t] * loss[t]
    (grad = 1 when None). Returns loss [len(rows)], dI, dq_I, dw, and dk_I [S, D_I]
    (the slot gradients scattered onto their key rows)."""
    rows = np.arange(q_I.shape[0]) if rows is None else np.asarray(rows)
    kh = _f64(k_I)
    idxh = _i64(idx)
    th = _f64(teacher)
    g = np.ones(q_I.shape[0]) if grad is None else _f64(grad)
    H, D = q_I.shape[1], q_I.shape[2]
    k = idxh.shape[1]
    loss = np.zeros(len(rows))
    dI = np.zeros((len(rows), k))
    dq = np.zeros((len(rows), H, D))
    dw = np.zeros((len(rows), H))
    dk = np.zeros(kh.shape)
    for r, t in enumerate(rows):
        l, a, b, c, e = indexer_kl_row(q_I[t], kh, w[t], idxh[t], th[t])
        loss[r] = l
        dI[r], dq[r], dw[r] = g[t] * a, g[t] * b, g[t] * c
        ok = idxh[t] >= 0
        np.add.at(dk, idxh[t][ok], g[t] * e[ok])
    return loss, dI, dq, dw, dk


# --------------------------------------------------- routing variants (pools, window)

def complete_block_topk(scores, k: int, block_size: int, cu_seqlens=None, rows=None):
    """Top-k over complete key blocks only: row t (offset o = t - start in its
    sequence) competes its blocks b < (o + 1) // B, the blocks all of whose keys are
    causal; the block that holds the query is left out unless it is complete. Same
    order and output convention as ``topk_select_row``; ids local to the sequence.

    "Support NoPE shapes and unaligned top-k in TileLang sparse MLA", the quoted GLM
    PR body, section "Why": k-pool selection picks among pools of keys, and the
    query's incomplete tail pool is handled apart (``kpool_expand``).
    """
    scores = np.asarray(scores)
    rows = np.arange(scores.shape[0]) if rows is None else np.asarray(rows)
    if cu_seqlens is None:
        starts = np.zeros(len(rows), dtype=np.int64)
    else:
        cu = _i64(cu_seqlens)
        starts = seq_bounds(int(cu[-1]), cu)[0][rows]
    idx = np.full((len(rows), k), -1, dtype=np.int32)
    val = np.full((len(rows), k), NEG_INF, dtype=np.float32)
    for r, t in enumerate(rows):
        n = (int(t - starts[r]) + 1) // block_size
        idx[r], val[r] = topk_select_row(scores[r], n, k)
    return idx, val


def kpool_expand(pool_idx, pool: int, cu_seqlens=None, T: int | None = None):
    """Token slots of a k-pool route, with the query's incomplete tail pool appended.

    Same passage as ``complete_block_topk`` (width 2048 + 3 = 2051 for 512 pools of
    four keys). Reading: slot i of row t's pool route (a local pool id c, or -1) gives
    the P slots i*P .. i*P + P - 1, holding the keys start + c*P .. start + c*P + P - 1
    (global rows; -1 for a -1 pool); then the keys of the query's own pool when it is
    incomplete (the o % P + 1 keys start + (o // P) * P .. t, o = t - start, when
    o % P != P - 1) fill the last P - 1 slots, -1 padded. Width k*P + P - 1.
    """
    pool_idx = _i64(pool_idx)
    Tn = pool_idx.shape[0] if T is None else T
    start, _ = seq_bounds(Tn, cu_seqlens)
    k = pool_idx.shape[1]
    out = np.full((Tn, k * pool + pool - 1), -1, dtype=np.int32)
    for t in range(Tn):
        s0 = int(start[t])
        for i, c in enumerate(pool_idx[t]):
            if c >= 0:
                out[t, i * pool:(i + 1) * pool] = range(s0 + c * pool, s0 + c * pool + pool)
        o = t - s0
        if o % pool != pool - 1:
            tail = list(range(s0 + (o // pool) * pool, t + 1))
            out[t, k * pool:k * pool + len(tail)] = tail
    return out


def append_window(idx, window: int, offset: int = 0, cu_seqlens=None):
    """Selected slots followed by a causal window of raw keys.

    "Add fused SBHD compressed sparse attention", "Scope" (compressed + window + sink).
    Reading: row t keeps its k selected slots and gains ``window`` slots holding
    offset + s for the keys s = t - window + 1 .. t of its own sequence (-1 where s
    falls before the sequence start); ``offset`` places the raw keys after another
    key table (e.g. compressed entries first). Width k + window.
    """
    idx = _i64(idx)
    T, k = idx.shape
    start, _ = seq_bounds(T, cu_seqlens)
    out = np.full((T, k + window), -1, dtype=np.int32)
    out[:, :k] = idx
    for t in range(T):
        for i in range(window):
            s = t - window + 1 + i
            if s >= start[t]:
                out[t, k + i] = offset + s
    return out
