/*
 * sa.h -- C ABI of the indexer-routed sparse-attention forward path on AMD MI355X
 * (gfx950). Four entry points, each a launch of hand-written HIP kernels on the
 * caller's stream:
 *
 *   sa_indexer_scores        multi-head ReLU indexer (dense scores, or fused with an
 *                            exact top-k so the score matrix is never stored)
 *   sa_topk_select           exact, deterministic top-k of score rows
 *   sa_sparse_mla_fwd        absorbed-MLA attention over selected latent rows
 *   sa_block_sparse_gqa_fwd  grouped-query attention over selected key blocks
 *
 * Sources (web pages on indexer-routed sparse attention in Megatron-LM):
 *   [QSA]  "Add trainable QSA sparse attention with a TileLang backend"
 *          (Megatron-LM issue #7060)
 *   [DSA]  "Enable DSA CP/absorbed/THD paths with TileLang fused ops"
 *          (Megatron-LM PR #3674)
 *   [NOPE] "Support NoPE shapes and unaligned top-k in TileLang sparse MLA"
 *          (Megatron-LM PR #7617), with the downstream GLM-5.3-Flash PR body it quotes
 *
 * Conventions shared by every call
 *   - Every pointer argument except `stream` is a DEVICE pointer (hipMalloc'd or a
 *     torch tensor's data). cu_seqlens included.
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronises; each call only enqueues kernels on `stream` (a hipStream_t; NULL
 *     means the default stream) and returns.
 *   - Inputs are read only and are left byte-identical ([NOPE] "Validation": input
 *     preservation). Outputs must not alias inputs or each other.
 *   - Tensors are dense, row-major, with the shapes given; no strides.
 *   - Packed variable-length (THD) layout ([DSA] "What does this PR do ?"): T rows are
 *     num_seqs sequences back to back; cu_seqlens is int32 [num_seqs+1], cu[0] = 0,
 *     cu[num_seqs] = T, non-decreasing; max_seqlen >= every cu[j+1]-cu[j]. Passing
 *     cu_seqlens = NULL means one sequence [0, T) (num_seqs and max_seqlen ignored).
 *     Causality is per sequence: key s is visible to query t iff start(t) <= s <= t.
 *   - Errors: argument checks run on the host before any launch and return a status
 *     without touching the stream ([QSA] "Additional context": fail fast on
 *     unsupported combinations). SA_ERR_LAUNCH reports hipGetLastError after a launch.
 *     Device-side contents (index values, cu_seqlens values) are NOT validated by
 *     libsa.so: an index outside its documented range is undefined behaviour. The
 *     debug build libsa_debug.so (same symbols, same kernels) checks them on the
 *     device before launching -- idx of sa_sparse_mla_fwd in [-1, S), and cu_seqlens
 *     (cu[0] = 0, cu[num_seqs] = T, every length in [0, max_seqlen]) -- and returns
 *     SA_ERR_SHAPE for a value out of range; those checks synchronise the stream.
 *     Route values of sa_block_sparse_gqa_fwd need no check: any value outside a
 *     query's blocks [0, own] contributes nothing.
 *   - Determinism: the same inputs give bitwise-identical outputs on every run,
 *     independent of other work on the device ([NOPE] "Validation": forward bit-exact
 *     replay). No call uses floating-point atomics.
 *   - Thread safety: calls hold no global mutable state and may be issued from any
 *     host thread.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 3

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,         /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,        /* a size is non-positive or inconsistent */
  SA_ERR_DTYPE = 3,        /* unknown dtype code */
  SA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned */
  SA_ERR_UNSUPPORTED = 5,  /* valid but unsupported combination (limits below) */
  SA_ERR_LAUNCH = 6,       /* a kernel launch failed */
  SA_ERR_WORKSPACE = 7     /* the workspace is smaller than the call needs */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* Human-readable name of a status code (static string). */
const char* sa_status_string(int status);

/* SA_ABI_VERSION of the built library. */
int sa_abi_version(void);

/*
 * sa_indexer_scores -- ReLU-weighted multi-head indexer.
 *
 * [QSA] "Describe the solution you'd like" (trainable indexer, streaming runner with
 * bounded memory, ReLU scores that tie at zero) and "Is your feature request related
 * to a problem?" (never materialise the [sequence, sequence / block_size] scores);
 * [DSA] file table (fused indexer forward). For query t and causal key s:
 *
 *     I[t,s] = sum_h w[t,h] * max( sum_d q_I[t,h,d] * k_I[s,d], 0 )
 *
 * accumulated in fp32 (bf16 products are exact in fp32). One k_I row per token is
 * shared by all indexer heads; any score scaling must be folded into w by the caller.
 * -0.0 results are stored as +0.0. With block_size B > 1 the row's score for block b
 * of its sequence is max of I[t,s] over the block's causal keys
 * s in [start + bB, min(start + bB + B - 1, t)].
 *
 * Inputs:
 *   q_I  [T, H_I, D_I]  dtype        k_I [T, D_I] dtype       w [T, H_I] fp32
 *   dtype  SA_F32 or SA_BF16 (q_I and k_I)
 *   H_I in {4, 8, 16, 32, 64}; D_I in {64, 128}; block_size in {1, 2, 4, 8, 16, 32,
 *   64, 128, 256}; otherwise SA_ERR_UNSUPPORTED.
 * Mode 1, dense (topk == 0): writes scores [T, ld] fp32; row t, column c holds the
 *   score of key start(t)+c (token mode) or of local block c (block mode) for the
 *   causal columns c < n(t), where n(t) = t-start(t)+1 (tokens) or
 *   (t-start(t))/B + 1 (blocks). Columns >= n(t) are not written.
 *   ld >= max_seqlen (tokens) or ceil(max_seqlen / B) (blocks); ld % 4 == 0.
 *   out_idx/out_val must be NULL.
 * Mode 2, fused selection (topk > 0): scores must be NULL. The causal keys stream
 *   tile by tile and each tile's scores are filtered on the fly; the score matrix is
 *   never stored. Writes out_idx [T, topk] int32 and, if out_val != NULL, out_val
 *   [T, topk] fp32, with exactly the result sa_topk_select gives on the dense scores
 *   (same indices, same order). Token mode: topk in [1, 2048]; block mode: topk in
 *   [1, 64]. force_own_block 0 or 1 as in sa_topk_select (block mode only; for 2,
 *   write the dense block scores and select them with sa_topk_select).
 *   Two ways to run it (same results, bit for bit):
 *   - ws == NULL: one pass; each row keeps an exact running top-k in on-chip
 *     memory ([QSA] "Describe the solution you'd like": streaming runner with
 *     bounded memory).
 *   - ws != NULL with ws_bytes >= sa_indexer_workspace_bytes(...): when that size is
 *     non-zero, two passes ([DSA] file table: the fused top-k's cached scratch
 *     buffers). Token mode (bf16, 64 indexer heads): the first pass appends, per row,
 *     the keys at or above a pivot drawn from a sample of the row's scores to the
 *     row's slice of the workspace (a per-tile partial selection; a few thousand
 *     entries per row), then the exact selection of sa_topk_select finishes each row;
 *     a row whose pivot kept fewer than topk keys is redone by the one-pass kernel.
 *     The workspace holds [T, cap] fp32 scores, [T, cap] int32 key ids and [T] int32
 *     counts. Block mode with sequences of more than 32 key tiles of 64 keys: the key
 *     range of each group of query rows is split over up to 4 workgroups, each
 *     keeping the exact top-k of its blocks, and a merge keeps the exact top-k of
 *     their union (the same blocks as one pass). The workspace holds [T, splits,
 *     topk] order keys and block ids, [T, splits] counts and [T] own-block values.
 *     Its contents on return are unspecified, and two calls in flight must not share
 *     one. A smaller ws_bytes returns SA_ERR_WORKSPACE; ws must be 16-byte aligned.
 *     When the size is zero, ws is ignored.
 */
sa_status sa_indexer_scores(const void* q_I, const void* k_I, const float* w, int dtype,
                            int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t max_seqlen, int32_t H_I, int32_t D_I, int32_t block_size,
                            float* scores, int64_t ld,
                            int32_t topk, int32_t force_own_block,
                            int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * sa_indexer_workspace_bytes -- workspace size for sa_indexer_scores mode 2.
 *
 * Bytes that the two-pass fused selection needs for these arguments (T, the widest
 * sequence max_seqlen -- T for one sequence --, dtype, H_I, D_I, block_size, topk);
 * 0 when the call runs in one pass (dense mode; token mode in fp32 or with H_I != 64;
 * block mode with sequences of at most 2048 keys). For T = 32768 one-sequence rows
 * at topk = 2048 it is about 1.3 GB; for 8192-token rows in blocks of 64 at topk = 16,
 * 4.2 MB. Host-only; no device access.
 */
size_t sa_indexer_workspace_bytes(int dtype, int32_t T, int32_t max_seqlen, int32_t H_I,
                                  int32_t D_I, int32_t block_size, int32_t topk);

/*
 * sa_indexer_scores_noalloc -- sa_indexer_scores without a caller workspace and
 * without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, results and
 * errors as sa_indexer_scores, minus ws/ws_bytes: when the call wants a workspace
 * (sa_indexer_workspace_bytes > 0) it uses a static device array of this library,
 * sa_noalloc_scratch_bytes() = 128 MiB, which every GPU the library runs on holds
 * from the library's load until the process ends; the first call on a device looks
 * up that device's copy. A call that needs more than the array holds returns
 * SA_ERR_WORKSPACE without launching anything (at topk = 2048 that is about 5000
 * rows of one 5000-token sequence; pass fewer rows per call, or use
 * sa_indexer_scores with a workspace). Nothing in the array has to start at zero:
 * every byte a call reads was written earlier by the same call. All calls on one
 * GPU share its array, so calls that overlap in time on one GPU (two streams, two
 * host threads) race and must be serialised by the caller.
 */
sa_status sa_indexer_scores_noalloc(const void* q_I, const void* k_I, const float* w, int dtype,
                                    int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                                    int32_t max_seqlen, int32_t H_I, int32_t D_I,
                                    int32_t block_size, float* scores, int64_t ld, int32_t topk,
                                    int32_t force_own_block, int32_t* out_idx, float* out_val,
                                    void* stream);

/* Bytes of the static device array that sa_indexer_scores_noalloc uses. */
size_t sa_noalloc_scratch_bytes(void);

/*
 * sa_topk_select -- exact, deterministic top-k of score rows.
 *
 * [QSA] "Describe the solution you'd like": exact selection keyed lexicographically
 * on (score, id), so ties (ReLU zeros) resolve identically on every run and rank;
 * [NOPE] "What does this PR do?": empty slots hold the -1 sentinel.
 *
 * Order: a precedes b iff score_a > score_b, or score_a == score_b and index_a <
 * index_b (-0.0 equals +0.0). Row t keeps the first min(topk, n(t)) candidates in
 * that order and writes them in ASCENDING index order to out_idx[t, 0..], then -1
 * up to topk. out_val (nullable) receives the scores in the same slots (+0.0 for a
 * zero score) and -inf on padding. NaN scores are not supported.
 *
 * Candidates of row t:
 *   cand_idx == NULL (dense causal rows, as written by sa_indexer_scores mode 1):
 *     columns c < n(t) of vals[t, :]; token mode (block_size 1) reports global key
 *     rows start(t)+c; block mode (block_size B > 1) reports local block ids c.
 *     force_own_block (block mode): 0 = the query's own block competes like the
 *     others; 1 = it (c = n(t)-1) is always kept and counts toward topk; 2 = only
 *     complete blocks compete, n(t) = (t-start(t)+1) / B, so the own block is left
 *     out while the query has not reached its last key (k-pool selection, [NOPE]
 *     quoted GLM body, "Why": the incomplete tail pool is appended apart, see
 *     sa_kpool_expand).
 *   cand_idx != NULL (explicit candidate lists): vals[t, c] with index cand_idx[t, c]
 *     for every column c < ld whose cand_idx is >= 0; the valid indices of a row must
 *     be strictly ascending left to right (-1 entries may sit anywhere). The layout
 *     arguments are ignored; force_own_block must be 0.
 * Sizes: ld % 4 == 0 (vals and cand_idx rows start 16-byte aligned), ld >= the
 *   widest row, widest row <= 65536; topk in [1, 65536].
 * Launches: one or more kernels on `stream` (dense single-sequence rows are split by
 *   width); a row that the fast pass cannot finish marks out_idx[t, 0] with INT32_MIN,
 *   and a last kernel of the same call completes it, so after the call (in stream
 *   order) every row holds its final result.
 */
sa_status sa_topk_select(const float* vals, const int32_t* cand_idx, int64_t ld,
                         int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                         int32_t max_seqlen, int32_t block_size, int32_t topk,
                         int32_t force_own_block, int32_t* out_idx, float* out_val,
                         void* stream);

/*
 * sa_sparse_mla_fwd -- absorbed-MLA sparse attention forward.
 *
 * [DSA] file table (sparse-MLA forward kernel); [NOPE] "What does this PR do?" and
 * the quoted GLM PR body, "Change": q and k share the 576-wide latent layout, the
 * value is the first 512 channels of the same latent row, -1 slots are masked, the
 * caller's softmax scale is used as given; a 512-wide (NoPE) q/kv is accepted
 * directly (it equals the zero-padded 576 case). For query t and head h over the
 * valid slots j (idx[t,j] >= 0):
 *
 *     l_j = scale * q[t,h,:] . kv[idx[t,j], :]          (d_qk channels)
 *     out[t,h,:] = sum_j softmax(l)_j * kv[idx[t,j], 0:d_v]
 *     lse[t,h]   = ln sum_j exp(l_j)
 *
 * fp32 softmax and accumulation; bf16 matrix products on MFMA for SA_BF16. A row
 * with no valid slot gives out = 0 and lse = -inf. Each slot counts once (a repeated
 * index counts twice). Slot order does not matter; topk need not be a multiple of
 * anything.
 *
 * sink (nullable, [H] fp32): a per-head logit that joins the softmax denominator and
 * carries no value ("Add fused SBHD compressed sparse attention", "Scope": the
 * compressed + window + sink attention): with Z = sum_j exp(l_j) + exp(sink[h]),
 * out = sum_j exp(l_j) kv[idx_j, 0:d_v] / Z and lse = ln Z; a row with no valid slot
 * gives out = 0 and lse = sink[h]. A window of raw keys is attended by appending its
 * slots to idx (sa_append_window).
 *
 * Inputs: q [T, H, d_qk], kv [S, d_qk] (dtype), idx [T, topk] int32 with values in
 *   [0, S) or -1. Outputs: out [T, H, d_v] (dtype), lse [T, H] fp32 (nullable).
 * Sizes: d_qk in {512, 576}; d_v == 512; H in [1, 128]; S >= 1; topk in [1, 8192] for
 *   fp32 and [1, 4096] for bf16, except [1, 3968] for bf16 with H > 64 and d_qk = 576
 *   (the index row shares the workgroup's LDS with the gather stages); larger values
 *   return SA_ERR_UNSUPPORTED.
 *   SA_BF16 needs H % 16 == 0 or H < 16 (heads are processed in groups of 32;
 *   partial groups are masked), and kv of at most 2^31 - 1 bytes (S * d_qk * 2).
 */
sa_status sa_sparse_mla_fwd(const void* q, const void* kv, const int32_t* idx, int dtype,
                            int32_t T, int32_t S, int32_t H, int32_t d_qk, int32_t d_v,
                            int32_t topk, float scale, const float* sink, void* out, float* lse,
                            void* stream);

/*
 * sa_sparse_mla_bwd -- gradients of sa_sparse_mla_fwd.
 *
 * [DSA] file table (sparse-MLA backward kernels); [NOPE] "Validation" (output and
 * Q/K gradients checked against an independent fp32 reference; the backward
 * accumulates with atomics, so it is checked numerically, not for bitwise replay).
 * Given the forward's inputs, its lse, and dout = dLoss/dout, with
 * p_j = exp(scale q.kv[idx_j] - lse), dp_j = dout . kv[idx_j, 0:d_v],
 * D = sum_j p_j dp_j (= dout . out, summed here from the p_j dp_j, so the forward's
 * rounded output is not needed) and ds_j = scale p_j (dp_j - D) for every valid slot
 * j of a row and head:
 *
 *     dq[t,h,:]       = sum_j ds_j kv[idx_j, :]
 *     dkv[idx_j, :]  += sum_(t,h) ds_j q[t,h,:]       (all d_qk channels)
 *     dkv[idx_j, :d_v] += sum_(t,h) p_j dout[t,h,:]   (the value channels)
 *
 * -1 slots contribute nothing; a repeated index contributes once per slot; a row with
 * no valid slot (lse = -inf) gets dq = 0. With a sink (the forward's sink, whose term
 * lse includes), p_j already shares its denominator with the sink; dsink (nullable
 * [H] fp32, zeroed by the call, needs sink) receives
 *     dsink[h] = -sum_t exp(sink[h] - lse[t,h]) D[t,h]
 * with atomics.
 * Inputs: q [T,H,d_qk], kv [S,d_qk], dout [T,H,d_v] (dtype), idx [T,topk], lse
 *   [T,H] fp32 (the forward's). Outputs: dq [T,H,d_qk] (dtype); dkv
 *   [S,d_qk] fp32, which the call zeroes and then accumulates into with
 *   floating-point atomics, so dkv's low bits may differ from run to run (every
 *   other output is deterministic). No output may overlap an input or another
 *   output: with bf16 at 64 or 128 heads the call keeps each row's D = dout . out in
 *   the first four bytes of that row of dq between its launches, then overwrites dq.
 * Sizes: d_qk in {512, 576}; d_v == 512; H in [1, 128]; topk >= 1 (at most 8192 for
 *   SA_F32). Pointers 16-byte aligned (lse and idx: 4-byte).
 */
sa_status sa_sparse_mla_bwd(const void* q, const void* kv, const int32_t* idx, const void* dout,
                            const float* lse, int dtype, int32_t T, int32_t S, int32_t H,
                            int32_t d_qk, int32_t d_v, int32_t topk, float scale, const float* sink,
                            void* dq, float* dkv, float* dsink, void* stream);

/*
 * sa_attn_teacher -- teacher distribution of the sparse KL indexer loss.
 *
 * [QSA] "Is your feature request related to a problem?" and "Describe the solution
 * you'd like" (sparse KL supervision of the indexer; a stage-2 teacher/KL loss); [DSA]
 * "What does this PR do ?" (streaming sparse-KL for the indexer loss). Reading of the
 * pages: the teacher of row t is the sparse attention's probability of each of its
 * slots, averaged over the H attention heads:
 *
 *     teacher[t,j] = (1/H) sum_h exp(scale q[t,h,:] . kv[idx[t,j],:] - lse[t,h])
 *
 * and 0 on -1 slots (so a row's valid entries sum to 1). q, kv, idx, scale and lse are
 * those of sa_sparse_mla_fwd (lse its output). teacher [T,topk] fp32 is overwritten:
 * for SA_BF16 one plain store per slot after the sum over all heads (deterministic);
 * for SA_F32 accumulated with floating-point atomics over the heads (low bits may vary
 * from run to run). Limits as sa_sparse_mla_fwd's d_qk and H.
 */
sa_status sa_attn_teacher(const void* q, const void* kv, const int32_t* idx, const float* lse,
                          int dtype, int32_t T, int32_t S, int32_t H, int32_t d_qk, int32_t topk,
                          float scale, float* teacher, void* stream);

/*
 * sa_indexer_kl_bwd -- sparse KL loss of the indexer and its backward.
 *
 * [QSA] (as above); [DSA] file table (fused indexer backward kernel). Over the valid
 * slots j of row t (key rows s_j = idx[t,j], global rows of k_I), with the indexer
 * scores I_j = sum_h w[t,h] max(z_hj, 0), z_hj = q_I[t,h,:] . k_I[s_j,:] (the
 * definition of sa_indexer_scores), the student softmax_j(I) and the given teacher p:
 *
 *     loss[t]    = sum_j p_j (log p_j - log softmax(I)_j)       (0 log 0 = 0)
 *     dI_j       = g_t (softmax(I)_j - p_j)
 *     dw[t,h]    = sum_j dI_j max(z_hj, 0)
 *     dq_I[t,h]  = sum_j dI_j w[t,h] [z_hj > 0] k_I[s_j]
 *     dk_I[s_j] += sum_h dI_j w[t,h] [z_hj > 0] q_I[t,h]
 *
 * i.e. the gradients of sum_t g_t loss[t], g = grad [T] fp32 (NULL: every g_t = 1). A
 * row without a valid slot has loss 0 and zero gradients. Only the topk selected
 * scores of a row are formed; no [T, T] matrix.
 * Inputs: q_I [T,H_I,D_I], k_I [S,D_I] (dtype), w [T,H_I] fp32, idx [T,topk] int32 in
 *   [-1, S), teacher [T,topk] fp32 (e.g. from sa_attn_teacher), grad [T] or NULL.
 * Outputs: loss [T] fp32, dq_I [T,H_I,D_I] (dtype), dw [T,H_I] fp32, dk_I [S,D_I] fp32
 *   (zeroed by the call, then accumulated with floating-point atomics: its low bits
 *   may vary from run to run).
 * Sizes: D_I in {64, 128}; SA_BF16 needs H_I in {16, 32, 64}; topk <= 4096.
 */
sa_status sa_indexer_kl_bwd(const void* q_I, const void* k_I, const float* w, const int32_t* idx,
                            const float* teacher, const float* grad, int dtype, int32_t T, int32_t S,
                            int32_t H_I, int32_t D_I, int32_t topk, float* loss, void* dq_I,
                            float* dw, float* dk_I, void* stream);

/*
 * sa_block_sparse_gqa_fwd -- grouped-query attention over selected key blocks.
 *
 * [QSA] "Describe the solution you'd like": sparse GQA attention over the blocks
 * chosen by the exact block TopK. For query t (sequence start c) and head h, the
 * attended keys are the set of s <= t whose local block (s - c) / block_size appears
 * among the slots of blk[t, :]; -1 slots and blocks past the query's own block add
 * nothing, and a block listed twice contributes its keys once. Head h reads kv head
 * g = h / (Hq / Hkv):
 *
 *     out[t,h,:] = softmax_s(scale * q[t,h,:] . k[s,g,:]) @ v[s,g,:]
 *     lse[t,h]   = ln sum_s exp(scale * q[t,h,:] . k[s,g,:])
 *
 * No key -> out = 0, lse = -inf.
 * Inputs: q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, Dv] (dtype), blk [T, nblk] int32
 *   local block ids in [0, ceil(len/block_size)) or -1. Outputs: out [T, Hq, Dv]
 *   (dtype), lse [T, Hq] fp32 (nullable).
 * Sizes: D == Dv == 128 or 64; Hq % Hkv == 0; Hq / Hkv <= 16; block_size a multiple
 *   of 16 up to 128; nblk in [1, 64].
 */
sa_status sa_block_sparse_gqa_fwd(const void* q, const void* k, const void* v,
                                  const int32_t* blk, int dtype, int32_t T,
                                  const int32_t* cu_seqlens, int32_t num_seqs,
                                  int32_t max_seqlen, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t Dv, int32_t block_size, int32_t nblk, float scale,
                                  void* out, float* lse, void* stream);

/*
 * sa_block_sparse_gqa_bwd -- gradients of sa_block_sparse_gqa_fwd.
 *
 * [QSA] "Is your feature request related to a problem?" and "Describe the solution
 * you'd like" (sparse GQA attention forward and backward; numerical and gradient
 * tests). Same key sets as the forward (the causal keys of the routed blocks, each
 * block once). With p_s = exp(scale q[t,h].k[s,g] - lse[t,h]), dp_s = dout[t,h].v[s,g],
 * D = sum_s p_s dp_s and ds_s = scale p_s (dp_s - D), for g = h / (Hq / Hkv):
 *
 *     dq[t,h]   = sum_s ds_s k[s,g]
 *     dk[s,g]  += sum_(t,h) ds_s q[t,h]
 *     dv[s,g]  += sum_(t,h) p_s dout[t,h]
 *
 * Inputs as the forward plus dout [T,Hq,Dv] (dtype) and the forward's lse [T,Hq] fp32.
 * Outputs: dq [T,Hq,D] (dtype); dk [T,Hkv,D] and dv [T,Hkv,Dv] fp32, which the call
 * zeroes and then accumulates into with floating-point atomics (their low bits may
 * differ from run to run; dq is deterministic). No output may overlap an input or
 * another output: in bf16 the call keeps each row's D in the first four bytes of that
 * row of dq between its launches, then overwrites dq. Limits as the forward.
 */
sa_status sa_block_sparse_gqa_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                                  const void* dout, const float* lse, int dtype, int32_t T,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t Dv, int32_t block_size,
                                  int32_t nblk, float scale, void* dq, float* dk, float* dv,
                                  void* stream);

/*
 * sa_kpool_expand -- token slots of a k-pool route, the incomplete tail pool appended.
 *
 * [NOPE] quoted GLM PR body, "Why": k-pool selection appends the query's incomplete
 * tail pool, so the top-k width is 2048 + 3. Reading: pools are runs of `pool` keys of
 * a sequence (pool c = keys start + c*pool .. + pool - 1); slot i of pools [T, kp]
 * (a local pool id, e.g. from sa_topk_select with force_own_block = 2, or -1) gives
 * out slots i*pool .. i*pool + pool - 1 (global key rows; -1 for a -1 pool); the last
 * pool - 1 slots hold the keys of the query's own pool while it is incomplete
 * (start + (o / pool) * pool .. t, o = t - start(t), when o % pool != pool - 1), -1
 * padded. out [T, kp*pool + pool - 1] int32 (2051 for 512 pools of 4), ready for
 * sa_sparse_mla_fwd. Pool ids must be below the row's complete pools.
 */
sa_status sa_kpool_expand(const int32_t* pools, int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                          int32_t max_seqlen, int32_t kp, int32_t pool, int32_t* out, void* stream);

/*
 * sa_append_window -- selected slots followed by a causal window of raw keys.
 *
 * [CSA] "Add fused SBHD compressed sparse attention", "Scope" (compressed + window +
 * sink attention). out [T, k + window] int32: out[t, 0:k] = idx[t, :]; out[t, k + i] =
 * offset + s for s = t - window + 1 + i when s >= start(t), else -1. With offset = the
 * rows of a table that precedes the raw keys (e.g. compressed entries, so kv = [that
 * table; raw keys]), the result indexes the concatenated table.
 */
sa_status sa_append_window(const int32_t* idx, int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t max_seqlen, int32_t k, int32_t window, int32_t offset, int32_t* out,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
