// C ABI of the sparse-attention library: host-side argument checks and launches.
// Every check runs before any launch; a failing check returns its status and
// leaves the stream untouched.
#include <hip/hip_runtime.h>

#include "../../include/sa.h"
#include "sa_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sa_status launch_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_LAUNCH; }

// Shared checks of the packed-sequence layout; returns the widest sequence.
sa_status check_layout(int32_t T, const int32_t* cu, int32_t num_seqs, int32_t max_seqlen,
                       int32_t* widest) {
  if (T < 0) return SA_ERR_SHAPE;
  if (cu == nullptr) {
    *widest = T;
    return SA_OK;
  }
  if (num_seqs < 1 || max_seqlen < 1) return SA_ERR_SHAPE;
  if (max_seqlen > T && T > 0) return SA_ERR_SHAPE;
  *widest = max_seqlen;
  return SA_OK;
}

// Debug build only (SA_DEBUG_CHECKS): device contents are validated before any
// launch; a value out of its documented range returns SA_ERR_SHAPE.
#ifdef SA_DEBUG_CHECKS
sa_status debug_offsets(const int32_t* cu, int32_t nseq, int32_t T, int32_t maxlen, hipStream_t st) {
  if (!cu) return SA_OK;
  bool ok = false;
  if (sa::debug_check_offsets(cu, nseq, T, maxlen, st, &ok) != hipSuccess) return SA_ERR_LAUNCH;
  return ok ? SA_OK : SA_ERR_SHAPE;
}
sa_status debug_range(const int32_t* v, int64_t n, int32_t lo, int32_t hi, hipStream_t st) {
  bool ok = false;
  if (sa::debug_check_range(v, n, lo, hi, st, &ok) != hipSuccess) return SA_ERR_LAUNCH;
  return ok ? SA_OK : SA_ERR_SHAPE;
}
#define SA_DEBUG_RETURN(expr)           \
  do {                                  \
    const sa_status dbg_ = (expr);      \
    if (dbg_ != SA_OK) return dbg_;     \
  } while (0)
#else
#define SA_DEBUG_RETURN(expr) \
  do {                        \
  } while (0)
#endif

}  // namespace

extern "C" {

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL: a required pointer is NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE: a size is non-positive or inconsistent";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE: unknown dtype";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: combination outside the supported limits";
    case SA_ERR_LAUNCH: return "SA_ERR_LAUNCH: kernel launch failed";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE: workspace smaller than the call needs";
    default: return "unknown sa_status";
  }
}

int sa_abi_version(void) { return SA_ABI_VERSION; }

size_t sa_indexer_workspace_bytes(int dtype, int32_t T, int32_t max_seqlen, int32_t H_I,
                                  int32_t D_I, int32_t block_size, int32_t topk) {
  (void)D_I;
  if (T <= 0 || max_seqlen <= 0 || topk <= 0) return 0;
  return sa::indexer_ws_bytes(dtype == SA_BF16, T, max_seqlen > T ? T : max_seqlen, H_I,
                              block_size, topk);
}

sa_status sa_indexer_scores(const void* q_I, const void* k_I, const float* w, int dtype,
                            int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t max_seqlen, int32_t H_I, int32_t D_I, int32_t block_size,
                            float* scores, int64_t ld, int32_t topk, int32_t force_own_block,
                            int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                            void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  int32_t widest = 0;
  sa_status st = check_layout(T, cu_seqlens, num_seqs, max_seqlen, &widest);
  if (st != SA_OK) return st;
  if (H_I < 1 || D_I < 1 || block_size < 1 || topk < 0) return SA_ERR_SHAPE;
  if (H_I != 4 && H_I != 8 && H_I != 16 && H_I != 32 && H_I != 64) return SA_ERR_UNSUPPORTED;
  if (D_I != 64 && D_I != 128) return SA_ERR_UNSUPPORTED;
  if (block_size != 1 && block_size != 2 && block_size != 4 && block_size != 8 && block_size != 16 &&
      block_size != 32 && block_size != 64 && block_size != 128 && block_size != 256)
    return SA_ERR_UNSUPPORTED;
  if (force_own_block && block_size == 1) return SA_ERR_UNSUPPORTED;
  if (force_own_block < 0 || force_own_block > 1) return SA_ERR_UNSUPPORTED;   // 2: dense + select
  const bool dense = topk == 0;
  if (T == 0) return SA_OK;
  if (!q_I || !k_I || !w) return SA_ERR_NULL;
  if (!aligned16(q_I) || !aligned16(k_I) || !aligned16(w)) return SA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  SA_DEBUG_RETURN(debug_offsets(cu_seqlens, num_seqs, T, widest, s));
  if (dense) {
    if (!scores) return SA_ERR_NULL;
    if (out_idx || out_val) return SA_ERR_SHAPE;
    const int64_t need = block_size == 1 ? widest : (widest + block_size - 1) / block_size;
    if (ld < need || ld % 4 != 0) return SA_ERR_SHAPE;
    if (!aligned16(scores)) return SA_ERR_ALIGN;
    return launch_status(sa::launch_indexer_dense(q_I, k_I, w, dtype == SA_BF16, T, cu_seqlens,
                                                  num_seqs, widest, H_I, D_I, block_size, scores,
                                                  ld, s));
  }
  if (scores) return SA_ERR_SHAPE;
  if (!out_idx) return SA_ERR_NULL;
  if (block_size == 1 ? topk > 2048 : topk > 64) return SA_ERR_UNSUPPORTED;
  if (ws) {
    if (ws_bytes < sa_indexer_workspace_bytes(dtype, T, widest, H_I, D_I, block_size, topk))
      return SA_ERR_WORKSPACE;
    if (!aligned16(ws)) return SA_ERR_ALIGN;
  }
  return launch_status(sa::launch_indexer_topk(q_I, k_I, w, dtype == SA_BF16, T, cu_seqlens,
                                               num_seqs, widest, H_I, D_I, block_size, topk,
                                               force_own_block, out_idx, out_val, ws, s));
}

sa_status sa_topk_select(const float* vals, const int32_t* cand_idx, int64_t ld, int32_t T,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                         int32_t block_size, int32_t topk, int32_t force_own_block,
                         int32_t* out_idx, float* out_val, void* stream) {
  if (T < 0 || ld < 1 || topk < 1 || block_size < 1) return SA_ERR_SHAPE;
  if (ld % 4 != 0) return SA_ERR_SHAPE;
  if (force_own_block < 0 || force_own_block > 2) return SA_ERR_UNSUPPORTED;
  if (topk > 65536) return SA_ERR_UNSUPPORTED;
  int32_t width = 0;
  if (cand_idx) {
    if (force_own_block) return SA_ERR_UNSUPPORTED;
    width = ld > INT32_MAX ? INT32_MAX : (int32_t)ld;
  } else {
    int32_t widest = 0;
    sa_status st = check_layout(T, cu_seqlens, num_seqs, max_seqlen, &widest);
    if (st != SA_OK) return st;
    if (force_own_block && block_size == 1) return SA_ERR_UNSUPPORTED;
    width = block_size == 1 ? widest : (widest + block_size - 1) / block_size;
    if (ld < width) return SA_ERR_SHAPE;
  }
  if (width > sa::topk_select_max_width()) return SA_ERR_UNSUPPORTED;
  if (T == 0) return SA_OK;
  if (!vals || !out_idx) return SA_ERR_NULL;
  if (!aligned16(vals) || (cand_idx && !aligned16(cand_idx))) return SA_ERR_ALIGN;
  if (!cand_idx) SA_DEBUG_RETURN(debug_offsets(cu_seqlens, num_seqs, T, max_seqlen,
                                               reinterpret_cast<hipStream_t>(stream)));
  return launch_status(sa::launch_topk_select(vals, cand_idx, ld, T, cand_idx ? nullptr : cu_seqlens,
                                              num_seqs, width, block_size, topk, force_own_block,
                                              out_idx, out_val, reinterpret_cast<hipStream_t>(stream)));
}

sa_status sa_sparse_mla_fwd(const void* q, const void* kv, const int32_t* idx, int dtype,
                            int32_t T, int32_t S, int32_t H, int32_t d_qk, int32_t d_v,
                            int32_t topk, float scale, const float* sink, void* out, float* lse,
                            void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  if (T < 0 || S < 1 || H < 1 || topk < 1 || d_qk < 1 || d_v < 1) return SA_ERR_SHAPE;
  if (d_qk != 512 && d_qk != 576) return SA_ERR_UNSUPPORTED;
  if (d_v != 512) return SA_ERR_UNSUPPORTED;
  if (H > 128) return SA_ERR_UNSUPPORTED;
  if (dtype == SA_BF16 && H >= 16 && H % 16 != 0) return SA_ERR_UNSUPPORTED;
  // the index row is staged in LDS (bf16); fp32 keeps the bound of its backward
  if (topk > (dtype == SA_BF16 ? 4096 : 8192)) return SA_ERR_UNSUPPORTED;
  if (dtype == SA_BF16 && !sa::sparse_mla_bf16_fits(H, d_qk, topk)) return SA_ERR_UNSUPPORTED;
  // the bf16 kernel addresses the RoPE channels of gathered rows with 32-bit byte
  // offsets from the start of kv
  if (dtype == SA_BF16 && (int64_t)S * d_qk * 2 > (int64_t)INT32_MAX) return SA_ERR_UNSUPPORTED;
  if (T == 0) return SA_OK;
  if (!q || !kv || !idx || !out) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return SA_ERR_ALIGN;
  SA_DEBUG_RETURN(debug_range(idx, (int64_t)T * topk, -1, S, reinterpret_cast<hipStream_t>(stream)));
  return launch_status(sa::launch_sparse_mla(q, kv, idx, dtype == SA_BF16, T, S, H, d_qk, d_v, topk,
                                             scale, sink, out, lse, reinterpret_cast<hipStream_t>(stream)));
}

sa_status sa_sparse_mla_bwd(const void* q, const void* kv, const int32_t* idx, const void* dout,
                            const float* lse, int dtype, int32_t T, int32_t S, int32_t H,
                            int32_t d_qk, int32_t d_v, int32_t topk, float scale, const float* sink,
                            void* dq, float* dkv, float* dsink, void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  if (T < 0 || S < 1 || H < 1 || topk < 1 || d_qk < 1 || d_v < 1) return SA_ERR_SHAPE;
  if (d_qk != 512 && d_qk != 576) return SA_ERR_UNSUPPORTED;
  if (d_v != 512) return SA_ERR_UNSUPPORTED;
  if (H > 128) return SA_ERR_UNSUPPORTED;
  if (dtype == SA_F32 && topk > 8192) return SA_ERR_UNSUPPORTED;   // per-slot terms staged in LDS
  if (!dkv) return SA_ERR_NULL;
  if (dsink && !sink) return SA_ERR_NULL;
  if (T > 0 && (!q || !kv || !idx || !dout || !lse || !dq)) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(dout) || !aligned16(dq) || !aligned16(dkv))
    return SA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T > 0) SA_DEBUG_RETURN(debug_range(idx, (int64_t)T * topk, -1, S, s));
  return launch_status(sa::launch_sparse_mla_bwd(q, kv, idx, dout, lse, dtype == SA_BF16, T, S, H, d_qk,
                                                 d_v, topk, scale, sink, dq, dkv, dsink, s));
}

sa_status sa_block_sparse_gqa_fwd(const void* q, const void* k, const void* v, const int32_t* blk,
                                  int dtype, int32_t T, const int32_t* cu_seqlens,
                                  int32_t num_seqs, int32_t max_seqlen, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t Dv, int32_t block_size, int32_t nblk,
                                  float scale, void* out, float* lse, void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  int32_t widest = 0;
  sa_status st = check_layout(T, cu_seqlens, num_seqs, max_seqlen, &widest);
  if (st != SA_OK) return st;
  if (Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || block_size < 1 || nblk < 1) return SA_ERR_SHAPE;
  if (Hq % Hkv != 0) return SA_ERR_SHAPE;
  if (Hq / Hkv > 16) return SA_ERR_UNSUPPORTED;
  if (!((D == 128 && Dv == 128) || (D == 64 && Dv == 64))) return SA_ERR_UNSUPPORTED;
  if (block_size % 16 != 0 || block_size > 128) return SA_ERR_UNSUPPORTED;
  if (nblk > sa::block_gqa_max_route()) return SA_ERR_UNSUPPORTED;
  if (T == 0) return SA_OK;
  if (!q || !k || !v || !blk || !out) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SA_ERR_ALIGN;
  SA_DEBUG_RETURN(debug_offsets(cu_seqlens, num_seqs, T, max_seqlen, reinterpret_cast<hipStream_t>(stream)));
  return launch_status(sa::launch_block_gqa(q, k, v, blk, dtype == SA_BF16, T, cu_seqlens, num_seqs,
                                            widest, Hq, Hkv, D, Dv, block_size, nblk, scale, out, lse,
                                            reinterpret_cast<hipStream_t>(stream)));
}

sa_status sa_attn_teacher(const void* q, const void* kv, const int32_t* idx, const float* lse,
                          int dtype, int32_t T, int32_t S, int32_t H, int32_t d_qk, int32_t topk,
                          float scale, float* teacher, void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  if (T < 0 || S < 1 || H < 1 || topk < 1 || d_qk < 1) return SA_ERR_SHAPE;
  if (d_qk != 512 && d_qk != 576) return SA_ERR_UNSUPPORTED;
  if (H > 128) return SA_ERR_UNSUPPORTED;
  if (T == 0) return SA_OK;
  if (!q || !kv || !idx || !lse || !teacher) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv)) return SA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  SA_DEBUG_RETURN(debug_range(idx, (int64_t)T * topk, -1, S, s));
  return launch_status(sa::launch_attn_teacher(q, kv, idx, lse, dtype == SA_BF16, T, H, d_qk, topk, scale,
                                               teacher, s));
}

sa_status sa_indexer_kl_bwd(const void* q_I, const void* k_I, const float* w, const int32_t* idx,
                            const float* teacher, const float* grad, int dtype, int32_t T, int32_t S,
                            int32_t H_I, int32_t D_I, int32_t topk, float* loss, void* dq_I,
                            float* dw, float* dk_I, void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  if (T < 0 || S < 1 || H_I < 1 || D_I < 1 || topk < 1) return SA_ERR_SHAPE;
  if (dtype == SA_BF16 && H_I != 16 && H_I != 32 && H_I != 64) return SA_ERR_UNSUPPORTED;
  if (D_I != 64 && D_I != 128) return SA_ERR_UNSUPPORTED;
  if (topk > sa::indexer_kl_max_topk()) return SA_ERR_UNSUPPORTED;
  if (!dk_I) return SA_ERR_NULL;
  if (T > 0 && (!q_I || !k_I || !w || !idx || !teacher || !loss || !dq_I || !dw)) return SA_ERR_NULL;
  if (!aligned16(q_I) || !aligned16(k_I) || !aligned16(dq_I)) return SA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T > 0) SA_DEBUG_RETURN(debug_range(idx, (int64_t)T * topk, -1, S, s));
  return launch_status(sa::launch_indexer_kl(q_I, k_I, w, idx, teacher, grad, dtype == SA_BF16, T, S, H_I,
                                             D_I, topk, loss, dq_I, dw, dk_I, s));
}

sa_status sa_block_sparse_gqa_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                                  const void* dout, const float* lse, int dtype, int32_t T,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t Dv, int32_t block_size,
                                  int32_t nblk, float scale, void* dq, float* dk, float* dv,
                                  void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_DTYPE;
  int32_t widest = 0;
  sa_status st = check_layout(T, cu_seqlens, num_seqs, max_seqlen, &widest);
  if (st != SA_OK) return st;
  if (Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || block_size < 1 || nblk < 1) return SA_ERR_SHAPE;
  if (Hq % Hkv != 0) return SA_ERR_SHAPE;
  if (Hq / Hkv > 16) return SA_ERR_UNSUPPORTED;
  if (!((D == 128 && Dv == 128) || (D == 64 && Dv == 64))) return SA_ERR_UNSUPPORTED;
  if (block_size % 16 != 0 || block_size > 128) return SA_ERR_UNSUPPORTED;
  if (nblk > sa::block_gqa_max_route()) return SA_ERR_UNSUPPORTED;
  if (!dk || !dv) return SA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !blk || !dout || !lse || !dq)) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return SA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T > 0) SA_DEBUG_RETURN(debug_offsets(cu_seqlens, num_seqs, T, max_seqlen, s));
  return launch_status(sa::launch_block_gqa_bwd(q, k, v, blk, dtype == SA_BF16, T, cu_seqlens, num_seqs,
                                                widest, Hq, Hkv, D, block_size, nblk, scale, dout, lse,
                                                dq, dk, dv, s));
}

sa_status sa_kpool_expand(const int32_t* pools, int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                          int32_t max_seqlen, int32_t kp, int32_t pool, int32_t* out, void* stream) {
  int32_t widest = 0;
  sa_status st = check_layout(T, cu_seqlens, num_seqs, max_seqlen, &widest);
  if (st != SA_OK) return st;
  if (kp < 1 || pool < 1) return SA_ERR_SHAPE;
  if ((int64_t)kp * pool + pool - 1 > INT32_MAX) return SA_ERR_UNSUPPORTED;
  if (T == 0) return SA_OK;
  if (!pools || !out) return SA_ERR_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  SA_DEBUG_RETURN(debug_offsets(cu_seqlens, num_seqs, T, max_seqlen, s));
  return launch_status(sa::launch_kpool_expand(pools, cu_seqlens, num_seqs, T, kp, pool, out, s));
}

sa_status sa_append_window(const int32_t* idx, int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t max_seqlen, int32_t k, int32_t window, int32_t offset, int32_t* out,
                           void* stream) {
  int32_t widest = 0;
  sa_status st = check_layout(T, cu_seqlens, num_seqs, max_seqlen, &widest);
  if (st != SA_OK) return st;
  if (k < 0 || window < 0 || k + window < 1 || offset < 0) return SA_ERR_SHAPE;
  if ((int64_t)offset + T > INT32_MAX) return SA_ERR_UNSUPPORTED;
  if (T == 0) return SA_OK;
  if ((k > 0 && !idx) || !out) return SA_ERR_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  SA_DEBUG_RETURN(debug_offsets(cu_seqlens, num_seqs, T, max_seqlen, s));
  return launch_status(sa::launch_append_window(idx, cu_seqlens, num_seqs, T, k, window, offset, out, s));
}

}  // extern "C"
