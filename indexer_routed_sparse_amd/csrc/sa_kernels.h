// Internal launch functions of the HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// topk_select.hip
int topk_select_max_width();
hipError_t launch_topk_select(const float* vals, const int32_t* cand, int64_t ld, int T,
                              const int32_t* cu, int nseq, int width, int block_size, int topk,
                              int force_own, int32_t* out_idx, float* out_val, hipStream_t st);
// Candidate rows [T, ld] whose first cnt[t] entries are valid (ascending ids); rows
// with cnt[t] < 0 are skipped and their outputs left untouched.
hipError_t launch_topk_select_counted(const float* vals, const int32_t* cand, const int32_t* cnt,
                                      int64_t ld, int T, int topk, int32_t* out_idx,
                                      float* out_val, hipStream_t st);

// sparse_mla.hip
// Whether the bf16 kernel's LDS (gather stages, q slices, P exchange, index row)
// fits one workgroup for this head count, width and top-k.
bool sparse_mla_bf16_fits(int H, int d_qk, int topk);
hipError_t launch_sparse_mla(const void* q, const void* kv, const int32_t* idx, bool bf16, int T,
                             int S, int H, int d_qk, int d_v, int topk, float scale, const float* sink,
                             void* out, float* lse, hipStream_t st);

// sparse_mla_bwd.hip: zeroes dkv [S, d_qk] (fp32), then accumulates into it.
hipError_t launch_sparse_mla_bwd(const void* q, const void* kv, const int32_t* idx, const void* dout,
                                 const float* lse, bool bf16, int T, int S, int H, int d_qk, int d_v,
                                 int topk, float scale, const float* sink, void* dq, float* dkv,
                                 float* dsink, hipStream_t st);

// indexer.hip
hipError_t launch_indexer_dense(const void* q, const void* k, const float* w, bool bf16, int T,
                                const int32_t* cu, int nseq, int maxlen, int H_I, int D_I,
                                int block_size, float* scores, int64_t ld, hipStream_t st);
// Workspace bytes of a fused selection (0 when the launch runs in one pass), and
// whether the launch takes the two-pass route when given a workspace.
size_t indexer_ws_bytes(bool bf16, int T, int maxlen, int H_I, int block_size, int topk);
bool indexer_two_pass(bool bf16, int H_I, int block_size, int topk);
hipError_t launch_indexer_topk(const void* q, const void* k, const float* w, bool bf16, int T,
                               const int32_t* cu, int nseq, int maxlen, int H_I, int D_I,
                               int block_size, int topk, int force_own, int32_t* out_idx,
                               float* out_val, void* ws, hipStream_t st);

// block_gqa.hip
// Largest route (blocks per query row) the bf16 kernel takes.
int block_gqa_max_route();
hipError_t launch_block_gqa(const void* q, const void* k, const void* v, const int32_t* blk,
                            bool bf16, int T, const int32_t* cu, int nseq, int maxlen, int Hq, int Hkv,
                            int D, int Dv, int block_size, int nblk, float scale, void* out, float* lse,
                            hipStream_t st);

// sa_checks.hip (called by the debug build's entry points only): whether every value
// of v[0..n) lies in [lo, hi); whether cu_seqlens is a valid offset array for T rows
// with sequences of at most maxlen rows. Both synchronise `st`.
hipError_t debug_check_range(const int32_t* v, int64_t n, int32_t lo, int32_t hi, hipStream_t st,
                             bool* ok);
hipError_t debug_check_offsets(const int32_t* cu, int nseq, int T, int maxlen, hipStream_t st,
                               bool* ok);

// sparse_mla_bwd.hip: teacher [T, topk] of the sparse KL loss (zeroed, then accumulated).
hipError_t launch_attn_teacher(const void* q, const void* kv, const int32_t* idx, const float* lse,
                               bool bf16, int T, int H, int d_qk, int topk, float scale, float* teacher,
                               hipStream_t st);

// indexer_kl.hip: sparse KL loss of the indexer and its gradients (dk zeroed first).
int indexer_kl_max_topk();
hipError_t launch_indexer_kl(const void* qI, const void* kI, const float* wI, const int32_t* idx,
                             const float* teacher, const float* grad, bool bf16, int T, int S, int H_I,
                             int D_I, int topk, float* loss, void* dq, float* dw, float* dk,
                             hipStream_t st);

// routes.hip: k-pool expansion with the incomplete tail pool; selected slots + window.
hipError_t launch_kpool_expand(const int32_t* pools, const int32_t* cu, int nseq, int T, int kp, int P,
                               int32_t* out, hipStream_t st);
hipError_t launch_append_window(const int32_t* idx, const int32_t* cu, int nseq, int T, int k, int W,
                                int offset, int32_t* out, hipStream_t st);

// block_gqa_bwd.hip: zeroes dk and dv [T, Hkv, D] (fp32), then accumulates into them.
hipError_t launch_block_gqa_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                                bool bf16, int T, const int32_t* cu, int nseq, int maxlen, int Hq,
                                int Hkv, int D, int block_size, int nblk, float scale,
                                const void* dout, const float* lse, void* dq, float* dk, float* dv,
                                hipStream_t st);

}  // namespace sa
