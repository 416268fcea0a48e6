// Allocation-free variant of sa_indexer_scores: the two-pass selection's workspace is
// a static device array of this library instead of caller memory.
//
// `scratch` below is a device symbol. In host code its name stands for a host-side
// shadow, not for device memory, so host code never uses it directly: the device
// address comes from hipGetSymbolAddress, looked up once per device (with that device
// current) on the first call there, and kept per device, since each GPU holds its own
// copy of the array at its own address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/sa.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t sa_noalloc_scratch_bytes(void) { return kScratchBytes; }

sa_status sa_indexer_scores_noalloc(const void* q_I, const void* k_I, const float* w, int dtype,
                                    int32_t T, const int32_t* cu_seqlens, int32_t num_seqs,
                                    int32_t max_seqlen, int32_t H_I, int32_t D_I,
                                    int32_t block_size, float* scores, int64_t ld, int32_t topk,
                                    int32_t force_own_block, int32_t* out_idx, float* out_val,
                                    void* stream) {
  const int32_t widest = cu_seqlens ? max_seqlen : T;
  const size_t need =
      topk > 0 ? sa_indexer_workspace_bytes(dtype, T, widest, H_I, D_I, block_size, topk) : 0;
  if (need > kScratchBytes) return SA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_ptr();
    if (!ws) return SA_ERR_LAUNCH;
  }
  // every part of the workspace that is read was written by the same call first
  return sa_indexer_scores(q_I, k_I, w, dtype, T, cu_seqlens, num_seqs, max_seqlen, H_I, D_I,
                           block_size, scores, ld, topk, force_own_block, out_idx, out_val, ws,
                           need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
