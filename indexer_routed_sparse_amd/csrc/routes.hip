// Route builders of the attention variants: k-pool expansion with the query's
// incomplete tail pool ("Support NoPE shapes and unaligned top-k in TileLang sparse
// MLA", quoted GLM PR body, section "Why": k-pool selection appends the query's
// incomplete tail pool, top-k width 2048 + 3) and a causal window of raw keys after the
// selected slots ("Add fused SBHD compressed sparse attention", section "Scope":
// compressed + window + sink). Integer work, one thread per output slot.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

// out [T, kp*P + P - 1]: slot i*P + r holds start + c*P + r for pool c = pools[t, i]
// (-1 for a -1 pool); the last P - 1 slots hold the incomplete own pool's keys.
__global__ void kpool_expand_kernel(const int32_t* __restrict__ pools, const int32_t* __restrict__ cu,
                                    int nseq, int T, int kp, int P, int32_t* __restrict__ out) {
  const int width = kp * P + P - 1;
  const int64_t n = (int64_t)T * width;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / width), j = (int)(e % width);
    const int s0 = cu ? seq_start_of(cu, nseq, t) : 0;
    int v = -1;
    if (j < kp * P) {
      const int c = pools[(int64_t)t * kp + j / P];
      if (c >= 0) v = s0 + c * P + j % P;
    } else {
      const int o = t - s0, r = j - kp * P;          // tail slot r
      if (o % P != P - 1 && r <= o % P) v = s0 + (o / P) * P + r;
    }
    out[e] = v;
  }
}

// out [T, k + W]: the k selected slots, then offset + s for the keys s = t - W + 1 .. t
// of the row's sequence (-1 before its start).
__global__ void append_window_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cu,
                                     int nseq, int T, int k, int W, int offset, int32_t* __restrict__ out) {
  const int width = k + W;
  const int64_t n = (int64_t)T * width;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / width), j = (int)(e % width);
    int v;
    if (j < k) {
      v = idx[(int64_t)t * k + j];
    } else {
      const int s0 = cu ? seq_start_of(cu, nseq, t) : 0;
      const int s = t - W + 1 + (j - k);
      v = s >= s0 ? offset + s : -1;
    }
    out[e] = v;
  }
}

int grid_for(int64_t n) { return (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096); }

}  // namespace

hipError_t launch_kpool_expand(const int32_t* pools, const int32_t* cu, int nseq, int T, int kp, int P,
                               int32_t* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(kpool_expand_kernel, dim3(grid_for((int64_t)T * (kp * P + P - 1))), dim3(256), 0, st,
                     pools, cu, cu ? nseq : 1, T, kp, P, out);
  return hipGetLastError();
}

hipError_t launch_append_window(const int32_t* idx, const int32_t* cu, int nseq, int T, int k, int W,
                                int offset, int32_t* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(append_window_kernel, dim3(grid_for((int64_t)T * (k + W))), dim3(256), 0, st, idx, cu,
                     cu ? nseq : 1, T, k, W, offset, out);
  return hipGetLastError();
}

}  // namespace sa
