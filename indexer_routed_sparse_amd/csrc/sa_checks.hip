// Device-content checks of the debug build (libsa_debug.so): each entry point of that
// build validates the index values and sequence offsets it is given before its
// launches and returns SA_ERR_SHAPE when one is out of range. The release build
// (libsa.so) never calls these: there, out-of-range contents are undefined behaviour.
// A check waits for its result (it synchronises the caller's stream).
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_kernels.h"

namespace sa {
namespace {

// One flag per device: a device symbol, addressed through hipGetSymbolAddress (its
// name in host code is only a host-side stand-in).
static __device__ int g_bad;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int* g_flag[kMaxDevices] = {};

int* flag_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_flag[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_bad)) != hipSuccess) return nullptr;
    g_flag[dev] = static_cast<int*>(p);
  }
  return g_flag[dev];
}

__global__ void zero_flag_kernel(int* flag) { flag[threadIdx.x] = 0; }   // one thread

// Every value of v[0..n) must lie in [lo, hi).
__global__ void range_kernel(const int32_t* __restrict__ v, int64_t n, int32_t lo, int32_t hi, int* flag) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    bad = bad || v[i] < lo || v[i] >= hi;
  if (bad) atomicOr(flag, 1);
}

// cu[0] = 0, cu[nseq] = T, and 0 <= cu[j+1] - cu[j] <= maxlen.
__global__ void offsets_kernel(const int32_t* __restrict__ cu, int nseq, int T, int maxlen, int* flag) {
  bool bad = false;
  for (int j = (int)threadIdx.x; j < nseq; j += (int)blockDim.x) {
    const int len = cu[j + 1] - cu[j];
    bad = bad || len < 0 || len > maxlen;
  }
  if (threadIdx.x == 0) bad = bad || cu[0] != 0 || cu[nseq] != T;
  if (bad) atomicOr(flag, 1);
}

// Runs `launch(flag)` after clearing the flag and waits for the result.
template <class F>
hipError_t run_check(hipStream_t st, bool* ok, F launch) {
  int* flag = flag_ptr();
  if (!flag) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(1), 0, st, flag);
  launch(flag);
  int host = 0;
  hipError_t e = hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  *ok = e == hipSuccess && host == 0;
  return e;
}

}  // namespace

hipError_t debug_check_range(const int32_t* v, int64_t n, int32_t lo, int32_t hi, hipStream_t st,
                             bool* ok) {
  if (n <= 0) { *ok = true; return hipSuccess; }
  return run_check(st, ok, [&](int* flag) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(range_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st,
                       v, n, lo, hi, flag);
  });
}

hipError_t debug_check_offsets(const int32_t* cu, int nseq, int T, int maxlen, hipStream_t st,
                               bool* ok) {
  return run_check(st, ok, [&](int* flag) {
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(256), 0, st, cu, nseq, T, maxlen, flag);
  });
}

}  // namespace sa
