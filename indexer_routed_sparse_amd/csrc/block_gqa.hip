// Grouped-query attention over selected key blocks (block-routed sparse GQA).
//
// Operation ("Add trainable QSA sparse attention with a TileLang backend", section
// "Describe the solution you'd like": sparse GQA attention over the blocks picked by
// the exact block TopK): query t attends to every causal key of the blocks listed in
// blk[t, :] (local block ids of its sequence, -1 skipped); head h uses kv head
// h / (Hq / Hkv).
//
// One workgroup per (token, kv head): the group's q rows stay in LDS, each selected
// block's keys and values are staged in LDS as fp32, and an online softmax (running
// max per head, exp2 domain) accumulates the output in registers. fp32 arithmetic
// throughout, no atomics.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNT = 256;

template <bool BF16>
SA_DEVICE float ld_elem(const void* p, int64_t i) {
  if constexpr (BF16) return bf_bits2f(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <bool BF16>
SA_DEVICE void st_elem(void* p, int64_t i, float v) {
  if constexpr (BF16) reinterpret_cast<uint16_t*>(p)[i] = f2bf_bits(v);
  else reinterpret_cast<float*>(p)[i] = v;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kNT) void block_gqa_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int Hq, int Hkv,
    int B, int nblk, float scale_log2, void* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float sm[];
  const int G = Hq / Hkv;                  // q heads per kv head (<= 16)
  float* sq = sm;                          // [G][D]   (pre-scaled q)
  float* sk = sq + 16 * D;                 // [B][D+1]
  float* sv = sk + B * (D + 1);            // [B][D]
  float* sp = sv + B * D;                  // [G][B]   logits, then probabilities
  float* salpha = sp + 16 * B;             // [G]
  float* sl = salpha + 16;                 // [G]      running sums
  float* smx = sl + 16;                    // [G]      running max

  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int start = cu ? seq_start_of(cu, nseq, t) : 0;

  for (int i = tid; i < G * D; i += kNT) {
    const int h = i / D, d = i % D;
    sq[i] = ld_elem<BF16>(q, ((int64_t)t * Hq + g * G + h) * D + d) * scale_log2;
  }
  if (tid < 16) { sl[tid] = 0.0f; smx[tid] = -__builtin_huge_valf(); }
  // each thread owns outputs (h, d) = i, i + kNT, ... of the G*D outputs
  constexpr int kPer = (16 * D + kNT - 1) / kNT;
  float acc[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) acc[r] = 0.0f;
  __syncthreads();

  const int32_t* brow = blk + (int64_t)t * nblk;
#pragma unroll 1
  for (int j = 0; j < nblk; ++j) {
    const int b = brow[j];
    if (b < 0) continue;
    const int lo = start + b * B;
    const int n = min(lo + B - 1, t) - lo + 1;   // causal keys in the block
    if (n <= 0) continue;
    for (int i = tid; i < n * D; i += kNT) {
      const int s = i / D, d = i % D;
      const int64_t row = ((int64_t)(lo + s) * Hkv + g) * D + d;
      sk[s * (D + 1) + d] = ld_elem<BF16>(k, row);
      sv[s * D + d] = ld_elem<BF16>(v, row);
    }
    __syncthreads();
    for (int i = tid; i < G * n; i += kNT) {
      const int h = i / n, s = i % n;
      float a = 0.0f;
      for (int d = 0; d < D; ++d) a = fmaf(sq[h * D + d], sk[s * (D + 1) + d], a);
      sp[h * B + s] = a;
    }
    __syncthreads();
    // per head: new running max, probabilities, rescale factor (one wave per head)
    for (int h = tid >> 6; h < G; h += kNT / 64) {
      const int L = tid & 63;
      float m = -__builtin_huge_valf();
      for (int s = L; s < n; s += 64) m = fmaxf(m, sp[h * B + s]);
      m = wave_max(m);
      const float m_old = smx[h];
      const float m_new = fmaxf(m_old, m);
      float ps = 0.0f;
      for (int s = L; s < n; s += 64) {
        const float p = exp2f(sp[h * B + s] - m_new);
        sp[h * B + s] = p;
        ps += p;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, 64);
      if (L == 0) {
        const float al = exp2f(m_old - m_new);   // 0 on the first block
        salpha[h] = al;
        sl[h] = sl[h] * al + ps;
        smx[h] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + r * kNT;
      if (i < G * D) {
        const int h = i / D, d = i % D;
        float a = acc[r] * salpha[h];
        for (int s = 0; s < n; ++s) a = fmaf(sp[h * B + s], sv[s * D + d], a);
        acc[r] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = tid + r * kNT;
    if (i < G * D) {
      const int h = i / D, d = i % D;
      const float l = sl[h];
      st_elem<BF16>(out, ((int64_t)t * Hq + g * G + h) * D + d, l > 0.0f ? acc[r] / l : 0.0f);
    }
  }
  if (lse && tid < G) {
    const float l = sl[tid];
    lse[(int64_t)t * Hq + g * G + tid] = l > 0.0f ? (smx[tid] + __log2f(l)) * kLn2 : -__builtin_huge_valf();
  }
}

template <bool BF16, int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                    const int32_t* cu, int nseq, int Hq, int Hkv, int B, int nblk, float scale,
                    void* out, float* lse, hipStream_t st) {
  const size_t shm = sizeof(float) * ((size_t)16 * D + (size_t)B * (D + 1) + (size_t)B * D + 16 * (size_t)B + 48);
  hipError_t e = hipFuncSetAttribute((const void*)block_gqa_kernel<BF16, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((block_gqa_kernel<BF16, D>), dim3(T, Hkv), dim3(kNT), shm, st, q, k, v, blk, cu,
                     nseq, Hq, Hkv, B, nblk, scale * kLog2e, out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_gqa(const void* q, const void* k, const void* v, const int32_t* blk,
                            bool bf16, int T, const int32_t* cu, int nseq, int Hq, int Hkv, int D,
                            int Dv, int block_size, int nblk, float scale, void* out, float* lse,
                            hipStream_t st) {
  (void)Dv;
  if (T == 0) return hipSuccess;
  if (bf16) {
    if (D == 64) return launch_d<true, 64>(q, k, v, blk, T, cu, nseq, Hq, Hkv, block_size, nblk, scale, out, lse, st);
    return launch_d<true, 128>(q, k, v, blk, T, cu, nseq, Hq, Hkv, block_size, nblk, scale, out, lse, st);
  }
  if (D == 64) return launch_d<false, 64>(q, k, v, blk, T, cu, nseq, Hq, Hkv, block_size, nblk, scale, out, lse, st);
  return launch_d<false, 128>(q, k, v, blk, T, cu, nseq, Hq, Hkv, block_size, nblk, scale, out, lse, st);
}

}  // namespace sa
