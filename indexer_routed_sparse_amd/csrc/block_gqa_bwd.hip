// Backward of block-routed sparse GQA: dq, dk and dv from the upstream gradient of the
// output ("Add trainable QSA sparse attention with a TileLang backend", sections "Is
// your feature request related to a problem?" and "Describe the solution you'd
// like": sparse GQA attention forward and backward).
//
// For query t, q head h (kv head g = h / (Hq / Hkv)) and attended key s (the causal
// keys of the routed blocks, each block once):
//   p_s = exp(scale q.k_s - lse), dp_s = dout . v_s, D = sum_s p_s dp_s,
//   ds_s = scale p_s (dp_s - D);
//   dq[t,h] = sum_s ds_s k_s;  dk[s,g] += sum_h ds_s q[t,h];  dv[s,g] += sum_h p_s dout[t,h].
// lse comes from the forward; D is summed from the p_s dp_s (a first pass).
//
// bf16 kernel (gfx950): one wave per (token, kv head), four per workgroup, each with
// its own LDS: the G <= 16 query heads of the group are the 16 rows of 16x16 MFMA tiles
// over 16-key sub-tiles of the route. S = Q K^T and dP = dout V^T take q and dout as A
// operands from registers and the staged key and value rows as B operands; P and dS
// come out with lane (c, n) holding heads 4c..4c+3 of key n, the A-operand layout of
// dS^T and P^T for dk = dS^T Q and dv = P^T dout, whose B operands are transposing LDS
// reads of q and dout; dq^T = K^T dS^T reads K^T transposed and dS^T through a small
// LDS transpose. dk and dv go to fp32 arrays by atomics.
// fp32 inputs use a plain kernel with the same arithmetic.
#include <type_traits>

#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kMaxRoute = 64;
constexpr int kSubMax = kMaxRoute * 8;   // 16-key sub-tiles per route: B <= 128

typedef float floatx4v_t __attribute__((ext_vector_type(4)));

SA_DEVICE floatx4v_t mfma16x32(bf16x8_t a, bf16x8_t b, floatx4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
SA_DEVICE floatx4v_t mfma16x16(short4_t a, short4_t b, floatx4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
SA_DEVICE short4_t pack4(float a, float b, float c, float d) {
  return __builtin_bit_cast(short4_t, make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d)));
}

template <int D>
constexpr int rb() { return D * 2 + 16; }   // padded LDS row bytes
template <int D>
constexpr int wave_lds() { return 4 * 16 * rb<D>() + 16 * 16 * 2 + kSubMax * 8; }

template <int D>
__global__ __launch_bounds__(kWaves * 64) void block_gqa_bwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int T, int Hq, int Hkv,
    int B, int nblk, float scale, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    uint16_t* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int RB = rb<D>();
  constexpr int KS = D / 32;           // k-steps of S and dP
  constexpr int NCB = D / 16;          // channel blocks of dq, dk, dv
  constexpr int CPR = D * 2 / 16;      // 16-byte chunks per row
  constexpr int NLD = 16 * CPR / 64;   // chunks per lane per 16 rows
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
  const int c4 = L >> 4, n = L & 15;
  const int unit = blockIdx.x * kWaves + w;           // (token, kv head)
  if ((int64_t)unit >= (int64_t)T * Hkv) return;      // whole wave; no workgroup barriers
  const int t = unit / Hkv, g = unit - t * Hkv;
  const int G = Hq / Hkv;
  char* q_l = lds + w * wave_lds<D>();                // [16 heads][RB]
  char* d_l = q_l + 16 * RB;                          // [16 heads][RB] dout
  char* k_l = d_l + 16 * RB;                          // [16 keys][RB]
  char* v_l = k_l + 16 * RB;                          // [16 keys][RB]
  char* s_l = v_l + 16 * RB;                          // [16 heads][16 keys] bf16
  int2* list = reinterpret_cast<int2*>(s_l + 16 * 16 * 2);
  const int c = cu ? seq_start_of(cu, nseq, t) : 0;
  const int own = (t - c) / B;

  // ---- route -> 16-key sub-tiles (s0, nkeys) in slot order; repeats skipped
  int nsub = 0;
  for (int base = 0; base < nblk; base += 64) {
    const int j = base + L;
    const int b = j < nblk ? blk[(int64_t)t * nblk + j] : -1;
    bool ok = b >= 0 && b <= own;
    for (int i = 0; i < nblk; ++i) {
      if (i >= j) break;
      ok = ok && blk[(int64_t)t * nblk + i] != b;
    }
    const int lo = c + b * B;
    const int nk = ok ? min(B, t - lo + 1) : 0;
    const int ns = (nk + 15) >> 4;
    const uint32_t incl = wave_incl_scan((uint32_t)ns);
    const int pos = nsub + (int)incl - ns;
    for (int h = 0; h < ns; ++h) list[pos + h] = make_int2(lo + 16 * h, min(16, nk - 16 * h));
    nsub += __shfl((int)incl, 63, 64);
  }
  // ---- q and dout of the group into LDS, zeros past G
  for (int e = L; e < 16 * CPR; e += 64) {
    const int hh = e / CPR, p = e % CPR;
    bf16x8_t a = bf16x8_t{}, b2 = bf16x8_t{};
    if (hh < G) {
      const int64_t off = ((int64_t)t * Hq + g * G + hh) * D + 8 * p;
      a = *reinterpret_cast<const bf16x8_t*>(q + off);
      b2 = *reinterpret_cast<const bf16x8_t*>(dout + off);
    }
    *reinterpret_cast<bf16x8_t*>(q_l + hh * RB + 16 * p) = a;
    *reinterpret_cast<bf16x8_t*>(d_l + hh * RB + 16 * p) = b2;
  }
  __builtin_amdgcn_wave_barrier();
  bf16x8_t qa[KS], ga[KS];                  // A operands: head n, dims 32 ks + 8 c4
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qa[ks] = *reinterpret_cast<const bf16x8_t*>(q_l + n * RB + 64 * ks + 16 * c4);
    ga[ks] = *reinterpret_cast<const bf16x8_t*>(d_l + n * RB + 64 * ks + 16 * c4);
  }
  float lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * c4 + i;
    lse2[i] = hh < G ? lse[(int64_t)t * Hq + g * G + hh] * kLog2e : -__builtin_huge_valf();
  }
  const float sc2 = scale * kLog2e;

  bf16x8_t nk_[NLD], nv_[NLD];
  auto load = [&](int i) __attribute__((always_inline)) {
    const int2 e = list[i];
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int cc = L + 64 * m, r = cc / CPR, p = cc % CPR;
      const int key = r < e.y ? e.x + r : e.x;
      const int64_t off = ((int64_t)key * Hkv + g) * D + 8 * p;
      nk_[m] = *reinterpret_cast<const bf16x8_t*>(k + off);
      nv_[m] = *reinterpret_cast<const bf16x8_t*>(v + off);
    }
  };
  auto stage = [&](int next) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int cc = L + 64 * m, r = cc / CPR, p = cc % CPR;
      *reinterpret_cast<bf16x8_t*>(k_l + r * RB + 16 * p) = nk_[m];
      *reinterpret_cast<bf16x8_t*>(v_l + r * RB + 16 * p) = nv_[m];
    }
    __builtin_amdgcn_wave_barrier();
    if (next < nsub) load(next);
  };
  auto scores = [&](int i, float (&P)[4], floatx4v_t& dP) __attribute__((always_inline)) {
    const bool ok = n < list[i].y;
    floatx4v_t S = floatx4v_t{};
    dP = floatx4v_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      S = mfma16x32(qa[ks], *reinterpret_cast<const bf16x8_t*>(k_l + n * RB + 64 * ks + 16 * c4), S);
      dP = mfma16x32(ga[ks], *reinterpret_cast<const bf16x8_t*>(v_l + n * RB + 64 * ks + 16 * c4), dP);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      P[e] = ok && lse2[e] > -__builtin_huge_valf() ? __builtin_amdgcn_exp2f(S[e] * sc2 - lse2[e]) : 0.0f;
  };

  // ---- pass 1: D per head
  float dpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (nsub > 0) load(0);
#pragma unroll 1
  for (int i = 0; i < nsub; ++i) {
    stage(i + 1);
    float P[4];
    floatx4v_t dP;
    scores(i, P, dP);
#pragma unroll
    for (int e = 0; e < 4; ++e) dpart[e] = fmaf(P[e], dP[e], dpart[e]);
    __builtin_amdgcn_wave_barrier();
  }
  float Dh[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) dpart[e] += __shfl_xor(dpart[e], off, 64);
    Dh[e] = dpart[e];
  }

  // ---- pass 2
  floatx4v_t acc[NCB];                      // dq^T: channels 16 cb + 4 c4 .. +3, head n
#pragma unroll
  for (int i = 0; i < NCB; ++i) acc[i] = floatx4v_t{};
  if (nsub > 0) load(0);
#pragma unroll 1
  for (int i = 0; i < nsub; ++i) {
    stage(i + 1);
    float P[4], dS[4];
    floatx4v_t dP;
    scores(i, P, dP);
#pragma unroll
    for (int e = 0; e < 4; ++e) dS[e] = P[e] * (dP[e] - Dh[e]) * scale;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<uint16_t*>(s_l + ((4 * c4 + e) * 16 + n) * 2) = f2bf_bits(dS[e]);
    const short4_t dsA = pack4(dS[0], dS[1], dS[2], dS[3]);
    const short4_t pA = pack4(P[0], P[1], P[2], P[3]);
    __builtin_amdgcn_wave_barrier();
    const short4_t dsB = *reinterpret_cast<const short4_t*>(s_l + (n * 16 + 4 * c4) * 2);
    const int2 e = list[i];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int toff = (16 * cb + 4 * (n & 3)) * 2;
      const int trow = 4 * c4 + (n >> 2);
      const short4_t kT = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(k_l + trow * RB + toff));
      acc[cb] = mfma16x16(kT, dsB, acc[cb]);
      const short4_t qB = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(q_l + trow * RB + toff));
      const short4_t gB = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(d_l + trow * RB + toff));
      const floatx4v_t dkt = mfma16x16(dsA, qB, floatx4v_t{});
      const floatx4v_t dvt = mfma16x16(pA, gB, floatx4v_t{});
      // lane (c4, n): keys 4c4..4c4+3, channel 16 cb + n
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = 4 * c4 + r;
        if (kr < e.y) {
          const int64_t off = ((int64_t)(e.x + kr) * Hkv + g) * D + 16 * cb + n;
          atomicAdd(dk + off, dkt[r]);
          atomicAdd(dv + off, dvt[r]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // ---- dq: lane (c4, n) holds channels 16 cb + 4 c4 .. +3 of head n
  if (n < G) {
    uint16_t* orow = dq + ((int64_t)t * Hq + g * G + n) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<uint2*>(orow + 16 * cb + 4 * c4) =
          make_uint2(pack_bf16x2(acc[cb][0], acc[cb][1]), pack_bf16x2(acc[cb][2], acc[cb][3]));
  }
}

// fp32: one workgroup per (token, q head) over the deduplicated route.
constexpr int kNT = 256;

template <int D>
__global__ __launch_bounds__(kNT) void block_gqa_bwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int Hq, int Hkv,
    int B, int nblk, float scale, const float* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv) {
  extern __shared__ float sm[];            // [keys] p, [keys] dp, [keys] key id, [4] reduce
  const int t = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int G = Hq / Hkv, g = h / G;
  const int c = cu ? seq_start_of(cu, nseq, t) : 0;
  const int own = (t - c) / B;
  const int cap = nblk * B;
  float* sp = sm;
  float* sdp = sp + cap;
  int* skey = reinterpret_cast<int*>(sdp + cap);
  float* red = reinterpret_cast<float*>(skey + cap);
  const float* qr = q + ((int64_t)t * Hq + h) * D;
  const float* gr = dout + ((int64_t)t * Hq + h) * D;
  const float l = lse[(int64_t)t * Hq + h];
  const int32_t* brow = blk + (int64_t)t * nblk;
  // key list of the route (slot order, repeats skipped), then p and dp per key
  int nkeys = 0;
  for (int j = 0; j < nblk; ++j) {
    const int b = brow[j];
    bool ok = b >= 0 && b <= own;
    for (int i = 0; i < j; ++i) ok = ok && brow[i] != b;
    if (!ok) continue;
    const int lo = c + b * B, nk = min(B, t - lo + 1);
    for (int r = tid; r < nk; r += kNT) skey[nkeys + r] = lo + r;
    nkeys += nk;
  }
  __syncthreads();
  float part = 0.0f;
  for (int i = tid; i < nkeys; i += kNT) {
    const int64_t off = ((int64_t)skey[i] * Hkv + g) * D;
    float s = 0.0f, dp = 0.0f;
    for (int d = 0; d < D; ++d) { s = fmaf(qr[d], k[off + d], s); dp = fmaf(gr[d], v[off + d], dp); }
    const float p = l > -__builtin_huge_valf() ? expf(s * scale - l) : 0.0f;
    sp[i] = p;
    sdp[i] = dp;
    part = fmaf(p, dp, part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if (L == 0) red[w] = part;
  __syncthreads();
  float Dv = 0.0f;
  for (int i = 0; i < kNT / 64; ++i) Dv += red[i];
  for (int i = tid; i < nkeys; i += kNT) {
    const float p = sp[i];
    const float ds = scale * p * (sdp[i] - Dv);
    const int64_t off = ((int64_t)skey[i] * Hkv + g) * D;
    for (int d = 0; d < D; ++d) {
      atomicAdd(dk + off + d, ds * qr[d]);
      atomicAdd(dv + off + d, p * gr[d]);
    }
    sdp[i] = ds;
  }
  __syncthreads();
  for (int d = tid; d < D; d += kNT) {
    float a = 0.0f;
    for (int i = 0; i < nkeys; ++i) a = fmaf(sdp[i], k[((int64_t)skey[i] * Hkv + g) * D + d], a);
    dq[((int64_t)t * Hq + h) * D + d] = a;
  }
}

__global__ void zero2_f32_kernel(float* __restrict__ a, float* __restrict__ b, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    a[i] = 0.0f;
    b[i] = 0.0f;
  }
}

template <int D>
hipError_t launch_bf16(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                       const int32_t* cu, int nseq, int Hq, int Hkv, int B, int nblk, float scale,
                       const void* dout, const float* lse, void* dq, float* dk, float* dv, hipStream_t st) {
  const size_t shm = (size_t)kWaves * wave_lds<D>();
  hipError_t e = hipFuncSetAttribute((const void*)block_gqa_bwd_bf16_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  const int64_t grid = ((int64_t)T * Hkv + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((block_gqa_bwd_bf16_kernel<D>), dim3((unsigned)grid), dim3(kWaves * 64), shm, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, blk, cu, nseq, T, Hq,
                     Hkv, B, nblk, scale, (const uint16_t*)dout, lse, (uint16_t*)dq, dk, dv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                      const int32_t* cu, int nseq, int Hq, int Hkv, int B, int nblk, float scale,
                      const void* dout, const float* lse, void* dq, float* dk, float* dv, hipStream_t st) {
  const size_t shm = (size_t)nblk * B * 12 + 16;
  hipError_t e = hipFuncSetAttribute((const void*)block_gqa_bwd_f32_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((block_gqa_bwd_f32_kernel<D>), dim3(T, Hq), dim3(kNT), shm, st, (const float*)q,
                     (const float*)k, (const float*)v, blk, cu, nseq, Hq, Hkv, B, nblk, scale,
                     (const float*)dout, lse, (float*)dq, dk, dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_gqa_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                                bool bf16, int T, const int32_t* cu, int nseq, int Hq, int Hkv, int D,
                                int block_size, int nblk, float scale, const void* dout,
                                const float* lse, void* dq, float* dk, float* dv, hipStream_t st) {
  hipLaunchKernelGGL(zero2_f32_kernel, dim3(1024), dim3(256), 0, st, dk, dv, (int64_t)T * Hkv * D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  const int ns = cu ? nseq : 1;
  if (bf16) {
    if (D == 64) return launch_bf16<64>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
    return launch_bf16<128>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
  }
  if (D == 64) return launch_f32<64>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
  return launch_f32<128>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
}

}  // namespace sa
