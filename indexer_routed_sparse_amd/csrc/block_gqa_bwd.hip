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
#include "gqa_group.h"
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

// Grouped bf16 backward: one workgroup per (group of GT consecutive tokens, kv head),
// eight waves, over the distinct blocks of the group's routes (gqa_group.h) in 32-key
// sub-tiles staged in LDS, twice: pass 1 forms D = sum p dp of every query row, pass
// 2 forms dS, dq (per row, in registers) and the sub-tile's dk and dv over all of the
// group's rows, added to dk and dv with one atomic per element and sub-tile instead
// of one per element and token. Wave w owns rows 16w .. 16w+15 (token row / G, head
// row mod G):
//   * S^T = K Q^T and dP^T = V dout^T on 16x16x32 MFMAs: key and value rows from
//     padded stages as A operands, the row's q and dout as B operands in registers;
//     lane (n, quad) holds keys 4 quad + e and 16 + 4 quad + e of row n;
//   * dq^T += K^T dS^T: K^T by transposing reads of a swizzled copy of the key rows,
//     dS^T as it stands in registers;
//   * dS and P (bf16) meet in LDS as [key][row]; wave w then takes its share of the
//     output tiles (16 keys x 16 channels) of dk = dS^T Q and dv = P^T dout over all
//     128 rows, with the group's q and dout rows in LDS read transposed.
template <int D>
constexpr int gb_stage_bytes() { return 32 * (D * 2 + 16) * 2 + 32 * D * 2; }   // K pad, V pad, K swz
constexpr int kXRB = kGrpRows * 2 + 16;                                           // [key][row] bf16 rows

size_t grp_bwd_lds_bytes(int D, int G, int nblk, int maxlen) {
  const size_t rows = (size_t)kGrpRows * D * 2 * 2;                    // q and dout rows
  const size_t st = D == 128 ? gb_stage_bytes<128>() : gb_stage_bytes<64>();
  return rows + 2 * st + 2 * 32 * (size_t)kXRB + grp_table_bytes(grp_tokens(G), nblk, maxlen);
}

template <int D>
SA_DEVICE int gswz(int row) { return D == 128 ? 2 * (row & 7) : 2 * (row & 3); }

template <int D>
__global__ __launch_bounds__(kGrpWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void block_gqa_bwd_group_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int T, int Hq, int Hkv,
    int B, int nblk, int GT, int nwords, float scale, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, uint16_t* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, int by_xcd) {
  constexpr int KS = D / 32;              // 32-wide k-steps of S^T and dP^T
  constexpr int NDT = D / 16;             // 16-channel tiles
  constexpr int CPR = D * 2 / 16;         // 16-byte chunks per row
  constexpr int KSB = D * 2 + 16;         // padded stage row bytes
  constexpr int RWB = D * 2;              // swizzled row bytes
  constexpr int NT = kGrpWaves * 64;
  constexpr int LDN = (2 * 32 * CPR + NT - 1) / NT;   // 16-byte loads per thread per sub-tile
  constexpr int NTILE = 2 * 2 * NDT;      // output tiles of dk and dv per sub-tile
  constexpr int TPW = NTILE / kGrpWaves;  // ... per wave
  static_assert(NTILE % kGrpWaves == 0, "tiles split evenly");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* q_l = lds;                                          // [128 rows][RWB] swizzled
  char* d_l = q_l + kGrpRows * RWB;                         // [128 rows][RWB] dout
  char* stg = d_l + kGrpRows * RWB;                         // [2][K pad | V pad | K swz]
  char* xs = stg + 2 * gb_stage_bytes<D>();                 // [dS | P][32 keys][kXRB]
  const GroupTables tbl = group_tables(xs + 2 * 32 * kXRB, GT, nblk, nwords);

  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int n = L & 15, quad = L >> 4;
  const int G = Hq / Hkv;
  const int ngrp = (T + GT - 1) / GT;
  int grp, g;
  if (by_xcd) {
    const int b = blockIdx.x, xcd = b & 7, nx = 8 / Hkv;
    g = xcd % Hkv;
    grp = (b >> 3) * nx + xcd / Hkv;
    if (grp >= ngrp) return;                             // whole workgroup leaves together
  } else {
    grp = (int)blockIdx.x / Hkv;
    g = (int)blockIdx.x - grp * Hkv;
  }
  grp = ngrp - 1 - grp;
  const int t0 = grp * GT;
  const int tlast = min(t0 + GT, T) - 1;
  const int base = cu ? seq_start_of(cu, nseq, t0) : 0;
  const int nrows = GT * G;

  // ---- the group's q and dout rows (zeros for rows past the group) into LDS
  for (int c = tid; c < kGrpRows * CPR; c += NT) {
    const int r = c / CPR, p = c % CPR;
    const int tau = r / G, h = r - tau * G;
    bf16x8_t a = bf16x8_t{}, b2 = bf16x8_t{};
    if (r < nrows && t0 + tau <= tlast) {
      const int64_t off = ((int64_t)(t0 + tau) * Hq + g * G + h) * D + 8 * p;
      a = *reinterpret_cast<const bf16x8_t*>(q + off);
      b2 = *reinterpret_cast<const bf16x8_t*>(dout + off);
    }
    const int so = r * RWB + ((p ^ gswz<D>(r)) << 4);
    *reinterpret_cast<bf16x8_t*>(q_l + so) = a;
    *reinterpret_cast<bf16x8_t*>(d_l + so) = b2;
  }
  const int nu = group_union<NT>(tbl, blk, cu, nseq, t0, tlast, GT, B, nblk, base, nwords);
  const int32_t* ulo = tbl.ulo;
  const uint32_t* umask = tbl.umask;

  // ---- this lane's row
  const int row = 16 * w + n;
  const int tau = row / G;
  const int tq = t0 + tau;
  const bool row_ok = row < nrows && tq <= tlast;
  const int hq = row - tau * G;
  bf16x8_t qb[KS], gb[KS];
  {
    const int64_t off = ((int64_t)(row_ok ? tq : t0) * Hq + g * G + hq) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(q + off + 32 * ks);
      const bf16x8_t y = *reinterpret_cast<const bf16x8_t*>(dout + off + 32 * ks);
      qb[ks] = row_ok ? x : bf16x8_t{};
      gb[ks] = row_ok ? y : bf16x8_t{};
    }
  }
  const float lse2 = row_ok ? lse[(int64_t)tq * Hq + g * G + hq] * kLog2e : -__builtin_huge_valf();
  const float sc2 = scale * kLog2e;
  uint32_t tile_tok = row_ok ? (1u << tau) : 0u;           // tokens of the wave's rows (uniform)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) tile_tok |= (uint32_t)__shfl_xor((int)tile_tok, off, 64);

  auto keys_of = [&](int u) { return min(B, tlast + 1 - ulo[u]); };
  auto advance = [&](int& uu, int& pp) __attribute__((always_inline)) {
    if (uu < nu) {
      ++pp;
      if (32 * pp >= keys_of(uu)) { ++uu; pp = 0; }
    }
  };
  auto loadTo = [&](bf16x8_t (&dst)[LDN], int uu, int pp) __attribute__((always_inline)) {
    const int lo = ulo[uu] + 32 * pp;
    const int nk = min(32, keys_of(uu) - 32 * pp);
#pragma unroll
    for (int m = 0; m < LDN; ++m) {
      const int c = tid + NT * m;                  // chunk: [K | V][row][CPR]
      const int isv = c >= 32 * CPR;
      const int cc = isv ? c - 32 * CPR : c;
      const int r = cc / CPR, p = cc % CPR;
      const int key = lo + (r < nk ? r : 0);
      const uint16_t* src = (isv ? v : k) + ((int64_t)key * Hkv + g) * D + 8 * p;
      dst[m] = (c < 2 * 32 * CPR) ? *reinterpret_cast<const bf16x8_t*>(src) : bf16x8_t{};
    }
  };
  auto storeFrom = [&](char* st, const bf16x8_t (&src)[LDN]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < LDN; ++m) {
      const int c = tid + NT * m;
      if (c < 2 * 32 * CPR) {
        const int isv = c >= 32 * CPR;
        const int cc = isv ? c - 32 * CPR : c;
        const int r = cc / CPR, p = cc % CPR;
        if (!isv) {
          *reinterpret_cast<bf16x8_t*>(st + r * KSB + 16 * p) = src[m];
          *reinterpret_cast<bf16x8_t*>(st + 64 * KSB + r * RWB + ((p ^ gswz<D>(r)) << 4)) = src[m];
        } else {
          *reinterpret_cast<bf16x8_t*>(st + 32 * KSB + r * KSB + 16 * p) = src[m];
        }
      }
    }
  };
  // S^T and dP^T of this wave's rows over the staged sub-tile; P (masked) and dP
  auto scores = [&](const char* st, int lo, int nk, uint32_t msk, float (&P)[8], float (&dPv)[8])
      __attribute__((always_inline)) {
    floatx4v_t S[2] = {floatx4v_t{}, floatx4v_t{}}, dP[2] = {floatx4v_t{}, floatx4v_t{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(st + (16 * kt + n) * KSB + 64 * ks + 16 * quad);
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(st + 32 * KSB + (16 * kt + n) * KSB + 64 * ks + 16 * quad);
        S[kt] = mfma16x32(ka, qb[ks], S[kt]);
        dP[kt] = mfma16x32(va, gb[ks], dP[kt]);
      }
    const bool in = row_ok && ((msk >> tau) & 1u) && lse2 > -__builtin_huge_valf();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 16 * kt + 4 * quad + e;
        const bool ok = in && kk < nk && lo + kk <= tq;
        P[4 * kt + e] = ok ? __builtin_amdgcn_exp2f(S[kt][e] * sc2 - lse2) : 0.0f;
        dPv[4 * kt + e] = dP[kt][e];
      }
  };

  // ---- pass 1: D = sum_s p_s dp_s of every row
  float dpart = 0.0f;
  {
    bf16x8_t nxA[LDN], nxB[LDN];
    int u = 0, pc = 0, ua = 0, pa = 0;
    advance(ua, pa);
    if (nu > 0) loadTo(nxA, 0, 0);
    if (ua < nu) loadTo(nxB, ua, pa);
    auto piece = [&](char* st, bf16x8_t (&buf)[LDN]) __attribute__((always_inline)) {
      storeFrom(st, buf);
      __syncthreads();
      int ub = ua, pb = pa;
      advance(ub, pb);
      if (ub < nu) loadTo(buf, ub, pb);
      const uint32_t msk = umask[u];
      if (msk & tile_tok) {                                   // uniform
        float P[8], dPv[8];
        scores(st, ulo[u] + 32 * pc, min(32, keys_of(u) - 32 * pc), msk, P, dPv);
#pragma unroll
        for (int i = 0; i < 8; ++i) dpart = fmaf(P[i], dPv[i], dpart);
      }
      u = ua; pc = pa; ua = ub; pa = pb;
    };
#pragma unroll 1
    while (u < nu) {
      piece(stg, nxA);
      if (u < nu) piece(stg + gb_stage_bytes<D>(), nxB);
    }
  }
  const float Drow = quad_sum(dpart);

  // ---- pass 2: dS, dq, dk, dv
  floatx4v_t dqa[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) dqa[i] = floatx4v_t{};
  char* xds = xs;
  char* xp = xs + 32 * kXRB;
  {
    bf16x8_t nxA[LDN], nxB[LDN];
    int u = 0, pc = 0, ua = 0, pa = 0;
    advance(ua, pa);
    __syncthreads();                                          // pass 1's stages are free
    if (nu > 0) loadTo(nxA, 0, 0);
    if (ua < nu) loadTo(nxB, ua, pa);
    auto piece = [&](char* st, bf16x8_t (&buf)[LDN]) __attribute__((always_inline)) {
      storeFrom(st, buf);
      __syncthreads();
      int ub = ua, pb = pa;
      advance(ub, pb);
      if (ub < nu) loadTo(buf, ub, pb);
      const int lo = ulo[u] + 32 * pc;
      const int nk = min(32, keys_of(u) - 32 * pc);
      const uint32_t msk = umask[u];
      float P[8], dS[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) { P[i] = 0.0f; dS[i] = 0.0f; }
      if (msk & tile_tok) {                                   // uniform
        float dPv[8];
        scores(st, lo, nk, msk, P, dPv);
#pragma unroll
        for (int i = 0; i < 8; ++i) dS[i] = P[i] * (dPv[i] - Drow) * scale;
        // dq^T += K^T dS^T; dS^T's B operand: k slots 0..3 = keys 4 quad + e, 4..7 = 16 + 4 quad + e
        bf16x2_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = __builtin_convertvector((float2_t){dS[2 * e], dS[2 * e + 1]}, bf16x2_t);
        const bf16x8_t dsb = __builtin_bit_cast(bf16x8_t, pk);
        const char* kswz = st + 64 * KSB;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int row0 = 4 * quad + (n >> 2);
          const int col = 16 * dt + 4 * (n & 3);
          const int off0 = row0 * RWB + (((col >> 3) ^ gswz<D>(row0)) << 4) + (col & 7) * 2;
          const int row1 = row0 + 16;
          const int off1 = row1 * RWB + (((col >> 3) ^ gswz<D>(row1)) << 4) + (col & 7) * 2;
          const short4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kswz + off0));
          const short4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kswz + off1));
          const short __attribute__((ext_vector_type(8))) a8 = {lo4[0], lo4[1], lo4[2], lo4[3],
                                                                hi4[0], hi4[1], hi4[2], hi4[3]};
          dqa[dt] = mfma16x32(__builtin_bit_cast(bf16x8_t, a8), dsb, dqa[dt]);
        }
      }
      // dS and P of this wave's rows -> [key][row] (zeros when the wave skipped)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kt + 4 * quad + e;
          *reinterpret_cast<uint16_t*>(xds + key * kXRB + row * 2) = f2bf_bits(dS[4 * kt + e]);
          *reinterpret_cast<uint16_t*>(xp + key * kXRB + row * 2) = f2bf_bits(P[4 * kt + e]);
        }
      __syncthreads();
      // dk = dS^T Q and dv = P^T dout over the 128 rows: tile (which, key tile, channel tile)
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tt = w * TPW + i;
        const int which = tt / (2 * NDT);                     // 0: dk, 1: dv
        const int ktile = (tt / NDT) & 1, dtile = tt % NDT;
        const char* xa = which ? xp : xds;
        const char* rb = which ? d_l : q_l;
        floatx4v_t acc = floatx4v_t{};
#pragma unroll
        for (int ks = 0; ks < kGrpRows / 32; ++ks) {
          // A: key 16 ktile + n, rows 32 ks + 4 quad + e and 32 ks + 16 + 4 quad + e
          const char* ar = xa + (16 * ktile + n) * kXRB + (32 * ks + 4 * quad) * 2;
          const uint2 alo = *reinterpret_cast<const uint2*>(ar);
          const uint2 ahi = *reinterpret_cast<const uint2*>(ar + 32);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(alo.x, alo.y, ahi.x, ahi.y));
          // B: the same rows, channel 16 dtile + n, by transposing reads
          const int r0 = 32 * ks + 4 * quad + (n >> 2);
          const int col = 16 * dtile + 4 * (n & 3);
          const int o0 = r0 * RWB + (((col >> 3) ^ gswz<D>(r0)) << 4) + (col & 7) * 2;
          const int r1 = r0 + 16;
          const int o1 = r1 * RWB + (((col >> 3) ^ gswz<D>(r1)) << 4) + (col & 7) * 2;
          const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(rb + o0));
          const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(rb + o1));
          const short __attribute__((ext_vector_type(8))) b8 = {b0[0], b0[1], b0[2], b0[3],
                                                                b1[0], b1[1], b1[2], b1[3]};
          acc = mfma16x32(a, __builtin_bit_cast(bf16x8_t, b8), acc);
        }
        // lane (quad, n): keys 16 ktile + 4 quad + e, channel 16 dtile + n
        float* dst = which ? dv : dk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 16 * ktile + 4 * quad + e;
          if (kk < nk) atomicAdd(dst + ((int64_t)(lo + kk) * Hkv + g) * D + 16 * dtile + n, acc[e]);
        }
      }
      u = ua; pc = pa; ua = ub; pa = pb;
    };
#pragma unroll 1
    while (u < nu) {
      piece(stg, nxA);
      if (u < nu) piece(stg + gb_stage_bytes<D>(), nxB);
    }
  }

  // ---- dq of this lane's row: channels 16 dt + 4 quad + e
  if (row_ok) {
    uint16_t* orow = dq + ((int64_t)tq * Hq + g * G + hq) * D + 4 * quad;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint32_t p0 = pack_bf16x2(dqa[dt][0], dqa[dt][1]);
      const uint32_t p1 = pack_bf16x2(dqa[dt][2], dqa[dt][3]);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(p0, p1);
    }
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

template <int D>
hipError_t launch_grouped(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                          const int32_t* cu, int nseq, int maxlen, int Hq, int Hkv, int B, int nblk,
                          float scale, const void* dout, const float* lse, void* dq, float* dk,
                          float* dv, hipStream_t st) {
  const int G = Hq / Hkv;
  const int GT = grp_tokens(G);
  const size_t shm = grp_bwd_lds_bytes(D, G, nblk, maxlen);
  hipError_t e = hipFuncSetAttribute((const void*)block_gqa_bwd_group_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  const int by_xcd = 8 % Hkv == 0;
  const int64_t ngrp = ((int64_t)T + GT - 1) / GT;
  const int64_t grid = by_xcd ? (ngrp + 8 / Hkv - 1) / (8 / Hkv) * 8 : ngrp * Hkv;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_gqa_bwd_group_kernel<D>), dim3((unsigned)grid), dim3(kGrpWaves * 64), shm, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, blk, cu, nseq, T, Hq,
                     Hkv, B, nblk, GT, grp_words(maxlen, GT), scale, (const uint16_t*)dout, lse,
                     (uint16_t*)dq, dk, dv, by_xcd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_gqa_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                                bool bf16, int T, const int32_t* cu, int nseq, int maxlen, int Hq,
                                int Hkv, int D, int block_size, int nblk, float scale,
                                const void* dout, const float* lse, void* dq, float* dk, float* dv,
                                hipStream_t st) {
  hipLaunchKernelGGL(zero2_f32_kernel, dim3(1024), dim3(256), 0, st, dk, dv, (int64_t)T * Hkv * D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  const int ns = cu ? nseq : 1;
  if (bf16) {
    // the grouped kernel when its rows, stages and set-up tables fit the LDS
    if (grp_bwd_lds_bytes(D, Hq / Hkv, nblk, maxlen) <= 160 * 1024) {
      if (D == 64)
        return launch_grouped<64>(q, k, v, blk, T, cu, ns, maxlen, Hq, Hkv, block_size, nblk, scale, dout,
                                  lse, dq, dk, dv, st);
      return launch_grouped<128>(q, k, v, blk, T, cu, ns, maxlen, Hq, Hkv, block_size, nblk, scale, dout,
                                 lse, dq, dk, dv, st);
    }
    if (D == 64) return launch_bf16<64>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
    return launch_bf16<128>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
  }
  if (D == 64) return launch_f32<64>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
  return launch_f32<128>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, dout, lse, dq, dk, dv, st);
}

}  // namespace sa
