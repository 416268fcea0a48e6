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
// bf16, where a token group's set-up tables fit the LDS: three launches after the dk/dv
// zero fill. The grouped kernel's D pass (D of every row into the first four bytes of
// its dq row), the key-major dk/dv kernel (one add per element per 64-key block and
// 2048-token chunk), then the grouped dq pass (D read back, dq written over it).
//
// bf16 otherwise (gfx950): one wave per (token, kv head), four per workgroup, each with
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

// Grouped bf16 passes of the backward: one workgroup per (group of GT consecutive
// tokens, kv head), eight waves, over the distinct blocks of the group's routes
// (gqa_group.h) in 32-key sub-tiles staged in LDS. MODE 1 forms D = sum p dp of every
// query row and leaves it, as fp32, in the first four bytes of the row's dq; MODE 2,
// launched after the key-major dk/dv kernel, reads it back and forms dS and dq (per
// row, in registers), then overwrites the row with dq. Wave w owns rows 16w .. 16w+15
// (token row / G, head row mod G):
//   * S^T = K Q^T and dP^T = V dout^T on 16x16x32 MFMAs: key and value rows from
//     padded stages as A operands, the row's q and dout as B operands in registers;
//     lane (n, quad) holds keys 4 quad + e and 16 + 4 quad + e of row n;
//   * dq^T += K^T dS^T: K^T by transposing reads of a swizzled copy of the key rows,
//     dS^T as it stands in registers.
template <int D>
constexpr int gb_stage_bytes() { return 32 * (D * 2 + 16) * 2 + 32 * D * 2; }   // K pad, V pad, K swz
constexpr int kXRB = kGrpRows * 2 + 16;                                           // [key][row] bf16 rows

size_t grp_bwd_lds_bytes(int D, int G, int nblk, int maxlen) {
  const size_t st = D == 128 ? gb_stage_bytes<128>() : gb_stage_bytes<64>();
  return 2 * st + grp_table_bytes(grp_tokens(G), nblk, maxlen);
}

template <int D>
SA_DEVICE int gswz(int row) { return D == 128 ? 2 * (row & 7) : 2 * (row & 3); }

template <int D, int MODE, int NWV>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(2)))
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
  constexpr int NT = NWV * 64;            // NWV waves own rows 16 w .. 16 w + 15
  constexpr int LDN = (2 * 32 * CPR + NT - 1) / NT;   // 16-byte loads per thread per sub-tile
  static_assert(MODE == 1 || MODE == 2, "D-only or dq-only");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* stg = lds;                                          // [2][K pad | V pad | K swz]
  const GroupTables tbl = group_tables(stg + 2 * gb_stage_bytes<D>(), GT, nblk, nwords);

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

  // ---- pass 1: D = sum_s p_s dp_s of every row (MODE 2: left in the first four bytes
  // of the row's dq by the MODE 1 launch)
  float dpart = 0.0f;
  if constexpr (MODE != 2) {
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
  float Drow;
  if constexpr (MODE == 2) {
    Drow = row_ok ? *reinterpret_cast<const float*>(dq + ((int64_t)tq * Hq + g * G + hq) * D) : 0.0f;
  } else {
    Drow = quad_sum(dpart);
  }
  if constexpr (MODE == 1) {
    if (row_ok && quad == 0) *reinterpret_cast<float*>(dq + ((int64_t)tq * Hq + g * G + hq) * D) = Drow;
    return;
  }

  // ---- pass 2: dS and dq
  floatx4v_t dqa[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) dqa[i] = floatx4v_t{};
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

// Key-major dk and dv (bf16), between the D-only and the dq-only launches of the
// grouped kernel: one workgroup per (64-key block K0 = 64 kb of the packed key rows,
// kv head, chunk of 256 consecutive tokens). Each fp32 atomic add costs the same
// whatever the lanes' layout, so the grouped kernel's adds (one per element of every
// 32-key sub-tile of every token group's union) bound it; here a key row gets one add
// per element from each chunk whose tokens attend it, and only the rows that do attend
// it are computed (the grouped kernel runs its whole group over every block of the
// union).
//   * set-up: thread i takes token t0 + i and ORs, over its routed blocks (0 <= b <=
//     own block, repeats included once), the causal keys that fall in the workgroup's
//     64 into a 64-bit mask; the tokens with a nonzero mask are listed in token order;
//   * the K and V rows of the block are staged once; the listed tokens' G query rows go
//     in tiles of 128 rows (128 / G tokens): wave w forms S^T = K Q^T and dP^T = V dout^T
//     of rows 16 w .. 16 w + 15 against the 64 keys (16x16x32 MFMAs, the rows' q and
//     dout from LDS as B operands), P from the token's mask and the forward's lse, dS
//     from D (left in the dq rows by the D-only launch); dS and P meet in LDS as
//     [key][row], and each wave contracts over the tile's rows for its share of the
//     16 x 16 output tiles of dk = dS^T Q and dv = P^T dout, kept in registers over the
//     tiles and added to dk and dv at the end.
constexpr int kKB = 64;          // keys per workgroup
constexpr int kCT = 2048;        // tokens per chunk

template <int D>
constexpr size_t kmaj_lds_bytes() {
  return (size_t)2 * kKB * (D * 2 + 16) + (size_t)2 * kGrpRows * D * 2 + (size_t)2 * kKB * kXRB +
         (size_t)kCT * 12 + (kCT / 64 + 16) * 4;
}

template <int D>
__global__ __launch_bounds__(kGrpWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void block_gqa_bwd_kmaj_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int T, int Hq, int Hkv,
    int B, int nblk, int maxlen, float scale, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const uint16_t* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int KS = D / 32;              // 32-wide k-steps of S^T and dP^T
  constexpr int NDT = D / 16;             // 16-channel tiles
  constexpr int CPR = D * 2 / 16;         // 16-byte chunks per row
  constexpr int KSB = D * 2 + 16;         // padded key row bytes
  constexpr int RWB = D * 2;              // swizzled q / dout row bytes
  constexpr int NT = kGrpWaves * 64;
  constexpr int NKT = kKB / 16;           // 16-key tiles
  constexpr int NTILE = 2 * NKT * NDT;    // output tiles of dk and dv
  constexpr int TPW = NTILE / kGrpWaves;  // ... per wave: all key tiles of DPW channel tiles
  constexpr int DPW = NDT / (kGrpWaves / 2);
  static_assert(NTILE % kGrpWaves == 0 && DPW * NKT == TPW, "tiles split evenly");
  constexpr int NR = kCT / NT;            // tokens per thread in the set-up
  static_assert(NR * NT == kCT, "whole rounds of tokens");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* k_l = lds;                                        // [64 keys][KSB]
  char* v_l = k_l + kKB * KSB;                            // [64 keys][KSB]
  char* q_l = v_l + kKB * KSB;                            // [128 rows][RWB] swizzled
  char* d_l = q_l + kGrpRows * RWB;                       // [128 rows][RWB] dout
  char* xds = d_l + kGrpRows * RWB;                       // dS [64 keys][kXRB]
  char* xp = xds + kKB * kXRB;                            // P  [64 keys][kXRB]
  uint64_t* lmask = reinterpret_cast<uint64_t*>(xp + kKB * kXRB);   // [kCT] key masks
  int* ltok = reinterpret_cast<int*>(lmask + kCT);                  // [kCT] tokens
  int* cnt = ltok + kCT;                                 // [NR][8] counts, then [16] key-mask words

  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int n = L & 15, quad = L >> 4;
  // The chunk's tokens attend keys in [t0 - maxlen + 1, t0 + kCT - 1] only (a sequence
  // holds at most maxlen rows), so blockIdx.y counts 64-key blocks from the one holding
  // key max(0, t0 - maxlen + 1).
  const int t0 = (int)blockIdx.x * kCT;
  const int K0 = (max(0, t0 - maxlen + 1) / kKB + (int)blockIdx.y) * kKB;
  const int g = (int)blockIdx.z;
  if (t0 + kCT - 1 < K0 || K0 >= T) return;               // no token of the chunk reaches the block
  const int G = Hq / Hkv;
  const int TT = kGrpRows / G;                            // tokens per row tile
  const int nrows = TT * G;
  if (TT == 0) return;                                    // G > 128: not launched

  // ---- the chunk's tokens that attend keys of the block, with their key masks (token
  // t0 + NT r + tid in step r of the set-up loop)
  uint64_t mr[NR], balr[NR];
  uint32_t mlo = 0u, mhi = 0u;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    uint64_t m = 0;
    const int t = t0 + NT * r + tid;
    if (t < T && t >= K0) {
      const int st = cu ? seq_start_of(cu, nseq, t) : 0;
      const int own = (t - st) / B;
      const int32_t* br = blk + (int64_t)t * nblk;
      for (int j0 = 0; j0 < nblk; j0 += 16) {
        int bb[16];                                         // 16 route loads in flight
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) bb[jj] = j0 + jj < nblk ? br[j0 + jj] : -1;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int b = bb[jj];
          if (b >= 0 && b <= own) {
            const int r0 = max(st + b * B, K0);
            const int r1 = min(min(st + b * B + B, t + 1), K0 + kKB);
            if (r0 < r1) {
              const int a = r0 - K0, e = r1 - K0;             // keys [a, e), 0 <= a < e <= 64
              const uint64_t below_e = e == 64 ? ~0ull : ((1ull << e) - 1ull);
              m |= below_e & ~((1ull << a) - 1ull);
            }
          }
        }
      }
    }
    mr[r] = m;
    balr[r] = __ballot(m != 0ull);
    mlo |= (uint32_t)m;
    mhi |= (uint32_t)(m >> 32);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    mlo |= (uint32_t)__shfl_xor((int)mlo, off, 64);
    mhi |= (uint32_t)__shfl_xor((int)mhi, off, 64);
  }
  if (L == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) cnt[kGrpWaves * r + w] = __popcll(balr[r]);
    cnt[kGrpWaves * NR + 2 * w] = (int)mlo;
    cnt[kGrpWaves * NR + 2 * w + 1] = (int)mhi;
  }
  __syncthreads();
  int nl = 0;
  uint64_t kmask = 0;                                     // keys any listed token attends
#pragma unroll
  for (int i = 0; i < kGrpWaves; ++i)
    kmask |= (uint64_t)(uint32_t)cnt[kGrpWaves * NR + 2 * i] | ((uint64_t)(uint32_t)cnt[kGrpWaves * NR + 2 * i + 1] << 32);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    int at = nl;                                          // listed before wave w of step r
#pragma unroll
    for (int i = 0; i < kGrpWaves; ++i) {
      at += i < w ? cnt[kGrpWaves * r + i] : 0;
      nl += cnt[kGrpWaves * r + i];
    }
    if (mr[r] != 0ull) {
      const int slot = at + __popcll(balr[r] & ((1ull << L) - 1ull));
      ltok[slot] = t0 + NT * r + tid;
      lmask[slot] = mr[r];
    }
  }
  if (nl == 0) return;                                    // uniform
  // ---- the block's K and V rows (zeros past T)
  for (int c = tid; c < 2 * kKB * CPR; c += NT) {
    const int isv = c >= kKB * CPR;
    const int cc = isv ? c - kKB * CPR : c;
    const int r = cc / CPR, p = cc % CPR;
    bf16x8_t x = bf16x8_t{};
    if (K0 + r < T) x = *reinterpret_cast<const bf16x8_t*>((isv ? v : k) + ((int64_t)(K0 + r) * Hkv + g) * D + 8 * p);
    *reinterpret_cast<bf16x8_t*>((isv ? v_l : k_l) + r * KSB + 16 * p) = x;
  }

  const float sc2 = scale * kLog2e;
  const int row = 16 * w + n;                             // this lane's row of a tile (S phase)
  floatx4v_t acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = floatx4v_t{};

  // The next row tile's q and dout rows, and the lse and D of this lane's row in it,
  // are loaded into registers while the current tile is computed.
  constexpr int NPF = kGrpRows * CPR / NT;                // 16-byte chunks per thread per tile
  static_assert(NPF * NT == kGrpRows * CPR, "whole chunks per thread");
  bf16x8_t pq[NPF], pd[NPF];
  float plse = 0.0f, pD = 0.0f;
  uint64_t pmask = 0ull;
  auto fetch = [&](int it) __attribute__((always_inline)) {
#pragma unroll
    for (int m2 = 0; m2 < NPF; ++m2) {
      const int c = tid + NT * m2, r = c / CPR, p = c % CPR;
      const int i = it + r / G, h = r % G;
      pq[m2] = bf16x8_t{};
      pd[m2] = bf16x8_t{};
      if (r < nrows && i < nl) {
        const int64_t off = ((int64_t)ltok[i] * Hq + g * G + h) * D + 8 * p;
        pq[m2] = *reinterpret_cast<const bf16x8_t*>(q + off);
        pd[m2] = *reinterpret_cast<const bf16x8_t*>(dout + off);
      }
    }
    const int ri = it + row / G;
    const bool ok = row < nrows && ri < nl;
    const int64_t hrow = (int64_t)(ok ? ltok[ri] : 0) * Hq + g * G + row % G;
    pmask = ok ? lmask[ri] : 0ull;
    plse = ok ? lse[hrow] * kLog2e : -__builtin_huge_valf();
    pD = ok ? *reinterpret_cast<const float*>(dq + hrow * D) : 0.0f;
  };
  __syncthreads();                     // the list (and the K and V rows) are in place
  fetch(0);

#pragma unroll 1
  for (int it = 0; it < nl; it += TT) {
#pragma unroll
    for (int m2 = 0; m2 < NPF; ++m2) {
      const int c = tid + NT * m2, r = c / CPR, p = c % CPR;
      const int so = r * RWB + ((p ^ gswz<D>(r)) << 4);
      *reinterpret_cast<bf16x8_t*>(q_l + so) = pq[m2];
      *reinterpret_cast<bf16x8_t*>(d_l + so) = pd[m2];
    }
    const uint64_t rmask = pmask;
    const float lse2 = plse;
    const float Drow = pD;
    if (it + TT < nl) fetch(it + TT);
    __syncthreads();
    bf16x8_t qb[KS], gb[KS];           // B operands: row 16 w + n, channels 32 ks + 8 quad
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int so = row * RWB + (((4 * ks + quad) ^ gswz<D>(row)) << 4);
      qb[ks] = *reinterpret_cast<const bf16x8_t*>(q_l + so);
      gb[ks] = *reinterpret_cast<const bf16x8_t*>(d_l + so);
    }
    // S^T and dP^T: lane (quad, n) holds keys 16 kt + 4 quad + e of row n
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      floatx4v_t S = floatx4v_t{}, dP = floatx4v_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(k_l + (16 * kt + n) * KSB + 64 * ks + 16 * quad);
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(v_l + (16 * kt + n) * KSB + 64 * ks + 16 * quad);
        S = mfma16x32(ka, qb[ks], S);
        dP = mfma16x32(va, gb[ks], dP);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kt + 4 * quad + e;
        const bool ok = ((rmask >> key) & 1ull) && lse2 > -__builtin_huge_valf();
        const float P = ok ? __builtin_amdgcn_exp2f(S[e] * sc2 - lse2) : 0.0f;
        const float dS = P * (dP[e] - Drow) * scale;
        *reinterpret_cast<uint16_t*>(xds + key * kXRB + row * 2) = f2bf_bits(dS);
        *reinterpret_cast<uint16_t*>(xp + key * kXRB + row * 2) = f2bf_bits(P);
      }
    }
    __syncthreads();
    // dk = dS^T Q and dv = P^T dout over the tile's rows. Wave w: dk (w < 4) or dv, channel
    // tiles DPW (w mod 4) + d, every key tile; each B operand (the rows' q or dout by
    // transposing reads) serves the four key tiles.
    {
      const int which = w >> 2;
      const char* xa = which ? xp : xds;
      const char* rb = which ? d_l : q_l;
#pragma unroll
      for (int ks = 0; ks < kGrpRows / 32; ++ks) {
        bf16x8_t bop[DPW];
#pragma unroll
        for (int d = 0; d < DPW; ++d) {
          // B: rows 32 ks + 4 quad + (n >> 2) (+16), channel 16 dtile + 4 (n & 3) ..
          const int dtile = DPW * (w & 3) + d;
          const int r0 = 32 * ks + 4 * quad + (n >> 2);
          const int col = 16 * dtile + 4 * (n & 3);
          const int o0 = r0 * RWB + (((col >> 3) ^ gswz<D>(r0)) << 4) + (col & 7) * 2;
          const int r1 = r0 + 16;
          const int o1 = r1 * RWB + (((col >> 3) ^ gswz<D>(r1)) << 4) + (col & 7) * 2;
          const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(rb + o0));
          const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(rb + o1));
          const short __attribute__((ext_vector_type(8))) b8 = {b0[0], b0[1], b0[2], b0[3],
                                                                b1[0], b1[1], b1[2], b1[3]};
          bop[d] = __builtin_bit_cast(bf16x8_t, b8);
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          // A: key 16 kt + n, rows 32 ks + 4 quad + e and 32 ks + 16 + 4 quad + e
          const char* ar = xa + (16 * kt + n) * kXRB + (32 * ks + 4 * quad) * 2;
          const uint2 alo = *reinterpret_cast<const uint2*>(ar);
          const uint2 ahi = *reinterpret_cast<const uint2*>(ar + 32);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(alo.x, alo.y, ahi.x, ahi.y));
#pragma unroll
          for (int d = 0; d < DPW; ++d) acc[kt * DPW + d] = mfma16x32(a, bop[d], acc[kt * DPW + d]);
        }
      }
    }
    __syncthreads();                   // every wave is done with this tile's rows and dS, P
  }
  // ---- one add per element: lane (quad, n) holds keys 16 ktile + 4 quad + e, channel 16 dtile + n
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ktile = i / DPW, dtile = DPW * (w & 3) + i % DPW;
    float* dst = (w >> 2) ? dv : dk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 16 * ktile + 4 * quad + e;
      if ((kmask >> key) & 1ull)
        atomicAdd(dst + ((int64_t)(K0 + key) * Hkv + g) * D + 16 * dtile + n, acc[i][e]);
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
  const int by_xcd = 8 % Hkv == 0;
  // D of every row (into the first four bytes of its dq row), then dk and dv key-major,
  // then dq
  // gt tokens per group (gt G <= 16 nwv rows), nwv waves per workgroup
  auto grouped = [&](auto kern, int gt, int nwv) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    const int64_t ng = ((int64_t)T + gt - 1) / gt;
    const int64_t gr = by_xcd ? (ng + 8 / Hkv - 1) / (8 / Hkv) * 8 : ng * Hkv;
    if (gr > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)gr), dim3(nwv * 64), shm, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, blk, cu, nseq, T, Hq, Hkv, B, nblk, gt,
                       grp_words(maxlen, gt), scale, (const uint16_t*)dout, lse, (uint16_t*)dq, dk, dv,
                       by_xcd);
    return hipGetLastError();
  };
  hipError_t e = grouped(block_gqa_bwd_group_kernel<D, 1, kGrpWaves>, GT, kGrpWaves);
  if (e != hipSuccess) return e;
  const size_t shk = kmaj_lds_bytes<D>();
  e = hipFuncSetAttribute((const void*)block_gqa_bwd_kmaj_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shk);
  if (e != hipSuccess) return e;
  const int64_t nkb = ((int64_t)maxlen + kCT + kKB - 1) / kKB + 1;   // blocks a chunk can reach
  if (nkb > 65535) return hipErrorInvalidValue;
  const dim3 kgrid((unsigned)((T + kCT - 1) / kCT), (unsigned)nkb, (unsigned)Hkv);
  hipLaunchKernelGGL((block_gqa_bwd_kmaj_kernel<D>), kgrid, dim3(kGrpWaves * 64), shk, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, blk, cu, nseq, T, Hq, Hkv, B, nblk, maxlen, scale,
                     (const uint16_t*)dout, lse, (const uint16_t*)dq, dk, dv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the dq pass in workgroups of four waves over 64-row groups: at 151 VGPRs three
  // of them share a CU, where one of eight waves fit
  const int GT4 = G >= 2 ? 64 / G : kGrpMaxTok;
  return grouped(block_gqa_bwd_group_kernel<D, 2, 4>, GT4, 4);
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
