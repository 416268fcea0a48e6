// Backward of absorbed-MLA sparse attention: dq and dkv from the upstream gradient of
// the output ("Enable DSA CP/absorbed/THD paths with TileLang fused ops", file table:
// sparse-MLA backward kernels; "Support NoPE shapes and unaligned top-k in TileLang
// sparse MLA", section "Validation": gradients are checked numerically because the
// backward accumulates with atomics).
//
// For query t, head h and valid slot j (latent row s = idx[t,j]):
//   p_j = exp(scale q.kv_s - lse),  dp_j = dout . kv_s[0:d_v],  D = sum_j p_j dp_j,
//   ds_j = scale p_j (dp_j - D);
//   dq[t,h]  = sum_j ds_j kv_s;      dkv[s] += sum_h ds_j q[t,h]  (+ p_j dout[t,h] on [0, d_v)).
// lse comes from the forward; the logits are recomputed, never stored. D (which
// equals dout . out) is summed from the p_j dp_j themselves in a first pass over the
// slots, so the ds_j of a row sum to zero as they must; taken from the forward's
// bf16 output instead, D is off by up to 2^-9 sum |dout out|, and that error, carried
// into every ds_j, dominates dq on rows whose few keys nearly cancel.
//
// bf16 kernel (gfx950): one workgroup per (token, group of 16 heads), four waves. The
// slots of the token are split into 16-key sub-tiles and the waves take turns (wave w
// takes sub-tiles w, w+4, ...), so the group's q and dout sit in LDS once and each
// wave stages only its own 16 gathered rows:
//   * S = Q K^T and dP = dout V^T (16 heads x 16 keys, 16x16x32 bf16 MFMA): q's A
//     operands are held in registers, dout's are read from LDS, the key rows are the
//     B operands as stored (row-major, one 16-byte read each);
//   * P and dS in registers: lane (g, n) holds heads 4g..4g+3 of key n, which is the
//     A-operand layout of dS^T and P^T for the 16x16x16 MFMAs of dkv, whose B operands
//     (q and dout, heads x channels) come from transposing LDS reads; the 16x16 dkv
//     block of a sub-tile is added into dkv (fp32) with atomics, one key row per
//     lane-quad;
//   * dq^T += K^T dS^T: K^T by transposing reads of the staged rows, dS^T through a
//     512-byte LDS transpose; 36 accumulators of 16x16 (all of d_qk x 16 heads) per
//     wave, summed over the four waves through LDS at the end;
//   * a first pass over the same sub-tiles computes only S and dP, for D.
// The next sub-tile's rows are loaded into registers while the current one is computed.
// fp32 inputs use a plain kernel with the same arithmetic.
#include <type_traits>

#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kHG = 16;           // heads per workgroup
constexpr int kSK = 16;           // keys per sub-tile

typedef float floatx4v_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

SA_DEVICE floatx4v_t mfma16x32(bf16x8_t a, bf16x8_t b, floatx4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
SA_DEVICE floatx4v_t mfma16x16(short4_t a, short4_t b, floatx4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

SA_DEVICE short4_t pack4(float a, float b, float c, float d) {
  const uint32_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
  return __builtin_bit_cast(short4_t, make_uint2(lo, hi));
}

// Byte strides of the LDS rows: 16 bytes of padding per row keep the 16 rows read by
// a 16-lane group on distinct banks.
template <int DQK>
constexpr int krow_bytes() { return DQK * 2 + 16; }
constexpr int drow_bytes() { return 512 * 2 + 16; }

template <int DQK>
constexpr size_t bwd_lds_bytes() {
  // q and dout of the group, one staged sub-tile per wave, one dS transpose per wave
  const size_t a = (size_t)kHG * krow_bytes<DQK>() + (size_t)kHG * drow_bytes() +
                   (size_t)kWaves * kSK * krow_bytes<DQK>() + (size_t)kWaves * kHG * kSK * 2 +
                   (size_t)kWaves * kHG * 4;
  // the end-of-kernel dq reduction reuses the staging area: half of d_qk per pass
  const size_t r = (size_t)kWaves * kHG * (DQK / 2) * 4;
  return a > r + (size_t)kHG * krow_bytes<DQK>() + (size_t)kHG * drow_bytes() ? a
                                                                              : r + (size_t)kHG * krow_bytes<DQK>() + (size_t)kHG * drow_bytes();
}

template <int DQK>
__global__ __launch_bounds__(kWaves * 64) void sparse_mla_bwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, int H, int topk, float scale,
    const float* __restrict__ sink, uint16_t* __restrict__ dq, float* __restrict__ dkv,
    float* __restrict__ dsink) {
  constexpr int KRB = krow_bytes<DQK>();
  constexpr int DRB = drow_bytes();
  constexpr int NK = DQK / 32;            // 32-wide k-steps of S
  constexpr int NV = 512 / 32;            // ... of dP
  constexpr int NCB = DQK / 16;           // 16-channel blocks of dq^T and dkv
  constexpr int NVB = 512 / 16;           // ... that carry the value part
  constexpr int CPR = DQK * 2 / 16;       // 16-byte chunks per key row
  constexpr int NLD = kSK * CPR / 64;     // row chunks per lane per sub-tile
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* q_l = lds;                                        // [16 heads][KRB]
  char* d_l = q_l + kHG * KRB;                            // [16 heads][DRB] dout
  char* k_l = d_l + kHG * DRB;                            // [waves][16 keys][KRB]
  char* s_l = k_l + kWaves * kSK * KRB;                   // [waves][16 heads][16 keys] bf16
  float* dD = reinterpret_cast<float*>(s_l + kWaves * kHG * kSK * 2);   // [waves][16] D partials

  const int t = blockIdx.x;
  const int h0 = blockIdx.y * kHG;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int g = L >> 4, n = L & 15;

  // ---- q and dout of the 16 heads into LDS (zeros past H)
  for (int c = tid; c < kHG * CPR; c += kWaves * 64) {
    const int hh = c / CPR, p = c % CPR;
    bf16x8_t v = bf16x8_t{};
    if (h0 + hh < H) v = *reinterpret_cast<const bf16x8_t*>(q + ((int64_t)t * H + h0 + hh) * DQK + 8 * p);
    *reinterpret_cast<bf16x8_t*>(q_l + hh * KRB + 16 * p) = v;
  }
  for (int c = tid; c < kHG * 64; c += kWaves * 64) {
    const int hh = c >> 6, p = c & 63;
    bf16x8_t v = bf16x8_t{};
    if (h0 + hh < H) v = *reinterpret_cast<const bf16x8_t*>(dout + ((int64_t)t * H + h0 + hh) * 512 + 8 * p);
    *reinterpret_cast<bf16x8_t*>(d_l + hh * DRB + 16 * p) = v;
  }
  __syncthreads();

  // per-lane constants: heads 4g..4g+3 (rows of the 16x16 tiles)
  float lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = h0 + 4 * g + i;
    const float l = hh < H ? lse[(int64_t)t * H + hh] : -__builtin_huge_valf();
    lse2[i] = l * kLog2e;
  }
  // q's A operands (head n, k-step ks): channels 32 ks + 8 g .. + 8
  bf16x8_t qa[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) qa[ks] = *reinterpret_cast<const bf16x8_t*>(q_l + n * KRB + 64 * ks + 16 * g);

  char* kt = k_l + w * kSK * KRB;
  char* st = s_l + w * kHG * kSK * 2;
  const int32_t* irow = idx + (int64_t)t * topk;
  const int nsub = (topk + kSK - 1) / kSK;
  const float sc2 = scale * kLog2e;

  // One index load per lane (slot kSK sub + (l mod 16), clamped to the last slot) and
  // lane shuffles hand each chunk its row: a sub-tile's row loads wait for one index
  // load, not for one per chunk.
  bf16x8_t nx[NLD];
  auto load = [&](int sub) __attribute__((always_inline)) {
    const int ix = irow[min(sub * kSK + (L & (kSK - 1)), topk - 1)];
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = L + 64 * m, r = c / CPR, p = c % CPR;
      int row = __shfl(ix, r, 64);
      row = row < 0 ? 0 : row;                 // masked slot (or past topk): any finite row
      nx[m] = *reinterpret_cast<const bf16x8_t*>(kv + (int64_t)row * DQK + 8 * p);
    }
  };
  // stages the sub-tile held in nx, then starts loading `next` (if any) into nx
  auto stage = [&](int next) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = L + 64 * m, r = c / CPR, p = c % CPR;
      *reinterpret_cast<bf16x8_t*>(kt + r * KRB + 16 * p) = nx[m];
    }
    __builtin_amdgcn_wave_barrier();
    if (next < nsub) load(next);
  };
  // S = Q K^T and dP = dout V^T of the staged sub-tile (heads 4g..4g+3 x key n per
  // lane) and P; returns whether key n's slot is valid
  auto scores = [&](int sub, float (&P)[4], floatx4v_t& dP) __attribute__((always_inline)) -> int {
    const int jn = sub * kSK + n;                           // slot of key column n
    const int rown = jn < topk ? irow[jn] : -1;
    floatx4v_t S = floatx4v_t{};
    dP = floatx4v_t{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(kt + n * KRB + 64 * ks + 16 * g);
      S = mfma16x32(qa[ks], b, S);
      if (ks < NV) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(d_l + n * DRB + 64 * ks + 16 * g);
        dP = mfma16x32(a, b, dP);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = rown >= 0 && lse2[i] > -__builtin_huge_valf();
      P[i] = ok ? __builtin_amdgcn_exp2f(S[i] * sc2 - lse2[i]) : 0.0f;
    }
    return rown;
  };

  // ---- pass 1: D = sum_j p_j dp_j per head
  float dpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (w < nsub) load(w);
#pragma unroll 1
  for (int sub = w; sub < nsub; sub += kWaves) {
    stage(sub + kWaves);
    float P[4];
    floatx4v_t dP;
    scores(sub, P, dP);
#pragma unroll
    for (int i = 0; i < 4; ++i) dpart[i] = fmaf(P[i], dP[i], dpart[i]);
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {          // sum over the 16 keys (lanes n) of each head
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) dpart[i] += __shfl_xor(dpart[i], off, 64);
    if (n == 0) dD[w * kHG + 4 * g + i] = dpart[i];
  }
  __syncthreads();
  float Dh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float d = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) d += dD[ww * kHG + 4 * g + i];
    Dh[i] = d;
  }
  // the sink's probability exp(sink - lse) times -D is its logit's gradient
  if (dsink && w == 0 && n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + 4 * g + i;
      if (hh < H) atomicAdd(dsink + hh, -__builtin_amdgcn_exp2f(sink[hh] * kLog2e - lse2[i]) * Dh[i]);
    }
  }

  floatx4v_t acc[NCB];   // dq^T: channel block cb, rows 16 cb + 4 g .. +3, column head n
#pragma unroll
  for (int i = 0; i < NCB; ++i) acc[i] = floatx4v_t{};

  // ---- pass 2: dS, dq, dkv
  if (w < nsub) load(w);
#pragma unroll 1
  for (int sub = w; sub < nsub; sub += kWaves) {
    stage(sub + kWaves);
    float P[4], dS[4];
    floatx4v_t dP;
    scores(sub, P, dP);
#pragma unroll
    for (int i = 0; i < 4; ++i) dS[i] = P[i] * (dP[i] - Dh[i]) * scale;
    // dS (heads x keys) transposed through LDS for the B operand of dq^T
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint16_t*>(st + ((4 * g + i) * kSK + n) * 2) = f2bf_bits(dS[i]);
    const short4_t dsA = pack4(dS[0], dS[1], dS[2], dS[3]);   // dS^T: key n, heads 4g..
    const short4_t pA = pack4(P[0], P[1], P[2], P[3]);        // P^T
    __builtin_amdgcn_wave_barrier();
    const short4_t dsB = *reinterpret_cast<const short4_t*>(st + (n * kSK + 4 * g) * 2);  // dS^T: keys 4g.., head n

    // key rows of this lane's dkv quad: keys 4g..4g+3
    int krow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = sub * kSK + 4 * g + i;
      krow[i] = j < topk ? irow[j] : -1;
    }
    const bool any_valid = ballot(krow[0] >= 0 || krow[1] >= 0 || krow[2] >= 0 || krow[3] >= 0) != 0;

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // transposing reads: rows 4g..4g+3 (keys or heads), channel 16 cb + n
      const int toff = 16 * cb + 4 * (n & 3);
      const short4_t kT = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (SA_LDS short4_t*)(kt + (4 * g + (n >> 2)) * KRB + toff * 2));
      acc[cb] = mfma16x16(kT, dsB, acc[cb]);
      if (any_valid) {
        const short4_t qB = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (SA_LDS short4_t*)(q_l + (4 * g + (n >> 2)) * KRB + toff * 2));
        floatx4v_t dk = mfma16x16(dsA, qB, floatx4v_t{});
        if (cb < NVB) {
          const short4_t gB = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (SA_LDS short4_t*)(d_l + (4 * g + (n >> 2)) * DRB + toff * 2));
          dk = mfma16x16(pA, gB, dk);
        }
        // lane (g, n): keys 4g..4g+3, channel 16 cb + n
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (krow[i] >= 0) atomicAdd(dkv + (int64_t)krow[i] * DQK + 16 * cb + n, dk[i]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- sum the waves' dq^T partials through LDS, half of d_qk per pass
  __syncthreads();
  float* red = reinterpret_cast<float*>(k_l);      // [waves][16 heads][DQK / 2]
  constexpr int HALF = DQK / 2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int cb = 0; cb < NCB / 2; ++cb) {
      const int cbb = half * (NCB / 2) + cb;
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(w * kHG + n) * HALF + 16 * cb + 4 * g + i] = acc[cbb][i];
    }
    __syncthreads();
    for (int e = tid; e < kHG * HALF; e += kWaves * 64) {
      const int hh = e / HALF, c = e % HALF;
      float s = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) s += red[(ww * kHG + hh) * HALF + c];
      if (h0 + hh < H) dq[((int64_t)t * H + h0 + hh) * DQK + half * HALF + c] = f2bf_bits(s);
    }
    __syncthreads();
  }
}

// bf16, 32 heads per workgroup (H a multiple of 32): one workgroup per (token, 32-head
// block), four waves on the same 32-key sub-tile, staged once in LDS (double-buffered,
// the next sub-tile's rows in registers meanwhile). Wave (hg, kh) = (w / 2, w % 2)
// forms S and dP of heads 16 hg .. +15 against keys 16 kh .. +15 (16x16x32 MFMAs, q's A
// operands in registers, dout's from LDS, the key rows as B operands), then P and dS.
// dS and P of the 32 heads x 32 keys meet in LDS; each wave then takes a quarter of
// the output tiles (16 x 16) of dkv = dS^T q + P^T dout and of dq = dS K, contracting
// over all 32 heads or all 32 keys: every kv row of a token receives one atomic add
// per element from each 32-head block (four at 128 heads) instead of one per 16-head
// group, and each row is gathered by half as many workgroups. dq accumulates in
// registers across sub-tiles. A first pass over the same sub-tiles forms D.
constexpr int kB32 = 32;          // heads per workgroup, keys per sub-tile
constexpr int kXR = kB32 * 2 + 16;  // [key][head] or [head][key] bf16 exchange rows (bytes)

template <int DQK>
constexpr size_t bwd32_lds_bytes() {
  return (size_t)kB32 * krow_bytes<DQK>() + (size_t)kB32 * drow_bytes() +
         (size_t)2 * kB32 * krow_bytes<DQK>() + (size_t)3 * kB32 * kXR + 2 * kB32 * sizeof(float);
}

template <int DQK>
__global__ __launch_bounds__(kWaves * 64) void sparse_mla_bwd_h32_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, int H, int topk, float scale,
    const float* __restrict__ sink, uint16_t* __restrict__ dq, float* __restrict__ dkv,
    float* __restrict__ dsink) {
  constexpr int KRB = krow_bytes<DQK>();
  constexpr int DRB = drow_bytes();
  constexpr int NK = DQK / 32;            // 32-wide k-steps of S
  constexpr int NV = 512 / 32;            // ... of dP
  constexpr int NCT = DQK / 16;           // 16-channel tiles of dkv and dq
  constexpr int NVT = 512 / 16;           // ... that carry the value part
  constexpr int TPW = 2 * NCT / kWaves;   // output tiles of dkv (and of dq) per wave
  constexpr int CPR = DQK * 2 / 16;       // 16-byte chunks per key row
  constexpr int NLD = (kB32 * CPR + kWaves * 64 - 1) / (kWaves * 64);   // chunks per thread
  static_assert((2 * NCT) % kWaves == 0, "tiles split evenly");
  static_assert(NLD * kWaves * 64 == kB32 * CPR, "every thread loads NLD chunks");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* q_l = lds;                                        // [32 heads][KRB]
  char* d_l = q_l + kB32 * KRB;                           // [32 heads][DRB]
  char* k_l = d_l + kB32 * DRB;                           // [2][32 keys][KRB]
  char* xS = k_l + 2 * kB32 * KRB;                        // dS  [32 keys][kXR] (heads)
  char* xP = xS + kB32 * kXR;                             // P   [32 keys][kXR]
  char* xT = xP + kB32 * kXR;                             // dS  [32 heads][kXR] (keys)
  float* dD = reinterpret_cast<float*>(xT + kB32 * kXR);  // [2 key halves][32 heads]

  const int t = blockIdx.x;
  const int h0 = blockIdx.y * kB32;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int g = L >> 4, n = L & 15;
  const int hg = w >> 1, kh = w & 1;

  // ---- q and dout of the 32 heads into LDS
  for (int c = tid; c < kB32 * CPR; c += kWaves * 64) {
    const int hh = c / CPR, p = c % CPR;
    *reinterpret_cast<bf16x8_t*>(q_l + hh * KRB + 16 * p) =
        *reinterpret_cast<const bf16x8_t*>(q + ((int64_t)t * H + h0 + hh) * DQK + 8 * p);
  }
  for (int c = tid; c < kB32 * 64; c += kWaves * 64) {
    const int hh = c >> 6, p = c & 63;
    *reinterpret_cast<bf16x8_t*>(d_l + hh * DRB + 16 * p) =
        *reinterpret_cast<const bf16x8_t*>(dout + ((int64_t)t * H + h0 + hh) * 512 + 8 * p);
  }
  __syncthreads();

  // heads 16 hg + 4 g + i of this lane (rows of its S / dP tile)
  float lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lse2[i] = lse[(int64_t)t * H + h0 + 16 * hg + 4 * g + i] * kLog2e;
  bf16x8_t qa[NK];                          // A operands: head 16 hg + n, channels 32 ks + 8 g
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
    qa[ks] = *reinterpret_cast<const bf16x8_t*>(q_l + (16 * hg + n) * KRB + 64 * ks + 16 * g);

  const int32_t* irow = idx + (int64_t)t * topk;
  const int nsub = (topk + kB32 - 1) / kB32;
  const float sc2 = scale * kLog2e;

  // Slot indices of a sub-tile: lane l holds slot 32 sub + (l mod 32), clamped to the
  // last slot (positions past topk are masked where they are used). Two registers
  // take turns: the one of sub-tile `sub` is reloaded with sub-tile sub + 2's indices
  // after its last use, and the loop body is written out twice with the two roles
  // swapped, so no in-flight load is ever copied (a copy would wait for every memory
  // operation issued before it, the dkv atomics included). The row loads take their
  // indices by lane shuffles a whole sub-tile after the index load was issued.
  auto idx_of = [&](int sub) __attribute__((always_inline)) {
    return irow[min(sub * kB32 + (L & 31), topk - 1)];
  };
  bf16x8_t nx[NLD];
  auto load = [&](int ix) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + kWaves * 64 * m, r = c / CPR, p = c % CPR;
      int row = __shfl(ix, r, 64);
      row = row < 0 ? 0 : row;                 // masked slot (or past topk): any finite row
      nx[m] = *reinterpret_cast<const bf16x8_t*>(kv + (int64_t)row * DQK + 8 * p);
    }
  };
  auto stage = [&](char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + kWaves * 64 * m, r = c / CPR, p = c % CPR;
      *reinterpret_cast<bf16x8_t*>(kt + r * KRB + 16 * p) = nx[m];
    }
  };
  // S and dP of this wave's 16 heads x 16 keys; P of the valid slots (ix: the
  // sub-tile's slot indices)
  auto scores = [&](const char* kt, int sub, int ix, float (&P)[4], floatx4v_t& dP) __attribute__((always_inline)) {
    const int rown = sub * kB32 + 16 * kh + n < topk ? __shfl(ix, 16 * kh + n, 64) : -1;
    const char* krow = kt + (16 * kh + n) * KRB + 16 * g;
    const char* drow = d_l + (16 * hg + n) * DRB + 16 * g;
    floatx4v_t S = floatx4v_t{};
    dP = floatx4v_t{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(krow + 64 * ks);
      S = mfma16x32(qa[ks], b, S);
      if (ks < NV) dP = mfma16x32(*reinterpret_cast<const bf16x8_t*>(drow + 64 * ks), b, dP);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      P[i] = rown >= 0 && lse2[i] > -__builtin_huge_valf() ? __builtin_amdgcn_exp2f(S[i] * sc2 - lse2[i]) : 0.0f;
  };

  // ---- pass 1: D = sum_j p_j dp_j per head
  float dpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto pass1 = [&](int sub, int& ixc, int ixn) __attribute__((always_inline)) {
    char* kt = k_l + (sub & 1) * kB32 * KRB;
    stage(kt);
    __syncthreads();
    if (sub + 1 < nsub) load(ixn);
    float P[4];
    floatx4v_t dP;
    scores(kt, sub, ixc, P, dP);
    ixc = idx_of(sub + 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) dpart[i] = fmaf(P[i], dP[i], dpart[i]);
  };
  int ixa = 0, ixb = 0;       // indices of sub-tiles of even / odd number
  if (nsub > 0) {
    ixa = idx_of(0);
    ixb = idx_of(1);
    load(ixa);
  }
#pragma unroll 1
  for (int sub = 0; sub < nsub; sub += 2) {
    pass1(sub, ixa, ixb);
    if (sub + 1 < nsub) pass1(sub + 1, ixb, ixa);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {          // over the 16 keys (lanes n) of the wave's half
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) dpart[i] += __shfl_xor(dpart[i], off, 64);
    if (n == 0) dD[kh * kB32 + 16 * hg + 4 * g + i] = dpart[i];
  }
  __syncthreads();
  float Dh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) Dh[i] = dD[16 * hg + 4 * g + i] + dD[kB32 + 16 * hg + 4 * g + i];
  // the sink's probability exp(sink - lse) times -D is its logit's gradient
  if (dsink && tid < kB32) {
    const int hh = h0 + tid;
    const float D = dD[tid] + dD[kB32 + tid];
    atomicAdd(dsink + hh, -__builtin_amdgcn_exp2f((sink[hh] - lse[(int64_t)t * H + hh]) * kLog2e) * D);
  }

  floatx4v_t dqa[TPW];       // dq tiles tt = w + 4 i: head tile tt / NCT, channel tile tt % NCT
#pragma unroll
  for (int i = 0; i < TPW; ++i) dqa[i] = floatx4v_t{};

  // ---- pass 2: dS; dkv and dq over the 32 heads / 32 keys
  auto pass2 = [&](int sub, int& ixc, int ixn) __attribute__((always_inline)) {
    char* kt = k_l + (sub & 1) * kB32 * KRB;
    stage(kt);
    __syncthreads();                   // also: every wave is done with the exchange rows
    float P[4], dS[4];
    floatx4v_t dP;
    scores(kt, sub, ixc, P, dP);
#pragma unroll
    for (int i = 0; i < 4; ++i) dS[i] = P[i] * (dP[i] - Dh[i]) * scale;
    {
      const int key = 16 * kh + n, head = 16 * hg + 4 * g;
      *reinterpret_cast<short4_t*>(xS + key * kXR + head * 2) = pack4(dS[0], dS[1], dS[2], dS[3]);
      *reinterpret_cast<short4_t*>(xP + key * kXR + head * 2) = pack4(P[0], P[1], P[2], P[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint16_t*>(xT + (head + i) * kXR + key * 2) = f2bf_bits(dS[i]);
    }
    // kv rows of this lane's dkv keys: 16 kt2 + 4 g + i
    int krow[2][4];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * kt2 + 4 * g + i;
        krow[kt2][i] = sub * kB32 + r < topk ? __shfl(ixc, r, 64) : -1;
      }
    ixc = idx_of(sub + 2);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      // The next sub-tile's rows are requested after the first third of the tiles: the
      // wait for them (at the next staging) then spans at most the atomics of the other
      // two thirds (48 at d_qk 576, within the 63 the wait counter can name), not the
      // atomics issued before the loads.
      if (i == TPW / 3 && sub + 1 < nsub) load(ixn);
      const int tt = w + kWaves * i;
      const int t2 = tt / NCT, ct = tt % NCT;
      const int toff = (16 * ct + 4 * (n & 3)) * 2;
      // dkv tile: keys 16 t2 + ..., channels 16 ct + ...; k = heads {4g + e, 16 + 4g + e}
      {
        const char* ar = xS + (16 * t2 + n) * kXR + 8 * g;
        const uint2 a0 = *reinterpret_cast<const uint2*>(ar);
        const uint2 a1 = *reinterpret_cast<const uint2*>(ar + 32);
        const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(q_l + (4 * g + (n >> 2)) * KRB + toff));
        const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(q_l + (16 + 4 * g + (n >> 2)) * KRB + toff));
        const short __attribute__((ext_vector_type(8))) b8 = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        floatx4v_t acc = mfma16x32(__builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y)),
                                   __builtin_bit_cast(bf16x8_t, b8), floatx4v_t{});
        if (ct < NVT) {
          const char* pr = xP + (16 * t2 + n) * kXR + 8 * g;
          const uint2 p0 = *reinterpret_cast<const uint2*>(pr);
          const uint2 p1 = *reinterpret_cast<const uint2*>(pr + 32);
          const short4_t c0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(d_l + (4 * g + (n >> 2)) * DRB + toff));
          const short4_t c1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(d_l + (16 + 4 * g + (n >> 2)) * DRB + toff));
          const short __attribute__((ext_vector_type(8))) c8 = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
          acc = mfma16x32(__builtin_bit_cast(bf16x8_t, make_uint4(p0.x, p0.y, p1.x, p1.y)),
                          __builtin_bit_cast(bf16x8_t, c8), acc);
        }
        // lane (g, n): keys 16 t2 + 4 g + e, channel 16 ct + n
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = t2 ? krow[1][e] : krow[0][e];
          if (r >= 0) atomicAdd(dkv + (int64_t)r * DQK + 16 * ct + n, acc[e]);
        }
      }
      // dq tile: heads 16 t2 + ..., channels 16 ct + ...; k = keys {4g + e, 16 + 4g + e}
      {
        const char* ar = xT + (16 * t2 + n) * kXR + 8 * g;
        const uint2 a0 = *reinterpret_cast<const uint2*>(ar);
        const uint2 a1 = *reinterpret_cast<const uint2*>(ar + 32);
        const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kt + (4 * g + (n >> 2)) * KRB + toff));
        const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kt + (16 + 4 * g + (n >> 2)) * KRB + toff));
        const short __attribute__((ext_vector_type(8))) b8 = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        dqa[i] = mfma16x32(__builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y)),
                           __builtin_bit_cast(bf16x8_t, b8), dqa[i]);
      }
    }
  };
  if (nsub > 0) {
    ixa = idx_of(0);
    ixb = idx_of(1);
    load(ixa);
  }
#pragma unroll 1
  for (int sub = 0; sub < nsub; sub += 2) {
    pass2(sub, ixa, ixb);
    if (sub + 1 < nsub) pass2(sub + 1, ixb, ixa);
  }

  // ---- dq: lane (g, n) of tile tt holds heads 16 (tt / NCT) + 4 g + e, channel 16 (tt % NCT) + n
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tt = w + kWaves * i;
    const int ht = tt / NCT, ct = tt % NCT;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dq[((int64_t)t * H + h0 + 16 * ht + 4 * g + e) * DQK + 16 * ct + n] = f2bf_bits(dqa[i][e]);
  }
}

// bf16 dkv with every head of a token in one workgroup (H = 16 NW heads, NW waves),
// for H in {64, 128}. Floating-point atomic adds into dkv run at a fixed rate per
// element whatever the lanes' address pattern, and they bound this backward; summing
// the whole token's heads before the adds issues one add per element of each gathered
// row instead of one per 32-head block. The token's q and dout (278 KB at 128 heads)
// do not both fit in LDS, so:
//   * dout of the H heads stays in LDS; wave w reads its S-phase A operands (heads
//     16 w + n, channel-contiguous) and, by transposing reads, the B operands of
//     dv = P^T dout (head-contiguous) from there;
//   * q passes through LDS once at the start, from which each wave keeps in registers
//     the A operands of S for its 16 heads and the B operands of dk = dS^T q for its
//     channel tiles (16 ct + n, ct = w + NW i) over all H heads;
//   * per 16-key sub-tile: S and dP of (wave's 16 heads) x 16 keys, P and dS into LDS
//     as [key][head]; then each wave contracts over all H heads for its channel tiles
//     and adds each 16x16 tile into the gathered rows (one add per element).
// A first pass over the same sub-tiles sums D = sum_j p_j dp_j per head; it is stored,
// as fp32, in the first four bytes of the head's dq row, which the dq kernel launched
// next reads before it overwrites the row (and dsink is formed here).
template <int DQK, int NW>
constexpr size_t dkv_lds_bytes() {
  constexpr size_t HH = 16 * NW;
  const size_t main = HH * drow_bytes() + (size_t)kSK * krow_bytes<DQK>() + 2 * (size_t)kSK * (HH * 2 + 16);
  const size_t qst = HH * krow_bytes<DQK>();        // q, staged once at the start
  return main > qst ? main : qst;
}

template <int DQK, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, int topk, float scale,
    const float* __restrict__ sink, uint16_t* __restrict__ dq, float* __restrict__ dkv,
    float* __restrict__ dsink) {
  constexpr int H = 16 * NW;
  constexpr int KRB = krow_bytes<DQK>();
  constexpr int DRB = drow_bytes();
  constexpr int XRB = H * 2 + 16;         // [key][head] bf16 exchange rows (bytes)
  constexpr int NK = DQK / 32;            // 32-wide k-steps of S
  constexpr int NV = 512 / 32;            // ... of dP
  constexpr int NCT = DQK / 16;           // 16-channel tiles of dkv
  constexpr int NVT = 512 / 16;           // ... that carry the value part
  constexpr int TPW = (NCT + NW - 1) / NW;  // channel tiles per wave (the last may be past NCT)
  constexpr int KS = H / 32;              // 32-head k-steps of the dkv contraction
  constexpr int CPR = DQK * 2 / 16;       // 16-byte chunks per key row
  constexpr int NT = NW * 64;
  constexpr int NLD = (kSK * CPR + NT - 1) / NT;   // chunks per thread (the last partial)
  static_assert(NW % 2 == 0, "whole 32-head k-steps");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* d_l = lds;                                        // [H heads][DRB] dout
  char* k_l = d_l + H * DRB;                              // [16 keys][KRB]
  char* xS = k_l + kSK * KRB;                             // dS [16 keys][XRB]
  char* xP = xS + kSK * XRB;                              // P  [16 keys][XRB]

  const int t = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int g = L >> 4, n = L & 15;

  // ---- q of the H heads through LDS into registers
  for (int c = tid; c < H * CPR; c += NT) {
    const int hh = c / CPR, p = c % CPR;
    *reinterpret_cast<bf16x8_t*>(lds + hh * KRB + 16 * p) =
        *reinterpret_cast<const bf16x8_t*>(q + ((int64_t)t * H + hh) * DQK + 8 * p);
  }
  __syncthreads();
  bf16x8_t qa[NK];                        // A operands of S: head 16 w + n, channels 32 ks + 8 g
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
    qa[ks] = *reinterpret_cast<const bf16x8_t*>(lds + (16 * w + n) * KRB + 64 * ks + 16 * g);
  bf16x8_t qb[TPW][KS];                   // B operands of dk: heads {32 s + 4 g + e, +16} x channel 16 ct + n
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ct = w + NW * i;
    const int toff = (16 * (ct < NCT ? ct : 0) + 4 * (n & 3)) * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(lds + (32 * s + 4 * g + (n >> 2)) * KRB + toff));
      const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(lds + (32 * s + 16 + 4 * g + (n >> 2)) * KRB + toff));
      const short __attribute__((ext_vector_type(8))) b8 = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      qb[i][s] = __builtin_bit_cast(bf16x8_t, b8);
    }
  }
  __syncthreads();                        // q's staging area becomes dout's and the key rows'
  for (int c = tid; c < H * 64; c += NT) {
    const int hh = c >> 6, p = c & 63;
    *reinterpret_cast<bf16x8_t*>(d_l + hh * DRB + 16 * p) =
        *reinterpret_cast<const bf16x8_t*>(dout + ((int64_t)t * H + hh) * 512 + 8 * p);
  }

  float lse2[4];                          // heads 16 w + 4 g + i (rows of this lane's S tile)
#pragma unroll
  for (int i = 0; i < 4; ++i) lse2[i] = lse[(int64_t)t * H + 16 * w + 4 * g + i] * kLog2e;
  const int32_t* irow = idx + (int64_t)t * topk;
  const int nsub = (topk + kSK - 1) / kSK;
  const float sc2 = scale * kLog2e;

  // Slot indices of a sub-tile: lane l holds slot 16 sub + (l mod 16), clamped to the
  // last slot. As in the 32-head kernel, two registers take turns and the loop body is
  // written out twice, so no in-flight load is copied (a copy would wait for the dkv
  // atomics issued before it).
  auto idx_of = [&](int sub) __attribute__((always_inline)) {
    return irow[min(sub * kSK + n, topk - 1)];
  };
  bf16x8_t nx[NLD], nx2[NLD];
  auto loadTo = [&](bf16x8_t (&buf)[NLD], int ix) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + NT * m, r = (c / CPR) & (kSK - 1), p = c % CPR;
      int row = __shfl(ix, r, 64);
      row = row < 0 ? 0 : row;                 // masked slot (or past topk): any finite row
      if (c < kSK * CPR) buf[m] = *reinterpret_cast<const bf16x8_t*>(kv + (int64_t)row * DQK + 8 * p);
    }
  };
  auto load = [&](int ix) __attribute__((always_inline)) { loadTo(nx, ix); };
  auto stageFrom = [&](const bf16x8_t (&buf)[NLD]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + NT * m, r = c / CPR, p = c % CPR;
      if (c < kSK * CPR) *reinterpret_cast<bf16x8_t*>(k_l + r * KRB + 16 * p) = buf[m];
    }
  };
  auto stage = [&]() __attribute__((always_inline)) { stageFrom(nx); };
  // kv row of key n of a sub-tile (-1: masked slot or past topk)
  auto row_of = [&](int sub, int ix) __attribute__((always_inline)) {
    return sub * kSK + n < topk ? __shfl(ix, n, 64) : -1;
  };
  // S and dP of this wave's 16 heads x the 16 keys; P of the valid slots
  auto scores = [&](int rown, float (&P)[4], floatx4v_t& dP) __attribute__((always_inline)) {
    const char* krow = k_l + n * KRB + 16 * g;
    const char* drow = d_l + (16 * w + n) * DRB + 16 * g;
    floatx4v_t S = floatx4v_t{};
    dP = floatx4v_t{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(krow + 64 * ks);
      S = mfma16x32(qa[ks], b, S);
      if (ks < NV) dP = mfma16x32(*reinterpret_cast<const bf16x8_t*>(drow + 64 * ks), b, dP);
      // a fence every few k-steps keeps the LDS reads from being hoisted all at once
      // (their registers would not fit beside q's operands)
      if (ks % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      P[i] = rown >= 0 && lse2[i] > -__builtin_huge_valf() ? __builtin_amdgcn_exp2f(S[i] * sc2 - lse2[i]) : 0.0f;
  };

  // ---- pass 1: D = sum_j p_j dp_j per head. No atomics here, so the rows go two
  // sub-tiles ahead: sub-tile s's rows sit in buffer s mod 2, requested at s - 2 with
  // the indices loaded at s - 4 (ja / jb), and its key rows (ra / rb) taken then.
  float dpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int ja = idx_of(0), jb = idx_of(1);
  int ra = row_of(0, ja), rb = row_of(1, jb);
  loadTo(nx, ja);
  if (nsub > 1) loadTo(nx2, jb);
  ja = idx_of(2);
  jb = idx_of(3);
  auto pass1 = [&](int sub, bf16x8_t (&buf)[NLD], int& jc, int& rc) __attribute__((always_inline)) {
    __syncthreads();                   // every wave is done with the previous key rows
    stageFrom(buf);
    __syncthreads();
    if (sub + 2 < nsub) loadTo(buf, jc);
    float P[4];
    floatx4v_t dP;
    scores(rc, P, dP);
    rc = row_of(sub + 2, jc);
    jc = idx_of(sub + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) dpart[i] = fmaf(P[i], dP[i], dpart[i]);
  };
#pragma unroll 1
  for (int sub = 0; sub < nsub; sub += 2) {
    pass1(sub, nx, ja, ra);
    if (sub + 1 < nsub) pass1(sub + 1, nx2, jb, rb);
  }
  int ixa = 0, ixb = 0;       // pass 2: indices of sub-tiles of even / odd number
  float Dh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {          // over the 16 keys (lanes n)
    float d = dpart[i];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) d += __shfl_xor(d, off, 64);
    Dh[i] = d;
  }
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * w + 4 * g + i;
      *reinterpret_cast<float*>(dq + ((int64_t)t * H + hh) * DQK) = Dh[i];
      // the sink's probability exp(sink - lse) times -D is its logit's gradient
      if (dsink)
        atomicAdd(dsink + hh, -__builtin_amdgcn_exp2f((sink[hh] - lse[(int64_t)t * H + hh]) * kLog2e) * Dh[i]);
    }
  }

  // ---- pass 2: dS; dkv = dS^T q + P^T dout over all H heads
  auto pass2 = [&](int sub, int& ixc, int ixn) __attribute__((always_inline)) {
    stage();
    __syncthreads();                   // also: every wave is done with the exchange rows
    if (sub + 1 < nsub) load(ixn);
    float P[4], dS[4];
    floatx4v_t dP;
    scores(row_of(sub, ixc), P, dP);
#pragma unroll
    for (int i = 0; i < 4; ++i) dS[i] = P[i] * (dP[i] - Dh[i]) * scale;
    {
      const int head = 16 * w + 4 * g;
      *reinterpret_cast<short4_t*>(xS + n * XRB + head * 2) = pack4(dS[0], dS[1], dS[2], dS[3]);
      *reinterpret_cast<short4_t*>(xP + n * XRB + head * 2) = pack4(P[0], P[1], P[2], P[3]);
    }
    int krow[4];                       // kv rows of this lane's dkv keys 4 g + e
#pragma unroll
    for (int e = 0; e < 4; ++e) krow[e] = sub * kSK + 4 * g + e < topk ? __shfl(ixc, 4 * g + e, 64) : -1;
    ixc = idx_of(sub + 2);
    __syncthreads();                   // also: every wave is done with the key rows
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ct = w + NW * i;
      if (ct < NCT) {
        const int toff = (16 * ct + 4 * (n & 3)) * 2;
        floatx4v_t acc = floatx4v_t{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const char* ar = xS + n * XRB + 64 * s + 8 * g;
          const uint2 a0 = *reinterpret_cast<const uint2*>(ar);
          const uint2 a1 = *reinterpret_cast<const uint2*>(ar + 32);
          acc = mfma16x32(__builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y)), qb[i][s], acc);
        }
        if (ct < NVT) {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const char* pr = xP + n * XRB + 64 * s + 8 * g;
            const uint2 p0 = *reinterpret_cast<const uint2*>(pr);
            const uint2 p1 = *reinterpret_cast<const uint2*>(pr + 32);
            const short4_t c0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(d_l + (32 * s + 4 * g + (n >> 2)) * DRB + toff));
            const short4_t c1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(d_l + (32 * s + 16 + 4 * g + (n >> 2)) * DRB + toff));
            const short __attribute__((ext_vector_type(8))) c8 = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            acc = mfma16x32(__builtin_bit_cast(bf16x8_t, make_uint4(p0.x, p0.y, p1.x, p1.y)),
                            __builtin_bit_cast(bf16x8_t, c8), acc);
          }
        }
        // lane (g, n): keys 4 g + e, channel 16 ct + n
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (krow[e] >= 0) atomicAdd(dkv + (int64_t)krow[e] * DQK + 16 * ct + n, acc[e]);
      }
      __builtin_amdgcn_sched_barrier(0);   // one tile's operands live at a time
    }
  };
  if (nsub > 0) {
    ixa = idx_of(0);
    ixb = idx_of(1);
    __syncthreads();                   // every wave is done with pass 1's key rows
    load(ixa);
  }
#pragma unroll 1
  for (int sub = 0; sub < nsub; sub += 2) {
    pass2(sub, ixa, ixb);
    if (sub + 1 < nsub) pass2(sub + 1, ixb, ixa);
  }
}

// bf16 dq with 64 heads per workgroup (H = 64 or 128), after the all-heads dkv kernel,
// which leaves D in the first four bytes of each head's dq row. dq needs q and dout
// only as the A operands of S and dP (channel-contiguous), so a wave keeps its 16
// heads' q and dout in VGPRs and its dq tiles (16 heads x d_qk) in AGPRs, and each
// gathered 32-key sub-tile serves 64 heads (the 32-head kernel gathers every row once
// per 32 heads). The token's slot indices are staged in LDS first, and the rows of
// sub-tile s + 1 are requested while sub-tile s is computed (one register buffer: a
// second one, for rows two sub-tiles ahead, took the registers the compiler uses to
// read the LDS operands ahead, and was slower). Per sub-tile each wave forms S and dP of its 16
// heads x 32 keys (16x16x32 MFMAs, key rows as B operands), dS into a wave-private LDS
// block as [head][key], and dq += dS K over the 32 keys (K^T by transposing reads): no
// exchange between waves, one barrier per sub-tile (two key stages).
constexpr int kQH = 64;            // heads per dq workgroup
constexpr int kXQ = 32 * 2 + 16;   // wave-private dS rows [16 heads][32 keys] bf16 (bytes)

template <int DQK>
constexpr size_t dq64_lds_bytes(int topk) {
  return (size_t)2 * kB32 * krow_bytes<DQK>() + (size_t)kWaves * 16 * kXQ +
         (size_t)((topk + kB32 - 1) / kB32) * kB32 * 4;
}

template <int DQK>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_bwd_dq64_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                const int32_t* __restrict__ idx, const uint16_t* __restrict__ dout,
                                const float* __restrict__ lse, int H, int topk, float scale,
                                uint16_t* __restrict__ dq) {
  constexpr int KRB = krow_bytes<DQK>();
  constexpr int NK = DQK / 32;            // 32-wide k-steps of S
  constexpr int NV = 512 / 32;            // ... of dP
  constexpr int NCT = DQK / 16;           // 16-channel tiles of dq
  constexpr int CPR = DQK * 2 / 16;       // 16-byte chunks per key row
  constexpr int NT = kWaves * 64;
  constexpr int NLD = kB32 * CPR / NT;    // chunks per thread per sub-tile
  static_assert(NLD * NT == kB32 * CPR, "every thread loads NLD chunks");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* k_l = lds;                                        // [2][32 keys][KRB]
  char* x_l = k_l + 2 * kB32 * KRB;                       // [4 waves][16 heads][kXQ]
  int* ix_l = reinterpret_cast<int*>(x_l + kWaves * 16 * kXQ);   // [nsub * 32] slots (-1 past topk)

  const int t = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int g = L >> 4, n = L & 15;
  const int hw = (int)blockIdx.y * kQH + 16 * w;          // the wave's first head
  const int nsub = (topk + kB32 - 1) / kB32;
  const float sc2 = scale * kLog2e;

  const int32_t* irow = idx + (int64_t)t * topk;
  for (int j = tid; j < nsub * kB32; j += NT) ix_l[j] = j < topk ? irow[j] : -1;

  bf16x8_t qa[NK], da[NV];                // A operands: head hw + n, channels 32 ks + 8 g
  {
    const int64_t hr = (int64_t)t * H + hw + n;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) qa[ks] = *reinterpret_cast<const bf16x8_t*>(q + hr * DQK + 32 * ks + 8 * g);
#pragma unroll
    for (int ks = 0; ks < NV; ++ks) da[ks] = *reinterpret_cast<const bf16x8_t*>(dout + hr * 512 + 32 * ks + 8 * g);
  }
  float lse2[4], Dh[4];                   // heads hw + 4 g + i (rows of the S tile)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t hr = (int64_t)t * H + hw + 4 * g + i;
    lse2[i] = lse[hr] * kLog2e;
    Dh[i] = *reinterpret_cast<const float*>(dq + hr * DQK);
  }
  floatx4v_t dqa[NCT];                    // dq tile ct: heads hw + 4 g + e, channel 16 ct + n
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) dqa[ct] = floatx4v_t{};
  __syncthreads();                        // the slot indices are in place

  auto load = [&](bf16x8_t (&nx)[NLD], int sub) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + NT * m, r = c / CPR, p = c % CPR;
      int row = ix_l[sub * kB32 + r];
      row = row < 0 ? 0 : row;                 // masked slot (or past topk): any finite row
      nx[m] = *reinterpret_cast<const bf16x8_t*>(kv + (int64_t)row * DQK + 8 * p);
    }
  };
  char* xw = x_l + w * 16 * kXQ;
  auto step = [&](int sub, bf16x8_t (&nx)[NLD]) __attribute__((always_inline)) {
    char* kt = k_l + (sub & 1) * kB32 * KRB;
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + NT * m, r = c / CPR, p = c % CPR;
      *reinterpret_cast<bf16x8_t*>(kt + r * KRB + 16 * p) = nx[m];
    }
    __syncthreads();                     // this stage is in place; the other one is free
    if (sub + 1 < nsub) load(nx, sub + 1);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int key = 16 * kh + n;
      const int rown = ix_l[sub * kB32 + key];
      const char* krow = kt + key * KRB + 16 * g;
      floatx4v_t S = floatx4v_t{}, dP = floatx4v_t{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(krow + 64 * ks);
        S = mfma16x32(qa[ks], b, S);
        if (ks < NV) dP = mfma16x32(da[ks], b, dP);
        if (ks % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float P = rown >= 0 && lse2[i] > -__builtin_huge_valf()
                            ? __builtin_amdgcn_exp2f(S[i] * sc2 - lse2[i]) : 0.0f;
        *reinterpret_cast<uint16_t*>(xw + (4 * g + i) * kXQ + key * 2) = f2bf_bits(P * (dP[i] - Dh[i]) * scale);
      }
    }
    __builtin_amdgcn_wave_barrier();      // the wave's dS rows are written (LDS runs in order)
    // dq += dS K: A = dS of head n, keys {4 g + e, 16 + 4 g + e}; B = K^T by transposing reads
    const char* ar = xw + n * kXQ + 8 * g;
    const uint2 a0 = *reinterpret_cast<const uint2*>(ar);
    const uint2 a1 = *reinterpret_cast<const uint2*>(ar + 32);
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int toff = (16 * ct + 4 * (n & 3)) * 2;
      const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kt + (4 * g + (n >> 2)) * KRB + toff));
      const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kt + (16 + 4 * g + (n >> 2)) * KRB + toff));
      const short __attribute__((ext_vector_type(8))) b8 = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      dqa[ct] = mfma16x32(a, __builtin_bit_cast(bf16x8_t, b8), dqa[ct]);
    }
    __builtin_amdgcn_wave_barrier();      // the dS rows are read before the next sub-tile's writes
  };
  bf16x8_t nx[NLD];
  load(nx, 0);
  // two steps per iteration (the two key stages): this form measured faster than one
#pragma unroll 1
  for (int sub = 0; sub < nsub; sub += 2) {
    step(sub, nx);
    if (sub + 1 < nsub) step(sub + 1, nx);
  }
  // lane (g, n) of tile ct: heads hw + 4 g + e, channel 16 ct + n
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dq[((int64_t)t * H + hw + 4 * g + e) * DQK + 16 * ct + n] = f2bf_bits(dqa[ct][e]);
}

// fp32: one workgroup per (token, head); plain arithmetic, dkv by atomics.
constexpr int kNT = 256;

__global__ __launch_bounds__(kNT) void sparse_mla_bwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ dout, const float* __restrict__ lse, int H, int d_qk, int d_v,
    int topk, float scale, const float* __restrict__ sink, float* __restrict__ dq,
    float* __restrict__ dkv, float* __restrict__ dsink) {
  extern __shared__ float sm[];        // [topk] p_j, then [topk] dp_j, then [kNT / 64] reduce slots
  float* sdp = sm + topk;
  float* red = sdp + topk;
  const int t = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const float* qr = q + ((int64_t)t * H + h) * d_qk;
  const float* gr = dout + ((int64_t)t * H + h) * d_v;
  const int32_t* ir = idx + (int64_t)t * topk;
  const float l = lse[(int64_t)t * H + h];
  // p_j = exp(scale q.kv - lse), dp_j = dout . v_j, and D = sum_j p_j dp_j
  float part = 0.0f;
  for (int j = tid; j < topk; j += kNT) {
    const int r = ir[j];
    float p = 0.0f, dp = 0.0f;
    if (r >= 0 && l > -__builtin_huge_valf()) {
      const float* kr = kv + (int64_t)r * d_qk;
      float s = 0.0f;
      for (int c = 0; c < d_qk; ++c) s = fmaf(qr[c], kr[c], s);
      for (int c = 0; c < d_v; ++c) dp = fmaf(gr[c], kr[c], dp);
      p = expf(s * scale - l);
    }
    sm[j] = p;
    sdp[j] = dp;
    part = fmaf(p, dp, part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if (L == 0) red[w] = part;
  __syncthreads();
  float D = 0.0f;
  for (int i = 0; i < kNT / 64; ++i) D += red[i];
  if (dsink && tid == 0) atomicAdd(dsink + h, -expf(sink[h] - l) * D);
  // ds_j = scale p_j (dp_j - D); dkv by atomics; sm[j] becomes ds_j
  for (int j = tid; j < topk; j += kNT) {
    const int r = ir[j];
    const float p = sm[j];
    const float ds = scale * p * (sdp[j] - D);
    if (r >= 0 && p != 0.0f) {
      for (int c = 0; c < d_qk; ++c) atomicAdd(dkv + (int64_t)r * d_qk + c, ds * qr[c]);
      for (int c = 0; c < d_v; ++c) atomicAdd(dkv + (int64_t)r * d_qk + c, p * gr[c]);
    }
    sm[j] = ds;
  }
  __syncthreads();
  for (int c = tid; c < d_qk; c += kNT) {
    float a = 0.0f;
    for (int j = 0; j < topk; ++j) {
      const int r = ir[j];
      if (r >= 0) a = fmaf(sm[j], kv[(int64_t)r * d_qk + c], a);
    }
    dq[((int64_t)t * H + h) * d_qk + c] = a;
  }
}

// Teacher of the sparse KL indexer loss: the head mean of the attention probability of
// every slot, p[t,j] = (1/H) sum_h exp(scale q[t,h].kv[idx_j] - lse[t,h]); 0 on -1 slots.
// Teacher, bf16: one workgroup per token, four waves; wave w owns heads
// [16 HB w, 16 HB (w + 1)), HB = 2 above 64 heads, else 1 (q slices of its heads as A
// operands in registers, its rows of the forward's lse). Four waves of up to 32 heads
// take one wave per SIMD and 76 KB of LDS, so two workgroups share a CU and two tokens'
// gathers are in flight there (eight waves of 16 heads held one workgroup per CU).
// The token's slots go in 16-key sub-tiles that the whole workgroup gathers once into
// LDS (double-buffered, the next sub-tile's rows in registers while the current one
// is computed); every wave forms S = Q K^T for its heads (16x16x32 MFMAs, key rows as
// B operands as stored) and sums exp(scale s - lse) over its 16 heads per key; the
// per-wave sums meet in LDS and one plain store per slot writes p_j / H.
constexpr int kTW = 4;            // waves of a teacher workgroup
constexpr int kTK = 16;           // keys per teacher sub-tile (32 measured 3-4 % slower:
                                  // its row buffer took registers the LDS reads use)

template <int DQK>
constexpr size_t teacher_lds_bytes() {
  return (size_t)2 * kTK * krow_bytes<DQK>() + (size_t)2 * kTW * kTK * sizeof(float);
}

template <int DQK, int NW, int HB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_teacher_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, int H, int topk, float scale, float* __restrict__ teacher) {
  constexpr int KRB = krow_bytes<DQK>();
  constexpr int NK = DQK / 32;
  constexpr int CPR = DQK * 2 / 16;
  constexpr int NT = NW * 64;
  constexpr int NLD = (kTK * CPR + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* stage = lds;                                                    // [2][kTK][KRB]
  float* part = reinterpret_cast<float*>(lds + 2 * kTK * KRB);          // [2][NW][kTK]
  const int t = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int g = L >> 4, n = L & 15;
  const int h0 = kHG * HB * w;                     // the wave's first head (HB blocks of 16)
  const int32_t* __restrict__ irow = idx + (int64_t)t * topk;
  const int nsub = (topk + kTK - 1) / kTK;
  const float sc2 = scale * kLog2e, invH = 1.0f / (float)H;

  bf16x8_t qa[HB][NK];
  float lse2[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int hq = h0 + kHG * hb + n;
    const uint16_t* qr = q + ((int64_t)t * H + (hq < H ? hq : 0)) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(qr + 32 * ks);
      qa[hb][ks] = hq < H ? x : bf16x8_t{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + kHG * hb + 4 * g + i;
      lse2[hb][i] = (hh < H ? lse[(int64_t)t * H + hh] : -__builtin_huge_valf()) * kLog2e;
    }
  }
  // Slot indices of a sub-tile: lane l holds slot kTK sub + (l mod kTK), clamped to the
  // last slot. As in the backward: two registers take turns (the loop body is written
  // out twice), each reloaded two sub-tiles ahead after its last use, and the row loads
  // take their indices by lane shuffles, so no load waits for an index load.
  auto idx_of = [&](int sub) __attribute__((always_inline)) {
    return irow[min(sub * kTK + (L & (kTK - 1)), topk - 1)];
  };
  bf16x8_t nx[NLD];
  auto load = [&](int ix) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + NT * m, r = c / CPR, p = c % CPR;
      int row = __shfl(ix, r < kTK ? r : 0, 64);
      row = row < 0 || c >= kTK * CPR ? 0 : row;
      nx[m] = *reinterpret_cast<const bf16x8_t*>(kv + (int64_t)row * DQK + 8 * p);
    }
  };
  // threads 0..kTK-1: slot sub kTK + tid; ok: the slot exists and is not -1
  auto finish = [&](int sub, bool ok) __attribute__((always_inline)) {
    const int j = sub * kTK + tid;
    if (j < topk) {
      const float* pp = part + (sub & 1) * NW * kTK + tid;
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < NW; ++v) sum += pp[v * kTK];
      teacher[(int64_t)t * topk + j] = ok ? sum * invH : 0.0f;
    }
  };
  bool okc = false;   // this lane's slot of the previous sub-tile is valid (threads < kTK)
  auto body = [&](int sub, int& ixc, int ixn) __attribute__((always_inline)) {
    char* kt = stage + (sub & 1) * kTK * KRB;
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int c = tid + NT * m, r = c / CPR, p = c % CPR;
      if (c < kTK * CPR) *reinterpret_cast<bf16x8_t*>(kt + r * KRB + 16 * p) = nx[m];
    }
    __syncthreads();
    if (sub + 1 < nsub) load(ixn);
    if (sub > 0 && tid < kTK) finish(sub - 1, okc);
    okc = sub * kTK + L < topk && ixc >= 0;
    ixc = idx_of(sub + 2);
    float* pw = part + (sub & 1) * NW * kTK + w * kTK;
#pragma unroll
    for (int half = 0; half < kTK / 16; ++half) {
      const char* kr = kt + (16 * half + n) * KRB + 16 * g;
      float ps = 0.0f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        if (h0 + kHG * hb < H) {                   // wave-uniform
          floatx4v_t S = floatx4v_t{};
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            S = mfma16x32(qa[hb][ks], *reinterpret_cast<const bf16x8_t*>(kr + 64 * ks), S);
            // a fence every few k-steps keeps the key-row reads from all being hoisted
            // (their registers would not fit beside two head blocks' q operands)
            if (ks % 6 == 5) __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ps += lse2[hb][i] > -__builtin_huge_valf() ? __builtin_amdgcn_exp2f(S[i] * sc2 - lse2[hb][i]) : 0.0f;
        }
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      if (g == 0) pw[16 * half + n] = ps;
    }
  };
  int ixa = 0, ixb = 0;       // indices of sub-tiles of even / odd number
  if (nsub > 0) {
    ixa = idx_of(0);
    ixb = idx_of(1);
    load(ixa);
  }
#pragma unroll 1
  for (int sub = 0; sub < nsub; sub += 2) {
    body(sub, ixa, ixb);
    if (sub + 1 < nsub) body(sub + 1, ixb, ixa);
  }
  __syncthreads();
  if (tid < kTK && nsub > 0) finish(nsub - 1, okc);
}

// Teacher, fp32: one workgroup per (token, head), plain arithmetic; each head adds its
// share exp(s - lse) / H to the slot with an atomic (the slots are zeroed first).
__global__ __launch_bounds__(kNT) void attn_teacher_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, int H, int d_qk, int topk, float scale, float* __restrict__ teacher) {
  const int t = blockIdx.x / H, h = blockIdx.x % H;
  const float* qr = q + ((int64_t)t * H + h) * d_qk;
  const float l = lse[(int64_t)t * H + h];
  const int32_t* ir = idx + (int64_t)t * topk;
  for (int j = threadIdx.x; j < topk; j += kNT) {
    const int r = ir[j];
    if (r < 0 || !(l > -__builtin_huge_valf())) continue;
    const float* kr = kv + (int64_t)r * d_qk;
    float s = 0.0f;
    for (int c = 0; c < d_qk; ++c) s = fmaf(qr[c], kr[c], s);
    atomicAdd(teacher + (int64_t)t * topk + j, expf(s * scale - l) / (float)H);
  }
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

template <int DQK>
hipError_t launch_bwd_bf16(const void* q, const void* kv, const int32_t* idx, const void* dout,
                           const float* lse, int T, int H, int topk, float scale, const float* sink,
                           void* dq, float* dkv, float* dsink, hipStream_t st) {
  const size_t shm = bwd_lds_bytes<DQK>();
  hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_bwd_bf16_kernel<DQK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_mla_bwd_bf16_kernel<DQK>), dim3(T, (H + kHG - 1) / kHG), dim3(kWaves * 64),
                     shm, st, (const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)dout,
                     lse, H, topk, scale, sink, (uint16_t*)dq, dkv, dsink);
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_bwd32(const void* q, const void* kv, const int32_t* idx, const void* dout,
                        const float* lse, int T, int H, int topk, float scale, const float* sink,
                        void* dq, float* dkv, float* dsink, hipStream_t st) {
  const size_t shm = bwd32_lds_bytes<DQK>();
  hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_bwd_h32_kernel<DQK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_mla_bwd_h32_kernel<DQK>), dim3(T, H / kB32), dim3(kWaves * 64), shm, st,
                     (const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)dout, lse, H, topk,
                     scale, sink, (uint16_t*)dq, dkv, dsink);
  return hipGetLastError();
}

// H = 16 NW in {64, 128} (slot rows that fit the dq kernel's LDS): dkv (and D, dsink)
// with all heads per workgroup, then dq by the 64-head kernel.
template <int DQK, int NW>
hipError_t launch_bwd_split(const void* q, const void* kv, const int32_t* idx, const void* dout,
                            const float* lse, int T, int topk, float scale, const float* sink,
                            void* dq, float* dkv, float* dsink, hipStream_t st) {
  const size_t shm_k = dkv_lds_bytes<DQK, NW>();
  hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_bwd_dkv_kernel<DQK, NW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm_k);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_mla_bwd_dkv_kernel<DQK, NW>), dim3(T), dim3(NW * 64), shm_k, st,
                     (const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)dout, lse, topk,
                     scale, sink, (uint16_t*)dq, dkv, dsink);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t shq = dq64_lds_bytes<DQK>(topk);
  e = hipFuncSetAttribute((const void*)sparse_mla_bwd_dq64_kernel<DQK>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)shq);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_mla_bwd_dq64_kernel<DQK>), dim3(T, 16 * NW / kQH), dim3(kWaves * 64), shq, st,
                     (const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)dout, lse, 16 * NW,
                     topk, scale, (uint16_t*)dq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla_bwd(const void* q, const void* kv, const int32_t* idx, const void* dout,
                                 const float* lse, bool bf16, int T, int S, int H, int d_qk, int d_v,
                                 int topk, float scale, const float* sink, void* dq, float* dkv,
                                 float* dsink, hipStream_t st) {
  const int64_t nkv = (int64_t)S * d_qk;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, st, dkv, nkv);
  if (dsink) hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(256), 0, st, dsink, (int64_t)H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  if (bf16) {
    const bool split = d_qk == 576 ? dq64_lds_bytes<576>(topk) <= 160 * 1024 : dq64_lds_bytes<512>(topk) <= 160 * 1024;
    if (H == 128 && split) {
      if (d_qk == 576) return launch_bwd_split<576, 8>(q, kv, idx, dout, lse, T, topk, scale, sink, dq, dkv, dsink, st);
      return launch_bwd_split<512, 8>(q, kv, idx, dout, lse, T, topk, scale, sink, dq, dkv, dsink, st);
    }
    if (H == 64 && split) {
      if (d_qk == 576) return launch_bwd_split<576, 4>(q, kv, idx, dout, lse, T, topk, scale, sink, dq, dkv, dsink, st);
      return launch_bwd_split<512, 4>(q, kv, idx, dout, lse, T, topk, scale, sink, dq, dkv, dsink, st);
    }
    if (H % kB32 == 0) {
      if (d_qk == 576) return launch_bwd32<576>(q, kv, idx, dout, lse, T, H, topk, scale, sink, dq, dkv, dsink, st);
      return launch_bwd32<512>(q, kv, idx, dout, lse, T, H, topk, scale, sink, dq, dkv, dsink, st);
    }
    if (d_qk == 576) return launch_bwd_bf16<576>(q, kv, idx, dout, lse, T, H, topk, scale, sink, dq, dkv, dsink, st);
    return launch_bwd_bf16<512>(q, kv, idx, dout, lse, T, H, topk, scale, sink, dq, dkv, dsink, st);
  }
  const size_t shm = (size_t)(2 * topk + kNT / 64) * sizeof(float);
  e = hipFuncSetAttribute((const void*)sparse_mla_bwd_f32_kernel,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sparse_mla_bwd_f32_kernel, dim3(T * H), dim3(kNT), shm, st, (const float*)q,
                     (const float*)kv, idx, (const float*)dout, lse, H, d_qk, d_v, topk, scale, sink,
                     (float*)dq, dkv, dsink);
  return hipGetLastError();
}

hipError_t launch_attn_teacher(const void* q, const void* kv, const int32_t* idx, const float* lse,
                               bool bf16, int T, int H, int d_qk, int topk, float scale, float* teacher,
                               hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipError_t e;
  if (!bf16) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, st, teacher, (int64_t)T * topk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_teacher_f32_kernel, dim3(T * H), dim3(kNT), 0, st, (const float*)q,
                       (const float*)kv, idx, lse, H, d_qk, topk, scale, teacher);
    return hipGetLastError();
  }
  const dim3 grid(T), block(kTW * 64);
  auto go = [&](auto kern, size_t shm) -> hipError_t {
    hipError_t r = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(kern, grid, block, shm, st, (const uint16_t*)q, (const uint16_t*)kv, idx, lse, H, topk,
                       scale, teacher);
    return hipGetLastError();
  };
  if (d_qk == 576)
    return H > 64 ? go(attn_teacher_bf16_kernel<576, kTW, 2>, teacher_lds_bytes<576>())
                  : go(attn_teacher_bf16_kernel<576, kTW, 1>, teacher_lds_bytes<576>());
  return H > 64 ? go(attn_teacher_bf16_kernel<512, kTW, 2>, teacher_lds_bytes<512>())
                : go(attn_teacher_bf16_kernel<512, kTW, 1>, teacher_lds_bytes<512>());
}

}  // namespace sa
