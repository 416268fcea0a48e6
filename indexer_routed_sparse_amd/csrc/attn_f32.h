// fp32 attention of one wave over a stream of 16-key sub-tiles, on 16x16x4 fp32
// MFMAs (v_mfma_f32_16x16x4_f32), with an online softmax in exp2 form.
//
// Lane layouts of the instruction (A 16x4, B 4x16, C 16x16): lane L supplies
// A[L%16][L/16] and B[L/16][L%16] and holds C[4(L/16) + i][L%16], i = 0..3.
//
// The wave owns up to 16 query heads, one per MFMA column n = L%16, and computes
//   S^T[key][h] = K[key] . q[h]    A = key rows, B = q^T. At k-step (j, i) the
//                                  channel is 16j + 4(L/16) + i, so a lane loads one
//                                  float4 of its key row and of its q row per j;
//   O^T[c][h] += V[key][c] P[key][h]   A = V^T, B = P^T. The S^T accumulator of lane
//                                  (n, g) holds keys 4g..4g+3 of head n, which is the
//                                  B operand of k-steps 0..3 as it stands. Row m of
//                                  channel tile 4a + b is channel 64a + 4m + b, so the
//                                  A values a lane needs for tiles 4a..4a+3 form one
//                                  float4 of a value row, and a lane's results for the
//                                  four tiles cover 16 consecutive channels.
// The softmax state of a head lives in the four lanes of its column: every rescale
// is lane-local and only the row max and the final sum cross lanes.
#pragma once

#include "sa_common.h"

namespace sa {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

SA_DEVICE f32x4_t mfma_f32_16x16x4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DQK, int DV>
struct WaveAttnF32 {
  static constexpr int NJ = DQK / 16;   // float4 k-chunks of a key row per lane
  static constexpr int NA = DV / 64;    // 64-channel groups of O^T
  static_assert(DQK % 16 == 0 && DV % 64 == 0, "tile shapes");
  f32x4_t O[4 * NA];
  float m;   // running max of head n's scaled logits, log2 units (same in its 4 lanes)
  float l;   // running sum over this lane's keys

  SA_DEVICE void init() {
#pragma unroll
    for (int i = 0; i < 4 * NA; ++i) O[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m = -__builtin_huge_valf();
    l = 0.0f;
  }

  // One sub-tile. sq: q rows of the 16 head columns in LDS, row stride ldq floats
  // (zero rows for absent heads). c2: softmax scale times log2(e). keys(r, kr, vr)
  // sets the key and value row pointers of key r (0..15) of the sub-tile and returns
  // false for a hole (the pointers must still address a readable row).
  template <class Keys>
  SA_DEVICE void tile(const float* sq, int ldq, float c2, const Keys& keys) {
    const int L = lane_id(), n = L & 15, g = L >> 4;
    const float* kr;
    const float* vr;
    const bool okn = keys(n, kr, vr);
    const uint32_t vm = (uint32_t)ballot(okn) & 0xFFFFu;   // validity of keys 0..15
    f32x4_t S = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const float* qp = sq + n * ldq + 4 * g;
    const float* kp = kr + 4 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(kp + 16 * j);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(qp + 16 * j);
      S = mfma_f32_16x16x4(a.x, b.x, S);
      S = mfma_f32_16x16x4(a.y, b.y, S);
      S = mfma_f32_16x16x4(a.z, b.z, S);
      S = mfma_f32_16x16x4(a.w, b.w, S);
    }
    // keys 4g + r of head n
    float s[4], mx = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = (vm >> (4 * g + r)) & 1u ? S[r] * c2 : -__builtin_huge_valf();
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const bool none = mn == -__builtin_huge_valf();          // no valid key yet
    const float al = none ? 1.0f : exp2f(m - mn);
    float p[4], ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = none ? 0.0f : exp2f(s[r] - mn);
      ps += p[r];
    }
    l = l * al + ps;
    m = mn;
#pragma unroll
    for (int i = 0; i < 4 * NA; ++i) O[i] *= al;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* kx;
      const float* vx;
      const bool ok = keys(4 * g + r, kx, vx);
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(vx + 64 * a + 4 * n);
        if (!ok) v = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        O[4 * a + 0] = mfma_f32_16x16x4(v.x, p[r], O[4 * a + 0]);
        O[4 * a + 1] = mfma_f32_16x16x4(v.y, p[r], O[4 * a + 1]);
        O[4 * a + 2] = mfma_f32_16x16x4(v.z, p[r], O[4 * a + 2]);
        O[4 * a + 3] = mfma_f32_16x16x4(v.w, p[r], O[4 * a + 3]);
      }
    }
  }

  // Normalises and stores head column n (if n < nh): out row at orow + n * ostride,
  // lse (natural log) at lrow[n] if lrow. sink: the head's sink logit (natural units,
  // nullptr for none), which joins the denominator only.
  SA_DEVICE void finish(int nh, const float* sink, float* orow, int64_t ostride, float* lrow) {
    const int L = lane_id(), n = L & 15, g = L >> 4;
    float lt = l + __shfl_xor(l, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (n >= nh) return;
    constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
    const float s2 = sink ? sink[n] * kLog2e : -__builtin_huge_valf();
    const float M = fmaxf(m, s2);
    const float em = m == -__builtin_huge_valf() ? 0.0f : exp2f(m - M);
    const float den = lt * em + (s2 == -__builtin_huge_valf() ? 0.0f : exp2f(s2 - M));
    const float inv = den > 0.0f ? em / den : 0.0f;
    float* o = orow + (int64_t)n * ostride + 16 * g;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4_t x = f32x4_t{O[4 * a + 0][r], O[4 * a + 1][r], O[4 * a + 2][r], O[4 * a + 3][r]} * inv;
        *reinterpret_cast<f32x4_t*>(o + 64 * a + 4 * r) = x;
      }
    if (lrow && g == 0) {
      float ls;
      if (lt > 0.0f) ls = (M + __log2f(den)) * kLn2;
      else ls = sink ? sink[n] : -__builtin_huge_valf();    // only the sink, or nothing
      lrow[n] = ls;
    }
  }
};

// Loads the q rows of `nh` heads (row stride DQK floats, from qrow) into the wave's LDS
// rows of stride DQK + 4; rows nh..15 are zero-filled.
template <int DQK>
SA_DEVICE void stage_q_f32(const float* __restrict__ qrow, int nh, float* sq) {
  constexpr int ldq = DQK + 4, C4 = DQK / 4;
  for (int i = lane_id(); i < 16 * C4; i += kWave) {
    const int h = i / C4, c = i - h * C4;
    f32x4_t x = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (h < nh) x = *reinterpret_cast<const f32x4_t*>(qrow + (int64_t)h * DQK + 4 * c);
    *reinterpret_cast<f32x4_t*>(sq + h * ldq + 4 * c) = x;
  }
}

}  // namespace sa
