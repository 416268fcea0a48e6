// Device helpers shared by the gfx950 kernels of the sparse-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SA_DEVICE __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

#define SA_LDS __attribute__((address_space(3)))

namespace sa {

constexpr int kWave = 64;

SA_DEVICE int lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane (wave-wide exclusive prefix count).
SA_DEVICE uint32_t mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

SA_DEVICE uint64_t ballot(bool p) { return __ballot(p); }

// Order-preserving map fp32 -> uint32 for finite values and +-inf: a > b as floats
// iff key(a) > key(b) as unsigned. -0.0 is canonicalised to +0.0 first so the two
// zeros tie. Every finite value maps above 0x007FFFFF, so 0 is free as "no value".
SA_DEVICE uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

SA_DEVICE float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
SA_DEVICE uint16_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

SA_DEVICE float bf_bits2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Packs two floats into one dword of two bf16 (low half = a).
SA_DEVICE uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f2bf_bits(a) | ((uint32_t)f2bf_bits(b) << 16);
}

// Start row of the packed sequence that holds row t (cu: int32 [nseq+1], ascending).
SA_DEVICE int seq_start_of(const int32_t* __restrict__ cu, int nseq, int t) {
  int lo = 0, hi = nseq;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (__ldg(cu + mid) <= t) lo = mid; else hi = mid;
  }
  return __ldg(cu + lo);
}

// Wave-wide inclusive scan of a 32-bit value: shifts by 1, 2, 4 and 8 inside each row
// of 16 lanes, then row 0's last lane into row 1 (and 2's into 3), then lane 31 into
// rows 2 and 3 (DPP row shifts and row broadcasts; out-of-row sources read 0).
SA_DEVICE uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// The values of lane i mod 32 and lane i mod 32 + 32 of `x`, in every lane i (one
// v_permlane32_swap, no LDS round trip): .x from the lower half, .y from the upper.
SA_DEVICE float2_t lane_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (float2_t){__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// The values of lanes i and i ^ 16 of `x` (one v_permlane16_swap): .x from the lane
// whose bit 4 is clear, .y from the one whose bit 4 is set.
SA_DEVICE float2_t lane_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (float2_t){__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Max and sum over the four lanes (i mod 16) + 16 r, r = 0..3 (the lanes that share a
// column of a 16x16 MFMA tile), in every one of them.
SA_DEVICE float quad_max(float x) {
  const float2_t a = lane_rows16(x);
  const float y = __builtin_elementwise_maximum(a.x, a.y);
  const float2_t b = lane_halves(y);
  return __builtin_elementwise_maximum(b.x, b.y);
}
SA_DEVICE float quad_sum(float x) {
  const float2_t a = lane_rows16(x);
  const float y = a.x + a.y;
  const float2_t b = lane_halves(y);
  return b.x + b.y;
}

// x from another lane through one DPP move (CTRL a constant dpp_ctrl code).
template <int CTRL>
SA_DEVICE float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max over the aligned groups of B lanes (B a power of two, 1..64), in every lane of
// each group: two quad permutes, the half-row and row mirrors, then the 16- and
// 32-lane swaps. Each step pairs every lane with one of the other half of its group,
// so no value goes through LDS.
SA_DEVICE float group_max(float x, int B) {
  // elementwise_maximum (v_maximum3) needs no quieting of its inputs, where fmaxf pays
  // a canonicalising max per operand; the values here are never NaN
  if (B >= 2) x = __builtin_elementwise_maximum(x, dpp_f32<0xB1>(x));    // quad_perm [1,0,3,2]
  if (B >= 4) x = __builtin_elementwise_maximum(x, dpp_f32<0x4E>(x));    // quad_perm [2,3,0,1]
  if (B >= 8) x = __builtin_elementwise_maximum(x, dpp_f32<0x141>(x));   // row_half_mirror
  if (B >= 16) x = __builtin_elementwise_maximum(x, dpp_f32<0x140>(x));  // row_mirror
  if (B >= 32) { const float2_t r = lane_rows16(x); x = __builtin_elementwise_maximum(r.x, r.y); }
  if (B >= 64) { const float2_t h = lane_halves(x); x = __builtin_elementwise_maximum(h.x, h.y); }
  return x;
}

SA_DEVICE float wave_max(float x) { return group_max(x, kWave); }

SA_DEVICE void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace sa
