// Grouped-query attention over selected key blocks (block-routed sparse GQA).
//
// Operation ("Add trainable QSA sparse attention with a TileLang backend", section
// "Describe the solution you'd like": sparse GQA attention over the blocks picked by
// the exact block TopK): query t attends to the set of causal keys s <= t whose local
// block (s - start(t)) / B is listed in blk[t, :] (local block ids of its sequence;
// -1 and blocks past the query's own are skipped; a block listed twice counts once);
// head h uses kv head h / (Hq / Hkv).
//
// bf16 kernel (gfx950): one wave per (token, kv head), four independent waves per
// workgroup. Routes differ from token to token, so the work is a gather: every wave
// streams the keys and values of its own blocks, and the kernel is bound by the
// L2/MALL -> CU bandwidth of those gathers, not by the matrix cores. When Hkv
// divides 8, the workgroups of each XCD serve a single kv head, so an XCD's L2
// caches the keys and values of one head instead of all of them.
//   * the wave's G <= 16 query heads are the 16 columns of 16x16x32 bf16 MFMAs:
//     S^T = K . Q^T (rows = 16 keys), then O^T = V^T . P^T (rows = 16 value
//     channels), so each lane owns one query head's softmax state and output column
//     and every rescale is lane-local;
//   * the route becomes a list of 32-key sub-tiles (one block = B/32 of them, the own
//     block cut at the query); key and value rows of a sub-tile are loaded straight
//     into VGPRs two sub-tiles ahead (no LDS on the load path), so many waves keep
//     many gathers in flight;
//   * K rows are the A operand as loaded; V rows are written to a per-wave LDS stage
//     and read back transposed with ds_read_b64_tr_b16, in the key order of the S^T
//     accumulator, which is P^T's operand layout;
//   * online softmax in exp2 form, fp32 accumulation, no atomics.
// fp32 inputs run a one-wave kernel on 16x16x4 fp32 MFMAs (attn_f32.h).
#include <type_traits>

#include "attn_f32.h"
#include "gqa_group.h"
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxRoute = 64;            // blocks per query row (API limit)
constexpr int kWavesPerGroup = 4;
constexpr float kHeadroom = 8.0f;        // log2 units a row's logits may exceed its reference

typedef float floatx4v_t __attribute__((ext_vector_type(4)));

// Per-wave LDS: value stage of one sub-tile (32 rows x D bf16, 16-byte chunks XOR-
// swizzled by 2 (row mod 8) so that the transposed reads of 16 rows x 32 bytes spread
// over the banks) and the wave's sub-tile list.
template <int D>
constexpr int stage_bytes() { return 32 * D * 2; }
constexpr int kListMax = kMaxRoute * 4;  // sub-tiles per row: B <= 128 -> 4 per block
template <int D>
constexpr int wave_lds_bytes() { return stage_bytes<D>() + kListMax * 8; }

template <int D>
SA_DEVICE int vswz(int row) { return D == 128 ? 2 * (row & 7) : 2 * (row & 3); }

template <int D>
__global__ __launch_bounds__(kWavesPerGroup * 64) void block_gqa_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int T, int Hq,
    int Hkv, int B, int nblk, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    int by_xcd) {
  constexpr int KS = D / 32;             // 32-wide k-steps of S^T
  constexpr int CPR = D * 2 / 16;        // 16-byte chunks per row
  constexpr int VL = 32 * CPR / 64;      // 16-byte value loads per lane per sub-tile
  constexpr int NDT = D / 16;            // 16-row value-channel tiles of O^T
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int w = threadIdx.x >> 6;
  const int L = threadIdx.x & 63;
  int t, g;
  if (by_xcd) {
    // Workgroups are dealt to the 8 XCDs in turn (workgroup b runs on XCD b mod 8).
    // Each XCD serves one kv head (8 / Hkv XCDs per head), so its L2 holds the keys
    // and values of that head only; a workgroup takes 4 consecutive tokens.
    const int b = blockIdx.x, xcd = b & 7, nx = 8 / Hkv;
    g = xcd % Hkv;
    t = ((b >> 3) * nx + xcd / Hkv) * kWavesPerGroup + w;
    if (t >= T) return;                                // whole wave leaves together
  } else {
    const int unit = blockIdx.x * kWavesPerGroup + w;   // (token, kv head) pair
    if ((int64_t)unit >= (int64_t)T * Hkv) return;
    t = unit / Hkv;
    g = unit - t * Hkv;
  }
  const int G = Hq / Hkv;
  char* stage = lds + w * wave_lds_bytes<D>();
  int2* list = reinterpret_cast<int2*>(stage + stage_bytes<D>());
  const int c = cu ? seq_start_of(cu, nseq, t) : 0;
  const int own = (t - c) / B;

  // ---- route -> sub-tile list (s0, nkeys), in slot order; a repeated block is
  //      skipped at its later slots
  int nsub = 0;
  for (int base = 0; base < nblk; base += 64) {
    const int j = base + L;
    const int b = j < nblk ? blk[(int64_t)t * nblk + j] : -1;
    bool ok = b >= 0 && b <= own;
    for (int i = 0; i < nblk; ++i) {                     // earlier slot with the same block?
      if (i >= j) break;
      ok = ok && blk[(int64_t)t * nblk + i] != b;
    }
    const int lo = c + b * B;
    const int nk = ok ? min(B, t - lo + 1) : 0;
    const int ns = (nk + 31) >> 5;
    const uint32_t incl = wave_incl_scan((uint32_t)ns);
    const int pos = nsub + (int)incl - ns;
    for (int h = 0; h < ns; ++h) list[pos + h] = make_int2(lo + 32 * h, min(32, nk - 32 * h));
    nsub += __shfl((int)incl, 63, 64);
  }
  __builtin_amdgcn_wave_barrier();

  // ---- q^T as B operands: column n = L & 15 (query head g*G + n), dims 32ks + 8(L>>4)
  const int n = L & 15;
  const int quad = L >> 4;
  const bool head_ok = n < G;
  bf16x8_t qb[KS];
  {
    const uint16_t* qr = q + ((int64_t)t * Hq + g * G + (head_ok ? n : 0)) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(qr + 32 * ks);
      qb[ks] = head_ok ? x : bf16x8_t{};
    }
  }

  // ---- loads of one sub-tile into registers
  struct Tile {
    bf16x8_t k[2][KS];     // A operands: key 16kt + (L&15), dims 32ks + 8(L>>4)
    bf16x8_t v[VL];        // value rows: chunk p = 64 j + L is row p / CPR, chunk p % CPR
  };
  auto load = [&](int i, Tile& tl) {
    const int2 e = list[i < nsub ? i : 0];
    const int s0 = e.x, nk = e.y;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = 16 * kt + n;
      const int key = r < nk ? s0 + r : s0;
      const uint16_t* kr = k + ((int64_t)key * Hkv + g) * D + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) tl.k[kt][ks] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * ks);
    }
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int p = 64 * j + L;
      const int r = p / CPR;
      const int key = r < nk ? s0 + r : s0;
      tl.v[j] = *reinterpret_cast<const bf16x8_t*>(v + ((int64_t)key * Hkv + g) * D + 8 * (p % CPR));
    }
  };

  floatx4v_t O[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) O[i] = floatx4v_t{};
  float m_run = -__builtin_huge_valf();   // log2 units, same in the 4 lanes of a head
  float l_run = 0.0f;                     // this lane's keys only

  Tile buf[2];
  if (nsub > 0) load(0, buf[0]);
  if (nsub > 1) load(1, buf[1]);

  auto step = [&](int i, Tile& tl) {
    const int nk = list[i].y;
    // value rows -> LDS stage (row-major, swizzled chunks)
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int p = 64 * j + L;
      const int r = p / CPR, ch = p % CPR;
      *reinterpret_cast<bf16x8_t*>(stage + r * (CPR * 16) + ((ch ^ vswz<D>(r)) << 4)) = tl.v[j];
    }
    // S^T = K . Q^T, two 16-key tiles
    floatx4v_t S[2] = {floatx4v_t{}, floatx4v_t{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl.k[kt][ks], qb[ks], S[kt], 0, 0, 0);
    // masked logits in log2 units; this lane's keys are 16 kt + 4 quad + e
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = 16 * kt + 4 * quad + e < nk;
        const float x = ok ? S[kt][e] * scale_log2 : -__builtin_huge_valf();
        S[kt][e] = x;
        mx = __builtin_elementwise_maximum(mx, x);
      }
    mx = quad_max(mx);
    const float m_new = __builtin_elementwise_maximum(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -inf
    m_run = m_new;
    if (ballot(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < NDT; ++i) O[i] *= alpha;
    }
    l_run *= alpha;
    // P^T as the B operand: k slots 0..3 = keys 4 quad + e, 4..7 = keys 16 + 4 quad + e
    float pf[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[4 * kt + e] = __builtin_amdgcn_exp2f(S[kt][e] - m_new);
        l_run += pf[4 * kt + e];
      }
    bf16x2_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = __builtin_convertvector((float2_t){pf[2 * e], pf[2 * e + 1]}, bf16x2_t);
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
    __builtin_amdgcn_wave_barrier();
    // O^T += V^T . P^T; V^T's A operand read transposed from the stage
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      // lane (quad, n) reads row 4 quad + n/4 (+16 for the second key half), channels
      // 16 dt + 4 (n & 3) .. +3: the transposed read hands it channel 16 dt + n of 4 keys
      short4_t lo, hi;
      {
        const int row0 = 4 * quad + (n >> 2);
        const int col = 16 * dt + 4 * (n & 3);
        const int off0 = row0 * (CPR * 16) + (((col >> 3) ^ vswz<D>(row0)) << 4) + (col & 7) * 2;
        const int row1 = row0 + 16;
        const int off1 = row1 * (CPR * 16) + (((col >> 3) ^ vswz<D>(row1)) << 4) + (col & 7) * 2;
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(stage + off0));
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(stage + off1));
      }
      const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                            hi[0], hi[1], hi[2], hi[3]};
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a8), pb, O[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

#pragma unroll 1
  for (int i = 0; i < nsub; i += 2) {
    step(i, buf[0]);
    if (i + 2 < nsub) load(i + 2, buf[0]);
    if (i + 1 < nsub) {
      step(i + 1, buf[1]);
      if (i + 3 < nsub) load(i + 3, buf[1]);
    }
  }

  // ---- normalise and write: lane owns head n, channels 16 dt + 4 quad + e
  const float l_tot = quad_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (head_ok) {
    uint16_t* orow = out + ((int64_t)t * Hq + g * G + n) * D + 4 * quad;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint32_t pk0 = pack_bf16x2(O[dt][0] * inv, O[dt][1] * inv);
      uint32_t pk1 = pack_bf16x2(O[dt][2] * inv, O[dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pk0, pk1);
    }
    if (lse && quad == 0)
      lse[(int64_t)t * Hq + g * G + n] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_huge_valf();
  }
}

// Grouped bf16 kernel: one workgroup per (group of GT consecutive tokens, kv head),
// eight waves. Neighbouring tokens' routes overlap, so the group loads every block of
// the union of its tokens' routes once, into LDS, and runs all of the group's
// GT x G query rows (at most 128: one 16-row column tile per wave) over it as a dense
// tile, masking each (row, key) by route membership and causality:
//   * set-up: the routes' blocks, as key rows start + b B, are marked in a bitmap over
//     the group's key range; a prefix count over its words numbers the distinct blocks
//     in ascending key order, and each route entry ORs its token into its block's mask;
//   * the blocks go in 32-key pieces, two per step (one barrier each): K and V rows
//     are copied straight from memory into a four-piece LDS ring by 16-byte
//     global_load_lds with a scalar row base and fixed per-lane offsets, the next
//     step's pieces while the current step's are computed; both regions are
//     XOR-swizzled per row, K for the operand reads of S^T = K . Q^T (16x16x32), V for
//     the transposed reads of O^T = V^T . P^T. The step is written out once per half of
//     the ring, so every LDS address is a lane offset plus an immediate, and each
//     piece's description (first key, keys, token mask) sits in scalar registers, read
//     from the tables once per block. Every wave copies every piece, so this per-piece
//     work is what the waves that skip a piece still pay;
//   * a wave skips the MFMAs of a piece none of its rows' tokens routes to; the two
//     pieces of a step share one online-softmax update (one max, one rescale test); a
//     row ignores masked keys exactly (p 0) and rescales O only when a logit passes the
//     row's reference by more than 2^8.
// Measured on the block-routed workload: two workgroups of four waves with two column
// tiles each, one sub-tile ahead, 0.89 ms; skipping per column tile 0.79; two sub-tiles
// ahead 0.77; eight waves of one tile (twice the waves per SIMD) 0.68; fixed softmax
// reference 0.58; copies with scalar bases and piece descriptions in scalar registers
// instead of per-lane 64-bit addresses and table reads per copy, 0.50; two pieces per
// barrier, 0.48 (the same change had measured 4 % slower while the copies still paid
// per-lane addresses). 256-row groups were no faster.
// Blocks are visited in ascending key order, the same for every row of the group.
constexpr int kGrpRing = 4;                      // pieces in the LDS ring (two steps)

template <int D>
constexpr int piece_bytes() { return 2 * 32 * D * 2; }   // K rows, then V rows

// K-region chunk swizzle: the 16 rows of an operand read land on distinct chunks.
template <int D>
SA_DEVICE int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }

size_t grp_lds_bytes(int D, int G, int nblk, int maxlen) {
  const size_t st = D == 128 ? piece_bytes<128>() : piece_bytes<64>();
  return kGrpRing * st + grp_table_bytes(grp_tokens(G), nblk, maxlen);
}

// 16-byte global -> LDS copy per lane: lane l writes LDS bytes [lds + 16 l, +16); lds
// and base are wave-uniform, voff is the lane's byte offset from base. Issued through inline asm so that later LDS reads are not ordered
// behind it; completion is tracked with s_waitcnt vmcnt. M0 is set here and nowhere
// else in these kernels.
SA_DEVICE void grp_dma16(uint32_t lds, const void* base, uint32_t voff) {
  // readfirstlane returns a signed int: zero-extend each half before recombining
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(sb)
               : "memory");
}

// s_waitcnt vmcnt(0) with the other counters left alone.
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);

template <int D>
__global__ __launch_bounds__(kGrpWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void block_gqa_group_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int T, int Hq,
    int Hkv, int B, int nblk, int GT, int nwords, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int by_xcd) {
  constexpr int KS = D / 32;             // 32-wide k-steps of S^T
  constexpr int CPR = D * 2 / 16;        // 16-byte chunks per row
  constexpr int RB = CPR * 16;           // bytes per row in a region
  constexpr int NDT = D / 16;            // 16-channel tiles of O^T
  constexpr int PB = piece_bytes<D>();
  constexpr int NT = kGrpWaves * 64;
  constexpr int DPP = 2 * 32 * CPR / 64; // 1 KiB copies per piece (K and V)
  static_assert(DPP % kGrpWaves == 0 && DPP % 2 == 0, "copies split evenly");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const GroupTables tbl = group_tables(lds + kGrpRing * PB, GT, nblk, nwords);
  const int32_t* ulo = tbl.ulo;
  const uint32_t* umask = tbl.umask;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(SA_LDS char*)lds;

  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int n = L & 15, quad = L >> 4;
  const int G = Hq / Hkv;
  const int ngrp = (T + GT - 1) / GT;
  int grp, g;
  if (by_xcd) {
    // workgroup b runs on XCD b mod 8; each XCD serves one kv head (8 / Hkv XCDs per
    // head); groups go from the last (the widest routes' unions) to the first
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

  // ---- set-up: distinct blocks of the group's routes, ascending, with token masks
  const int nu = group_union<NT>(tbl, blk, cu, nseq, t0, tlast, GT, B, nblk, base, nwords);

  // ---- this lane's query row: column tile w, row 16 w + n (token tau, head h)
  const int row = 16 * w + n;
  const int tau = row / G;
  const int tq = t0 + tau;
  const bool row_ok = tau < GT && row < GT * G && tq <= tlast;
  const int hq = row - tau * G;
  bf16x8_t qb[KS];
  {
    const uint16_t* qr = q + ((int64_t)(row_ok ? tq : t0) * Hq + g * G + hq) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(qr + 32 * ks);
      qb[ks] = row_ok ? x : bf16x8_t{};
    }
  }
  uint32_t tile_tok = row_ok ? (1u << tau) : 0u;     // tokens of the wave's rows (uniform)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) tile_tok |= (uint32_t)__shfl_xor((int)tile_tok, off, 64);

  floatx4v_t O[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) O[i] = floatx4v_t{};
  float m_run = -__builtin_huge_valf();   // log2 units, same in the 4 lanes of a row
  float l_run = 0.0f;                     // this lane's keys only

  // pieces: for each distinct block u, keys ulo[u] .. min(ulo[u] + B, tlast + 1) - 1 in
  // 32-key pieces, walked in order. A piece's description (block, piece of the block,
  // first key, keys, keys of its block, token mask) is wave-uniform and lives in scalar
  // registers; the LDS tables are read once per block.
  struct Piece {
    int u, pc, lo, nk, kof;
    uint32_t m;
  };
  auto first_of = [&](int u) __attribute__((always_inline)) {
    Piece p{u, 0, 0, 0, 0, 0u};
    if (u < nu) {
      p.lo = __builtin_amdgcn_readfirstlane(ulo[u]);
      p.m = (uint32_t)__builtin_amdgcn_readfirstlane((int)umask[u]);
      p.kof = min(B, tlast + 1 - p.lo);
      p.nk = min(32, p.kof);
    }
    return p;
  };
  auto next_of = [&](const Piece& a) __attribute__((always_inline)) {
    Piece p = a;
    if (a.u < nu) {
      if (32 * (a.pc + 1) < a.kof) {
        p.pc = a.pc + 1;
        p.lo = a.lo + 32;
        p.nk = min(32, a.kof - 32 * p.pc);
      } else {
        p = first_of(a.u + 1);
      }
    }
    return p;
  };

  // copies: wave w moves DP1 of a piece's 1 KiB runs (K rows, then V rows); lane L of
  // run j holds row r, chunk slot L mod CPR (the swizzled chunk ch of the source row).
  // Rows past a piece's last key repeat its first key.
  constexpr int DP1 = DPP / kGrpWaves;
  uint32_t voff[DP1], voff0[DP1];
  int vrow[DP1];
#pragma unroll
  for (int i = 0; i < DP1; ++i) {
    const int j = w * DP1 + i;
    const int isv = j >= DPP / 2;
    const int jj = j - isv * (DPP / 2);
    const int r = jj * (64 / CPR) + L / CPR;
    const int ch = (L % CPR) ^ (isv ? vswz<D>(r) : kswz<D>(r));
    vrow[i] = r;
    voff0[i] = (uint32_t)ch * 16u;
    voff[i] = (uint32_t)r * (uint32_t)(Hkv * D * 2) + voff0[i];
  }
  auto fetch = [&](const Piece& p, int slot) __attribute__((always_inline)) {
    if (p.u < nu) {                                     // uniform
#pragma unroll
      for (int i = 0; i < DP1; ++i) {
        const int j = w * DP1 + i;
        const int isv = j >= DPP / 2;
        const int jj = j - isv * (DPP / 2);
        const uint16_t* src = (isv ? v : k) + ((int64_t)p.lo * Hkv + g) * D;
        grp_dma16(lds0 + (uint32_t)(slot * PB + isv * 32 * RB + jj * 1024), src,
                  vrow[i] < p.nk ? voff[i] : voff0[i]);
      }
    }
  };

  // S^T of one piece: rows = keys 16 kt + (0..15), columns = the wave's 16 query rows
  auto logits = [&](const char* st, floatx4v_t* S) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int r = 16 * kt + n;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(st + r * RB + (((4 * ks + quad) ^ kswz<D>(r)) << 4));
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], S[kt], 0, 0, 0);
      }
  };
  // O^T += V^T . P^T of one piece (P^T: this lane's 8 keys 4 quad + e, 16 + 4 quad + e)
  auto values = [&](const char* st, bf16x8_t pb) __attribute__((always_inline)) {
    const char* vst = st + 32 * RB;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int row0 = 4 * quad + (n >> 2);
      const int col = 16 * dt + 4 * (n & 3);
      const int off0 = row0 * RB + (((col >> 3) ^ vswz<D>(row0)) << 4) + (col & 7) * 2;
      const int row1 = row0 + 16;
      const int off1 = row1 * RB + (((col >> 3) ^ vswz<D>(row1)) << 4) + (col & 7) * 2;
      const short4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(vst + off0));
      const short4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(vst + off1));
      const short __attribute__((ext_vector_type(8))) a8 = {lo4[0], lo4[1], lo4[2], lo4[3],
                                                            hi4[0], hi4[1], hi4[2], hi4[3]};
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a8), pb, O[dt], 0, 0, 0);
    }
  };

  Piece p0 = first_of(0);
  Piece p1 = next_of(p0);
  fetch(p0, 0);
  fetch(p1, 1);
  // one step: pieces p0 and p1 in ring slots SA and SA + 1 (constants, so every LDS
  // address is a lane offset plus an immediate); wait for their copies (the only ones
  // in flight), barrier, copy the next step's two pieces into the other half of the ring
  // (free once every wave has passed the barrier), then compute both pieces with one
  // online-softmax update
  auto step2 = [&](auto sa_c) __attribute__((always_inline)) {
    constexpr int SA = decltype(sa_c)::value;
    const Piece p2 = next_of(p1);
    const Piece p3 = next_of(p2);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    fetch(p2, (SA + 2) & 3);
    fetch(p3, (SA + 3) & 3);
    const char* stA = lds + SA * PB;
    const char* stB = stA + PB;
    const bool cA = (p0.m & tile_tok) != 0u, cB = (p1.m & tile_tok) != 0u;
    if (cA || cB) {
      floatx4v_t S[4] = {floatx4v_t{}, floatx4v_t{}, floatx4v_t{}, floatx4v_t{}};
      if (cA) logits(stA, S);
      __builtin_amdgcn_sched_barrier(0);          // (keeps the register peak of the two pieces apart)
      if (cB) logits(stB, S + 2);
      // keys 4 quad + e (+16) of a piece count below its lim: the row routes there, the
      // key is in the piece and causal for the row
      const int limA = (row_ok && ((p0.m >> tau) & 1u)) ? min(p0.nk, tq - p0.lo + 1) - 4 * quad : 0;
      const int limB = (row_ok && ((p1.m >> tau) & 1u)) ? min(p1.nk, tq - p1.lo + 1) - 4 * quad : 0;
      // logits in log2 units relative to the row's reference m_run (absolute for a row
      // that has no reference yet), -inf where the row does not route to the piece: one
      // fma per logit; only a piece in which some row's causal limit falls (uniform
      // test) masks key by key
      const bool seen = m_run != -__builtin_huge_valf();
      const float ref = seen ? -m_run : 0.0f;
      const float bA = limA > 0 ? ref : -__builtin_huge_valf();
      const float bB = limB > 0 ? ref : -__builtin_huge_valf();
      float x[16];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[4 * kt + e] = fmaf(S[kt][e], scale_log2, bA);
          x[8 + 4 * kt + e] = fmaf(S[2 + kt][e], scale_log2, bB);
        }
      if (ballot(limA > 0 && limA < 20)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[4 * kt + e] = 16 * kt + e < limA ? x[4 * kt + e] : -__builtin_huge_valf();
      }
      if (ballot(limB > 0 && limB < 20)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[8 + 4 * kt + e] = 16 * kt + e < limB ? x[8 + 4 * kt + e] : -__builtin_huge_valf();
      }
      float mx[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = __builtin_elementwise_maximum(x[2 * i], x[2 * i + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = __builtin_elementwise_maximum(mx[2 * i], mx[2 * i + 1]);
      float m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx[0], mx[1]),
                                              __builtin_elementwise_maximum(mx[2], mx[3]));
      m = quad_max(m);
      // fixed reference: a row takes a new one at its first keys and when a max passes
      // the reference by more than 2^8; O and l are rescaled then only
      const bool up = m > -__builtin_huge_valf() && (!seen || m > kHeadroom);
      if (ballot(up)) {                                  // uniform
        const float alpha = up && seen ? __builtin_amdgcn_exp2f(-m) : 1.0f;
        const float shift = up ? m : 0.0f;
        m_run = up ? (seen ? m_run + m : m) : m_run;
#pragma unroll
        for (int i = 0; i < NDT; ++i) O[i] *= alpha;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] -= shift;
      }
      // P of each piece (bf16, the B operand of O^T += V^T . P^T), then its values
      auto probs = [&](int o) __attribute__((always_inline)) {
        float pf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[i] = __builtin_amdgcn_exp2f(x[o + i]);
        l_run += ((pf[0] + pf[1]) + (pf[2] + pf[3])) + ((pf[4] + pf[5]) + (pf[6] + pf[7]));
        bf16x2_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = __builtin_convertvector((float2_t){pf[2 * e], pf[2 * e + 1]}, bf16x2_t);
        return __builtin_bit_cast(bf16x8_t, pk);
      };
      if (cA) values(stA, probs(0));
      __builtin_amdgcn_sched_barrier(0);
      if (cB) values(stB, probs(8));
    }
    p0 = p2;
    p1 = p3;
  };
#pragma unroll 1
  for (;;) {                                            // uniform exits
    if (p0.u >= nu) break;
    step2(std::integral_constant<int, 0>{});
    if (p0.u >= nu) break;
    step2(std::integral_constant<int, 2>{});
  }

  // ---- normalise and write: lane owns row 16 w + n, channels 16 dt + 4 quad + e
  const float l_tot = quad_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
    uint16_t* orow = out + ((int64_t)tq * Hq + g * G + hq) * D + 4 * quad;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint32_t pk0 = pack_bf16x2(O[dt][0] * inv, O[dt][1] * inv);
      uint32_t pk1 = pack_bf16x2(O[dt][2] * inv, O[dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(pk0, pk1);
    }
    if (lse && quad == 0)
      lse[(int64_t)tq * Hq + g * G + hq] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_huge_valf();
  }
}

// fp32 inputs: one wave per (token, kv head) on 16x16x4 fp32 MFMAs (the wave routine
// of attn_f32.h). The route becomes a list of 16-key sub-tiles as in the bf16 kernel,
// the G query heads are the MFMA columns and key and value rows are read straight
// from memory.
template <int D>
__global__ __launch_bounds__(64) void block_gqa_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ cu, int nseq, int Hq, int Hkv,
    int B, int nblk, float scale_log2, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int ldq = D + 4;
  constexpr int kList16 = kMaxRoute * 8;  // 16-key sub-tiles per row: B <= 128 -> 8 per block
  __shared__ __attribute__((aligned(16))) float sq[16 * ldq];
  __shared__ int2 list[kList16];
  const int t = blockIdx.x, g = blockIdx.y, L = threadIdx.x;
  const int G = Hq / Hkv;
  const int c = cu ? seq_start_of(cu, nseq, t) : 0;
  const int own = (t - c) / B;
  const int32_t* __restrict__ brow = blk + (int64_t)t * nblk;
  int nsub = 0;
  for (int base = 0; base < nblk; base += 64) {
    const int j = base + L;
    const int b = j < nblk ? brow[j] : -1;
    bool ok = b >= 0 && b <= own;
    for (int i = 0; i < j && ok; ++i) ok = brow[i] != b;   // a repeated block counts once
    const int lo = c + b * B;
    const int nk = ok ? min(B, t - lo + 1) : 0;
    const int ns = (nk + 15) >> 4;
    const uint32_t incl = wave_incl_scan((uint32_t)ns);
    const int pos = nsub + (int)incl - ns;
    for (int h = 0; h < ns; ++h) list[pos + h] = make_int2(lo + 16 * h, min(16, nk - 16 * h));
    nsub += __shfl((int)incl, 63, 64);
  }
  stage_q_f32<D>(q + ((int64_t)t * Hq + g * G) * D, G, sq);
  __syncthreads();
  WaveAttnF32<D, D> at;
  at.init();
#pragma unroll 1
  for (int i = 0; i < nsub; ++i) {
    const int2 e = list[i];
    auto keys = [&](int r, const float*& kr, const float*& vr) {
      const int64_t row = ((int64_t)(e.x + (r < e.y ? r : 0)) * Hkv + g) * D;
      kr = k + row;
      vr = v + row;
      return r < e.y;
    };
    at.tile(sq, ldq, scale_log2, keys);
  }
  at.finish(G, nullptr, out + ((int64_t)t * Hq + g * G) * D, D,
            lse ? lse + (int64_t)t * Hq + g * G : nullptr);
}

template <int D>
hipError_t launch_grouped(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                          const int32_t* cu, int nseq, int maxlen, int Hq, int Hkv, int B, int nblk,
                          float scale, void* out, float* lse, hipStream_t st) {
  const int G = Hq / Hkv;
  const int GT = grp_tokens(G);
  const int nwords = grp_words(maxlen, GT);
  const size_t shm = grp_lds_bytes(D, G, nblk, maxlen);
  if (shm > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)block_gqa_group_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  const int by_xcd = 8 % Hkv == 0;
  const int64_t ngrp = ((int64_t)T + GT - 1) / GT;
  int64_t grid = by_xcd ? (ngrp + 8 / Hkv - 1) / (8 / Hkv) * 8 : ngrp * Hkv;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_gqa_group_kernel<D>), dim3((unsigned)grid), dim3(kGrpWaves * 64), shm,
                     st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, blk, cu, nseq, T,
                     Hq, Hkv, B, nblk, GT, nwords, scale * kLog2e, (uint16_t*)out, lse, by_xcd);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                       const int32_t* cu, int nseq, int Hq, int Hkv, int B, int nblk, float scale,
                       void* out, float* lse, hipStream_t st) {
  const size_t shm = (size_t)kWavesPerGroup * wave_lds_bytes<D>();
  const int by_xcd = 8 % Hkv == 0;
  int64_t grid;
  if (by_xcd) {
    const int64_t groups = ((int64_t)T + kWavesPerGroup - 1) / kWavesPerGroup;
    const int nx = 8 / Hkv;
    grid = (groups + nx - 1) / nx * 8;
  } else {
    grid = ((int64_t)T * Hkv + kWavesPerGroup - 1) / kWavesPerGroup;
  }
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_gqa_bf16_kernel<D>), dim3((unsigned)grid), dim3(kWavesPerGroup * 64), shm,
                     st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, blk, cu, nseq, T,
                     Hq, Hkv, B, nblk, scale * kLog2e, (uint16_t*)out, lse, by_xcd);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const void* q, const void* k, const void* v, const int32_t* blk, int T,
                      const int32_t* cu, int nseq, int Hq, int Hkv, int B, int nblk, float scale,
                      void* out, float* lse, hipStream_t st) {
  hipLaunchKernelGGL((block_gqa_f32_kernel<D>), dim3(T, Hkv), dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, blk, cu, nseq, Hq, Hkv, B, nblk,
                     scale * kLog2e, (float*)out, lse);
  return hipGetLastError();
}

}  // namespace

int block_gqa_max_route() { return kMaxRoute; }

hipError_t launch_block_gqa(const void* q, const void* k, const void* v, const int32_t* blk,
                            bool bf16, int T, const int32_t* cu, int nseq, int maxlen, int Hq, int Hkv,
                            int D, int Dv, int block_size, int nblk, float scale, void* out, float* lse,
                            hipStream_t st) {
  (void)Dv;
  if (T == 0) return hipSuccess;
  const int ns = cu ? nseq : 1;
  if (bf16) {
    // the grouped kernel when its set-up tables fit the LDS (rows up to ~150K keys)
    if (grp_lds_bytes(D, Hq / Hkv, nblk, maxlen) <= 160 * 1024) {
      if (D == 64)
        return launch_grouped<64>(q, k, v, blk, T, cu, ns, maxlen, Hq, Hkv, block_size, nblk, scale, out, lse, st);
      return launch_grouped<128>(q, k, v, blk, T, cu, ns, maxlen, Hq, Hkv, block_size, nblk, scale, out, lse, st);
    }
    if (D == 64) return launch_bf16<64>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, out, lse, st);
    return launch_bf16<128>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, out, lse, st);
  }
  if (D == 64) return launch_f32<64>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, out, lse, st);
  return launch_f32<128>(q, k, v, blk, T, cu, ns, Hq, Hkv, block_size, nblk, scale, out, lse, st);
}

}  // namespace sa
