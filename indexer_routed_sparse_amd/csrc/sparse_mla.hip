// Absorbed-MLA sparse attention forward over selected latent rows.
//
// Operation ("Support NoPE shapes and unaligned top-k in TileLang sparse MLA",
// section "What does this PR do?", and the GLM-5.3-Flash PR body quoted there,
// section "Change"): for query t and head h, softmax over the valid slots j of
// scale * q[t,h,:] . kv[idx[t,j], :] (d_qk = 576 or 512 channels), weights applied
// to kv[idx[t,j], 0:512]; -1 slots are masked; the caller's scale is used as given.
//
// bf16 kernel (gfx950), one workgroup per query token, NW = ceil(H / 32) waves:
//   * logits: wave w computes S^T = K . Q^T for heads [32w, 32w+32) (32x32x16 bf16
//     MFMA, rows = keys, columns = heads); the token's q slices are its B operands,
//     loaded once and held in VGPRs and LDS;
//   * the selected latent rows of a 32-key tile are gathered straight from HBM/L2
//     into LDS with 16-byte global_load_lds (no register staging), double
//     buffered: the gather of tile n+1 is in flight while tile n is computed;
//   * the LDS tile is row-major with an XOR swizzle of the 16-byte chunks so that
//     both the K reads (ds_read_b128) and the V reads are free of bank conflicts;
//   * P = exp2(S - m) is packed to bf16 in the A-operand layout of P . V: the S^T
//     accumulator layout already is that layout up to a permutation of keys inside
//     the tile. Each wave publishes its 32 heads' P in LDS;
//   * values: wave w accumulates O for ALL heads over output channels
//     [512w/NW, 512(w+1)/NW), so every V element is read from LDS once per tile (the
//     gfx950 transposing read ds_read_b64_tr_b16, same key permutation as P) instead
//     of once per wave; the transposing read is the slowest LDS path, and this
//     split cuts its traffic by NW;
//   * softmax with a fixed per-head reference: the first tile's max; a later tile
//     max above it by more than 2^16 restarts the pass with the largest max seen, so
//     O is never rescaled;
//   * fp32 accumulation throughout; no atomics, so results are bitwise
//     reproducible.
// fp32 inputs run a one-wave kernel on 16x16x4 fp32 MFMAs (attn_f32.h).
#include <type_traits>

#include "sa_common.h"
#include "attn_f32.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS tile of kBK = 32 gathered latent rows. The first 512 channels of each row
// (64 chunks of 16 bytes) form the main region, row-major with a 1 KiB row stride;
// the 64 RoPE channels (8 chunks) of all rows form a second region. Chunks are
// XOR-swizzled so that the K reads (ds_read_b128, 16 rows per cycle) and the V
// transpose reads (4 rows x 4 chunks per 32 lanes) hit distinct banks.
SA_DEVICE int swz_main(int R) { return ((R & 3) << 2) | ((R >> 2) & 3); }
SA_DEVICE int swz_rope(int R) { return (R >> 1) & 7; }

// 16-byte global -> LDS copy per lane: lane l writes LDS bytes [lds + 16 l, +16).
// `lds` is wave-uniform. The address is a wave-uniform 64-bit base plus a per-lane
// 32-bit byte offset. Issued through inline asm so that the compiler does not order
// later LDS reads behind it; completion is tracked with s_waitcnt vmcnt. M0 is set
// here and nowhere else in these kernels.
SA_DEVICE void lds_dma16(uint32_t lds, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base)
               : "memory");
}

constexpr int kBK = 32;        // keys per tile
SA_DEVICE int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }
typedef int int4_t __attribute__((ext_vector_type(4)));

// 32x32x16 bf16 MFMA with the accumulator in VGPRs. The compiler gives every MFMA
// builtin an AGPR accumulator; the 256 AGPRs hold O here, and a builtin logit tile
// would push one O tile out of them on every key tile (32 copies each way, and a wait
// for the P . V MFMAs before the copy back). The caller keeps the MFMA-to-VALU wait
// states: mfma32_last() ends with them (a VALU read of a 16-pass MFMA result needs 19
// independent cycles).
SA_DEVICE floatx16_t mfma32_first(bf16x8_t a, bf16x8_t b) {
  floatx16_t c;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  return c;
}
SA_DEVICE floatx16_t mfma32_acc(bf16x8_t a, bf16x8_t b, floatx16_t c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
SA_DEVICE floatx16_t mfma32_last(bf16x8_t a, bf16x8_t b, floatx16_t c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(c) : "v"(a), "v"(b));
  return c;
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most `vm` vector-memory
// operations of this wave are outstanding and ignores the other counters.
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <int DQK>
constexpr int mla_tile_bytes() { return kBK * 64 * 16 + (DQK == 576 ? kBK * 8 * 16 : 0); }

template <int NW, int DQK, int NST, int NKL>
constexpr size_t mla_lds_bytes(int topk) {
  return (size_t)NST * mla_tile_bytes<DQK>() + (size_t)NKL * NW * 64 * 16 +
         (size_t)NW * 2 * 64 * 16 + (size_t)NW * 32 * 4 + (size_t)((topk + kBK - 1) / kBK) * kBK * 4;
}

// NW waves. Wave w computes the logits and probabilities of heads [32w, 32w+32)
// (S^T = K . Q^T, its q slices held as B operands: NKL k-steps in LDS, the rest in
// VGPRs) and publishes its P tile in LDS; then every wave accumulates O for ALL
// heads over its own 512/NW output channels, so each V element is read from LDS
// by one wave only. NST gather stages.
template <int NW, int DQK, int NST, int NKL, bool NEG>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                            const int32_t* __restrict__ idx, int H, int topk, float scale_log2,
                            const float* __restrict__ sink, uint16_t* __restrict__ out,
                            float* __restrict__ lse) {
  constexpr int NK = DQK / 16;            // MFMA k-steps of S^T = K . Q^T
  constexpr int NKM = 32;                 // k-steps in the main region
  constexpr int NKR = NK - NKL;           // k-steps whose q slices stay in VGPRs
  constexpr int NDB = 16 / NW;            // 32-wide dv blocks owned by each wave
  constexpr int NACC = NW * NDB;          // O accumulators per wave (always 16)
  constexpr bool ROPE = DQK == 576;
  constexpr int TILE_BYTES = mla_tile_bytes<DQK>();
  constexpr int ROPE_OFF = kBK * 64 * 16;
  constexpr int MAIN_PER_WAVE = kBK / NW;               // one DMA per row
  constexpr int ROPE_PER_WAVE = ROPE ? 4 / NW + (4 % NW ? 1 : 0) : 0;
  constexpr int DA = 4;                   // K-operand prefetch distance (k-steps)
  static_assert(NW == 1 || NW == 2 || NW == 4, "waves");
  static_assert(NACC == 16, "accumulators");
  // fp32 P values stay below 2^16 times the reference; a larger tile max restarts
  constexpr float kThr = 16.0f;

  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* tiles = lds;                                           // NST tiles
  char* s_q = lds + NST * TILE_BYTES;                          // [NKL][NW*64] x 16 B
  char* s_p = s_q + NKL * NW * 64 * 16;                        // [NW][2][64] x 16 B
  float* s_inv = reinterpret_cast<float*>(s_p + NW * 2 * 64 * 16);       // [NW*32]
  int32_t* s_idx = reinterpret_cast<int32_t*>(s_inv + NW * 32);          // [ntiles*32]
  __shared__ int s_restart;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int L = tid & 63;
  const int hl = L >> 5;        // lane half
  const int head = 32 * w + (L & 31);
  const bool head_ok = head < H;
  const int ntiles_all = (topk + kBK - 1) / kBK;
  __shared__ int s_wlast[NW];

  // ---- stage the index row (and find its last valid slot); q for this wave's 32
  //      heads as B-operand slices
  {
    const int32_t* __restrict__ irow = idx + (int64_t)t * topk;
    int last = 0;
    for (int j = tid; j < ntiles_all * kBK; j += NW * 64) {
      const int32_t v = j < topk ? irow[j] : -1;
      s_idx[j] = v;
      last = v >= 0 ? j + 1 : last;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off, 64));
    if (L == 0) s_wlast[w] = last;
  }
  if (tid == 0) s_restart = 0;
  bf16x8_t qv[NKR > 0 ? NKR : 1];
  {
    const uint16_t* qrow = q + ((int64_t)t * H + (head_ok ? head : 0)) * DQK + 8 * hl;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * n);
      if (!head_ok) v = bf16x8_t{};
      if (n < NKR) qv[n < NKR ? n : 0] = v;
      else *reinterpret_cast<bf16x8_t*>(s_q + ((n - NKR) * NW * 64 + tid) * 16) = v;
    }
  }

  // ---- per-lane LDS offsets
  // K reads (A operand): row R = L&31, chunk 2n + hl.
  int a_off[8];
  int a_rope[4];
  {
    const int R = L & 31;
    const int f = swz_main(R);
#pragma unroll
    for (int cls = 0; cls < 8; ++cls) a_off[cls] = (R * 64 + ((2 * cls + hl) ^ f)) * 16;
    const int gr = swz_rope(R);
#pragma unroll
    for (int j = 0; j < 4; ++j) a_rope[j] = ROPE_OFF + (R * 8 + ((2 * j + hl) ^ gr)) * 16;
  }
  // V transpose reads: lane L = 16g + s reads row 4(g/2) + s/4 (+16m + 8r) and
  // columns 16(g%2) + 4(s%4) (+32nt), 8 bytes.
  int v_off[2][4];      // [r][nt & 3]
  {
    const int g = L >> 4, s = L & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int R = 8 * r + 4 * (g >> 1) + (s >> 2);
      const int f = swz_main(R);
      const int col = 16 * (g & 1) + 4 * (s & 3);
#pragma unroll
      for (int nc = 0; nc < 4; ++nc) {
        const int c = 4 * nc + (col >> 3);
        v_off[r][nc] = (R * 64 + (c ^ f)) * 16 + (col & 7) * 2;
      }
    }
  }
  __syncthreads();
  // Tiles after the last valid slot hold only masked slots: they change neither O nor
  // l, and are not visited (a row without a valid slot visits none).
  int ntiles = 0;
  {
    int last = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) last = max(last, s_wlast[i]);
    ntiles = (int)uniform_i((last + kBK - 1) / kBK);
  }

  // Gather of one tile: this wave's MAIN_PER_WAVE row DMAs (1 KiB each: channels
  // 0..511 of rows R = MAIN_PER_WAVE w + j, contiguous, so that their indices come in
  // 16-byte LDS reads) and ROPE_PER_WAVE RoPE DMAs (channels 512..575 of 8 rows each).
  // gather_rows() reads the row indices from LDS; gather_dma(j) issues DMA j. The DMAs of the next tile are spread over the logit MFMAs, so the wave
  // never stalls on a burst of memory instructions.
  constexpr int ND = MAIN_PER_WAVE + ROPE_PER_WAVE;
  struct Rows { int main[MAIN_PER_WAVE]; int rope[ROPE_PER_WAVE > 0 ? ROPE_PER_WAVE : 1]; };
  auto gather_rows = [&](int tile) {
    Rows r;
    const int32_t* ir = s_idx + tile * kBK;
    const int4_t* ir4 = reinterpret_cast<const int4_t*>(ir + MAIN_PER_WAVE * w);
#pragma unroll
    for (int v = 0; v < MAIN_PER_WAVE / 4; ++v) {
      const int4_t x = ir4[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) r.main[4 * v + e] = __builtin_amdgcn_readfirstlane(x[e]);
    }
    if constexpr (ROPE) {
#pragma unroll
      for (int j = 0; j < ROPE_PER_WAVE; ++j) {
        const int ii = w + NW * j;
        r.rope[j] = ii < 4 ? ir[8 * ii + (L >> 3)] : 0;
      }
    }
    return r;
  };
  auto gather_dma = [&](int tile, const Rows& r, int j) {
    const uint32_t base = (uint32_t)(uintptr_t)(SA_LDS char*)(tiles + (tile % NST) * TILE_BYTES);
    if (j < MAIN_PER_WAVE) {
      const int R = MAIN_PER_WAVE * w + j;            // wave-uniform row
      int row = r.main[j < MAIN_PER_WAVE ? j : 0];
      row = row < 0 ? 0 : row;   // masked slot: any finite row keeps P*V finite
      lds_dma16(base + R * 1024, kv + (int64_t)row * DQK, (uint32_t)((L ^ swz_main(R)) * 16));
    } else if constexpr (ROPE) {
      const int jr = j - MAIN_PER_WAVE;
      const int ii = w + NW * jr;                     // rope instruction: rows 8ii..8ii+7
      if (ii < 4) {
        const int R = 8 * ii + (L >> 3);
        const int rr = r.rope[jr < ROPE_PER_WAVE ? jr : 0];
        const int row = rr < 0 ? 0 : rr;
        const int c = (L & 7) ^ swz_rope(R);
        lds_dma16(base + ROPE_OFF + ii * 1024, kv, (uint32_t)(row * (DQK * 2) + 1024 + 16 * c));
      }
    }
  };
  auto gather = [&](int tile) {
    const Rows r = gather_rows(tile);
#pragma unroll
    for (int j = 0; j < ND; ++j) gather_dma(tile, r, j);
  };

  // O[hb * NDB + db]: heads [32hb, 32hb+32) x channels 32(NDB w + db) + [0, 32).
  // With one wave, the last two accumulators are summed per key tile in a temporary
  // and added into VGPRs, which keeps the 16 accumulators, S and the operands within
  // the register file without spilling.
  constexpr int NOA = NW == 1 ? NACC - 2 : NACC;
  floatx16_t O[NACC];
  float m_ref = -__builtin_huge_valf();   // softmax reference (log2 units), per head
  float m_seen = -__builtin_huge_valf();
  float l_run = 0.0f;

#pragma unroll 1
  for (;;) {   // one pass over the tiles; repeated only if a tile max outgrows m_ref
#pragma unroll
    for (int i = 0; i < NACC; ++i) O[i] = floatx16_t{};
    l_run = 0.0f;
    bool grow = false;   // a tile max above m_ref + kThr (kept in a register: no branch)
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
      if (p < ntiles) gather(p);
#pragma unroll 1
    for (int tile = 0; tile < ntiles; ++tile) {
      // wait for this tile's gather; the newer ones (up to NST-2) may stay in flight
      const int newer = min(ntiles - 1 - tile, NST - 2);
      if (newer >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * (MAIN_PER_WAVE + ROPE_PER_WAVE)));
      else if (newer == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(MAIN_PER_WAVE + ROPE_PER_WAVE));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __syncthreads();               // tile resident in all waves' view; P of tile-1 consumed
      // the next gather goes to the stage read in tile-1; its DMAs ride along the
      // logit MFMAs below
      const int gtile = tile + NST - 1;
      const bool do_gather = gtile < ntiles;
      Rows grows;   // read after the first logit MFMA is issued (first DMA at k-step 2)
      const int my_slot = s_idx[tile * kBK + (L & (kBK - 1))];   // consumed after S
      const char* tb = tiles + (tile % NST) * TILE_BYTES;

      // ---- S^T = K . Q^T over d_qk, K slices prefetched DA k-steps ahead
      auto a_at = [&](int n) {
        const int off = n < NKM ? a_off[n & 7] + (n >> 3) * 256 : a_rope[(n - NKM) & 3];
        return *reinterpret_cast<const bf16x8_t*>(tb + off);
      };
      auto q_at = [&](int n) {
        return n < NKR ? qv[n < NKR ? n : 0]
                       : *reinterpret_cast<const bf16x8_t*>(s_q + ((n - NKR) * NW * 64 + tid) * 16);
      };
      floatx16_t S;
      {
        // K slices and the LDS-held q slices are both read DA k-steps ahead of use
        bf16x8_t ring[DA], qring[DA];
#pragma unroll
        for (int i = 0; i < DA; ++i) {
          ring[i] = a_at(i);
          if (i >= NKR) qring[i] = q_at(i);
        }
#pragma unroll
        for (int n = 0; n < NK; ++n) {
          const bf16x8_t a = ring[n % DA];
          const bf16x8_t b = n < NKR ? qv[n < NKR ? n : 0] : qring[n % DA];
          if (n + DA < NK) {
            ring[n % DA] = a_at(n + DA);
            if (n + DA >= NKR) qring[n % DA] = q_at(n + DA);
          }
          if (n == 0) S = mfma32_first(a, b);
          else if (n == NK - 1) S = mfma32_last(a, b, S);
          else S = mfma32_acc(a, b, S);
          if (n == 0) grows = gather_rows(do_gather ? gtile : tile);
          // the next gather's DMAs, spread over the k-steps from k-step 2 on (the row
          // indices read at the top of the tile have arrived by then)
#pragma unroll
          for (int j = 0; j < ND; ++j)
            if (2 + (j * (NK - 2)) / ND == n && do_gather) gather_dma(gtile, grows, j);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- logits in log2 units, tile max per head, reference update, then P (bf16,
      //      round to nearest even) in the A-operand layout of P . V (keys permuted
      //      inside the tile: half m holds S slots 8m..8m+7), published for every
      //      wave. A tile whose 32 slots are all valid (wave-uniform test) skips the
      //      masking; scaling is monotone, so the max of the scaled logits is the
      //      scaled max (or min, for a negative scale). Both variants are emitted
      //      whole, so the compiler keeps a uniform branch instead of computing both.
      const uint64_t vmask = ballot(L < kBK && my_slot >= 0);
      auto softmax = [&](auto full_t) {
        constexpr bool FULL = decltype(full_t)::value;
        float mx;
        uint32_t okbits = 0xFFFFu;          // bit sg: slot sg of this lane is valid
        if constexpr (FULL) {
          // NEG (a negative scale, chosen at launch): the largest scaled logit is the
          // smallest raw one
          float e = S[0];
#pragma unroll
          for (int sg = 1; sg < 15; sg += 2)
            e = NEG ? __builtin_elementwise_minimum(__builtin_elementwise_minimum(e, S[sg]), S[sg + 1])
                    : __builtin_elementwise_maximum(__builtin_elementwise_maximum(e, S[sg]), S[sg + 1]);
          e = NEG ? __builtin_elementwise_minimum(e, S[15]) : __builtin_elementwise_maximum(e, S[15]);
          mx = e * scale_log2;
        } else {
          // the volatile asm keeps the mask arithmetic inside this rarely taken branch
          // (otherwise it is hoisted above the branch and paid by every full tile)
          uint64_t vm = vmask;
          asm volatile("" : "+s"(vm));
          okbits = 0;
          mx = -__builtin_huge_valf();
#pragma unroll
          for (int sg = 0; sg < 16; ++sg) {
            const int key = 8 * (sg >> 2) + 4 * hl + (sg & 3);
            const bool ok = (vm >> key) & 1ull;
            okbits |= ok ? 1u << sg : 0u;
            mx = __builtin_elementwise_maximum(mx, ok ? S[sg] * scale_log2 : -__builtin_huge_valf());
          }
        }
        const float2_t mh = lane_halves(mx);
        mx = __builtin_elementwise_maximum(mh.x, mh.y);
        m_seen = __builtin_elementwise_maximum(m_seen, mx);
        if (m_ref == -__builtin_huge_valf()) m_ref = mx;   // first valid tile (O, l still 0)
        grow |= mx > m_ref + kThr;                          // published after the pass
        const float m_use = (m_ref == -__builtin_huge_valf()) ? 0.0f : m_ref;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float pf[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = fmaf(S[8 * m + e], scale_log2, -m_use);
            pf[e] = __builtin_amdgcn_exp2f(FULL || ((okbits >> (8 * m + e)) & 1u) ? x : -__builtin_huge_valf());
          }
          // pairwise, so that the sum is not one dependent chain
          l_run += ((pf[0] + pf[1]) + (pf[2] + pf[3])) + ((pf[4] + pf[5]) + (pf[6] + pf[7]));
          bf16x2_t pk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pk[e] = __builtin_convertvector((float2_t){pf[2 * e], pf[2 * e + 1]}, bf16x2_t);
          *reinterpret_cast<bf16x8_t*>(s_p + ((w * 2 + m) * 64 + L) * 16) = __builtin_bit_cast(bf16x8_t, pk);
        }
      };
      if ((uint32_t)vmask == 0xFFFFFFFFu) softmax(std::true_type{});
      else softmax(std::false_type{});
      // ---- O[hb][db] += P[hb] . V[:, dv block NDB w + db]; V's B operand is read
      //      with the same key permutation through the LDS transpose read. The first
      //      V operands do not depend on P and are read before the barrier.
      auto v_at = [&](int m, int nt) {
        const int off = m * (16 * 1024) + (nt >> 2) * 256;
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(tb + off + v_off[0][nt & 3]));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(tb + off + v_off[1][nt & 3]));
        const short __attribute__((ext_vector_type(8))) b8 = {lo[0], lo[1], lo[2], lo[3],
                                                              hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8_t, b8);
      };
      constexpr int NB = 2 * NDB;          // B operands per tile, order (db, m)
      constexpr int DV = NW == 1 ? 2 : 4;  // prefetch distance
      bf16x8_t ring[DV];
#pragma unroll
      for (int i = 0; i < DV; ++i) ring[i] = v_at(i & 1, NDB * w + (i >> 1));
      __syncthreads();               // every wave's P tile visible
      bf16x8_t Pa[NW][2];
      floatx16_t T;   // one-wave kernel: per-tile partial of the last two accumulators
#pragma unroll
      for (int hb = 0; hb < NW; ++hb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          Pa[hb][m] = *reinterpret_cast<const bf16x8_t*>(s_p + ((hb * 2 + m) * 64 + L) * 16);
      {
#pragma unroll
        for (int st = 0; st < NB; ++st) {
          const int db = st >> 1, m = st & 1;
          const bf16x8_t b = ring[st % DV];
          if (st + DV < NB) ring[st % DV] = v_at((st + DV) & 1, NDB * w + ((st + DV) >> 1));
#pragma unroll
          for (int hb = 0; hb < NW; ++hb) {
            const int a = hb * NDB + db;
            if (a < NOA) {
              O[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Pa[hb][m], b, O[a], 0, 0, 0);
            } else if (m == 0) {
              T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Pa[hb][0], b, floatx16_t{}, 0, 0, 0);
            } else {
              T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Pa[hb][1], b, T, 0, 0, 0);
              O[a] += T;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // A tile max above m_ref + kThr anywhere in the pass: redo the pass with the
    // largest max seen so far as the reference (all gathers have completed).
    if (grow) s_restart = 1;
    __syncthreads();
    const bool restart = s_restart != 0;
    __syncthreads();
    if (!restart) break;
    if (tid == 0) s_restart = 0;
    m_ref = m_seen;
  }

  // ---- epilogue: per-head 1/l through LDS, normalise, write bf16 out and lse
  const float2_t lh = lane_halves(l_run);
  const float l_tot = lh.x + lh.y;
  if (!sink) {
    if (hl == 0) s_inv[head] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (lse && hl == 0 && head_ok) {
      lse[(int64_t)t * H + head] =
          l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : -__builtin_huge_valf();
    }
  } else if (hl == 0) {
    // a sink logit joins the denominator: relative to M = max(m_ref, sink) it is
    // l_tot 2^(m_ref - M) + 2^(sink - M); the slots' weights are O 2^(m_ref - M) / that
    const float s2 = (head_ok ? sink[head] : 0.0f) * kLog2e;
    if (l_tot > 0.0f) {
      const float M = __builtin_elementwise_maximum(m_ref, s2);
      const float a = __builtin_amdgcn_exp2f(m_ref - M);
      const float den = l_tot * a + __builtin_amdgcn_exp2f(s2 - M);
      s_inv[head] = a / den;
      if (lse && head_ok) lse[(int64_t)t * H + head] = (M + __log2f(den)) * kLn2;
    } else {
      s_inv[head] = 0.0f;                              // no slot: out = 0, lse = sink
      if (lse && head_ok) lse[(int64_t)t * H + head] = sink[head];
    }
  }
  __syncthreads();
  uint16_t* __restrict__ orow = out + (int64_t)t * H * 512;
#pragma unroll
  for (int hb = 0; hb < NW; ++hb) {
#pragma unroll
    for (int sg = 0; sg < 16; ++sg) {
      const int hh = 32 * hb + 8 * (sg >> 2) + 4 * hl + (sg & 3);
      if (hh < H) {
        const float a = s_inv[hh];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          orow[(int64_t)hh * 512 + 32 * (NDB * w + db) + (L & 31)] = f2bf_bits(O[hb * NDB + db][sg] * a);
      }
    }
  }
}

// fp32 inputs: one wave per (token, group of 16 heads) on 16x16x4 fp32 MFMAs (the
// wave routine of attn_f32.h): the group's q rows sit in LDS, the selected kv rows are
// read as key rows (all d_qk channels) and as value rows (the first 512), 16 slots at
// a time; -1 slots and the slots past topk are holes.
template <int DQK>
__global__ __launch_bounds__(64) void sparse_mla_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ idx,
    int H, int topk, float scale_log2, const float* __restrict__ sink, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int ldq = DQK + 4;
  __shared__ __attribute__((aligned(16))) float sq[16 * ldq];
  const int t = blockIdx.x, h0 = 16 * (int)blockIdx.y;
  const int nh = min(16, H - h0);
  stage_q_f32<DQK>(q + ((int64_t)t * H + h0) * DQK, nh, sq);
  __syncthreads();
  const int32_t* __restrict__ ir = idx + (int64_t)t * topk;
  WaveAttnF32<DQK, 512> at;
  at.init();
  const int nsub = (topk + 15) / 16;
#pragma unroll 1
  for (int i = 0; i < nsub; ++i) {
    auto keys = [&](int r, const float*& kr, const float*& vr) {
      const int j = 16 * i + r;
      const int id = j < topk ? ir[j] : -1;
      kr = vr = kv + (int64_t)(id >= 0 ? id : 0) * DQK;
      return id >= 0;
    };
    at.tile(sq, ldq, scale_log2, keys);
  }
  at.finish(nh, sink ? sink + h0 : nullptr, out + ((int64_t)t * H + h0) * 512, 512,
            lse ? lse + (int64_t)t * H + h0 : nullptr);
}

constexpr int kStages = 2;
constexpr size_t kLdsLimit = 160 * 1024;

// k-steps of q kept in LDS (the rest stay in VGPRs): one wave has LDS to spare and
// keeps all of q there; two waves keep 20 k-steps there, four waves 12 (24 k-steps in
// VGPRs is the most that compiles without spills; each k-step moved out of LDS saves
// 1 KiB of LDS reads per wave and key tile).
template <int NW, int DQK>
constexpr int q_in_lds() { return NW == 1 ? DQK / 16 : (NW == 2 ? 20 : 12); }

template <int NW, int DQK>
size_t lds_bytes(int topk) { return mla_lds_bytes<NW, DQK, kStages, q_in_lds<NW, DQK>()>(topk); }

int waves_for(int H) { return H <= 32 ? 1 : (H <= 64 ? 2 : 4); }

template <int NW, int DQK>
hipError_t launch_bf16(const void* q, const void* kv, const int32_t* idx, int T, int H, int topk,
                       float scale, const float* sink, void* out, float* lse, hipStream_t st) {
  constexpr int NKL = q_in_lds<NW, DQK>();
  const size_t shm = mla_lds_bytes<NW, DQK, kStages, NKL>(topk);
  if (shm > kLdsLimit) return hipErrorInvalidValue;
  auto kern = scale < 0.0f ? sparse_mla_bf16_kernel<NW, DQK, kStages, NKL, true>
                           : sparse_mla_bf16_kernel<NW, DQK, kStages, NKL, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(T), dim3(NW * 64), shm, st, (const uint16_t*)q, (const uint16_t*)kv,
                     idx, H, topk, scale * kLog2e, sink, (uint16_t*)out, lse);
  return hipGetLastError();
}

template <int DQK>
hipError_t dispatch_bf16(const void* q, const void* kv, const int32_t* idx, int T, int H,
                         int topk, float scale, const float* sink, void* out, float* lse,
                         hipStream_t st) {
  switch (waves_for(H)) {
    case 1: return launch_bf16<1, DQK>(q, kv, idx, T, H, topk, scale, sink, out, lse, st);
    case 2: return launch_bf16<2, DQK>(q, kv, idx, T, H, topk, scale, sink, out, lse, st);
    default: return launch_bf16<4, DQK>(q, kv, idx, T, H, topk, scale, sink, out, lse, st);
  }
}

}  // namespace

bool sparse_mla_bf16_fits(int H, int d_qk, int topk) {
  size_t b;
  switch (waves_for(H)) {
    case 1: b = d_qk == 576 ? lds_bytes<1, 576>(topk) : lds_bytes<1, 512>(topk); break;
    case 2: b = d_qk == 576 ? lds_bytes<2, 576>(topk) : lds_bytes<2, 512>(topk); break;
    default: b = d_qk == 576 ? lds_bytes<4, 576>(topk) : lds_bytes<4, 512>(topk); break;
  }
  return b <= kLdsLimit;
}

hipError_t launch_sparse_mla(const void* q, const void* kv, const int32_t* idx, bool bf16, int T,
                             int S, int H, int d_qk, int d_v, int topk, float scale, const float* sink,
                             void* out, float* lse, hipStream_t st) {
  (void)S;
  if (T == 0) return hipSuccess;
  if (bf16) {
    if (d_qk == 576) return dispatch_bf16<576>(q, kv, idx, T, H, topk, scale, sink, out, lse, st);
    return dispatch_bf16<512>(q, kv, idx, T, H, topk, scale, sink, out, lse, st);
  }
  const dim3 grid(T, (H + 15) / 16);
  if (d_qk == 576)
    hipLaunchKernelGGL((sparse_mla_f32_kernel<576>), grid, dim3(64), 0, st, (const float*)q,
                       (const float*)kv, idx, H, topk, scale * kLog2e, sink, (float*)out, lse);
  else
    hipLaunchKernelGGL((sparse_mla_f32_kernel<512>), grid, dim3(64), 0, st, (const float*)q,
                       (const float*)kv, idx, H, topk, scale * kLog2e, sink, (float*)out, lse);
  return hipGetLastError();
}

}  // namespace sa
