// Multi-head ReLU indexer, streamed over causal key tiles, with either a dense
// score write or a fused exact top-k that never stores the score matrix.
//
// Operation ("Add trainable QSA sparse attention with a TileLang backend", sections
// "Is your feature request related to a problem?" and "Describe the solution you'd
// like": a trainable indexer with ReLU scores, a streaming runner with bounded
// memory, exact block TopK without the [sequence, sequence / block] matrix; and
// "Enable DSA CP/absorbed/THD paths with TileLang fused ops", file table: fused
// indexer forward):  I[t,s] = sum_h w[t,h] * max(q[t,h,:] . k[s,:], 0).
//
// Layout of the work (gfx950):
//   * a workgroup owns a run of consecutive query tokens of ONE sequence; its waves
//     each own 64 (token, head) rows = 64 / H_I tokens, so every token's heads and
//     its selection state belong to a single wave;
//   * key tiles of 64 rows stream through LDS by 16-byte global_load_lds (double
//     buffered, XOR-swizzled chunks for conflict-free operand reads);
//   * scores of a tile come from MFMA (bf16 32x32x16, or fp32 32x32x2) with rows =
//     (token, head) and columns = keys; the epilogue applies ReLU, the head weight
//     and the head sum in registers (one cross-half lane add) and stages one fp32
//     score per (token, key) in LDS;
//   * dense mode writes the staged scores; fused mode appends the keys that beat
//     the token's current k-th best key to an LDS candidate buffer (ballot/mbcnt
//     compaction, ascending key order), and when the buffer is full the owning wave
//     shrinks it back to exactly topk entries with a radix select (4 passes of 8-bit
//     digits over order-preserving keys) and a stable in-place compaction. Because
//     keys arrive in ascending index order, a later key equal to the k-th best can
//     never enter (it loses the index tie-break), so a strict ">" filter is exact.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kKT = 64;       // keys per tile
constexpr int kMaxWaves = 4;

struct IdxArgs {
  const void* q;
  const void* k;
  const float* w;
  int T;
  const int32_t* cu;
  int nseq;
  int B;                 // block size (1 = tokens)
  int nwave;             // waves per workgroup
  int chunks;            // token chunks per sequence (grid.x)
  // dense
  float* scores;
  int64_t ld;
  // fused
  int topk;
  int cap;               // candidate buffer entries per token
  int force_own;
  int32_t* out_idx;
  float* out_val;
  // two-pass selection through a workspace (64 heads): candidate rows [T, ws_cap]
  // (score, key id) and the number each row holds (-1: left to the exact kernel)
  float* ws_val;
  int32_t* ws_idx;
  int32_t* ws_cnt;
  int ws_cap;
  // block mode with a workspace: the key tiles of each token chunk split over nsplit
  // workgroups (grid.z), each leaving its exact partial top-k [T, nsplit, topk] (order
  // keys, block ids, counts) for a merge kernel; the own block's value per token
  int nsplit;
  uint32_t* sp_key;
  int32_t* sp_id;
  int32_t* sp_cnt;
  float* sp_own;
};

// Launch modes of the 64-head kernel.
constexpr int kDense = 0;    // write the scores
constexpr int kFused = 1;    // exact running top-k in LDS candidate buffers
constexpr int kAppend = 2;   // keys above a sampled pivot appended to the workspace
constexpr int kSample = 1024;   // pivot sample size (16 key tiles)

template <int CPR>
SA_DEVICE int kswz(int r) {
  if constexpr (CPR == 8) return (r >> 1) & 7;
  else return r & 15;
}

SA_DEVICE void lds_dma16(uint32_t lds, const void* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(src)
               : "memory");
}

// Same copy with a wave-uniform 64-bit base and a per-lane 32-bit byte offset.
SA_DEVICE void lds_dma16_sv(uint32_t lds, const void* base, uint32_t voff) {
  // readfirstlane returns a signed int: zero-extend each half before recombining
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(sb)
               : "memory");
}

// 32x32x16 bf16 MFMA with the A operand in AGPRs and the accumulator in VGPRs (the
// builtin would put the accumulator in AGPRs, and every epilogue read would need a
// copy). A VALU read of the result needs 19 wait states after the MFMA; the caller
// provides them.
SA_DEVICE floatx16_t idx_mfma_first(bf16x8_t a, bf16x8_t b) {
  floatx16_t c;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "a"(a), "v"(b));
  return c;
}
SA_DEVICE floatx16_t idx_mfma_acc(bf16x8_t a, bf16x8_t b, floatx16_t c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "a"(a), "v"(b));
  return c;
}

// ---- wave-level exact top-k shrink of a candidate buffer (keys, idx) of n entries,
//      stored in ascending index order. Keeps the first `k` under (key desc, index
//      asc) in place, in index order, and returns the smallest kept key.
SA_DEVICE uint32_t wave_shrink(uint32_t* keys, int32_t* ids, int n, int k, uint32_t* hist) {
  const int L = lane_id();
  uint32_t prefix = 0, need = (uint32_t)k;
  int mode = 2;            // 1: keep key >= thr; 2: keep key > thr + first `need` == thr
  uint32_t thr = 0;
#pragma unroll 1
  for (int p = 0; p < 4; ++p) {
    const int sh = 24 - 8 * p;
#pragma unroll
    for (int r = 0; r < 4; ++r) hist[4 * L + r] = 0u;
    __builtin_amdgcn_wave_barrier();
    for (int e = L; e < n; e += kWave) {
      const uint32_t kk = keys[e];
      if (p == 0 || (kk >> (sh + 8)) == prefix) atomicAdd(&hist[(kk >> sh) & 255u], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    // lane L owns bins 255-4L .. 252-4L (descending)
    uint32_t c[4], s = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) { c[r] = hist[255 - 4 * L - r]; s += c[r]; }
    uint32_t run = wave_incl_scan(s) - s;
    int found = -1;
    uint32_t above_f = 0, cnt_f = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t above = run;
      run += c[r];
      if (above < need && run >= need) { found = 255 - 4 * L - r; above_f = above; cnt_f = c[r]; }
    }
    const uint64_t fb = ballot(found >= 0);
    const int src = (int)__builtin_ctzll(fb);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(found, src);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)above_f, src);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)cnt_f, src);
    __builtin_amdgcn_wave_barrier();
    prefix = (prefix << 8) | d;
    need -= above;
    if (cnt == need) { mode = 1; thr = prefix << sh; break; }
    if (p == 3) thr = prefix;
  }
  // stable compaction, 64 entries per round; a round's reads precede its writes
  int out = 0;
  uint32_t eqseen = 0, kmin = 0xFFFFFFFFu;
  for (int base = 0; base < n; base += kWave) {
    const int e = base + L;
    const bool in = e < n;
    const uint32_t kk = in ? keys[e] : 0u;
    const int32_t id = in ? ids[e] : 0;
    const bool gt = in && (mode == 1 ? kk >= thr : kk > thr);
    const bool eq = in && mode == 2 && kk == thr;
    const uint64_t eb = ballot(eq);
    const uint32_t er = eqseen + mbcnt(eb);
    const bool take = gt || (eq && er < need);
    const uint64_t tb = ballot(take);
    const int pos = out + (int)mbcnt(tb);
    __builtin_amdgcn_wave_barrier();
    if (take) { keys[pos] = kk; ids[pos] = id; kmin = kmin < kk ? kmin : kk; }
    out += __popcll(tb);
    eqseen += (uint32_t)__popcll(eb);
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(kmin, off, kWave);
    kmin = kmin < o ? kmin : o;
  }
  return kmin;
}

// Appends the lanes with `take` set (ascending lane = ascending index) to a token
// buffer, shrinking it first when it would overflow. `tau` is the filter (a key
// must be > tau). Returns the new count; updates tau.
SA_DEVICE int wave_append(uint32_t* keys, int32_t* ids, int n, int cap, int k, uint32_t* hist,
                          uint32_t& tau, uint32_t kk, int32_t id, bool valid) {
  bool take = valid && kk > tau;
  uint64_t tb = ballot(take);
  int cnt = __popcll(tb);
  if (cnt == 0) return n;
  if (n + cnt > cap) {
    tau = wave_shrink(keys, ids, n, k, hist);
    n = k;
    take = valid && kk > tau;
    tb = ballot(take);
    cnt = __popcll(tb);
  }
  const int pos = n + (int)mbcnt(tb);
  if (take) { keys[pos] = kk; ids[pos] = id; }
  __builtin_amdgcn_wave_barrier();
  return n + cnt;
}

template <bool BF16, int HI, int DI>
__global__ __launch_bounds__(kMaxWaves * 64) void indexer_kernel(IdxArgs a) {
  using elem_t = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int ESZ = sizeof(elem_t);
  constexpr int CPR = DI * ESZ / 16;          // 16-byte chunks per key row
  constexpr int TILE_BYTES = kKT * CPR * 16;
  constexpr int KSTEPS = BF16 ? DI / 16 : DI / 2;
  constexpr int TW = 64 / HI;                 // tokens per wave
  static_assert(64 % HI == 0 && HI >= 4, "heads");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int nw = a.nwave;
  const int QT = nw * TW;                     // tokens per workgroup
  char* ktiles = lds;                                             // 2 tiles
  float* stage = reinterpret_cast<float*>(lds + 2 * TILE_BYTES);  // [QT][64]
  uint32_t* hist = reinterpret_cast<uint32_t*>(stage + QT * kKT); // [nw][256]
  int* s_n = reinterpret_cast<int*>(hist + nw * 256);             // [QT]
  uint32_t* s_tau = reinterpret_cast<uint32_t*>(s_n + QT);        // [QT]
  float* s_bmax = reinterpret_cast<float*>(s_tau + QT);           // [QT]
  float* s_own = s_bmax + QT;                                     // [QT]
  uint32_t* bkeys = reinterpret_cast<uint32_t*>(s_own + QT);      // [QT][cap]
  int32_t* bids = reinterpret_cast<int32_t*>(bkeys + (size_t)QT * a.cap);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int L = tid & 63;
  const int hl = L >> 5;
  const bool fused = a.topk > 0;

  // ---- token range of this workgroup
  const int seq = blockIdx.y;
  const int chunk = a.chunks - 1 - (int)blockIdx.x;   // longest rows first
  const int cs = a.cu ? __ldg(a.cu + seq) : 0;
  const int ce = a.cu ? __ldg(a.cu + seq + 1) : a.T;
  const int t0 = cs + chunk * QT;
  if (t0 >= ce) return;
  const int t1 = min(t0 + QT, ce);
  const int ntiles = (t1 - 1 - cs) / kKT + 1;
  // key tiles [tb, te) of this workgroup: all of them, or, split over grid.z
  // workgroups, an equal share in whole blocks (so a block's running max stays in one
  // workgroup)
  int tb = 0, te = ntiles;
  const bool split = a.nsplit > 1;
  if (split) {
    const int tpb = a.B > kKT ? a.B / kKT : 1;          // tiles per block
    const int units = (ntiles + tpb - 1) / tpb;
    const int per = (units + a.nsplit - 1) / a.nsplit;
    tb = min((int)blockIdx.z * per * tpb, ntiles);
    te = min(tb + per * tpb, ntiles);
  }

  // ---- this wave's A operand (q rows) and head weights
  const int wt0 = t0 + w * TW;               // first token of this wave
  using aslice_t = typename std::conditional<BF16, bf16x8_t, float>::type;
  aslice_t qa[2][KSTEPS];
  float wr[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = 32 * mt + (L & 31);        // wave-local row
    const int tok = wt0 + r / HI;
    const int h = r % HI;
    const bool ok = tok < t1;
    const elem_t* qrow = reinterpret_cast<const elem_t*>(a.q) + ((int64_t)(ok ? tok : t0) * HI + h) * DI;
#pragma unroll
    for (int n = 0; n < KSTEPS; ++n) {
      if constexpr (BF16) {
        bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * n + 8 * hl);
        qa[mt][n] = ok ? v : bf16x8_t{};
      } else {
        const float v = qrow[2 * n + hl];
        qa[mt][n] = ok ? v : 0.0f;
      }
    }
#pragma unroll
    for (int sg = 0; sg < 16; ++sg) {
      const int rr = 32 * mt + 8 * (sg >> 2) + 4 * hl + (sg & 3);
      const int tk = wt0 + rr / HI;
      wr[mt][sg] = tk < t1 ? __ldg(a.w + (int64_t)tk * HI + rr % HI) : 0.0f;
    }
  }

  // ---- per-token state (visible to every wave before its first use: the tile loop's
  //      barrier comes first, except in a split workgroup whose window holds no tile)
  for (int i = tid; i < QT; i += nw * 64) {
    s_n[i] = 0;
    s_tau[i] = 0u;
    s_bmax[i] = -__builtin_huge_valf();
    s_own[i] = 0.0f;
  }
  if (tb >= te) __syncthreads();            // uniform

  // B operand offsets (K^T slices) inside a tile: row = 32*nt + (L&31)
  int b_off[2][KSTEPS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = 32 * nt + (L & 31);
#pragma unroll
    for (int n = 0; n < KSTEPS; ++n) {
      if constexpr (BF16) {
        const int c = 2 * n + hl;
        b_off[nt][n] = (r * CPR + (c ^ kswz<CPR>(r))) * 16;
      } else {
        const int ch = 2 * n + hl;             // float index in the row
        const int c = ch >> 2;
        b_off[nt][n] = (r * CPR + (c ^ kswz<CPR>(r))) * 16 + (ch & 3) * 4;
      }
    }
  }

  auto gather = [&](int tile) {
    const uint32_t base = (uint32_t)(uintptr_t)(SA_LDS char*)(ktiles + (tile & 1) * TILE_BYTES);
    const int k0 = cs + tile * kKT;
    for (int ii = w; ii < CPR; ii += nw) {   // CPR instructions of 64 chunks per tile
      const int p = 64 * ii + L;
      const int r = p / CPR;
      const int c = (p % CPR) ^ kswz<CPR>(r);
      const int row = min(k0 + r, a.T - 1);
      lds_dma16(base + ii * 1024, reinterpret_cast<const char*>(a.k) + ((int64_t)row * DI) * ESZ + 16 * c);
    }
  };

  if (tb < te) gather(tb);
#pragma unroll 1
  for (int tile = tb; tile < te; ++tile) {
    wait_vmcnt0();
    __syncthreads();                      // tile resident; previous tile fully consumed
    if (tile + 1 < te) gather(tile + 1);
    const char* tb = ktiles + (tile & 1) * TILE_BYTES;
    const int k0 = cs + tile * kKT;

    // ---- S = Q . K^T for 64 rows x 64 keys
    floatx16_t S[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[mt][nt] = floatx16_t{};
    // bf16: the K^T slices are read DA k-steps ahead of their MFMAs (read just before
    // each MFMA pair, every k-step waited out a whole LDS latency)
    constexpr int DA = 4;
    bf16x8_t ring[BF16 ? DA : 1][2];
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < DA; ++i)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) ring[i][nt] = *reinterpret_cast<const bf16x8_t*>(tb + b_off[nt][i]);
    }
#pragma unroll
    for (int n = 0; n < KSTEPS; ++n) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if constexpr (BF16) {
          const bf16x8_t b = ring[n % DA][nt];
          if (n + DA < KSTEPS) ring[n % DA][nt] = *reinterpret_cast<const bf16x8_t*>(tb + b_off[nt][n + DA]);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            S[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][n], b, S[mt][nt], 0, 0, 0);
        } else {
          const float b = *reinterpret_cast<const float*>(tb + b_off[nt][n]);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            S[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[mt][n], b, S[mt][nt], 0, 0, 0);
        }
      }
      if constexpr (BF16) __builtin_amdgcn_sched_barrier(0);   // keep each k-step's read-ahead in place
    }

    // ---- ReLU, head weight, head sum; stage one score per (token, key)
    float* wst = stage + (w * TW) * kKT;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int key = 32 * nt + (L & 31);
      if constexpr (HI >= 8) {
        float acc[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int sg = 0; sg < 16; ++sg) {
            const int tl = (32 * mt + 8 * (sg >> 2)) / HI;
            acc[tl] = fmaf(wr[mt][sg], __builtin_elementwise_maximum(S[mt][nt][sg], 0.0f), acc[tl]);
          }
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          const float2_t h = lane_halves(acc[i]);   // own + the other lane half's
          const float v = h.x + h.y;
          if (hl == 0) wst[i * kKT + key] = v;
        }
      } else {   // HI == 4: each token's 4 rows sit in one lane
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) v = fmaf(wr[mt][4 * g + j], __builtin_elementwise_maximum(S[mt][nt][4 * g + j], 0.0f), v);
            const int tl = 8 * mt + 2 * g + hl;
            wst[tl * kKT + key] = v;
          }
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- blocks of at least a tile: every token of the wave gets at most one block
    //      value per tile, so all TW tokens are handled in one pass, HI lanes per token
    //      (lane j of token i takes keys j KPL .. j KPL + KPL - 1 of the staged row)
    if (a.B >= kKT) {
      constexpr int KPL = kKT / HI;
      const int i = L / HI, j = L % HI;
      const int t = wt0 + i;
      const int qi = w * TW + i;
      const bool live = t < t1 && k0 <= t;   // the token has a causal key in this tile
      float m = -__builtin_huge_valf();
      if (live) {
        const float* src = wst + i * kKT + j * KPL;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          float sc = src[e];
          if (sc == 0.0f) sc = 0.0f;           // -0 -> +0
          if (k0 + j * KPL + e <= t) m = __builtin_elementwise_maximum(m, sc);
        }
      }
      m = group_max(m, HI);
      const int B = a.B;
      const int blk = (k0 - cs) / B;
      bool emit = live;
      if (B > kKT) {
        // running max over the tiles of a block; the value goes out at its last tile
        m = __builtin_elementwise_maximum(m, live ? s_bmax[qi] : -__builtin_huge_valf());
        const bool last = ((k0 - cs + kKT) % B == 0) || (k0 + kKT > t);
        if (live && j == 0) s_bmax[qi] = last ? -__builtin_huge_valf() : m;
        emit = live && last;
      }
      emit = emit && j == 0;
      if (!fused) {
        if (emit) a.scores[(int64_t)t * a.ld + blk] = m;
      } else {
        uint32_t kk = order_key(m);
        if (emit && a.force_own && blk == (t - cs) / B) {
          kk = 0xFFFFFFFFu;
          s_own[qi] = m == 0.0f ? 0.0f : m;
        }
        uint32_t tau = emit ? s_tau[qi] : 0u;
        int n = emit ? s_n[qi] : 0;
        bool take = emit && kk > tau;
        // a full buffer is first cut back to topk by the whole wave, one token at a time
        uint64_t full = ballot(take && n + 1 > a.cap);
#pragma unroll 1
        while (full) {                          // uniform
          const int srcl = (int)__builtin_ctzll(full);
          const int qs = w * TW + srcl / HI;
          const int ns = __builtin_amdgcn_readlane(n, srcl);
          const uint32_t tnew = wave_shrink(bkeys + (size_t)qs * a.cap, bids + (size_t)qs * a.cap, ns,
                                            a.topk, hist + w * 256);
          if (L == srcl) {
            tau = tnew;
            n = a.topk;
            take = kk > tau;
          }
          full &= full - 1;
        }
        if (take) {
          bkeys[(size_t)qi * a.cap + n] = kk;
          bids[(size_t)qi * a.cap + n] = blk;
          ++n;
        }
        if (emit) {
          s_n[qi] = n;
          s_tau[qi] = tau;
        }
      }
      __builtin_amdgcn_wave_barrier();
      continue;
    }

    // ---- per token of this wave: dense write, or fused selection
#pragma unroll 1
    for (int i = 0; i < TW; ++i) {
      const int t = wt0 + i;
      if (t >= t1) break;
      if (k0 > t) continue;                 // no causal key of t in this tile
      const int qi = w * TW + i;
      float sc = wst[i * kKT + L];
      if (sc == 0.0f) sc = 0.0f;             // -0 -> +0
      const int kg = k0 + L;
      const bool valid = kg <= t;            // kg >= cs always
      const int off = kg - cs;
      if (a.B == 1) {
        if (!fused) {
          if (valid) a.scores[(int64_t)t * a.ld + off] = sc;
        } else {
          uint32_t tau = s_tau[qi];
          const int n = wave_append(bkeys + (size_t)qi * a.cap, bids + (size_t)qi * a.cap, s_n[qi],
                                    a.cap, a.topk, hist + w * 256, tau, order_key(sc), kg, valid);
          __builtin_amdgcn_wave_barrier();
          if (L == 0) { s_n[qi] = n; s_tau[qi] = tau; }
          __builtin_amdgcn_wave_barrier();
        }
      } else {
        // block scores: max over the block's causal keys
        const int B = a.B;
        const int own = (t - cs) / B;
        float m = valid ? sc : -__builtin_huge_valf();
        bool emit;
        int blk;
        if (B <= kKT) {
          m = group_max(m, B);
          blk = off / B;
          emit = (L % B == 0) && (k0 + L <= t);
        } else {
          m = wave_max(m);
          m = __builtin_elementwise_maximum(m, s_bmax[qi]);
          blk = (k0 - cs) / B;
          const bool last_of_block = ((k0 - cs + kKT) % B == 0) || (k0 + kKT > t);
          __builtin_amdgcn_wave_barrier();
          if (L == 0) s_bmax[qi] = last_of_block ? -__builtin_huge_valf() : m;
          __builtin_amdgcn_wave_barrier();
          emit = last_of_block && L == 0;
        }
        if (!fused) {
          if (emit) a.scores[(int64_t)t * a.ld + blk] = m;
        } else {
          uint32_t kk = order_key(m);
          if (emit && a.force_own && blk == own) {
            kk = 0xFFFFFFFFu;
            s_own[qi] = m == 0.0f ? 0.0f : m;
          }
          uint32_t tau = s_tau[qi];
          const int n = wave_append(bkeys + (size_t)qi * a.cap, bids + (size_t)qi * a.cap, s_n[qi],
                                    a.cap, a.topk, hist + w * 256, tau, kk, blk, emit);
          __builtin_amdgcn_wave_barrier();
          if (L == 0) { s_n[qi] = n; s_tau[qi] = tau; }
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
  }

  if (!fused) return;
  // ---- final selection and output, per token of this wave
#pragma unroll 1
  for (int i = 0; i < TW; ++i) {
    const int t = wt0 + i;
    if (t >= t1) break;
    const int qi = w * TW + i;
    uint32_t* keys = bkeys + (size_t)qi * a.cap;
    int32_t* ids = bids + (size_t)qi * a.cap;
    int n = s_n[qi];
    if (n > a.topk) { wave_shrink(keys, ids, n, a.topk, hist + w * 256); n = a.topk; }
    const int own = a.B > 1 ? (t - cs) / a.B : -1;
    if (split) {
      // this workgroup's exact partial top-k, in ascending block order, for the merge
      const size_t slot = (size_t)t * a.nsplit + blockIdx.z;
      for (int j = L; j < n; j += kWave) {
        a.sp_key[slot * a.topk + j] = keys[j];
        a.sp_id[slot * a.topk + j] = ids[j];
      }
      if (L == 0) {
        a.sp_cnt[slot] = n;
        const int own_tile = own * a.B / kKT;
        if (a.force_own && own_tile >= tb && own_tile < te) a.sp_own[t] = s_own[qi];
      }
      continue;
    }
    int32_t* orow = a.out_idx + (int64_t)t * a.topk;
    float* vrow = a.out_val ? a.out_val + (int64_t)t * a.topk : nullptr;
    for (int j = L; j < a.topk; j += kWave) {
      if (j < n) {
        const int32_t id = ids[j];
        orow[j] = id;
        if (vrow) vrow[j] = (a.force_own && id == own) ? s_own[qi] : key_value(keys[j]);
      } else {
        orow[j] = -1;
        if (vrow) vrow[j] = -__builtin_huge_valf();
      }
    }
  }
}

// Merge of the partial block top-k lists of a split launch: one wave per token. The
// token's candidates (at most nsplit x topk <= 256) sit in split order, which is
// ascending block order (the splits cover consecutive key ranges and each list is
// ascending); a candidate is kept when fewer than topk others beat it under (key
// desc, block asc), and the kept ones are written in that same order.
constexpr int kMergeWaves = 4;
constexpr int kMergeMax = 256;          // candidates per token: nsplit <= 4, topk <= 64

__global__ __launch_bounds__(kMergeWaves * 64) void indexer_merge_kernel(IdxArgs a) {
  constexpr int R = kMergeMax / kWave;
  const int L = lane_id();
  const int t = (int)blockIdx.x * kMergeWaves + (int)(threadIdx.x >> 6);
  if (t >= a.T) return;                    // whole wave
  const int topk = a.topk;
  // offsets of the splits' lists in the concatenation
  int cnt[4] = {0, 0, 0, 0};
  int m = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (p < a.nsplit) {
      cnt[p] = __ldg(a.sp_cnt + (size_t)t * a.nsplit + p);
      m += cnt[p];
    }
  }
  uint32_t key[R];
  int32_t id[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = L + kWave * r;           // concatenated position
    key[r] = 0u;
    id[r] = INT32_MAX;
    if (c < m) {
      int p = 0, base = 0;
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (p == q && c >= base + cnt[q]) { base += cnt[q]; p = q + 1; }
      const size_t e = ((size_t)t * a.nsplit + p) * topk + (c - base);
      key[r] = a.sp_key[e];
      id[r] = a.sp_id[e];
    }
  }
  // rank of each candidate: how many others beat it
  int rank[R] = {};
#pragma unroll 1
  for (int j = 0; j < m; ++j) {
    const int r0 = j / kWave, l0 = j % kWave;
    uint32_t kj = 0u;
    int32_t ij = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r == r0) {
        kj = (uint32_t)__builtin_amdgcn_readlane((int)key[r], l0);
        ij = __builtin_amdgcn_readlane(id[r], l0);
      }
#pragma unroll
    for (int r = 0; r < R; ++r) rank[r] += (kj > key[r] || (kj == key[r] && ij < id[r])) ? 1 : 0;
  }
  int32_t* orow = a.out_idx + (int64_t)t * topk;
  float* vrow = a.out_val ? a.out_val + (int64_t)t * topk : nullptr;
  const int cs = a.cu ? seq_start_of(a.cu, a.nseq, t) : 0;
  const int own = (t - cs) / a.B;
  int pos = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool keep = L + kWave * r < m && rank[r] < topk;
    const uint64_t b = ballot(keep);
    if (keep) {
      const int o = pos + (int)mbcnt(b);
      orow[o] = id[r];
      if (vrow) vrow[o] = (a.force_own && id[r] == own) ? a.sp_own[t] : key_value(key[r]);
    }
    pos += __popcll(b);
  }
  for (int j = pos + L; j < topk; j += kWave) {
    orow[j] = -1;
    if (vrow) vrow[j] = -__builtin_huge_valf();
  }
}

// ---- exact wave-level top-k of a candidate buffer, radix digits taken from the top
//      of the occupied key range. keys[0..n) (order keys in [lo, hi]) and ids[0..n)
//      are in ascending index order; keeps the first k under (key desc, index asc) in
//      place, stable, and returns the smallest kept key. Each pass histograms the
//      window that holds the k-th key into 256 buckets of width 2^shift, so it takes
//      ceil(bits(hi - lo) / 8) passes at most, and ends early when the bucket of the
//      k-th key is taken whole.
SA_DEVICE uint32_t wave_select(uint32_t* keys, int32_t* ids, int n, int k, uint32_t* hist,
                               uint32_t lo, uint32_t hi) {
  const int L = lane_id();
  uint32_t wlo = 0, whi = hi - lo;         // window (offsets from lo) holding the k-th key
  uint32_t need = (uint32_t)k;             // keys still to take from the window
  int mode = 1;                            // 1: keep >= thr; 2: keep > thr + first `need` == thr
  uint32_t thr = lo;
#pragma unroll 1
  for (;;) {
    const uint32_t span = whi - wlo;
    const int shift = span >= 256u ? (32 - __builtin_clz(span)) - 8 : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) hist[4 * L + r] = 0u;
    __builtin_amdgcn_wave_barrier();
    int e = L;
#pragma unroll 1
    for (; e + 192 < n; e += 256) {       // four independent reads in flight
      uint32_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = keys[e + 64 * u] - lo;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (x[u] >= wlo && x[u] <= whi) atomicAdd(&hist[(x[u] - wlo) >> shift], 1u);
    }
#pragma unroll 1
    for (; e < n; e += 64) {
      const uint32_t x = keys[e] - lo;
      if (x >= wlo && x <= whi) atomicAdd(&hist[(x - wlo) >> shift], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    // lane L owns buckets 255-4L .. 252-4L (descending)
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) { c[r] = hist[255 - 4 * L - r]; sum += c[r]; }
    uint32_t run = wave_incl_scan(sum) - sum;
    int found = -1;
    uint32_t above_f = 0, cnt_f = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t above = run;
      run += c[r];
      if (above < need && run >= need) { found = 255 - 4 * L - r; above_f = above; cnt_f = c[r]; }
    }
    const int src = (int)__builtin_ctzll(ballot(found >= 0));
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(found, src);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)above_f, src);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)cnt_f, src);
    __builtin_amdgcn_wave_barrier();
    need -= above;
    const uint32_t blo = wlo + (d << shift);
    if (cnt == need) { mode = 1; thr = lo + blo; break; }      // bucket taken whole
    if (shift == 0) { mode = 2; thr = lo + blo; break; }       // k-th key's exact value
    wlo = blo;
    whi = min(whi, blo + ((1u << shift) - 1u));
  }
  // stable compaction, 64 entries per round, four rounds per batch: a batch reads
  // its 256 entries first, then writes only below its own start, so the reads of
  // later batches never see a write
  int out = 0;
  uint32_t eqseen = 0, kmin = 0xFFFFFFFFu;
#pragma unroll 1
  for (int base = 0; base < n; base += 4 * kWave) {
    uint32_t kk[4];
    int32_t id[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = base + 64 * u + L;
      kk[u] = e < n ? keys[e] : 0u;
      id[u] = e < n ? ids[e] : 0;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = base + 64 * u + L < n;
      const bool gt = in && (mode == 1 ? kk[u] >= thr : kk[u] > thr);
      const bool eq = in && mode == 2 && kk[u] == thr;
      const uint64_t eb = ballot(eq);
      const uint32_t er = eqseen + mbcnt(eb);
      const bool take = gt || (eq && er < need);
      const uint64_t tb = ballot(take);
      const int pos = out + (int)mbcnt(tb);
      if (take) { keys[pos] = kk[u]; ids[pos] = id[u]; kmin = kmin < kk[u] ? kmin : kk[u]; }
      out += __popcll(tb);
      eqseen += (uint32_t)__popcll(eb);
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(kmin, off, kWave);
    kmin = kmin < o ? kmin : o;
  }
  return kmin;
}

// ---- one-pass cut-back of a candidate buffer: keys[0..n) (order keys in [lo, hi]),
//      ids[0..n), ascending index order, in a buffer of `cap` entries (cap a multiple
//      of 4, both arrays 16-byte aligned). Histograms [lo, hi] into 256 buckets, finds
//      the lowest bucket b such that the buckets from b up hold at least k keys, and
//      keeps (stably, in place) every key >= the lower edge of b. The kept set always
//      contains the exact top-k, so the caller may raise its threshold to that edge
//      minus one. Returns the number kept; if the buckets from b up hold more than
//      `limit` keys (massive ties) nothing is dropped and n is returned.
//      Lane L takes entries 4L..4L+3 of each 256-entry batch with 16-byte reads (reads
//      past n are clamped into the buffer and masked), the loops run on a wave-uniform
//      count, and the compaction places each kept entry by ballot counts.
SA_DEVICE int wave_cut(uint32_t* keys, int32_t* ids, int n, int cap, int k, int limit, uint32_t* hist,
                       uint32_t lo, uint32_t hi, uint32_t& edge) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
  const int L = lane_id();
  n = __builtin_amdgcn_readfirstlane(n);
  const uint32_t span = hi - lo;
  const int shift = span >= 256u ? (32 - __builtin_clz(span)) - 8 : 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) hist[4 * L + r] = 0u;
  __builtin_amdgcn_wave_barrier();
#pragma unroll 1
  for (int base = 0; base < n; base += 512) {   // two batches of reads in flight
    u32x4_t x[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      x[u] = *reinterpret_cast<const u32x4_t*>(keys + min(base + 256 * u + 4 * L, cap - 4));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {     // masked entries add 0 to bucket 0: no branch
        const bool in = base + 256 * u + 4 * L + j < n;
        atomicAdd(&hist[in ? (x[u][j] - lo) >> shift : 0u], in ? 1u : 0u);
      }
  }
  __builtin_amdgcn_wave_barrier();
  uint32_t c[4], sum = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) { c[r] = hist[255 - 4 * L - r]; sum += c[r]; }
  uint32_t run = wave_incl_scan(sum) - sum;
  int found = -1;
  uint32_t upto_f = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t above = run;
    run += c[r];
    if (above < (uint32_t)k && run >= (uint32_t)k) { found = 255 - 4 * L - r; upto_f = run; }
  }
  const int src = (int)__builtin_ctzll(ballot(found >= 0));
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(found, src);
  const int kept = __builtin_amdgcn_readlane((int)upto_f, src);
  __builtin_amdgcn_wave_barrier();
  if (kept > limit) { edge = lo; return n; }
  edge = lo + (d << shift);
  const uint32_t thr = edge;
  // A batch's reads all land before its writes, and every write goes at or below its
  // own source, below the next batch's reads.
  int out = 0;
#pragma unroll 1
  for (int base = 0; base < n; base += 4 * kWave) {
    const int e = min(base + 4 * L, cap - 4);
    const u32x4_t kk = *reinterpret_cast<const u32x4_t*>(keys + e);
    const i32x4_t id = *reinterpret_cast<const i32x4_t*>(ids + e);
    __builtin_amdgcn_wave_barrier();
    bool take[4];
    uint32_t below = 0, cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      take[j] = base + 4 * L + j < n && kk[j] >= thr;
      const uint64_t tb = ballot(take[j]);
      below += mbcnt(tb);                 // kept entries of the lower lanes, slot j
      cnt += (uint32_t)__popcll(tb);
    }
    int pos = out + (int)below;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (take[j]) { keys[pos] = kk[j]; ids[pos] = id[j]; }
      pos += take[j] ? 1 : 0;
    }
    out += (int)cnt;
    __builtin_amdgcn_wave_barrier();
  }
  return out;
}

// Token scores with 64 indexer heads (bf16): one token per wave, so the 64 heads are
// the 64 rows of the wave's MFMA tiles and a token's whole state stays in the wave.
//   * key tiles of 64 rows stream through LDS (global_load_lds, double buffered); the
//     K^T operand slices are read DA k-steps ahead of their MFMAs;
//   * the ReLU, head weight and head sum run on the accumulators: each lane sums its
//     32 (head, key) products, one lane-half swap completes the 64-head sum, and lane
//     L ends up holding the score of key k0 + L, so no score goes through LDS;
//   * dense mode stores the scores (one coalesced 256-byte row segment per tile);
//     fused mode compares each lane's key with the running threshold held in a
//     register and appends the winners, in index order, to the token's LDS candidate
//     buffer; a nearly full buffer is cut back by wave_cut (one histogram pass keeps
//     the buckets that hold the top k, and the kept edge becomes the new threshold),
//     or by the exact wave_select when ties defeat the histogram; the exact select also
//     finishes the row. Keys arrive in ascending index order, so a later key equal to
//     a kept one never wins and the strict filter is exact.
// MODE kAppend (first pass of the two-pass selection): before the stream, the
// workgroup scores a sample of kSample evenly spaced causal keys; each wave bisects
// its token's sample for a pivot that about k plus 4.3 standard deviations of the
// sample rank reach, then appends every key at or above it, in index order, to the
// token's workspace row and records how many it appended. A row whose count falls
// below k (or overflows the row) is marked -1 and redone by the kFused launch, so
// the pivot never decides a result; sa_topk_select finishes the other rows.
// With ws_cnt set, a kFused launch only runs the workgroups holding a marked row.
// SPREAD (the dense and append launches): a wave spreads its share of the next
// gather over the first key half's MFMAs instead of issuing it right after the
// barrier.
template <int DI, int MODE>
__global__ __launch_bounds__(kMaxWaves * 64) void indexer64_kernel(IdxArgs args) {
  const IdxArgs a = args;   // local copy: lambdas capture it without a private-memory copy of the kernel argument
  constexpr bool SPREAD = MODE != kFused;
  constexpr bool APPEND = MODE == kAppend;
  constexpr int CPR = DI * 2 / 16;            // 16-byte chunks per key row
  constexpr int TILE_BYTES = kKT * CPR * 16;
  constexpr int KSTEPS = DI / 16;
  constexpr int DA = 4;                       // K^T operand prefetch distance (k-steps)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* ktiles = lds;                                              // 2 tiles
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds + 2 * TILE_BYTES);   // [4][256]
  uint32_t* bkeys = hist + kMaxWaves * 256;                         // [4][cap]
  int32_t* bids = reinterpret_cast<int32_t*>(bkeys + (size_t)kMaxWaves * a.cap);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int L = tid & 63;
  const int hl = L >> 5;
  const bool fused = MODE == kFused;

  const int seq = blockIdx.y;
  const int chunk = a.chunks - 1 - (int)blockIdx.x;   // longest rows first
  const int cs = a.cu ? __ldg(a.cu + seq) : 0;
  const int ce = a.cu ? __ldg(a.cu + seq + 1) : a.T;
  const int t0 = cs + chunk * kMaxWaves;
  if (t0 >= ce) return;
  const int t1 = min(t0 + kMaxWaves, ce);
  if constexpr (MODE == kFused) {
    if (a.ws_cnt) {                                    // redo only marked rows (uniform test)
      bool marked = false;
      for (int i = t0; i < t1; ++i) marked = marked || __ldg(a.ws_cnt + i) < 0;
      if (!marked) return;
    }
  }
  const int ntiles = (t1 - 1 - cs) / kKT + 1;
  const int t = t0 + w;                                // this wave's token
  const bool active = t < t1;
  const int my_tiles = active ? (t - cs) / kKT + 1 : 0;

  // A operands (q rows = heads) and head weights of this wave's token
  bf16x8_t qa[2][KSTEPS];
  float wr[2][16];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)(active ? t : t0) * 64 * DI;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint16_t* qh = qrow + (32 * mt + (L & 31)) * DI + 8 * hl;
#pragma unroll
      for (int n = 0; n < KSTEPS; ++n) qa[mt][n] = *reinterpret_cast<const bf16x8_t*>(qh + 16 * n);
#pragma unroll
      for (int sg = 0; sg < 16; ++sg)
        wr[mt][sg] = __ldg(a.w + (int64_t)(active ? t : t0) * 64 + 32 * mt + 8 * (sg >> 2) + 4 * hl + (sg & 3));
    }
  }
  int b_off[2][KSTEPS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = 32 * nt + (L & 31);
#pragma unroll
    for (int n = 0; n < KSTEPS; ++n) b_off[nt][n] = (r * CPR + ((2 * n + hl) ^ kswz<CPR>(r))) * 16;
  }

  // Tile gather: CPR / 4 copies of 1 KiB per wave. Copy ii moves chunk p = 64 ii + L,
  // i.e. row p / CPR, swizzled chunk; its byte offset inside the tile's rows is fixed,
  // so a full tile needs only a scalar base per tile.
  constexpr int NG = CPR / kMaxWaves;
  uint32_t g_off[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int p = 64 * (w + kMaxWaves * j) + L;
    const int r = p / CPR;
    g_off[j] = (uint32_t)(r * DI * 2 + 16 * ((p % CPR) ^ kswz<CPR>(r)));
  }
  auto gather_one = [&](int tile, int j) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(uintptr_t)(SA_LDS char*)(ktiles + (tile & 1) * TILE_BYTES);
    const int k0 = __builtin_amdgcn_readfirstlane(cs + tile * kKT);
    if (k0 + kKT <= a.T) {
      const char* src = reinterpret_cast<const char*>(a.k) + (int64_t)k0 * DI * 2;
      lds_dma16_sv(base + (w + kMaxWaves * j) * 1024, src, g_off[j]);
    } else {                                // last tile of the key array: clamp rows
      const int p = 64 * (w + kMaxWaves * j) + L;
      const int r = p / CPR;
      const int c = (p % CPR) ^ kswz<CPR>(r);
      const int row = min(k0 + r, a.T - 1);
      lds_dma16(base + (w + kMaxWaves * j) * 1024,
                reinterpret_cast<const char*>(a.k) + ((int64_t)row * DI) * 2 + 16 * c);
    }
  };
  auto gather = [&](int tile) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(uintptr_t)(SA_LDS char*)(ktiles + (tile & 1) * TILE_BYTES);
    const int k0 = __builtin_amdgcn_readfirstlane(cs + tile * kKT);
    if (k0 + kKT <= a.T) {
      const char* src = reinterpret_cast<const char*>(a.k) + (int64_t)k0 * DI * 2;
#pragma unroll
      for (int j = 0; j < NG; ++j) lds_dma16_sv(base + (w + kMaxWaves * j) * 1024, src, g_off[j]);
    } else {
#pragma unroll
      for (int j = 0; j < NG; ++j) gather_one(tile, j);
    }
  };

  uint32_t* keys = bkeys + (size_t)w * a.cap;
  int32_t* ids = bids + (size_t)w * a.cap;
  uint32_t* whist = hist + w * 256;
  // Cut-backs are synchronised: a wave whose buffer has less than one tile of room
  // left records the tile in s_req, and after the next barrier every wave holding
  // more than k candidates cuts back at once, so no wave waits on another's cut-back.
  __shared__ int s_req;
  if (tid == 0) s_req = -1;
  int n = 0;                       // candidates held
  uint32_t tau = 0u;               // a key must exceed this to enter; every held key is
                                   // >= tau (after a cut-back the smallest kept key == tau)
  uint32_t kmax = 0u;              // largest key this lane appended

  // S = Q . K^T of one tile in two key halves, S0 = keys 0..31 and S1 = keys 32..63,
  // each as two 32x32 blocks of heads (mt). The accumulators live in VGPRs (inline-asm
  // MFMAs) so that the epilogue reads them without copies; the q slices are the A
  // operands, held in AGPRs. K^T operand slices are read DA k-steps ahead, over the
  // 2 x KSTEPS slices of a tile in order (half nt, k-step kn: slice KSTEPS nt + kn).
  constexpr int NSL = 2 * KSTEPS;
  constexpr int VPP = 32 / KSTEPS;            // epilogue values per k-step
  floatx16_t S0[2], S1[2];
  bf16x8_t ring[DA];
  auto slice_load = [&](const char* tb, int i) __attribute__((always_inline)) {
    ring[i % DA] = *reinterpret_cast<const bf16x8_t*>(tb + b_off[i / KSTEPS][i % KSTEPS]);
  };
  auto tile_start = [&](const char* tb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < DA; ++i) slice_load(tb, i);
  };
  // ReLU, head weight, head sum of one key half: each lane sums its 32 (head, key)
  // products in (mt, sg) order; one lane-half swap completes the 64-head sum.
  auto epi_part = [&](const floatx16_t (&S)[2], int j, float acc) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < VPP; ++u) {
      const int v = VPP * j + u, mt = v >> 4, sg = v & 15;
      acc = fmaf(wr[mt][sg], __builtin_elementwise_maximum(S[mt][sg], 0.0f), acc);
    }
    return acc;
  };
  auto epi_end = [&](float acc) __attribute__((always_inline)) {
    const float2_t h2 = lane_halves(acc);
    return h2.x + h2.y;
  };
  // The MFMAs of key half nt of the tile at tb into Sd; with EPI, the epilogue of Se
  // rides along, one slice per k-step. Se's last MFMA was issued before this call:
  // the leading s_nops give a VALU read of its result the wait states it needs.
  auto half = [&](auto epi_t, const char* tb, int nt, floatx16_t (&Sd)[2], const floatx16_t (&Se)[2],
                  int gtile = -1) __attribute__((always_inline)) -> float {
    constexpr bool EPI = decltype(epi_t)::value;
    float acc = 0.0f;
    // The empty asm statements keep the epilogue where it is written: Se passes through
    // one here (so its ReLUs are not hoisted into a common block before the caller's
    // branch), and each k-step's partial sum through another (so its slice is not
    // sunk past the later MFMAs).
    floatx16_t E[2] = {Se[0], Se[1]};
    if constexpr (EPI) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(E[0]), "+v"(E[1]));
#pragma unroll
    for (int kn = 0; kn < KSTEPS; ++kn) {
      const int i = KSTEPS * nt + kn;
      const bf16x8_t b = ring[i % DA];
      if (i + DA < NSL) slice_load(tb, i + DA);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        Sd[mt] = kn == 0 ? idx_mfma_first(qa[mt][0], b) : idx_mfma_acc(qa[mt][kn], b, Sd[mt]);
      if constexpr (EPI) {
        acc = epi_part(E, kn, acc);
        asm volatile("" : "+v"(acc));
      }
      // a tile gather's DMAs, one per k-step from the first: each DMA's issue then
      // overlaps the MFMAs instead of stalling the wave before them, and the copy
      // still starts early in the tile
      if (gtile >= 0 && kn < NG) gather_one(gtile, kn);
      __builtin_amdgcn_sched_barrier(0);
    }
    return EPI ? epi_end(acc) : 0.0f;
  };
  // epilogue of one half without MFMAs (the wave's last tile)
  auto epi_only = [&](const floatx16_t (&Se)[2]) __attribute__((always_inline)) -> float {
    floatx16_t E[2] = {Se[0], Se[1]};
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(E[0]), "+v"(E[1]));
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) acc = epi_part(E, j, acc);
    return epi_end(acc);
  };
  // lane L's score of key k0 + L (+0.0 for -0.0): keys 0..31 from tot0, 32..63 from tot1
  auto score_of = [&](float tot0, float tot1) __attribute__((always_inline)) {
    const float sc = hl ? tot1 : tot0;
    return sc == 0.0f ? 0.0f : sc;
  };
  // Cut-back: one histogram pass keeps the buckets that hold the top k (a little more
  // than k keys); only when ties leave the buffer nearly full is the exact select run.
  auto cut_back = [&]() __attribute__((always_inline)) {
    uint32_t hi = kmax;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hi = max(hi, (uint32_t)__shfl_xor(hi, off, kWave));
    // after a cut-back one more tile (kKT keys) must still fit: kept <= cap - kKT
    const int limit = a.topk + (a.cap - a.topk - kKT) / 2;
    uint32_t edge;
    const int kept = wave_cut(keys, ids, n, a.cap, a.topk, limit, whist, tau, hi, edge);
    if (kept <= limit) {
      n = kept;
      tau = edge - 1u;                  // every held key is > edge - 1 = tau
      if (edge == 0u) tau = 0u;
    } else {
      tau = wave_select(keys, ids, n, a.topk, whist, tau, hi);
      n = a.topk;
    }
  };
  auto select = [&](float sc, int tile) __attribute__((always_inline)) {
    const int kg = cs + tile * kKT + L;
    const bool valid = kg <= t;            // kg >= cs always
    if constexpr (APPEND) {
      const bool take = valid && order_key(sc) > tau;
      const uint64_t tb2 = ballot(take);
      if (tb2 == 0) return;
      const int pos = n + (int)mbcnt(tb2);
      if (take && pos < a.ws_cap) {
        a.ws_val[(int64_t)t * a.ws_cap + pos] = sc;
        a.ws_idx[(int64_t)t * a.ws_cap + pos] = kg;
      }
      n += __popcll(tb2);
      return;
    }
    if (!fused) {
      if (valid) a.scores[(int64_t)t * a.ld + (kg - cs)] = sc;
      return;
    }
    const uint32_t kk = order_key(sc);
    bool take = valid && kk > tau;
    uint64_t tb2 = ballot(take);
    if (tb2 == 0) return;
    int cnt = __popcll(tb2);
    if (n + cnt > a.cap) {                // cannot happen after a requested cut-back
      cut_back();
      take = valid && kk > tau;
      tb2 = ballot(take);
      cnt = __popcll(tb2);
    }
    const int pos = n + (int)mbcnt(tb2);
    if (take) { keys[pos] = kk; ids[pos] = kg; kmax = max(kmax, kk); }
    n += cnt;
    if (n > a.cap - kKT && L == 0) s_req = tile;
    __builtin_amdgcn_wave_barrier();
  };

  if constexpr (APPEND) {
    // ---- pivot from a sample of the workgroup's causal keys (when some token of the
    //      workgroup has more keys than its workspace row holds): sample key j of
    //      kSample is cs + j * n0 / kSample, n0 = keys of the first token, so every
    //      sample key is causal for all four tokens
    if (t1 - cs > a.ws_cap) {
      const int n0 = t0 - cs + 1;
      auto sgather = [&](int st) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)(uintptr_t)(SA_LDS char*)(ktiles + (st & 1) * TILE_BYTES);
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          const int p = 64 * (w + kMaxWaves * j) + L;
          const int r = p / CPR;
          const int c = (p % CPR) ^ kswz<CPR>(r);
          const int key = cs + (int)(((int64_t)(st * kKT + r) * n0) / kSample);
          lds_dma16(base + (w + kMaxWaves * j) * 1024,
                    reinterpret_cast<const char*>(a.k) + (int64_t)key * DI * 2 + 16 * c);
        }
      };
      constexpr int NS = kSample / kKT;
      uint32_t xs[NS];
      sgather(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        wait_vmcnt0();
        __syncthreads();                  // sample tile st resident; tile st-1 read by all
        if (st + 1 < NS) sgather(st + 1);
        const char* tb = ktiles + (st & 1) * TILE_BYTES;
        tile_start(tb);
        half(std::false_type{}, tb, 0, S0, S1);
        const float s0 = half(std::true_type{}, tb, 1, S1, S0);
        xs[st] = order_key(score_of(s0, epi_only(S1)));
      }
      __syncthreads();                    // every wave is done with the sample tiles
      const int nt = t - cs + 1;
      if (active && nt > a.ws_cap) {
        // the k-th key's expected sample rank r0, aimed at r0 + 4.3 sqrt(r0) + 1
        const float r0 = (float)kSample * (float)a.topk / (float)nt;
        const uint32_t target = (uint32_t)(r0 + 4.3f * __builtin_sqrtf(r0)) + 1u;
        uint32_t P = 0u;                  // largest key that `target` sample keys reach
#pragma unroll 1
        for (int b = 31; b >= 0; --b) {
          const uint32_t cnd = P | (1u << b);
          uint32_t cnt = 0;
#pragma unroll
          for (int i = 0; i < NS; ++i) cnt += (uint32_t)__popcll(ballot(xs[i] >= cnd));
          if (cnt >= target) P = cnd;
        }
        tau = P > 0u ? P - 1u : 0u;       // append keys >= P
      }
    }
  }

  // Software pipeline over key halves: iteration `tile` runs the first half's MFMAs of
  // tile+1 with the epilogue of tile's second half, selects tile, then runs the second
  // half's MFMAs of tile+1 with the epilogue of its first half (kept in tot0).
  float tot0 = 0.0f;
  gather(0);
  wait_vmcnt0();
  __syncthreads();                        // tile 0 resident, s_req initialised
  if (ntiles > 1) gather(1);
  if (my_tiles > 0) {
    tile_start(ktiles);
    half(std::false_type{}, ktiles, 0, S0, S1);
    tot0 = half(std::true_type{}, ktiles, 1, S1, S0);
  }
#pragma unroll 1
  for (int tile = 0; tile < ntiles; ++tile) {
    wait_vmcnt0();
    __syncthreads();                      // tile+1 resident; every wave is done with tile
    // The gather of tile+2 refills the buffer every wave finished reading before the
    // barrier. With SPREAD (the dense launch) a wave with MFMAs to issue spreads its
    // DMAs over the first half, which measured faster there; the fused launch issues
    // them at once, before a possible cut-back (spreading them measured slower there).
    const int gt = tile + 2 < ntiles ? tile + 2 : -1;
    const bool spread = SPREAD && tile + 1 < my_tiles;
    if (gt >= 0 && !spread) gather(gt);
    if (fused && s_req == tile - 1 && n > a.topk) cut_back();
    if (tile >= my_tiles) continue;       // wave-uniform: no causal key of t left
    if (tile + 1 < my_tiles) {
      const char* tb = ktiles + ((tile + 1) & 1) * TILE_BYTES;
      tile_start(tb);
      const float tot1 = half(std::true_type{}, tb, 0, S0, S1, SPREAD ? gt : -1);
      select(score_of(tot0, tot1), tile);
      tot0 = half(std::true_type{}, tb, 1, S1, S0);
    } else {
      select(score_of(tot0, epi_only(S1)), tile);
    }
  }

  if constexpr (APPEND) {
    if (active && L == 0) {
      const int nv = t - cs + 1;
      a.ws_cnt[t] = n <= a.ws_cap && (n >= a.topk || n == nv) ? n : -1;
    }
    return;
  }
  if (!fused || !active) return;
  if (n > a.topk) {
    uint32_t hi = kmax;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hi = max(hi, (uint32_t)__shfl_xor(hi, off, kWave));
    wave_select(keys, ids, n, a.topk, whist, tau, hi);
    n = a.topk;
  }
  __builtin_amdgcn_wave_barrier();
  int32_t* orow = a.out_idx + (int64_t)t * a.topk;
  float* vrow = a.out_val ? a.out_val + (int64_t)t * a.topk : nullptr;
  for (int j = L; j < a.topk; j += kWave) {
    if (j < n) {
      orow[j] = ids[j];
      if (vrow) vrow[j] = key_value(keys[j]);
    } else {
      orow[j] = -1;
      if (vrow) vrow[j] = -__builtin_huge_valf();
    }
  }
}

// 64-head launches. Dense (topk == 0), fused with LDS candidate buffers, or the
// append pass of the two-pass selection (a.ws_val set).
template <int DI>
hipError_t launch_64(const IdxArgs& a0, int maxlen, hipStream_t st) {
  IdxArgs a = a0;
  constexpr int CPR = DI * 2 / 16;
  constexpr int TILE_BYTES = kKT * CPR * 16;
  const int mode = a.topk == 0 ? kDense : a.ws_val ? kAppend : kFused;
  a.cap = 0;
  if (mode == kFused) {
    // room above k: at least two tiles, so that a cut-back always frees a tile, and as
    // much more as the LDS holds (each cut-back then frees more room: fewer of them)
    const size_t fixed = 2 * (size_t)TILE_BYTES + (size_t)kMaxWaves * 256 * 4 + 256;   // + static LDS
    const int fit = (int)((160 * 1024 - fixed) / ((size_t)kMaxWaves * 8));
    const int extra = a.topk < 256 ? 256 : (a.topk > 1024 ? 1024 : a.topk);
    a.cap = max(a.topk + extra, min(fit, 2 * a.topk + 2 * kKT));
    a.cap &= ~63;                         // 16-byte aligned buffers for the cut-back's reads
  }
  const size_t shm = mode == kAppend
                         ? 2 * (size_t)TILE_BYTES
                         : 2 * (size_t)TILE_BYTES + (size_t)kMaxWaves * 256 * 4 + (size_t)kMaxWaves * a.cap * 8;
  if (shm > 160 * 1024) return hipErrorInvalidValue;
  a.nwave = kMaxWaves;
  a.chunks = (maxlen + kMaxWaves - 1) / kMaxWaves;
  const void* kern = mode == kDense   ? (const void*)indexer64_kernel<DI, kDense>
                     : mode == kFused ? (const void*)indexer64_kernel<DI, kFused>
                                      : (const void*)indexer64_kernel<DI, kAppend>;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  const dim3 grid(a.chunks, a.nseq), block(kMaxWaves * 64);
  if (mode == kDense)
    hipLaunchKernelGGL((indexer64_kernel<DI, kDense>), grid, block, shm, st, a);
  else if (mode == kFused)
    hipLaunchKernelGGL((indexer64_kernel<DI, kFused>), grid, block, shm, st, a);
  else
    hipLaunchKernelGGL((indexer64_kernel<DI, kAppend>), grid, block, shm, st, a);
  return hipGetLastError();
}

template <bool BF16, int HI, int DI>
hipError_t launch_hi(const IdxArgs& a0, int maxlen, hipStream_t st) {
  IdxArgs a = a0;
  const bool fused = a.topk > 0;
  constexpr int CPR = DI * (BF16 ? 2 : 4) / 16;
  constexpr int TILE_BYTES = kKT * CPR * 16;
  constexpr int TW = 64 / HI;
  auto lds_for = [&](int nw) {
    const int QT = nw * TW;
    size_t b = 2 * (size_t)TILE_BYTES + (size_t)QT * kKT * 4 + (size_t)nw * 256 * 4 + (size_t)QT * 16;
    if (fused) b += (size_t)QT * a.cap * 8;
    return b;
  };
  if (fused) {
    const int extra = a.topk < 64 ? 64 : (a.topk > 1024 ? 1024 : a.topk);
    a.cap = a.topk + extra;
  }
  int nw = kMaxWaves;
  const size_t budget = 160 * 1024 - 256;
  while (nw > 1 && lds_for(nw) > budget) nw >>= 1;
  if (lds_for(nw) > budget) return hipErrorInvalidValue;
  a.nwave = nw;
  const int QT = nw * TW;
  a.chunks = (maxlen + QT - 1) / QT;
  const size_t shm = lds_for(nw);
  hipError_t e = hipFuncSetAttribute((const void*)indexer_kernel<BF16, HI, DI>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((indexer_kernel<BF16, HI, DI>), dim3(a.chunks, a.nseq, a.nsplit > 1 ? a.nsplit : 1),
                     dim3(nw * 64), shm, st, a);
  return hipGetLastError();
}

template <bool BF16, int DI>
hipError_t launch_di(const IdxArgs& a, int H_I, int maxlen, hipStream_t st) {
  switch (H_I) {
    case 4: return launch_hi<BF16, 4, DI>(a, maxlen, st);
    case 8: return launch_hi<BF16, 8, DI>(a, maxlen, st);
    case 16: return launch_hi<BF16, 16, DI>(a, maxlen, st);
    case 32: return launch_hi<BF16, 32, DI>(a, maxlen, st);
    default: return launch_hi<BF16, 64, DI>(a, maxlen, st);
  }
}

hipError_t launch_any(const IdxArgs& a, bool bf16, int H_I, int D_I, int maxlen, hipStream_t st) {
  if (bf16 && H_I == 64 && a.B == 1) return D_I == 64 ? launch_64<64>(a, maxlen, st) : launch_64<128>(a, maxlen, st);
  if (bf16) return D_I == 64 ? launch_di<true, 64>(a, H_I, maxlen, st) : launch_di<true, 128>(a, H_I, maxlen, st);
  return D_I == 64 ? launch_di<false, 64>(a, H_I, maxlen, st) : launch_di<false, 128>(a, H_I, maxlen, st);
}

}  // namespace

hipError_t launch_indexer_dense(const void* q, const void* k, const float* w, bool bf16, int T,
                                const int32_t* cu, int nseq, int maxlen, int H_I, int D_I,
                                int block_size, float* scores, int64_t ld, hipStream_t st) {
  if (T == 0) return hipSuccess;
  IdxArgs a{};
  a.q = q; a.k = k; a.w = w; a.T = T; a.cu = cu; a.nseq = cu ? nseq : 1; a.B = block_size;
  a.scores = scores; a.ld = ld; a.topk = 0;
  return launch_any(a, bf16, H_I, D_I, cu ? maxlen : T, st);
}

bool indexer_two_pass(bool bf16, int H_I, int block_size, int topk) {
  return bf16 && H_I == 64 && block_size == 1 && topk > 0;
}

// Entries per workspace row: the keys of a whole row when every row fits, else enough
// for the pivot's count with margin. Sample key j of kSample stands for maxlen /
// kSample keys; the pivot aims at r0 + 4.3 sqrt(r0) + 1 sample keys (r0 = kSample k /
// maxlen), and the row holds the count that the sample reaches with that many keys
// 4.3 standard deviations below its mean: c = maxlen / kSample * (z/2 + sqrt(z^2/4 +
// target))^2. Rounded up to 64 entries.
int indexer_ws_cap(int topk, int maxlen) {
  const double z = 4.3;
  const double r0 = (double)kSample * topk / (double)maxlen;
  const double target = r0 + z * std::sqrt(r0) + 2.0;
  const double root = z / 2 + std::sqrt(z * z / 4 + target);
  int64_t cap = (int64_t)std::ceil((double)maxlen / kSample * root * root) + 64;
  cap = std::max<int64_t>(cap, topk);
  cap = std::min<int64_t>(cap, maxlen);
  return (int)((cap + 63) / 64 * 64);
}

// Workgroups over which block mode splits each token chunk's key tiles when a
// workspace is given: about 32 tiles each, at most 4 (so that a token's partial lists
// hold at most 4 x 64 candidates); 1 (no split) for rows of up to 32 tiles.
int indexer_block_splits(int maxlen, int block_size, int topk) {
  if (block_size == 1 || topk <= 0) return 1;
  const int tiles = (maxlen + kKT - 1) / kKT;
  const int ns = (tiles + 31) / 32;
  return ns < 1 ? 1 : (ns > 4 ? 4 : ns);
}

size_t indexer_ws_bytes(bool bf16, int T, int maxlen, int H_I, int block_size, int topk) {
  if (T <= 0) return 0;
  const int ns = indexer_block_splits(maxlen, block_size, topk);
  if (ns > 1)   // partial lists: keys, block ids, counts; the own block's value
    return (size_t)T * ns * topk * 8 + (size_t)T * ns * 4 + (size_t)T * 4;
  if (!indexer_two_pass(bf16, H_I, block_size, topk)) return 0;
  const int cap = indexer_ws_cap(topk, maxlen);
  return (size_t)T * cap * 8 + (size_t)T * 4;
}

hipError_t launch_indexer_topk(const void* q, const void* k, const float* w, bool bf16, int T,
                               const int32_t* cu, int nseq, int maxlen, int H_I, int D_I,
                               int block_size, int topk, int force_own, int32_t* out_idx,
                               float* out_val, void* ws, hipStream_t st) {
  if (T == 0) return hipSuccess;
  IdxArgs a{};
  a.q = q; a.k = k; a.w = w; a.T = T; a.cu = cu; a.nseq = cu ? nseq : 1; a.B = block_size;
  a.topk = topk; a.force_own = force_own; a.out_idx = out_idx; a.out_val = out_val;
  const int width = cu ? maxlen : T;
  const int ns = indexer_block_splits(width, block_size, topk);
  if (ws && ns > 1) {
    // block mode: partial top-k lists of ns key ranges per token chunk, then the merge
    a.nsplit = ns;
    a.sp_key = static_cast<uint32_t*>(ws);
    a.sp_id = reinterpret_cast<int32_t*>(a.sp_key + (size_t)T * ns * topk);
    a.sp_cnt = a.sp_id + (size_t)T * ns * topk;
    a.sp_own = reinterpret_cast<float*>(a.sp_cnt + (size_t)T * ns);
    hipError_t e = launch_any(a, bf16, H_I, D_I, width, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(indexer_merge_kernel, dim3((T + kMergeWaves - 1) / kMergeWaves),
                       dim3(kMergeWaves * 64), 0, st, a);
    return hipGetLastError();
  }
  if (!ws || !indexer_two_pass(bf16, H_I, block_size, topk))
    return launch_any(a, bf16, H_I, D_I, width, st);
  // two passes through the workspace: [T, cap] scores, [T, cap] key ids, [T] counts
  const int cap = indexer_ws_cap(topk, width);
  a.ws_cap = cap;
  a.ws_val = static_cast<float*>(ws);
  a.ws_idx = reinterpret_cast<int32_t*>(a.ws_val + (size_t)T * cap);
  a.ws_cnt = a.ws_idx + (size_t)T * cap;
  hipError_t e = D_I == 64 ? launch_64<64>(a, width, st) : launch_64<128>(a, width, st);
  if (e != hipSuccess) return e;
  e = launch_topk_select_counted(a.ws_val, a.ws_idx, a.ws_cnt, cap, T, topk, out_idx, out_val, st);
  if (e != hipSuccess) return e;
  // rows whose pivot missed: the exact single-pass kernel, on their workgroups only
  IdxArgs r = a;
  r.ws_val = nullptr;
  r.ws_idx = nullptr;
  return D_I == 64 ? launch_64<64>(r, width, st) : launch_64<128>(r, width, st);
}

}  // namespace sa
