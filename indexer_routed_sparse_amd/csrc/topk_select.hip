// Exact deterministic top-k of score rows, one 512-thread workgroup per row.
//
// Order (per "Add trainable QSA sparse attention with a TileLang backend", section
// "Describe the solution you'd like": a lexicographic (score, id) key): higher score
// first, then smaller index. Candidates sit in ascending index order, so "smaller
// index" is "earlier position" and ties at the k-th score are resolved by a
// position-ordered prefix count.
//
// The row is read from HBM once into registers: wave w owns the contiguous span
// [w*seg, (w+1)*seg) of the row (seg a multiple of 256), one float4 per lane per
// 256-position chunk. The selection then never touches HBM again:
//
//   1. pivot: for rows wider than the candidate buffer, one wave bisects the order
//      key over a 512-entry sample (one value per lane, spread over all chunks of
//      every wave) for a value that about k plus four standard deviations of the
//      sample rank keys reach. In dense mode the sample is loaded ahead of the row,
//      so the bisection runs while the row is still arriving. The pivot almost
//      always keeps at least k and at most kCap keys; correctness never depends
//      on it, since both bounds are checked exactly.
//   2. count the keys >= pivot per wave (float compares, ballot popcounts), then
//      compact them, in position order, into an LDS buffer of kCap entries.
//   3. exact radix select over the compacted candidates: keys are offset by the
//      candidate minimum and 12-bit digits are taken from the top of the occupied
//      range. As soon as the bin holding the k-th key has at most 64 members, one
//      wave ranks those members directly instead of running another pass.
//   4. rank by a block-wide prefix count and write the indices in ascending order.
//
// Rows whose pivot fails (fewer than k or more than kCap keys above it) are marked
// and redone by a second, persistent launch that runs the same radix select over
// every key held in registers; a single launch of that kind serves all rows when
// topk exceeds kCap. With force_own_block the query's own block (the last column)
// is taken out of the competition and written after the others, which is where
// ascending order puts it.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kNT = 512;                 // threads per row
constexpr int kNW = kNT / kWave;         // waves per row
constexpr int kSpan = 4 * kWave;         // positions per wave chunk
constexpr int kCap = 6144;               // candidate buffer entries
constexpr int kPer = kCap / kNT;         // candidates per thread in the exact stage
constexpr int kDigit = 12;               // radix digit bits
constexpr int kBins = 1 << kDigit;
constexpr int kSmall = 64;               // bins this small are ranked by one wave
constexpr int kRetryGrid = 512;          // workgroups of the persistent retry launch
constexpr int32_t kRetry = INT32_MIN;    // out_idx[t, 0] of a row left to the retry launch
// LDS (about 52 KB, so three rows fit a CU): candidate values and 16-bit positions,
// the first histogram, per-wave partials, broadcast slots, the small-bin gather
// list. The value array also holds the pivot sample (before compaction) and the
// second histogram (once candidates sit in registers); after the select, the
// output is staged by rank over values/positions/first histogram: positions from
// byte 0, values from byte kStageVal.
constexpr size_t kOffPos = kCap * sizeof(uint32_t);
constexpr size_t kOffHist = kOffPos + kCap * sizeof(uint16_t);
constexpr size_t kOffRed = kOffHist + kBins * sizeof(uint32_t);
constexpr size_t kOffBc = kOffRed + 8 * kNW * sizeof(uint32_t);
constexpr size_t kOffGath = kOffBc + 8 * sizeof(uint32_t);
constexpr size_t kSmemBytes = kOffGath + kSmall * sizeof(uint32_t);
constexpr size_t kStageVal = kCap * sizeof(uint32_t);
static_assert(kBins * sizeof(uint32_t) <= kCap * sizeof(uint32_t), "second histogram fits");
static_assert(kStageVal + kCap * sizeof(float) <= kOffRed, "staging fits");
static_assert(kNT * sizeof(uint32_t) <= kCap * sizeof(uint32_t), "sample fits");

SA_DEVICE float qnan() { return __uint_as_float(0x7FC00000u); }

// Order key of a non-NaN value; NaN marks an excluded slot and maps to 0.
SA_DEVICE uint32_t key_or_zero(float f) { return f == f ? order_key(f) : 0u; }

SA_DEVICE uint32_t mbcnt_add(uint64_t mask, uint32_t acc) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, acc));
}

// Wave-wide inclusive prefix sum with DPP row shifts and row broadcasts.
SA_DEVICE uint32_t dpp_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Wave-wide max (result valid in lane 63).
SA_DEVICE uint32_t dpp_max_to_last(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));
  return x;
}

// Wave-wide min (result valid in lane 63).
SA_DEVICE uint32_t dpp_min_to_last(uint32_t x) { return ~dpp_max_to_last(~x); }

// Sum of the per-wave partials red[0..w) (exclusive) and of all of them.
SA_DEVICE uint32_t wave_offset(const uint32_t* red, int w, uint32_t* total) {
  uint32_t below = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kNW; ++i) {
    const uint32_t x = red[i];
    below += i < w ? x : 0u;
    all += x;
  }
  *total = all;
  return below;
}

struct Smem {
  uint32_t* cval;  // [kCap] candidate value bits, position order
  uint16_t* cpos;  // [kCap] candidate positions
  uint32_t* hist;  // [kBins] first histogram, zero on entry to a select
  uint32_t* spos;  // [<= kCap] staged output positions by rank
  float* sval;     // [<= kCap] staged output values by rank
  uint32_t* red;   // [8][kNW] per-wave partials
  uint32_t* bc;    // [8] broadcast slots; bc[4] is the gather counter, zero on entry
  uint32_t* gath;  // [kSmall] members of a small bin
};

SA_DEVICE Smem smem_layout(unsigned char* raw) {
  Smem sm;
  sm.cval = reinterpret_cast<uint32_t*>(raw);
  sm.cpos = reinterpret_cast<uint16_t*>(raw + kOffPos);
  sm.hist = reinterpret_cast<uint32_t*>(raw + kOffHist);
  sm.spos = reinterpret_cast<uint32_t*>(raw);
  sm.sval = reinterpret_cast<float*>(raw + kStageVal);
  sm.red = reinterpret_cast<uint32_t*>(raw + kOffRed);
  sm.bc = reinterpret_cast<uint32_t*>(raw + kOffBc);
  sm.gath = reinterpret_cast<uint32_t*>(raw + kOffGath);
  return sm;
}

// Result of a select: the k-th largest key is base + thr (offset domain). mode 1:
// every key >= base + thr is taken (exactly k of them). mode 2: keys > base + thr are
// taken plus the first `need` keys equal to it in position order.
struct Cut {
  uint32_t base, thr, need;
  int mode;
};

SA_DEVICE bool take_gt(uint32_t k, const Cut& c) {
  if (k == 0u) return false;
  const uint32_t d = k - c.base;
  return c.mode == 1 ? d >= c.thr : d > c.thr;
}

SA_DEVICE bool take_eq(uint32_t k, const Cut& c) {
  return k != 0u && c.mode == 2 && k - c.base == c.thr;
}

// Exact radix select of the k-th largest among the nonzero order keys x (held N per
// thread). The caller guarantees that at least k keys are nonzero, that sm.hist and
// bc[4] are zero on entry and that sm.cval is no longer read by any thread once
// every thread has entered. Uses red rows 4..7, bc and gath.
template <int N>
SA_DEVICE Cut radix_select(const uint32_t (&x)[N], uint32_t k, const Smem& sm) {
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const uint32_t kk = x[r];
    kmin = kk != 0u ? min(kmin, kk) : kmin;
    kmax = max(kmax, kk);
  }
  kmin = dpp_min_to_last(kmin);
  kmax = dpp_max_to_last(kmax);
  if (l == kWave - 1) { sm.red[6 * kNW + w] = kmin; sm.red[7 * kNW + w] = kmax; }
  __syncthreads();
  uint32_t gmin = 0xFFFFFFFFu, gmax = 0u;
#pragma unroll
  for (int i = 0; i < kNW; ++i) { gmin = min(gmin, sm.red[6 * kNW + i]); gmax = max(gmax, sm.red[7 * kNW + i]); }

  Cut cut{gmin, 0u, k, 2};
  const uint32_t span = gmax - gmin;
  int hi = span ? 32 - __builtin_clz(span) : 0;  // occupied offset bits
  uint32_t prefix = 0;
  int buf = 0;
  uint32_t* const second = sm.cval;
#pragma unroll 1
  while (hi > 0) {
    const int s = hi > kDigit ? hi - kDigit : 0;
    const int nbits = hi - s;
    const int nb = 1 << nbits;
    uint32_t* H = buf ? second : sm.hist;
    uint32_t* Hn = buf ? sm.hist : second;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const uint32_t kk = x[r];
      const uint32_t d = kk - gmin;
      const bool in = kk != 0u && (hi >= 32 || (d >> hi) == prefix);
      if (in) atomicAdd(&H[(d >> s) & (uint32_t)(nb - 1)], 1u);
      if ((r & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // bound live addresses
    }
    for (int b = tid; b < kBins; b += kNT) Hn[b] = 0u;  // next pass's buffer
    __syncthreads();
    // suffix counts from the top bin: thread i owns bins nb-1-8i .. nb-8-8i
    constexpr int kPT = kBins / kNT;
    uint32_t loc[kPT], tsum = 0;
#pragma unroll
    for (int r = 0; r < kPT; ++r) {
      const int b = nb - 1 - kPT * tid - r;
      loc[r] = b >= 0 ? H[b] : 0u;
      tsum += loc[r];
    }
    const uint32_t inc = dpp_incl_scan(tsum);
    if (l == kWave - 1) sm.red[4 * kNW + w] = inc;
    __syncthreads();
    uint32_t tot;
    uint32_t run = inc - tsum + wave_offset(sm.red + 4 * kNW, w, &tot);
#pragma unroll
    for (int r = 0; r < kPT; ++r) {
      const uint32_t above = run;
      run += loc[r];
      if (above < cut.need && run >= cut.need) {
        sm.bc[1] = (uint32_t)(nb - 1 - kPT * tid - r);
        sm.bc[2] = above;
        sm.bc[3] = loc[r];
      }
    }
    __syncthreads();
    const uint32_t d = sm.bc[1], above = sm.bc[2], cnt = sm.bc[3];
    prefix = (prefix << nbits) | d;
    cut.need -= above;
    if (cnt == cut.need) {  // the whole bin is taken
      cut.mode = 1;
      cut.thr = prefix << s;
      return cut;
    }
    if (s > 0 && cnt <= (uint32_t)kSmall) {
      // gather the bin's members; one wave finds the need-th largest among them
#pragma unroll
      for (int r = 0; r < N; ++r) {
        const uint32_t kk = x[r];
        if (kk != 0u && ((kk - gmin) >> s) == prefix) sm.gath[atomicAdd(&sm.bc[4], 1u)] = kk - gmin;
      }
      __syncthreads();
      if (w == 0) {
        const bool mine = (uint32_t)l < cnt;
        const uint32_t me = mine ? sm.gath[l] : 0u;
        uint32_t gt = 0, eq = 0;
#pragma unroll 1
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)me, (int)j);
          gt += o > me ? 1u : 0u;
          eq += o == me ? 1u : 0u;
        }
        if (mine && gt < cut.need && cut.need <= gt + eq) {
          sm.bc[5] = me;
          sm.bc[6] = cut.need - gt;
        }
      }
      __syncthreads();
      cut.thr = sm.bc[5];
      cut.need = sm.bc[6];
      return cut;
    }
    hi = s;
    buf ^= 1;
  }
  cut.thr = prefix;  // exact offset of the k-th key; `need` of its ties are taken
  return cut;
}

struct RowArgs {
  int row0;  // first row of this launch
  const float* vals;
  const int32_t* cand;
  int64_t ld;
  const int32_t* cu;
  int nseq, block_size, topk, force_own;
  int32_t* out_idx;
  float* out_val;
};

// KIND 0: pivot + candidate buffer (topk <= kCap). Rows whose pivot fails get
//         kRetry in their first output slot and nothing else.
// KIND 1: radix select over the keys held in registers (any topk); selected
//         positions go straight to out_idx and become ids in a copy-out pass.
template <int CH, int KIND>
SA_DEVICE void select_row(int t, const RowArgs& a, const Smem& sm) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int topk = a.topk;

  int start = 0, n;
  if (a.cand) {
    n = (int)a.ld;
  } else {
    if (a.cu) start = seq_start_of(a.cu, a.nseq, t);
    const int off = t - start;
    n = (a.block_size == 1) ? off + 1 : off / a.block_size + 1;
  }
  const bool own = !a.cand && a.block_size > 1 && a.force_own;
  const int n1 = own ? n - 1 : n;          // competing positions
  const int k1 = own ? topk - 1 : topk;    // slots they compete for
  const float* __restrict__ row = a.vals + (int64_t)t * a.ld;
  const int32_t* __restrict__ crow = a.cand ? a.cand + (int64_t)t * a.ld : nullptr;
  int32_t* __restrict__ orow = a.out_idx + (int64_t)t * topk;
  float* __restrict__ vrow = a.out_val ? a.out_val + (int64_t)t * topk : nullptr;
  const int32_t idbase = a.block_size == 1 ? start : 0;

  const int seg = (n1 + kNW * kSpan - 1) / (kNW * kSpan) * kSpan;
  const int ws = w * seg;
  const int we = min(ws + seg, n1);
  const int m = we > ws ? (we - ws + kSpan - 1) / kSpan : 0;  // chunks of this wave

  for (int b = tid; b < kBins; b += kNT) sm.hist[b] = 0u;
  if (tid == 0) sm.bc[4] = 0u;

  // Dense rows that will need a pivot: fetch the sample before the row so that it
  // arrives first (loads complete in order). Lane l samples chunk l % m.
  const bool early = KIND == 0 && !crow && n1 > kCap && k1 < n1;
  float smp = qnan();
  if (early) {
    const int ps = ws + (m > 0 ? l % m : 0) * kSpan + 4 * l;
    if (m > 0 && ps < we) smp = row[ps];
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- load the wave's span; excluded slots become NaN
  float v[4 * CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float4 x = make_float4(qnan(), qnan(), qnan(), qnan());
    if (c < m) {
      const int pos = ws + c * kSpan + 4 * l;
      if (pos < we) {
        x = *reinterpret_cast<const float4*>(row + pos);
        if (crow) {
          const int4 ci = *reinterpret_cast<const int4*>(crow + pos);
          if (ci.x < 0) x.x = qnan();
          if (ci.y < 0) x.y = qnan();
          if (ci.z < 0) x.z = qnan();
          if (ci.w < 0) x.w = qnan();
        }
        if (pos + 4 > we) {
          if (pos + 1 >= we) x.y = qnan();
          if (pos + 2 >= we) x.z = qnan();
          if (pos + 3 >= we) x.w = qnan();
        }
      }
    }
    v[4 * c + 0] = x.x;
    v[4 * c + 1] = x.y;
    v[4 * c + 2] = x.z;
    v[4 * c + 3] = x.w;
  }

  int nvalid = n1;
  if (crow) {
    uint32_t cv = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < m)
#pragma unroll
        for (int j = 0; j < 4; ++j) cv += __popcll(ballot(v[4 * c + j] == v[4 * c + j]));
    if (l == 0) sm.red[0 * kNW + w] = cv;
    __syncthreads();
    uint32_t tot;
    wave_offset(sm.red + 0 * kNW, w, &tot);
    nvalid = (int)tot;
  }
  const int nsel = k1 < nvalid ? k1 : nvalid;

  if (nsel > 0) {
    if constexpr (KIND == 0) {
      if (nvalid <= k1) {
        // every valid key is taken: stage by rank = valid keys before it
        uint32_t cg = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (c < m)
#pragma unroll
            for (int j = 0; j < 4; ++j) cg += __popcll(ballot(v[4 * c + j] == v[4 * c + j]));
        if (l == 0) sm.red[2 * kNW + w] = cg;
        __syncthreads();
        uint32_t tot;
        uint32_t og = wave_offset(sm.red + 2 * kNW, w, &tot);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if (c < m) {
            bool g[4];
            uint64_t bg[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) { g[j] = v[4 * c + j] == v[4 * c + j]; bg[j] = ballot(g[j]); }
            uint32_t lg = mbcnt_add(bg[3], mbcnt_add(bg[2], mbcnt_add(bg[1], mbcnt_add(bg[0], og))));
            const uint32_t pos = (uint32_t)(ws + c * kSpan + 4 * l);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (g[j]) {
                sm.spos[lg] = pos + j;
                sm.sval[lg] = v[4 * c + j] + 0.0f;
              }
              lg += g[j] ? 1u : 0u;
            }
            og += __popcll(bg[0]) + __popcll(bg[1]) + __popcll(bg[2]) + __popcll(bg[3]);
          }
        }
      } else {
        float pf = -__builtin_huge_valf();
        if (nvalid > kCap) {
          uint32_t* s_samp = sm.cval;
          if (!early) {
            const int cl = m > 0 ? l % m : 0;
#pragma unroll
            for (int c = 0; c < CH; ++c) smp = c == cl ? v[4 * c] : smp;
          }
          s_samp[tid] = m > 0 ? key_or_zero(smp) : 0u;
          __syncthreads();
          if (w == 0) {
            uint32_t xs[kNT / kWave];
#pragma unroll
            for (int i = 0; i < kNT / kWave; ++i) xs[i] = s_samp[l + kWave * i];
            uint32_t sv = 0;
#pragma unroll
            for (int i = 0; i < kNT / kWave; ++i) sv += __popcll(ballot(xs[i] != 0u));
            const float r0 = (float)sv * (float)k1 / (float)nvalid;
            const uint32_t target = (uint32_t)(r0 + 4.0f * __builtin_sqrtf(r0)) + 4u;
            const uint32_t enough = target + target / 4u;
            // Largest P (in key bits, high to low) with >= target sample keys at or
            // above it; refining stops once the sample count at P is within 25% of
            // target, which for smooth data happens after 10-16 bits.
            uint32_t P = 0, at_p = sv;
            if (target <= sv) {
#pragma unroll 1
              for (int b = 31; b >= 0 && at_p > enough; --b) {
                const uint32_t cnd = P | (1u << b);
                uint32_t cnt = 0;
#pragma unroll
                for (int i = 0; i < kNT / kWave; ++i) cnt += __popcll(ballot(xs[i] >= cnd));
                if (cnt >= target) { P = cnd; at_p = cnt; }
              }
            }
            if (l == 0) sm.bc[0] = P;
          }
          __syncthreads();
          const uint32_t P = sm.bc[0];
          if (P > 0x007FFFFFu) pf = key_value(P);  // lower P selects every valid key
        }
        // candidates: keys >= pivot, counted per wave
        uint32_t cc = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (c < m)
#pragma unroll
            for (int j = 0; j < 4; ++j) cc += __popcll(ballot(v[4 * c + j] >= pf));
        if (l == 0) sm.red[1 * kNW + w] = cc;
        __syncthreads();
        uint32_t C;
        uint32_t run = wave_offset(sm.red + 1 * kNW, w, &C);
        if (C < (uint32_t)k1 || C > (uint32_t)kCap) {
          if (tid == 0) orow[0] = kRetry;
          return;  // uniform
        }
        // compact in position order
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if (c < m) {
            bool p[4];
            uint64_t b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) { p[j] = v[4 * c + j] >= pf; b[j] = ballot(p[j]); }
            uint32_t o = mbcnt_add(b[3], mbcnt_add(b[2], mbcnt_add(b[1], mbcnt_add(b[0], run))));
            const uint32_t pos = (uint32_t)(ws + c * kSpan + 4 * l);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (p[j]) {
                sm.cval[o] = __float_as_uint(v[4 * c + j]);
                sm.cpos[o] = (uint16_t)(pos + j);
              }
              o += p[j] ? 1u : 0u;
            }
            run += __popcll(b[0]) + __popcll(b[1]) + __popcll(b[2]) + __popcll(b[3]);
          }
        }
        __syncthreads();
        uint32_t ck[kPer], cp[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          const uint32_t i = (uint32_t)(tid * kPer + r);
          ck[r] = i < C ? key_or_zero(__uint_as_float(sm.cval[i])) : 0u;
          cp[r] = i < C ? sm.cpos[i] : 0u;
        }
        const Cut c2 = radix_select<kPer>(ck, (uint32_t)k1, sm);
        // ranks: block-wide exclusive count of (greater, equal) in position order
        uint32_t ng = 0, ne = 0;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          ng += take_gt(ck[r], c2) ? 1u : 0u;
          ne += take_eq(ck[r], c2) ? 1u : 0u;
        }
        const uint32_t pk = ng | (ne << 16);  // both <= kCap < 2^16
        const uint32_t inc = dpp_incl_scan(pk);
        if (l == kWave - 1) sm.red[2 * kNW + w] = inc;
        __syncthreads();
        uint32_t tot;
        const uint32_t base = inc - pk + wave_offset(sm.red + 2 * kNW, w, &tot);
        uint32_t gb = base & 0xFFFFu, eb = base >> 16;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          const bool g = take_gt(ck[r], c2), e = take_eq(ck[r], c2);
          if (g || (e && eb < c2.need)) {
            const uint32_t rank = gb + (eb < c2.need ? eb : c2.need);
            sm.spos[rank] = cp[r];
            sm.sval[rank] = key_value(ck[r]);
          }
          gb += g ? 1u : 0u;
          eb += e ? 1u : 0u;
        }
      }
      // coalesced copy-out of the staged entries: positions -> reported ids
      __syncthreads();
      for (int i = tid; i < nsel; i += kNT) {
        const uint32_t pos = sm.spos[i];
        orow[i] = crow ? crow[pos] : idbase + (int32_t)pos;
        if (vrow) vrow[i] = sm.sval[i];
      }
    } else {
      uint32_t key[4 * CH];
#pragma unroll
      for (int e = 0; e < 4 * CH; ++e) key[e] = key_or_zero(v[e]);
      Cut cut{0u, 0u, 0u, 0};  // mode 0: every valid key
      if (nvalid > k1) cut = radix_select<4 * CH>(key, (uint32_t)k1, sm);
      // position-ordered ranks straight from the registers
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c < m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t kk = key[4 * c + j];
            cg += __popcll(ballot(cut.mode == 0 ? kk != 0u : take_gt(kk, cut)));
            ce += __popcll(ballot(take_eq(kk, cut)));
          }
      if (l == 0) { sm.red[2 * kNW + w] = cg; sm.red[3 * kNW + w] = ce; }
      __syncthreads();
      uint32_t tot;
      uint32_t og = wave_offset(sm.red + 2 * kNW, w, &tot);
      uint32_t oe = wave_offset(sm.red + 3 * kNW, w, &tot);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < m) {
          bool g[4], e[4];
          uint64_t bg[4], be[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t kk = key[4 * c + j];
            g[j] = cut.mode == 0 ? kk != 0u : take_gt(kk, cut);
            e[j] = take_eq(kk, cut);
            bg[j] = ballot(g[j]);
            be[j] = ballot(e[j]);
          }
          uint32_t lg = mbcnt_add(bg[3], mbcnt_add(bg[2], mbcnt_add(bg[1], mbcnt_add(bg[0], og))));
          uint32_t le = mbcnt_add(be[3], mbcnt_add(be[2], mbcnt_add(be[1], mbcnt_add(be[0], oe))));
          const uint32_t pos = (uint32_t)(ws + c * kSpan + 4 * l);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (g[j] || (e[j] && le < cut.need)) {
              const uint32_t rank = lg + (le < cut.need ? le : cut.need);
              orow[rank] = (int32_t)(pos + j);
              if (vrow) vrow[rank] = key_value(key[4 * c + j]);
            }
            lg += g[j] ? 1u : 0u;
            le += e[j] ? 1u : 0u;
          }
          og += __popcll(bg[0]) + __popcll(bg[1]) + __popcll(bg[2]) + __popcll(bg[3]);
          oe += __popcll(be[0]) + __popcll(be[1]) + __popcll(be[2]) + __popcll(be[3]);
        }
      }
      __syncthreads();
      // copy-out: positions -> reported ids
      for (int i = tid; i < nsel; i += kNT) {
        const int32_t pos = orow[i];
        orow[i] = crow ? crow[pos] : idbase + pos;
      }
    }
  }
  int filled = nsel;
  if (own) {
    if (tid == 0) {
      orow[nsel] = n - 1;
      if (vrow) vrow[nsel] = row[n - 1] + 0.0f;
    }
    ++filled;
  }
  for (int i = filled + tid; i < topk; i += kNT) {
    orow[i] = -1;
    if (vrow) vrow[i] = -__builtin_huge_valf();
  }
}

// Three 8-wave workgroups per CU (LDS allows it) need at most 80 VGPRs; rows wider
// than 8K positions do not fit that budget without spilling and run two per CU.
template <int CH>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(CH <= 8 ? 6 : 1)))
void topk_pivot_kernel(RowArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  select_row<CH, 0>(a.row0 + (int)blockIdx.x, a, smem_layout(smem_raw));
}

template <int CH>
__global__ __launch_bounds__(kNT) void topk_full_kernel(RowArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  select_row<CH, 1>(a.row0 + (int)blockIdx.x, a, smem_layout(smem_raw));
}

// Persistent redo of the rows the pivot pass marked: workgroup b owns rows
// b, b + grid, ...; it lists its marked rows, then selects them one by one.
template <int CH>
__global__ __launch_bounds__(kNT) void topk_retry_kernel(RowArgs a, int T) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const Smem sm = smem_layout(smem_raw);
  __shared__ uint32_t s_count;
  __shared__ int32_t s_rows[kNT];
  const int tid = threadIdx.x;
  const int stride = (int)gridDim.x;
  for (int base = blockIdx.x; base < T; base += stride * kNT) {
    if (tid == 0) s_count = 0u;
    __syncthreads();
    const int t = base + tid * stride;
    if (t < T && a.out_idx[(int64_t)t * a.topk] == kRetry) s_rows[atomicAdd(&s_count, 1u)] = t;
    __syncthreads();
    const uint32_t cnt = s_count;
    for (uint32_t i = 0; i < cnt; ++i) {
      select_row<CH, 1>(s_rows[i], a, sm);
      __syncthreads();
    }
    __syncthreads();  // every thread has read s_count before it is reset
  }
}

template <class K>
hipError_t set_smem(K kernel) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
}

template <int CH>
hipError_t launch_rows(const RowArgs& a, int r0, int r1, bool big, hipStream_t st) {
  static bool attr_set = false;  // per instantiation; setting it twice is harmless
  if (!attr_set) {
    hipError_t e = set_smem(&topk_pivot_kernel<CH>);
    if (e == hipSuccess) e = set_smem(&topk_full_kernel<CH>);
    if (e == hipSuccess) e = set_smem(&topk_retry_kernel<CH>);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  RowArgs b = a;
  b.row0 = r0;
  if (big)
    hipLaunchKernelGGL((topk_full_kernel<CH>), dim3(r1 - r0), dim3(kNT), kSmemBytes, st, b);
  else
    hipLaunchKernelGGL((topk_pivot_kernel<CH>), dim3(r1 - r0), dim3(kNT), kSmemBytes, st, b);
  return hipGetLastError();
}

template <int CH>
hipError_t launch_retry(const RowArgs& a, int T, hipStream_t st) {
  const int grid = T < kRetryGrid ? T : kRetryGrid;
  hipLaunchKernelGGL((topk_retry_kernel<CH>), dim3(grid), dim3(kNT), kSmemBytes, st, a, T);
  return hipGetLastError();
}

constexpr int kRowSpan = kNW * kSpan;  // positions per chunk index across the workgroup

// Chunks per lane for a row of `width` positions: 1, 2, 4, ..., 32.
int chunk_class(int width) {
  int ch = 1;
  while (ch < 32 && width > kRowSpan * ch) ch *= 2;
  return ch;
}

hipError_t launch_class(int ch, const RowArgs& a, int r0, int r1, bool big, hipStream_t st) {
  switch (ch) {
    case 1: return launch_rows<1>(a, r0, r1, big, st);
    case 2: return launch_rows<2>(a, r0, r1, big, st);
    case 4: return launch_rows<4>(a, r0, r1, big, st);
    case 8: return launch_rows<8>(a, r0, r1, big, st);
    case 16: return launch_rows<16>(a, r0, r1, big, st);
    default: return launch_rows<32>(a, r0, r1, big, st);
  }
}

hipError_t retry_class(int ch, const RowArgs& a, int T, hipStream_t st) {
  switch (ch) {
    case 1: return launch_retry<1>(a, T, st);
    case 2: return launch_retry<2>(a, T, st);
    case 4: return launch_retry<4>(a, T, st);
    case 8: return launch_retry<8>(a, T, st);
    case 16: return launch_retry<16>(a, T, st);
    default: return launch_retry<32>(a, T, st);
  }
}

}  // namespace

int topk_select_max_width() { return kRowSpan * 32; }

// Dense rows of a single sequence have known widths (t + 1 tokens, t / B + 1
// blocks), so their rows are split by width class and each class runs with the
// fewest registers that hold it, which lets more rows share a CU.
hipError_t launch_topk_select(const float* vals, const int32_t* cand, int64_t ld, int T,
                              const int32_t* cu, int nseq, int width, int block_size, int topk,
                              int force_own, int32_t* out_idx, float* out_val, hipStream_t st) {
  const RowArgs a{0, vals, cand, ld, cu, nseq, block_size, topk, force_own, out_idx, out_val};
  const bool big = topk > kCap;
  const int top = chunk_class(width);
  hipError_t e = hipSuccess;
  if (!cand && !cu) {
    int r0 = 0;
    for (int ch = 1; ch <= top && r0 < T && e == hipSuccess; ch *= 2) {
      const int64_t rows_fit = (int64_t)kRowSpan * ch * block_size;  // rows with width <= span
      const int r1 = ch == top || rows_fit >= T ? T : (int)rows_fit;
      if (r1 > r0) e = launch_class(ch, a, r0, r1, big, st);
      r0 = r1;
    }
  } else {
    e = launch_class(top, a, 0, T, big, st);
  }
  if (e != hipSuccess || big) return e;
  return retry_class(top, a, T, st);
}

}  // namespace sa
