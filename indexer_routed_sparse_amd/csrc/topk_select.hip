// Exact deterministic top-k of score rows, one workgroup per row (512 threads for rows
// up to 16K positions, 1024 for wider ones).
//
// Order (per "Add trainable QSA sparse attention with a TileLang backend", section
// "Describe the solution you'd like": a lexicographic (score, id) key): higher score
// first, then smaller index. Candidates sit in ascending index order, so "smaller
// index" is "earlier position" and ties at the k-th score are resolved by a
// position-ordered prefix count.
//
// The row is read from HBM once into registers: wave w owns the contiguous span
// [w*seg, (w+1)*seg) of the row (seg a multiple of 256), one float4 per lane per
// 256-position chunk. The selection then never touches HBM again, and since every
// sweep over the row costs vector instructions for all of it, the row is swept only
// twice:
//
//   1. pivot: one wave bisects the order key over a sample of 512 evenly spaced
//      positions for a value that about k plus three standard deviations of the
//      sample rank keys reach. The sample is loaded ahead of the row, so for dense
//      rows the bisection runs while the row is still arriving. A pivot that keeps
//      fewer than k keys or more than the candidate buffer holds is searched again
//      with another margin; correctness never depends on it, since both bounds are
//      checked exactly.
//   2. count the keys >= pivot per wave (one compare and a ballot popcount per
//      value), then compact them, in position order, into an LDS buffer.
//   3. exact radix select over the candidates, which thread t holds in registers as
//      the contiguous slots [t*R, t*R + R) (R = candidates per thread, rounded up to
//      even): 10-bit digits of the key offset within the exact candidate range; as
//      soon as the bin holding the k-th key is taken whole or has at most 64 members
//      (one wave ranks those directly), the threshold is known.
//   4. rank by a block-wide prefix count over the slots and write each selected id
//      at its rank.
//
// Rows whose pivot fails three times are marked and redone by a second, persistent
// launch that runs the same radix select over every key held in registers; a single
// launch of that kind serves all rows whose candidate buffer cannot hold topk. With
// force_own_block the query's own block (the last column) is taken out of the
// competition and written after the others, which is where ascending order puts it.
#include <type_traits>

#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kSpan = 4 * kWave;         // positions per wave chunk
constexpr int kCapSmall = 4096;          // candidate buffer entries, rows up to 16K wide
constexpr int kCapLarge = 5120;          // candidate buffer entries, wider rows
constexpr int kDigit = 10;               // radix digit bits
constexpr int kBins = 1 << kDigit;
constexpr int kSmall = 64;               // bins this small are ranked by one wave
constexpr int kSample = 512;             // pivot sample entries (the first 512 threads)
constexpr int kRetryGrid = 512;          // workgroups of the persistent retry launch
constexpr int32_t kRetry = INT32_MIN;    // out_idx[t, 0] of a row left to the retry launch
static_assert(kBins <= kCapSmall, "second histogram fits the value array");

// LDS of one row of NT threads (37 KB with 4096 candidate entries, so four rows
// share a CU; 45 KB with 5120). The value array also holds the pivot sample (before
// compaction) and the second histogram (once the candidates sit in registers).
template <int CAP, int NT>
struct Smem {
  static constexpr int kNT = NT;                          // threads per row
  static constexpr int kNW = NT / kWave;                  // waves per row
  static constexpr int kCap = CAP;
  static constexpr int kPer = (CAP + 2 * NT - 1) / (2 * NT) * 2;  // most slots per thread
  static constexpr int kPT = kBins / NT;                  // bins per thread in the scan
  static_assert(kPT >= 1 && kBins % NT == 0, "scan covers the bins");
  uint32_t cval[CAP];    // candidate value bits, position order
  uint32_t cpos[CAP];    // candidate positions
  uint32_t hist[kBins];  // first histogram, zero on entry to a select
  uint32_t red[8][kNW];  // per-wave partials
  uint32_t bc[8];        // broadcast slots; bc[4] is the gather counter, zero on entry
  uint32_t gath[kSmall]; // members of a small bin
};

SA_DEVICE float qnan() { return __uint_as_float(0x7FC00000u); }

// Order key of a non-NaN value; NaN marks an excluded slot and maps to 0.
SA_DEVICE uint32_t key_or_zero(float f) { return f == f ? order_key(f) : 0u; }

SA_DEVICE int bit_width(uint32_t x) { return x ? 32 - __builtin_clz(x) : 0; }

SA_DEVICE uint32_t mbcnt_add(uint64_t mask, uint32_t acc) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, acc));
}

SA_DEVICE uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

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

// Inclusive prefix of op over lanes 0..15 of each row of 16 lanes (DPP row shifts).
template <class Op>
SA_DEVICE uint32_t row_scan16(uint32_t x, uint32_t id, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  return x;
}

// Sum of the per-wave partials red[0..w) (exclusive) and of all NW of them: lane i
// reads red[i], a 16-lane prefix sum follows, and two lanes are read back.
template <int NW>
SA_DEVICE uint32_t wave_offset(const uint32_t* red, int w, uint32_t* total) {
  static_assert(NW <= 16, "one DPP row holds the partials");
  const int l = lane_id();
  const uint32_t inc = row_scan16(l < NW ? red[l] : 0u, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  *total = (uint32_t)__builtin_amdgcn_readlane((int)inc, NW - 1);
  return w > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)inc, w - 1) : 0u;
}

// Result of a select. mode 0: every valid key is taken. mode 1: every key >= thr is
// taken (exactly k of them). mode 2: keys > thr are taken plus the first `need` keys
// equal to thr in position order.
struct Cut {
  uint32_t thr, need;
  int mode;
};

SA_DEVICE bool take_gt(uint32_t k, const Cut& c) {
  return c.mode == 0 ? k != 0u : c.mode == 1 ? k >= c.thr : k > c.thr;
}

SA_DEVICE bool take_eq(uint32_t k, const Cut& c) { return c.mode == 2 && k == c.thr; }

// Exact radix select of the k-th largest among the nonzero order keys x[0..R) of
// every thread (R uniform). The caller guarantees that at least k keys are nonzero,
// that sm.hist and bc[4] are zero on entry and that sm.cval is no longer read by any
// thread once every thread has entered. Digits are taken over the exact key range
// of the nonzero keys.
template <int N, class S>
SA_DEVICE Cut radix_select_in(const uint32_t (&x)[N], int R, uint32_t k, S& sm, uint32_t lo, uint32_t hi);

template <int N, class S>
SA_DEVICE Cut radix_select(const uint32_t (&x)[N], int R, uint32_t k, S& sm) {
  constexpr int kNW = S::kNW;
  const int tid = threadIdx.x, w = (int)uniform((uint32_t)tid / kWave), l = lane_id();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    if (r < R) {
      const uint32_t kk = x[r];
      kmin = kk != 0u ? min(kmin, kk) : kmin;
      kmax = max(kmax, kk);
    }
  }
  kmin = dpp_min_to_last(kmin);
  kmax = dpp_max_to_last(kmax);
  if (l == kWave - 1) { sm.red[6][w] = kmin; sm.red[7][w] = kmax; }
  __syncthreads();
  uint32_t lo, hi;
  {
    const uint32_t rl = row_scan16(l < kNW ? sm.red[6][l] : 0xFFFFFFFFu, 0xFFFFFFFFu,
                                   [](uint32_t a, uint32_t b) { return min(a, b); });
    const uint32_t rh = row_scan16(l < kNW ? sm.red[7][l] : 0u, 0u,
                                   [](uint32_t a, uint32_t b) { return max(a, b); });
    lo = (uint32_t)__builtin_amdgcn_readlane((int)rl, kNW - 1);
    hi = (uint32_t)__builtin_amdgcn_readlane((int)rh, kNW - 1);
  }
  return radix_select_in<N>(x, R, k, sm, lo, hi);
}

// The select proper, given bounds: every nonzero key in use lies in [lo, hi] (lo > 0;
// invalid slots hold 0 < lo). The bounds may be loose: they only set the digit width.
template <int N, class S>
SA_DEVICE Cut radix_select_in(const uint32_t (&x)[N], int R, uint32_t k, S& sm, uint32_t lo, uint32_t hi) {
  constexpr int kNT = S::kNT, kNW = S::kNW, kPT = S::kPT;
  const int tid = threadIdx.x, w = (int)uniform((uint32_t)tid / kWave), l = lane_id();
  int s = bit_width(hi - lo) - kDigit;
  s = s > 0 ? s : 0;
  uint32_t need = k;
  int buf = 0;
#pragma unroll 1
  for (;;) {
    uint32_t* H = buf ? sm.cval : sm.hist;
    uint32_t* Hn = buf ? sm.hist : sm.cval;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      if (r < R) {
        const uint32_t kk = x[r];
        if (kk >= lo && kk <= hi) atomicAdd(&H[(kk - lo) >> s], 1u);
      }
    }
    __syncthreads();
    for (int b = tid; b < kBins; b += kNT) Hn[b] = 0u;  // next pass's buffer
    // suffix counts from the top bin: thread i owns bins nb-1-4i .. nb-4-4i
    uint32_t loc[kPT], tsum = 0;
#pragma unroll
    for (int r = 0; r < kPT; ++r) {
      loc[r] = H[kBins - 1 - kPT * tid - r];
      tsum += loc[r];
    }
    const uint32_t inc = dpp_incl_scan(tsum);
    if (l == kWave - 1) sm.red[4][w] = inc;
    __syncthreads();
    uint32_t tot;
    uint32_t run = inc - tsum + wave_offset<kNW>(sm.red[4], w, &tot);
#pragma unroll
    for (int r = 0; r < kPT; ++r) {
      const uint32_t above = run;
      run += loc[r];
      if (above < need && run >= need) {
        sm.bc[1] = (uint32_t)(kBins - 1 - kPT * tid - r);
        sm.bc[2] = above;
        sm.bc[3] = loc[r];
      }
    }
    __syncthreads();
    const uint32_t bs = sm.bc[1], above = sm.bc[2], cnt = sm.bc[3];
    need -= above;
    const uint32_t blo = lo + (bs << s);
    const uint32_t bhi = min(hi, blo + ((1u << s) - 1u));
    if (cnt == need) return Cut{blo, 0u, 1};  // the whole bin is taken
    if (blo == bhi) return Cut{blo, need, 2};  // one key value: ties by position
    if (cnt <= (uint32_t)kSmall) {
      // gather the bin's members; one wave finds the need-th largest among them
#pragma unroll
      for (int r = 0; r < N; ++r) {
        if (r < R) {
          const uint32_t kk = x[r];
          if (kk >= blo && kk <= bhi) sm.gath[atomicAdd(&sm.bc[4], 1u)] = kk;
        }
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
        if (mine && gt < need && need <= gt + eq) {
          sm.bc[5] = me;
          sm.bc[6] = need - gt;
          sm.bc[7] = eq;
        }
      }
      __syncthreads();
      const uint32_t thr = sm.bc[5], ne = sm.bc[6], eq = sm.bc[7];
      return ne == eq ? Cut{thr, 0u, 1} : Cut{thr, ne, 2};
    }
    lo = blo;
    hi = bhi;
    s = bit_width(hi - lo) - kDigit;
    s = s > 0 ? s : 0;
    buf ^= 1;
  }
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
  const int32_t* cnt;  // candidate rows only: valid entries per row (< 0: skip the row)
};

// KIND 0: pivot + candidate buffer (topk <= its capacity). Rows whose pivot fails get
//         kRetry in their first output slot and nothing else.
// KIND 1: radix select over the keys held in registers (any topk).
// CAND: rows come with explicit candidate ids (a.cand), -1 marking a hole.
template <int CH, int KIND, bool CAND, class S>
SA_DEVICE void select_row(int t, const RowArgs& a, S& sm) {
  constexpr int kCap = S::kCap, kPer = S::kPer, kNT = S::kNT, kNW = S::kNW;
  const int tid = threadIdx.x;
  const int w = (int)uniform((uint32_t)tid / kWave);  // wave-uniform, so spans live in SGPRs
  const int l = lane_id();
  const int topk = a.topk;

  int start = 0, n;
  if (CAND) {
    n = a.cnt ? (int)uniform((uint32_t)__ldg(a.cnt + t)) : (int)a.ld;
    if (n < 0) return;                     // uniform: the row is left to its owner
  } else {
    if (a.cu) start = seq_start_of(a.cu, a.nseq, t);
    const int off = t - start;
    n = (a.block_size == 1)   ? off + 1
        : a.force_own == 2    ? (off + 1) / a.block_size     // complete blocks only
                              : off / a.block_size + 1;
  }
  const bool own = !CAND && a.block_size > 1 && a.force_own == 1;
  const int n1 = own ? n - 1 : n;          // competing positions
  const int k1 = own ? topk - 1 : topk;    // slots they compete for
  const float* __restrict__ row = a.vals + (int64_t)t * a.ld;
  const int32_t* __restrict__ crow = CAND ? a.cand + (int64_t)t * a.ld : nullptr;
  int32_t* __restrict__ orow = a.out_idx + (int64_t)t * topk;
  float* __restrict__ vrow = a.out_val ? a.out_val + (int64_t)t * topk : nullptr;
  const int32_t idbase = a.block_size == 1 ? start : 0;

  const int seg = (n1 + kNW * kSpan - 1) / (kNW * kSpan) * kSpan;
  const int ws = w * seg;
  const int we = min(ws + seg, n1);
  const int m = we > ws ? (we - ws + kSpan - 1) / kSpan : 0;  // chunks of this wave
  const int mfull = we > ws ? (we - ws) / kSpan : 0;         // chunks without a tail

  for (int b = tid; b < kBins; b += kNT) sm.hist[b] = 0u;
  if (tid == 0) sm.bc[4] = 0u;

  // Pivot search (wave 0) over the sample keys in sm.cval[0..kSample): the largest key P,
  // in key bits from high to low, that at least `target` sample keys reach, where
  // target sits z sample standard deviations above the expected sample rank of the
  // k-th key; refining stops once the sample count at P is within 12.5% of target.
  // Ends with a barrier; returns the pivot value (-inf: every key is a candidate).
  // Searches made while the row sits in registers re-read the sample from LDS at
  // every step instead of holding it.
  auto pivot_search = [&](auto hold, float z, int nv) __attribute__((always_inline)) -> float {
    if (w == 0) {
      uint32_t xs[kSample / kWave];
      uint32_t sv = 0;
#pragma unroll
      for (int i = 0; i < kSample / kWave; ++i) {
        if constexpr (!decltype(hold)::value) asm volatile("" ::: "memory");
        xs[i] = sm.cval[l + kWave * i];
        sv += __popcll(ballot(xs[i] != 0u));
      }
      const float r0 = (float)sv * (float)k1 / (float)nv;
      const float aim = r0 + z * __builtin_sqrtf(r0);
      const uint32_t target = (uint32_t)(aim > 0.0f ? aim : 0.0f) + 4u;
      const uint32_t enough = target + target / 8u;
      uint32_t Pw = 0, at_p = sv;
      if (target <= sv) {
#pragma unroll 1
        for (int b = 31; b >= 0 && at_p > enough; --b) {
          const uint32_t cnd = Pw | (1u << b);
          uint32_t cnt = 0;
#pragma unroll
          for (int i = 0; i < kSample / kWave; ++i) {
            if constexpr (!decltype(hold)::value) asm volatile("" ::: "memory");
            const uint32_t x = decltype(hold)::value ? xs[i] : sm.cval[l + kWave * i];
            cnt += __popcll(ballot(x >= cnd));
          }
          if (cnt >= target) { Pw = cnd; at_p = cnt; }
        }
      }
      if (l == 0) sm.bc[0] = Pw;
    }
    __syncthreads();
    const uint32_t P = uniform(sm.bc[0]);
    return P > 0x007FFFFFu ? key_value(P) : -__builtin_huge_valf();
  };

  // Rows that may need a select fetch the pivot sample (512 evenly spaced positions)
  // before the row, so that it arrives first (loads complete in order) and, for dense
  // rows, the search runs while the row is still arriving.
  const bool early = KIND == 0 && !CAND && k1 < n1;
  float smp = qnan();
  int32_t scand = 0;
  if (KIND == 0 && k1 < n1 && tid < kSample) {
    const int ps = (int)(((uint32_t)tid * (uint32_t)n1) / kSample);
    smp = row[ps];
    if (CAND) scand = crow[ps];
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- load the wave's span; excluded slots become NaN. Dense rows issue all CH
  // float4 loads unconditionally (lanes past the span end read the last aligned float4
  // inside it, or the row's first one), so every load is in flight at once and the
  // wait for the sample, loaded first, counts exactly CH later loads.
  float v[4 * CH];
  const uint32_t lane4 = 4u * (uint32_t)l;
  const uint32_t lastp = we > ws ? (uint32_t)(we - 1) & ~3u : 0u;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float4 x = make_float4(qnan(), qnan(), qnan(), qnan());
    const uint32_t p = min(uniform((uint32_t)(ws + c * kSpan)) + lane4, lastp);
    if constexpr (CAND) {
      if (c < m) {
        x = *reinterpret_cast<const float4*>(row + p);
        const int4 ci = *reinterpret_cast<const int4*>(crow + p);
        if (ci.x < 0) x.x = qnan();
        if (ci.y < 0) x.y = qnan();
        if (ci.z < 0) x.z = qnan();
        if (ci.w < 0) x.w = qnan();
      }
    } else {
      x = *reinterpret_cast<const float4*>(row + p);
    }
    v[4 * c + 0] = x.x;
    v[4 * c + 1] = x.y;
    v[4 * c + 2] = x.z;
    v[4 * c + 3] = x.w;
  }
  float pf = -__builtin_huge_valf();
  if (early) {
    if (tid < kSample) sm.cval[tid] = key_or_zero(smp);
    __syncthreads();
    pf = pivot_search(std::true_type{}, 3.0f, n1);
  }

  // mask the positions past the span end (after the pivot search, so that the
  // sample is stored without waiting for the row)
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c >= mfull) {  // a tail chunk or one past the span
      const int pos = ws + c * kSpan + 4 * l;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (pos + j >= we) v[4 * c + j] = qnan();
    }
  }

  int nvalid = n1;
  if (crow) {
    uint32_t cv = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < m)
#pragma unroll
        for (int j = 0; j < 4; ++j) cv += __popcll(ballot(v[4 * c + j] == v[4 * c + j]));
    if (l == 0) sm.red[0][w] = cv;
    __syncthreads();
    uint32_t tot;
    wave_offset<kNW>(sm.red[0], w, &tot);
    nvalid = (int)tot;
  }
  const int nsel = k1 < nvalid ? k1 : nvalid;

  if (nsel > 0) {
    if constexpr (KIND == 0) {
      if (nvalid <= k1) {
        // every valid key is taken: rank = valid keys before it in position order
        uint32_t cg = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (c < m)
#pragma unroll
            for (int j = 0; j < 4; ++j) cg += __popcll(ballot(v[4 * c + j] == v[4 * c + j]));
        if (l == 0) sm.red[2][w] = cg;
        __syncthreads();
        uint32_t tot;
        uint32_t og = uniform(wave_offset<kNW>(sm.red[2], w, &tot));
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if (c < m) {
            bool g[4];
            uint64_t bg[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) { g[j] = v[4 * c + j] == v[4 * c + j]; bg[j] = ballot(g[j]); }
            uint32_t lg = mbcnt_add(bg[3], mbcnt_add(bg[2], mbcnt_add(bg[1], mbcnt_add(bg[0], og))));
            const int32_t pos = ws + c * kSpan + 4 * l;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (g[j]) {
                orow[lg] = crow ? crow[pos + j] : idbase + pos + j;
                if (vrow) vrow[lg] = v[4 * c + j] + 0.0f;
              }
              lg += g[j] ? 1u : 0u;
            }
            og += __popcll(bg[0]) + __popcll(bg[1]) + __popcll(bg[2]) + __popcll(bg[3]);
          }
        }
      } else {
        uint32_t C = 0, run = 0;
        float z = 3.0f;
        if constexpr (CAND) {  // (dense rows found their pivot before loading)
          if (tid < kSample) sm.cval[tid] = scand < 0 ? 0u : key_or_zero(smp);
          __syncthreads();
          pf = pivot_search(std::false_type{}, z, nvalid);
        }
        // The row's largest key bounds the candidates for the radix select from above
        // (the pivot bounds them from below), so the select needs no range pass: each
        // wave's maximum (a DPP reduction) rides the count's barrier. fmaxf skips the NaNs
        // of excluded slots; +1 covers a -0.0 maximum beside a +0.0 key.
        {
          float vmax = -__builtin_huge_valf();
#pragma unroll
          for (int c = 0; c < CH; ++c)
            if (c < m)
#pragma unroll
              for (int j = 0; j < 4; ++j) vmax = fmaxf(vmax, v[4 * c + j]);
          const uint32_t kx = dpp_max_to_last(key_or_zero(vmax));
          if (l == kWave - 1) sm.red[7][w] = kx == 0xFFFFFFFFu ? kx : kx + 1u;
        }
        // A pivot that keeps fewer than k keys or more than the buffer holds is searched again
        // with a wider or narrower margin.
#pragma unroll 1
        for (int attempt = 0;; ++attempt) {
          uint32_t cc = 0;
#pragma unroll
          for (int c = 0; c < CH; ++c)
            if (c < m)
#pragma unroll
              for (int j = 0; j < 4; ++j) cc += __popcll(ballot(v[4 * c + j] >= pf));
          if (l == 0) sm.red[1][w] = cc;
          __syncthreads();
          run = uniform(wave_offset<kNW>(sm.red[1], w, &C));
          C = uniform(C);
          if (C >= (uint32_t)k1 && C <= (uint32_t)kCap) break;  // uniform
          if (attempt == 2) {
            if (tid == 0) orow[0] = kRetry;
            return;  // uniform
          }
          z = C < (uint32_t)k1 ? z + 4.0f : z - 3.0f;
          pf = pivot_search(std::false_type{}, z, nvalid);
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
            const uint32_t pos = uniform((uint32_t)(ws + c * kSpan)) + lane4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (p[j]) {
                sm.cval[o] = __float_as_uint(v[4 * c + j]);
                sm.cpos[o] = pos + j;
              }
              o += p[j] ? 1u : 0u;
            }
            run += __popcll(b[0]) + __popcll(b[1]) + __popcll(b[2]) + __popcll(b[3]);
          }
          __builtin_amdgcn_sched_barrier(0);  // one chunk at a time bounds the live masks
        }
        __syncthreads();
        // thread t holds candidates [t*R, t*R + R), in position order
        const int R = (int)((C + 2 * kNT - 1) / (2 * kNT)) * 2;
        uint32_t ck[kPer], cp[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          ck[r] = 0u;
          cp[r] = 0u;
          if (r < R) {
            const uint32_t i = (uint32_t)(tid * R + r);
            if (i < C) {
              ck[r] = order_key(__uint_as_float(sm.cval[i]));
              cp[r] = sm.cpos[i];
            }
          }
        }
        uint32_t rlo, rhi;
        {
          const uint32_t kp = order_key(pf);   // every candidate is >= pf
          rlo = kp > 0u ? kp : 1u;
          const uint32_t rh = row_scan16(l < kNW ? sm.red[7][l] : 0u, 0u,
                                         [](uint32_t a, uint32_t b) { return max(a, b); });
          rhi = (uint32_t)__builtin_amdgcn_readlane((int)rh, kNW - 1);
          rhi = rhi > rlo ? rhi : rlo;
        }
        const Cut c2 = radix_select_in<kPer>(ck, R, (uint32_t)k1, sm, rlo, rhi);
        // ranks: block-wide exclusive count of (greater, equal) in position order
        uint32_t ng = 0, ne = 0;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          if (r < R) {
            ng += take_gt(ck[r], c2) ? 1u : 0u;
            ne += take_eq(ck[r], c2) ? 1u : 0u;
          }
        }
        const uint32_t pk = ng | (ne << 16);  // both <= kCap < 2^16
        const uint32_t inc = dpp_incl_scan(pk);
        if (l == kWave - 1) sm.red[2][w] = inc;
        __syncthreads();
        uint32_t tot;
        const uint32_t base = inc - pk + wave_offset<kNW>(sm.red[2], w, &tot);
        uint32_t gb = base & 0xFFFFu, eb = base >> 16;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          if (r < R) {
            const bool g = take_gt(ck[r], c2), e = take_eq(ck[r], c2);
            if (g || (e && eb < c2.need)) {
              const uint32_t rank = gb + (eb < c2.need ? eb : c2.need);
              orow[rank] = crow ? crow[cp[r]] : idbase + (int32_t)cp[r];
              if (vrow) vrow[rank] = key_value(ck[r]);
            }
            gb += g ? 1u : 0u;
            eb += e ? 1u : 0u;
          }
        }
      }
    } else {
      uint32_t key[4 * CH];
#pragma unroll
      for (int e = 0; e < 4 * CH; ++e) key[e] = key_or_zero(v[e]);
      Cut cut{0u, 0u, 0};  // mode 0: every valid key
      if (nvalid > k1) cut = radix_select<4 * CH>(key, 4 * CH, (uint32_t)k1, sm);
      // position-ordered ranks straight from the registers
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c < m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t kk = key[4 * c + j];
            cg += __popcll(ballot(take_gt(kk, cut)));
            ce += __popcll(ballot(take_eq(kk, cut)));
          }
      if (l == 0) { sm.red[2][w] = cg; sm.red[3][w] = ce; }
      __syncthreads();
      uint32_t tot;
      uint32_t og = wave_offset<kNW>(sm.red[2], w, &tot);
      uint32_t oe = wave_offset<kNW>(sm.red[3], w, &tot);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < m) {
          bool g[4], e[4];
          uint64_t bg[4], be[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t kk = key[4 * c + j];
            g[j] = take_gt(kk, cut);
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
              orow[rank] = crow ? crow[pos + j] : idbase + (int32_t)(pos + j);
              if (vrow) vrow[rank] = key_value(key[4 * c + j]);
            }
            lg += g[j] ? 1u : 0u;
            le += e[j] ? 1u : 0u;
          }
          og += __popcll(bg[0]) + __popcll(bg[1]) + __popcll(bg[2]) + __popcll(bg[3]);
          oe += __popcll(be[0]) + __popcll(be[1]) + __popcll(be[2]) + __popcll(be[3]);
        }
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

// Candidate buffer of a width class: rows up to 16K take 4096 entries, wider rows 5120.
constexpr int cap_of(int nt, int ch) { return nt * ch <= 512 * 8 ? kCapSmall : kCapLarge; }

// Width classes (threads per row, chunks per lane): rows up to 16K run 512 threads
// with up to 32 values per lane in at most 64 registers (four rows per CU); rows up
// to 32K run 1024 threads with 32 values per lane (two rows per CU); rows up to 64K
// run 1024 threads with 64 values per lane.
template <int CH, int NT, bool CAND>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(CH <= 8 ? 8 : 4)))
void topk_pivot_kernel(RowArgs a) {
  __shared__ Smem<cap_of(NT, CH), NT> sm;
  select_row<CH, 0, CAND>(a.row0 + (int)blockIdx.x, a, sm);
}

template <int CH, int NT, bool CAND>
__global__ __launch_bounds__(NT) void topk_full_kernel(RowArgs a) {
  __shared__ Smem<kCapSmall, NT> sm;
  select_row<CH, 1, CAND>(a.row0 + (int)blockIdx.x, a, sm);
}

// Persistent redo of the rows the pivot pass marked: workgroup b owns rows
// b, b + grid, ...; it lists its marked rows, then selects them one by one.
template <int CH, int NT, bool CAND>
__global__ __launch_bounds__(NT) void topk_retry_kernel(RowArgs a, int T) {
  __shared__ Smem<kCapSmall, NT> sm;
  __shared__ uint32_t s_count;
  __shared__ int32_t s_rows[NT];
  const int tid = threadIdx.x;
  const int stride = (int)gridDim.x;
  for (int base = blockIdx.x; base < T; base += stride * NT) {
    if (tid == 0) s_count = 0u;
    __syncthreads();
    const int t = base + tid * stride;
    if (t < T && a.out_idx[(int64_t)t * a.topk] == kRetry) s_rows[atomicAdd(&s_count, 1u)] = t;
    __syncthreads();
    const uint32_t cnt = s_count;
    for (uint32_t i = 0; i < cnt; ++i) {
      select_row<CH, 1, CAND>(s_rows[i], a, sm);
      __syncthreads();
    }
    __syncthreads();  // every thread has read s_count before it is reset
  }
}

template <int CH, int NT, bool CAND>
hipError_t launch_rows_as(const RowArgs& a, int r0, int r1, hipStream_t st) {
  RowArgs b = a;
  b.row0 = r0;
  // Rows wider than k but at most 2k wide keep most of their keys as candidates: a radix
  // select over the registers-held row costs less than sampling, pivoting and compacting
  // them (rows up to k wide take every key, which the pivot kernel does without a select).
  constexpr int64_t kSpanRow = (int64_t)(NT / kWave) * kSpan * CH;
  if (a.topk > cap_of(NT, CH) || (kSpanRow > (int64_t)a.topk && kSpanRow <= 2 * (int64_t)a.topk))
    hipLaunchKernelGGL((topk_full_kernel<CH, NT, CAND>), dim3(r1 - r0), dim3(NT), 0, st, b);
  else
    hipLaunchKernelGGL((topk_pivot_kernel<CH, NT, CAND>), dim3(r1 - r0), dim3(NT), 0, st, b);
  return hipGetLastError();
}

template <int CH, int NT>
hipError_t launch_rows(const RowArgs& a, int r0, int r1, hipStream_t st) {
  return a.cand ? launch_rows_as<CH, NT, true>(a, r0, r1, st)
                : launch_rows_as<CH, NT, false>(a, r0, r1, st);
}

template <int CH, int NT>
hipError_t launch_retry(const RowArgs& a, int T, hipStream_t st) {
  const int grid = T < kRetryGrid ? T : kRetryGrid;
  if (a.cand)
    hipLaunchKernelGGL((topk_retry_kernel<CH, NT, true>), dim3(grid), dim3(NT), 0, st, a, T);
  else
    hipLaunchKernelGGL((topk_retry_kernel<CH, NT, false>), dim3(grid), dim3(NT), 0, st, a, T);
  return hipGetLastError();
}

struct WidthClass {
  int nt, ch;
  int64_t span() const { return (int64_t)(nt / kWave) * kSpan * ch; }  // widest row
};
constexpr WidthClass kClasses[] = {{512, 1}, {512, 2}, {512, 4}, {512, 8}, {1024, 8}, {1024, 16}};
constexpr int kNumClasses = sizeof(kClasses) / sizeof(kClasses[0]);

// Narrowest class that holds rows of `width` positions.
int class_of(int width) {
  int c = 0;
  while (c + 1 < kNumClasses && width > kClasses[c].span()) ++c;
  return c;
}

hipError_t launch_class(int c, const RowArgs& a, int r0, int r1, hipStream_t st) {
  switch (c) {
    case 0: return launch_rows<1, 512>(a, r0, r1, st);
    case 1: return launch_rows<2, 512>(a, r0, r1, st);
    case 2: return launch_rows<4, 512>(a, r0, r1, st);
    case 3: return launch_rows<8, 512>(a, r0, r1, st);
    case 4: return launch_rows<8, 1024>(a, r0, r1, st);
    default: return launch_rows<16, 1024>(a, r0, r1, st);
  }
}

hipError_t retry_class(int c, const RowArgs& a, int T, hipStream_t st) {
  switch (c) {
    case 0: return launch_retry<1, 512>(a, T, st);
    case 1: return launch_retry<2, 512>(a, T, st);
    case 2: return launch_retry<4, 512>(a, T, st);
    case 3: return launch_retry<8, 512>(a, T, st);
    case 4: return launch_retry<8, 1024>(a, T, st);
    default: return launch_retry<16, 1024>(a, T, st);
  }
}

}  // namespace

int topk_select_max_width() { return (int)kClasses[kNumClasses - 1].span(); }

// Dense rows of a single sequence have known widths (t + 1 tokens, t / B + 1
// blocks), so their rows are split by width class and each class runs with the
// fewest registers that hold it, which lets more rows share a CU.
hipError_t launch_topk_select(const float* vals, const int32_t* cand, int64_t ld, int T,
                              const int32_t* cu, int nseq, int width, int block_size, int topk,
                              int force_own, int32_t* out_idx, float* out_val, hipStream_t st) {
  const RowArgs a{0, vals, cand, ld, cu, nseq, block_size, topk, force_own, out_idx, out_val, nullptr};
  const int top = class_of(width);
  hipError_t e = hipSuccess;
  bool pivoted = false;  // some class ran the pivot kernel, so rows may await the retry
  if (!cand && !cu) {
    int r0 = 0;
    for (int c = 0; c <= top && r0 < T && e == hipSuccess; ++c) {
      const int64_t rows_fit = kClasses[c].span() * block_size;  // rows with width <= span
      const int r1 = c == top || rows_fit >= T ? T : (int)rows_fit;
      if (r1 > r0) {
        e = launch_class(c, a, r0, r1, st);
        pivoted |= topk <= cap_of(kClasses[c].nt, kClasses[c].ch);
      }
      r0 = r1;
    }
  } else {
    e = launch_class(top, a, 0, T, st);
    pivoted = topk <= cap_of(kClasses[top].nt, kClasses[top].ch);
  }
  if (e != hipSuccess || !pivoted) return e;
  return retry_class(top, a, T, st);
}

// Candidate rows counted by a first pass hold only the keys at or above a sampled pivot,
// a few standard deviations more than topk, so every row takes the register radix
// select over all of its candidates: a second sample, pivot and compaction would cost
// more than they remove.
hipError_t launch_topk_select_counted(const float* vals, const int32_t* cand, const int32_t* cnt,
                                      int64_t ld, int T, int topk, int32_t* out_idx,
                                      float* out_val, hipStream_t st) {
  const RowArgs a{0, vals, cand, ld, nullptr, 1, 1, topk, 0, out_idx, out_val, cnt};
  switch (class_of((int)ld)) {
    case 0: hipLaunchKernelGGL((topk_full_kernel<1, 512, true>), dim3(T), dim3(512), 0, st, a); break;
    case 1: hipLaunchKernelGGL((topk_full_kernel<2, 512, true>), dim3(T), dim3(512), 0, st, a); break;
    case 2: hipLaunchKernelGGL((topk_full_kernel<4, 512, true>), dim3(T), dim3(512), 0, st, a); break;
    case 3: hipLaunchKernelGGL((topk_full_kernel<8, 512, true>), dim3(T), dim3(512), 0, st, a); break;
    case 4: hipLaunchKernelGGL((topk_full_kernel<8, 1024, true>), dim3(T), dim3(1024), 0, st, a); break;
    default: hipLaunchKernelGGL((topk_full_kernel<16, 1024, true>), dim3(T), dim3(1024), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace sa
