// Exact deterministic top-k of score rows: one workgroup per row, the row held in
// registers, an LDS radix select on order-preserving keys, and a ballot/mbcnt
// compaction that writes the chosen indices in ascending order.
//
// Order (per "Add trainable QSA sparse attention with a TileLang backend", section
// "Describe the solution you'd like": a lexicographic (score, id) key): higher score
// first, then smaller index. Because candidates are laid out by ascending index,
// "smaller index" is "earlier position", so ties at the k-th score are resolved by a
// position-ordered prefix count.
//
// Radix select: keys are 32-bit; three LDS histogram passes over digits of 11, 11
// and 10 bits find the k-th largest key tau and how many keys equal to tau are
// still needed. A pass stops early when the bin holding the k-th key is taken
// whole. Each thread holds CH float4 chunks; chunk c of thread i covers positions
// 4*(c*NT + i) .. +3, so a row of up to NT*4*CH candidates is read from HBM once.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kBins = 2048;

template <int NT>
SA_DEVICE uint32_t block_excl_scan(uint32_t v, uint32_t* sm_waves, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  uint32_t inc = wave_incl_scan(v);
  if (l == kWave - 1) sm_waves[w] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    uint32_t s = sm_waves[i];
    base += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

template <int NT, int CH>
__global__ __launch_bounds__(NT) void topk_select_kernel(
    const float* __restrict__ vals, const int32_t* __restrict__ cand, int64_t ld,
    const int32_t* __restrict__ cu, int nseq, int block_size, int topk, int force_own,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val) {
  constexpr int NW = NT / kWave;
  constexpr int E = 4 * CH;  // candidates per thread
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sm_waves[NW];
  __shared__ uint32_t sm_tab[2][CH * NW];
  __shared__ uint32_t sm_found[2];

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();

  int start = 0, n;
  if (cand) {
    n = (int)ld;
  } else {
    if (cu) start = seq_start_of(cu, nseq, t);
    const int off = t - start;
    n = (block_size == 1) ? off + 1 : off / block_size + 1;
  }
  const int own = (!cand && block_size > 1 && force_own) ? n - 1 : -1;
  const float* __restrict__ row = vals + (int64_t)t * ld;
  const int32_t* __restrict__ crow = cand ? cand + (int64_t)t * ld : nullptr;

  // ---- load: one HBM pass; invalid slots get key 0
  uint32_t key[E];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int pos = 4 * (c * NT + tid);
    if (pos < n) {
      const float4 v = *reinterpret_cast<const float4*>(row + pos);
      int4 ci = make_int4(0, 0, 0, 0);
      if (crow) ci = *reinterpret_cast<const int4*>(crow + pos);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      const int cc[4] = {ci.x, ci.y, ci.z, ci.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = (pos + j < n) && (cc[j] >= 0);
        uint32_t kk = ok ? order_key(vv[j]) : 0u;
        if (pos + j == own) kk = 0xFFFFFFFFu;  // forced: above every real key
        key[4 * c + j] = kk;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) key[4 * c + j] = 0u;
    }
  }

  // ---- radix select of the topk-th largest key
  // mode 0: take every valid key; 1: take keys >= thr; 2: keys > thr plus the first
  // `need` keys == thr in position order.
  int mode = 2;
  uint32_t prefix = 0, thr = 0;
  uint32_t need = (uint32_t)topk;
  uint32_t nvalid = 0;
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int sh = p == 0 ? 21 : (p == 1 ? 10 : 0);
    const int nbits = p == 2 ? 10 : 11;
    const int nb = 1 << nbits;
    for (int b = tid; b < kBins; b += NT) hist[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t kk = key[e];
      const bool in = (kk != 0u) && (p == 0 || (kk >> (sh + nbits)) == prefix);
      if (in) atomicAdd(&hist[(kk >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // suffix counts from the top bin down: thread i owns bins nb-1-(i*per .. i*per+per-1)
    constexpr int kMaxPer = kBins / NT;
    const int per = nb / NT > 0 ? nb / NT : 1;
    uint32_t loc[kMaxPer > 0 ? kMaxPer : 1];
    uint32_t tsum = 0;
#pragma unroll
    for (int r = 0; r < (kMaxPer > 0 ? kMaxPer : 1); ++r) {
      const int bi = tid * per + r;
      loc[r] = (r < per && bi < nb) ? hist[nb - 1 - bi] : 0u;
      tsum += loc[r];
    }
    uint32_t total;
    uint32_t running = block_excl_scan<NT>(tsum, sm_waves, &total);
    if (p == 0) {
      nvalid = total;
      if (total <= need) { mode = 0; break; }
    }
#pragma unroll
    for (int r = 0; r < (kMaxPer > 0 ? kMaxPer : 1); ++r) {
      const uint32_t above = running;
      running += loc[r];
      if (r < per && above < need && running >= need) {
        sm_found[0] = (uint32_t)(nb - 1 - (tid * per + r));
        sm_found[1] = above;
      }
    }
    __syncthreads();
    const uint32_t d = sm_found[0];
    const uint32_t above = sm_found[1];
    const uint32_t cnt = hist[d];
    __syncthreads();
    prefix = (prefix << nbits) | d;
    need -= above;
    if (cnt == need) { mode = 1; thr = prefix << sh; break; }
    if (p == 2) thr = prefix;
  }

  // ---- position-ordered ranks of the "greater" and "equal" flags
  auto flags = [&](uint32_t kk, bool& gt, bool& eq) {
    if (mode == 0) { gt = kk != 0u; eq = false; }
    else if (mode == 1) { gt = kk >= thr; eq = false; }
    else { gt = kk > thr; eq = kk == thr; }
  };
  uint32_t wgt[CH], weq[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    uint32_t sg = 0, se = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bool gt, eq;
      flags(key[4 * c + j], gt, eq);
      sg += __popcll(ballot(gt));
      se += __popcll(ballot(eq));
    }
    wgt[c] = sg;
    weq[c] = se;
  }
  if (l == 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) { sm_tab[0][c * NW + w] = wgt[c]; sm_tab[1][c * NW + w] = weq[c]; }
  }
  __syncthreads();
  if (w == 0) {
    // exclusive scan over the (chunk, wave) table in position order
    constexpr int M = CH * NW;
    constexpr int PL = (M + kWave - 1) / kWave;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      uint32_t v[PL];
      uint32_t s = 0;
#pragma unroll
      for (int r = 0; r < PL; ++r) { const int i = l * PL + r; v[r] = i < M ? sm_tab[a][i] : 0u; s += v[r]; }
      uint32_t ex = wave_incl_scan(s) - s;
#pragma unroll
      for (int r = 0; r < PL; ++r) { const int i = l * PL + r; if (i < M) sm_tab[a][i] = ex; ex += v[r]; }
    }
  }
  __syncthreads();

  const uint32_t nsel = nvalid < (uint32_t)topk ? nvalid : (uint32_t)topk;
  int32_t* __restrict__ orow = out_idx + (int64_t)t * topk;
  float* __restrict__ vrow = out_val ? out_val + (int64_t)t * topk : nullptr;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    uint32_t gb = sm_tab[0][c * NW + w];
    uint32_t eb = sm_tab[1][c * NW + w];
    bool gts[4], eqs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      flags(key[4 * c + j], gts[j], eqs[j]);
      gb += mbcnt(ballot(gts[j]));
      eb += mbcnt(ballot(eqs[j]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool gt = gts[j];
      const bool eq = eqs[j];
      const bool sel = gt || (eq && eb < need);
      const uint32_t rank = gb + (eb < need ? eb : need);
      if (sel && rank < (uint32_t)topk) {
        const int pos = 4 * (c * NT + tid) + j;
        const int32_t id = crow ? crow[pos] : (block_size == 1 ? start + pos : pos);
        orow[rank] = id;
        if (vrow) {
          float v = (pos == own) ? row[pos] : key_value(key[4 * c + j]);
          if (v == 0.0f) v = 0.0f;
          vrow[rank] = v;
        }
      }
      gb += gt ? 1u : 0u;
      eb += eq ? 1u : 0u;
    }
  }
  for (int i = (int)nsel + tid; i < topk; i += NT) {
    orow[i] = -1;
    if (vrow) vrow[i] = -__builtin_huge_valf();
  }
}

template <int NT, int CH>
hipError_t launch(const float* vals, const int32_t* cand, int64_t ld, int T, const int32_t* cu,
                  int nseq, int block_size, int topk, int force_own, int32_t* out_idx,
                  float* out_val, hipStream_t st) {
  hipLaunchKernelGGL((topk_select_kernel<NT, CH>), dim3(T), dim3(NT), 0, st, vals, cand, ld, cu,
                     nseq, block_size, topk, force_own, out_idx, out_val);
  return hipGetLastError();
}

}  // namespace

int topk_select_max_width() { return 1024 * 4 * 16; }

hipError_t launch_topk_select(const float* vals, const int32_t* cand, int64_t ld, int T,
                              const int32_t* cu, int nseq, int width, int block_size, int topk,
                              int force_own, int32_t* out_idx, float* out_val, hipStream_t st) {
  if (width <= 256 * 4) return launch<256, 1>(vals, cand, ld, T, cu, nseq, block_size, topk, force_own, out_idx, out_val, st);
  if (width <= 1024 * 4) return launch<1024, 1>(vals, cand, ld, T, cu, nseq, block_size, topk, force_own, out_idx, out_val, st);
  if (width <= 1024 * 8) return launch<1024, 2>(vals, cand, ld, T, cu, nseq, block_size, topk, force_own, out_idx, out_val, st);
  if (width <= 1024 * 16) return launch<1024, 4>(vals, cand, ld, T, cu, nseq, block_size, topk, force_own, out_idx, out_val, st);
  if (width <= 1024 * 32) return launch<1024, 8>(vals, cand, ld, T, cu, nseq, block_size, topk, force_own, out_idx, out_val, st);
  return launch<1024, 16>(vals, cand, ld, T, cu, nseq, block_size, topk, force_own, out_idx, out_val, st);
}

}  // namespace sa
