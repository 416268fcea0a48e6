// Token groups of the block-routed GQA kernels: the distinct blocks that a group of
// consecutive tokens routes to, in ascending key order, each with the mask of the
// group's tokens that route to it. Shared by the forward and the backward.
#pragma once

#include "sa_common.h"

namespace sa {

constexpr int kGrpRows = 128;            // query rows of a group (8 column tiles of 16)
constexpr int kGrpMaxTok = 32;           // tokens of a group (token mask width)
constexpr int kGrpWaves = 8;             // one column tile each

// Tokens per group for G query heads per kv head: 128 / G rows' worth, at most 32.
inline int grp_tokens(int G) { return G >= 4 ? kGrpRows / G : kGrpMaxTok; }
// Bitmap words over a group's key range (a sequence of maxlen keys plus GT - 1).
inline int grp_words(int maxlen, int GT) { return (maxlen + GT + 31) / 32 + 1; }
// Bytes of the set-up tables: bitmap, prefix counts, block key rows, token masks, and
// 16 words of scratch.
inline size_t grp_table_bytes(int GT, int nblk, int maxlen) {
  return 2 * (size_t)grp_words(maxlen, GT) * 4 + 2 * (size_t)GT * nblk * 4 + 64;
}

struct GroupTables {
  uint32_t* bits;   // [nwords]  bitmap over key rows base .. base + 32 nwords - 1
  uint32_t* pre;    // [nwords]  exclusive prefix counts of the bitmap words
  int32_t* ulo;     // [GT nblk] first key row of distinct block u
  uint32_t* umask;  // [GT nblk] tokens of the group that route to block u
  uint32_t* red;    // [16]      scratch
};

SA_DEVICE GroupTables group_tables(char* p, int GT, int nblk, int nwords) {
  GroupTables g;
  g.bits = reinterpret_cast<uint32_t*>(p);
  g.pre = g.bits + nwords;
  g.ulo = reinterpret_cast<int32_t*>(g.pre + nwords);
  g.umask = reinterpret_cast<uint32_t*>(g.ulo + GT * nblk);
  g.red = g.umask + GT * nblk;
  return g;
}

// Builds the tables for tokens t0 .. tlast (all threads of the workgroup call it; it
// ends with a barrier) and returns the number of distinct blocks. base = start of
// t0's sequence. A route entry counts when 0 <= b <= the token's own block; its block
// is the key row start(t) + b B, so entries of different tokens (or sequences) that
// name the same rows meet in one entry. Blocks are numbered in ascending key order.
template <int NT>
SA_DEVICE int group_union(const GroupTables& tb, const int32_t* __restrict__ blk,
                          const int32_t* __restrict__ cu, int nseq, int t0, int tlast, int GT,
                          int B, int nblk, int base, int nwords) {
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  for (int i = tid; i < nwords; i += NT) tb.bits[i] = 0u;
  __syncthreads();
  const int ne = GT * nblk;
  for (int e = tid; e < ne; e += NT) {
    const int tau = e / nblk, j = e - tau * nblk;
    const int t = t0 + tau;
    if (t <= tlast) {
      const int st = cu ? seq_start_of(cu, nseq, t) : 0;
      const int b = blk[(int64_t)t * nblk + j];
      if (b >= 0 && b <= (t - st) / B) {
        const int r = st + b * B - base;
        atomicOr(&tb.bits[r >> 5], 1u << (r & 31));
      }
    }
  }
  __syncthreads();
  {
    const int wpt = (nwords + NT - 1) / NT;
    uint32_t cnt = 0;
    for (int r = 0; r < wpt; ++r) {
      const int i = tid * wpt + r;
      if (i < nwords) cnt += (uint32_t)__popc(tb.bits[i]);
    }
    const uint32_t inc = wave_incl_scan(cnt);
    if (L == 63) tb.red[w] = inc;
    __syncthreads();
    uint32_t run = inc - cnt;
    for (int i = 0; i < w; ++i) run += tb.red[i];
    if (tid == NT - 1) tb.red[15] = run + cnt;                 // distinct blocks
    for (int r = 0; r < wpt; ++r) {
      const int i = tid * wpt + r;
      if (i < nwords) {
        tb.pre[i] = run;
        run += (uint32_t)__popc(tb.bits[i]);
      }
    }
  }
  for (int i = tid; i < ne; i += NT) tb.umask[i] = 0u;
  __syncthreads();
  const int nu = (int)tb.red[15];
  for (int e = tid; e < ne; e += NT) {
    const int tau = e / nblk, j = e - tau * nblk;
    const int t = t0 + tau;
    if (t <= tlast) {
      const int st = cu ? seq_start_of(cu, nseq, t) : 0;
      const int b = blk[(int64_t)t * nblk + j];
      if (b >= 0 && b <= (t - st) / B) {
        const int r = st + b * B - base;
        const int u = (int)(tb.pre[r >> 5] + (uint32_t)__popc(tb.bits[r >> 5] & ((1u << (r & 31)) - 1u)));
        tb.ulo[u] = r + base;
        atomicOr(&tb.umask[u], 1u << tau);
      }
    }
  }
  __syncthreads();
  return nu;
}

}  // namespace sa
