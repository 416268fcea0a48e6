// Sparse KL loss of the indexer over the selected slots, with its backward into the
// indexer ("Add trainable QSA sparse attention with a TileLang backend": sparse KL
// supervision of the indexer, a stage-2 teacher/KL loss; "Enable DSA CP/absorbed/THD
// paths with TileLang fused ops": streaming sparse-KL for the indexer loss and the
// fused indexer backward). Reading of the pages: over the valid slots j of row t
// (keys s_j = idx[t,j]) the teacher p_j is given (the head-mean sparse attention
// probability), the student is softmax_j(I_j) of the indexer scores
// I_j = sum_h w[t,h] relu(z_hj), z_hj = q_I[t,h] . k_I[s_j], and
//   loss[t] = sum_j p_j (log p_j - log softmax(I)_j),
//   dI_j = g_t (softmax(I)_j sum_i p_i - p_j)   (sum_i p_i < 1 when a sink holds mass),
//   dw[t,h] = sum_j dI_j relu(z_hj),
//   dq_I[t,h] = sum_j dI_j w[t,h] [z_hj > 0] k_I[s_j],
//   dk_I[s_j] += sum_h dI_j w[t,h] [z_hj > 0] q_I[t,h]       (atomics, fp32),
// g_t the weight of row t in the summed loss. Only the k selected scores of a row are
// ever formed ("streaming": no [T, T] matrix).
//
// bf16 kernel (gfx950): one workgroup per row, four waves taking turns over 16-slot
// sub-tiles; the row's slot indices are staged in LDS first. The row's heads are the
// rows of 16x16x32 MFMA tiles (q_I as A operands in registers, the 16 gathered key
// rows as B operands). Pass 1 reads the rows straight into B operands and forms the
// scores I_j into LDS; the row's log-sum-exp, loss and dI follow; pass 2 stages the
// rows in LDS and recomputes z per sub-tile for dw, dq_I^T += K^T dz^T (K^T by
// transposing reads of the staged rows, dz^T through a small LDS transpose) and
// dk_I = dz^T q_I (q_I by transposing LDS reads), added to k_I's gradient with atomics.
// In both passes each wave requests its next sub-tile's rows before computing the
// current one.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;
constexpr int kSK = 16;
constexpr int kMaxTopk = 4096;

typedef float floatx4v_t __attribute__((ext_vector_type(4)));

SA_DEVICE floatx4v_t mfma16x32(bf16x8_t a, bf16x8_t b, floatx4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
SA_DEVICE floatx4v_t mfma16x16(short4_t a, short4_t b, floatx4v_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
SA_DEVICE short4_t pack4(float a, float b, float c, float d) {
  return __builtin_bit_cast(short4_t, make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d)));
}

template <int DI>
constexpr int rowb() { return DI * 2 + 16; }

// slots of the score array, rounded up so that the areas after it stay 16-byte aligned
SA_DEVICE __host__ inline int score_slots(int topk) { return (topk + 3) & ~3; }

template <int NHB, int DI>
constexpr size_t kl_lds_bytes(int topk) {
  const size_t head = (size_t)16 * NHB * rowb<DI>() + (size_t)score_slots(topk) * 8 + 64;
  const size_t work = (size_t)kWaves * (kSK * rowb<DI>() + 16 * NHB * kSK * 2) + (size_t)kWaves * 16 * NHB * 4;
  const size_t red = (size_t)kWaves * 16 * NHB * (DI / 2) * 4;    // dq_I reduction, half of DI per pass
  return head + (work > red ? work : red);
}

// NHB blocks of 16 indexer heads, DI head dim.
template <int NHB, int DI>
__global__ __launch_bounds__(kWaves * 64) void indexer_kl_bf16_kernel(
    const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI, const float* __restrict__ wI,
    const int32_t* __restrict__ idx, const float* __restrict__ teacher, const float* __restrict__ grad,
    int topk, float* __restrict__ loss, uint16_t* __restrict__ dq, float* __restrict__ dw,
    float* __restrict__ dk) {
  constexpr int H = 16 * NHB;
  constexpr int RB = rowb<DI>();
  constexpr int KS = DI / 32;
  constexpr int NDB = DI / 16;
  constexpr int CPR = DI * 2 / 16;
  constexpr int NLD = kSK * CPR / 64;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* q_l = lds;                                              // [H][RB]
  float* Il = reinterpret_cast<float*>(q_l + H * RB);           // [topk] scores, then dI
  int32_t* il = reinterpret_cast<int32_t*>(Il + score_slots(topk));   // [topk] slot indices
  float* bc = reinterpret_cast<float*>(il + score_slots(topk));       // [16] broadcast slots
  char* work = reinterpret_cast<char*>(bc + 16);
  const int t = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const int g = L >> 4, n = L & 15;
  char* kt = work + w * (kSK * RB + H * kSK * 2);               // staged key rows
  char* zt = kt + kSK * RB;                                     // dz transpose [H][16] bf16
  float* dwp = reinterpret_cast<float*>(work + kWaves * (kSK * RB + H * kSK * 2));   // [waves][H]

  for (int c = tid; c < H * CPR; c += kWaves * 64) {
    const int hh = c / CPR, p = c % CPR;
    *reinterpret_cast<bf16x8_t*>(q_l + hh * RB + 16 * p) =
        *reinterpret_cast<const bf16x8_t*>(qI + ((int64_t)t * H + hh) * DI + 8 * p);
  }
  // the row's slot indices, staged once: every later row load takes its index from LDS
  for (int j = tid; j < topk; j += kWaves * 64) il[j] = idx[(int64_t)t * topk + j];
  __syncthreads();
  bf16x8_t qa[NHB][KS];                // head 16 hb + n, dims 32 ks + 8 g
  float wr[NHB][4];                    // w of heads 16 hb + 4 g + i
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[hb][ks] = *reinterpret_cast<const bf16x8_t*>(q_l + (16 * hb + n) * RB + 64 * ks + 16 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[hb][i] = wI[(int64_t)t * H + 16 * hb + 4 * g + i];
  }
  const int nsub = (topk + kSK - 1) / kSK;
  auto slot = [&](int j) __attribute__((always_inline)) { return j < topk ? il[j] : -1; };

  // z tiles of one sub-tile from the B operands kb (key n, dims 32 ks + 8 g)
  auto ztiles = [&](const bf16x8_t (&kb)[KS], floatx4v_t (&Z)[NHB]) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      Z[hb] = floatx4v_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) Z[hb] = mfma16x32(qa[hb][ks], kb[ks], Z[hb]);
    }
  };
  // key row of slot column n of a sub-tile, read straight into B operands
  auto kload = [&](int sub, bf16x8_t (&kb)[KS]) __attribute__((always_inline)) {
    const int row = slot(sub * kSK + n);
    const uint16_t* kr = kI + (int64_t)(row < 0 ? 0 : row) * DI + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * ks);
  };

  // ---- pass 1: scores of the slots (-inf on -1 slots). The wave's next sub-tile is
  //      requested before the current one is computed; the loop body is written out
  //      twice with the two operand buffers swapped, so no in-flight load is copied.
  auto pass1 = [&](int sub, const bf16x8_t (&kb)[KS], bf16x8_t (&kn)[KS]) __attribute__((always_inline)) {
    if (sub + kWaves < nsub) kload(sub + kWaves, kn);
    floatx4v_t Z[NHB];
    ztiles(kb, Z);
    float acc = 0.0f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(wr[hb][i], __builtin_elementwise_maximum(Z[hb][i], 0.0f), acc);
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    const int j = sub * kSK + n;
    if (g == 0 && j < topk) Il[j] = il[j] >= 0 ? acc : -__builtin_huge_valf();
  };
  {
    bf16x8_t kbA[KS], kbB[KS];
    if (w < nsub) kload(w, kbA);
#pragma unroll 1
    for (int sub = w; sub < nsub; sub += 2 * kWaves) {
      pass1(sub, kbA, kbB);
      if (sub + kWaves < nsub) pass1(sub + kWaves, kbB, kbA);
    }
  }
  __syncthreads();
  // ---- row max, log-sum-exp, loss and dI (block-wide over the slots)
  float m = -__builtin_huge_valf();
  for (int j = tid; j < topk; j += kWaves * 64) m = __builtin_elementwise_maximum(m, Il[j]);
  m = wave_max(m);
  if (L == 0) bc[w] = m;
  __syncthreads();
  m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(bc[0], bc[1]),
                                    __builtin_elementwise_maximum(bc[2], bc[3]));
  const float* prow = teacher + (int64_t)t * topk;
  float se = 0.0f, pm = 0.0f;
  for (int j = tid; j < topk; j += kWaves * 64) {
    if (Il[j] > -__builtin_huge_valf()) {
      se += __builtin_amdgcn_exp2f((Il[j] - m) * kLog2e);
      pm += prow[j];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    se += __shfl_xor(se, off, 64);
    pm += __shfl_xor(pm, off, 64);
  }
  if (L == 0) { bc[4 + w] = se; bc[12 + w] = pm; }
  __syncthreads();
  const bool any = m > -__builtin_huge_valf();
  const float lsum = any ? m + __log2f(bc[4] + bc[5] + bc[6] + bc[7]) * kLn2 : 0.0f;   // log sum exp I
  const float pmass = bc[12] + bc[13] + bc[14] + bc[15];                              // teacher mass
  const float gt = grad ? grad[t] : 1.0f;
  float lpart = 0.0f;
  for (int j = tid; j < topk; j += kWaves * 64) {
    const float I = Il[j];
    float d = 0.0f;
    if (I > -__builtin_huge_valf()) {
      const float ls = I - lsum;                                  // log student
      const float p = prow[j];
      if (p > 0.0f) lpart += p * (__log2f(p) * kLn2 - ls);
      d = gt * (__builtin_amdgcn_exp2f(ls * kLog2e) * pmass - p);
    }
    Il[j] = d;                                                    // every thread owns its own j
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lpart += __shfl_xor(lpart, off, 64);
  if (L == 0) bc[8 + w] = lpart;
  __syncthreads();
  if (tid == 0) loss[t] = any ? bc[8] + bc[9] + bc[10] + bc[11] : 0.0f;

  // ---- pass 2: dw, dq_I^T, dk_I
  floatx4v_t acc[NHB][NDB];            // dq_I^T: dims 16 db + 4 g .. +3, head 16 hb + n
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[hb][db] = floatx4v_t{};
  float dwl[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dwl[hb][i] = 0.0f;
  // the 16 key rows of a sub-tile, as 16-byte chunks of this lane
  auto rload = [&](int sub, bf16x8_t (&nx)[NLD]) __attribute__((always_inline)) {
#pragma unroll
    for (int mm = 0; mm < NLD; ++mm) {
      const int c = L + 64 * mm, r = c / CPR, p = c % CPR;
      const int row = slot(sub * kSK + r);
      nx[mm] = *reinterpret_cast<const bf16x8_t*>(kI + (int64_t)(row < 0 ? 0 : row) * DI + 8 * p);
    }
  };
  // Pass 2 body: stages the sub-tile's rows (held in nx) for the transposing reads of
  // K^T and reads its B operands back from there; the wave's next sub-tile is requested
  // into nn first (again two buffers taking turns).
  auto pass2 = [&](int sub, const bf16x8_t (&nx)[NLD], bf16x8_t (&nn)[NLD]) __attribute__((always_inline)) {
#pragma unroll
    for (int mm = 0; mm < NLD; ++mm) {
      const int c = L + 64 * mm, r = c / CPR, p = c % CPR;
      *reinterpret_cast<bf16x8_t*>(kt + r * RB + 16 * p) = nx[mm];
    }
    if (sub + kWaves < nsub) rload(sub + kWaves, nn);
    __builtin_amdgcn_wave_barrier();
    bf16x8_t kb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = *reinterpret_cast<const bf16x8_t*>(kt + n * RB + 64 * ks + 16 * g);
    floatx4v_t Z[NHB];
    ztiles(kb, Z);
    const int j = sub * kSK + n;
    const float dI = slot(j) >= 0 ? Il[j] : 0.0f;
    short4_t dzA[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float dz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = Z[hb][i];
        dwl[hb][i] = fmaf(dI, __builtin_elementwise_maximum(z, 0.0f), dwl[hb][i]);
        dz[i] = z > 0.0f ? dI * wr[hb][i] : 0.0f;
        *reinterpret_cast<uint16_t*>(zt + ((16 * hb + 4 * g + i) * kSK + n) * 2) = f2bf_bits(dz[i]);
      }
      dzA[hb] = pack4(dz[0], dz[1], dz[2], dz[3]);               // dz^T: key n, heads 16hb+4g..
    }
    __builtin_amdgcn_wave_barrier();
    int krow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) krow[i] = slot(sub * kSK + 4 * g + i);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int toff = (16 * db + 4 * (n & 3)) * 2;
      const int trow = 4 * g + (n >> 2);
      const short4_t kT = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS short4_t*)(kt + trow * RB + toff));
      floatx4v_t dkt = floatx4v_t{};
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const short4_t dzB = *reinterpret_cast<const short4_t*>(zt + ((16 * hb + n) * kSK + 4 * g) * 2);
        acc[hb][db] = mfma16x16(kT, dzB, acc[hb][db]);
        const short4_t qB = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (SA_LDS short4_t*)(q_l + (16 * hb + trow) * RB + toff));
        dkt = mfma16x16(dzA[hb], qB, dkt);
      }
      // lane (g, n): keys 4g..4g+3, dim 16 db + n
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (krow[i] >= 0) atomicAdd(dk + (int64_t)krow[i] * DI + 16 * db + n, dkt[i]);
    }
    __builtin_amdgcn_wave_barrier();
  };
  {
    bf16x8_t nxA[NLD], nxB[NLD];
    if (w < nsub) rload(w, nxA);
#pragma unroll 1
    for (int sub = w; sub < nsub; sub += 2 * kWaves) {
      pass2(sub, nxA, nxB);
      if (sub + kWaves < nsub) pass2(sub + kWaves, nxB, nxA);
    }
  }
  // dw: sum over the keys (lanes n), then over the waves
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = dwl[hb][i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
      if (n == 0) dwp[w * H + 16 * hb + 4 * g + i] = v;
    }
  __syncthreads();
  for (int h = tid; h < H; h += kWaves * 64)
    dw[(int64_t)t * H + h] = dwp[h] + dwp[H + h] + dwp[2 * H + h] + dwp[3 * H + h];
  __syncthreads();
  // dq_I: the waves' dq_I^T partials summed through LDS, half of DI per pass
  float* red = reinterpret_cast<float*>(work);       // [waves][H][DI / 2]
  constexpr int HALF = DI / 2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[(w * H + 16 * hb + n) * HALF + 16 * db + 4 * g + i] = acc[hb][half * (NDB / 2) + db][i];
    __syncthreads();
    for (int e = tid; e < H * HALF; e += kWaves * 64) {
      const int hh = e / HALF, c = e % HALF;
      float s = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) s += red[(ww * H + hh) * HALF + c];
      dq[((int64_t)t * H + hh) * DI + half * HALF + c] = f2bf_bits(s);
    }
    __syncthreads();
  }
}

// fp32 (and any head count): one workgroup per row, plain arithmetic.
constexpr int kNT = 256;

__global__ __launch_bounds__(kNT) void indexer_kl_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ kI, const float* __restrict__ wI,
    const int32_t* __restrict__ idx, const float* __restrict__ teacher, const float* __restrict__ grad,
    int H, int DI, int topk, float* __restrict__ loss, float* __restrict__ dq, float* __restrict__ dw,
    float* __restrict__ dk) {
  extern __shared__ float sm[];              // [topk] scores then dI, [16] reduce slots
  float* red = sm + topk;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, L = tid & 63;
  const float* q = qI + (int64_t)t * H * DI;
  const float* wr = wI + (int64_t)t * H;
  const int32_t* ir = idx + (int64_t)t * topk;
  float m = -__builtin_huge_valf();
  for (int j = tid; j < topk; j += kNT) {
    const int r = ir[j];
    float I = -__builtin_huge_valf();
    if (r >= 0) {
      I = 0.0f;
      for (int h = 0; h < H; ++h) {
        float z = 0.0f;
        for (int d = 0; d < DI; ++d) z = fmaf(q[h * DI + d], kI[(int64_t)r * DI + d], z);
        I = fmaf(wr[h], fmaxf(z, 0.0f), I);
      }
    }
    sm[j] = I;
    m = fmaxf(m, I);
  }
  m = wave_max(m);
  if (L == 0) red[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float se = 0.0f, pm = 0.0f;
  for (int j = tid; j < topk; j += kNT) {
    if (sm[j] > -__builtin_huge_valf()) {
      se += expf(sm[j] - m);
      pm += teacher[(int64_t)t * topk + j];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    se += __shfl_xor(se, off, 64);
    pm += __shfl_xor(pm, off, 64);
  }
  if (L == 0) { red[4 + w] = se; red[12 + w] = pm; }
  __syncthreads();
  const bool any = m > -__builtin_huge_valf();
  const float lsum = any ? m + logf(red[4] + red[5] + red[6] + red[7]) : 0.0f;
  const float pmass = red[12] + red[13] + red[14] + red[15];
  const float gt = grad ? grad[t] : 1.0f;
  float lpart = 0.0f;
  for (int j = tid; j < topk; j += kNT) {
    float d = 0.0f;
    if (sm[j] > -__builtin_huge_valf()) {
      const float ls = sm[j] - lsum, p = teacher[(int64_t)t * topk + j];
      if (p > 0.0f) lpart += p * (logf(p) - ls);
      d = gt * (expf(ls) * pmass - p);
    }
    sm[j] = d;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lpart += __shfl_xor(lpart, off, 64);
  if (L == 0) red[8 + w] = lpart;
  __syncthreads();
  if (tid == 0) loss[t] = any ? red[8] + red[9] + red[10] + red[11] : 0.0f;
  // dw and dq: thread per (head, dim) entry; dk by atomics, one slot per thread
  for (int e = tid; e < H * DI; e += kNT) {
    const int h = e / DI, d = e % DI;
    float a = 0.0f, b = 0.0f;
    for (int j = 0; j < topk; ++j) {
      const int r = ir[j];
      if (r < 0) continue;
      float z = 0.0f;
      for (int c = 0; c < DI; ++c) z = fmaf(q[h * DI + c], kI[(int64_t)r * DI + c], z);
      if (z > 0.0f) a = fmaf(sm[j] * wr[h], kI[(int64_t)r * DI + d], a);
      if (d == 0) b = fmaf(sm[j], fmaxf(z, 0.0f), b);
    }
    dq[(int64_t)t * H * DI + e] = a;
    if (d == 0) dw[(int64_t)t * H + h] = b;
  }
  for (int j = tid; j < topk; j += kNT) {
    const int r = ir[j];
    if (r < 0) continue;
    for (int h = 0; h < H; ++h) {
      float z = 0.0f;
      for (int c = 0; c < DI; ++c) z = fmaf(q[h * DI + c], kI[(int64_t)r * DI + c], z);
      if (z > 0.0f)
        for (int d = 0; d < DI; ++d) atomicAdd(dk + (int64_t)r * DI + d, sm[j] * wr[h] * q[h * DI + d]);
    }
  }
}

__global__ void zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

template <int NHB, int DI>
hipError_t launch_kl(const void* qI, const void* kI, const float* wI, const int32_t* idx,
                     const float* teacher, const float* grad, int T, int topk, float* loss, void* dq,
                     float* dw, float* dk, hipStream_t st) {
  const size_t shm = kl_lds_bytes<NHB, DI>(topk);
  hipError_t e = hipFuncSetAttribute((const void*)indexer_kl_bf16_kernel<NHB, DI>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((indexer_kl_bf16_kernel<NHB, DI>), dim3(T), dim3(kWaves * 64), shm, st,
                     (const uint16_t*)qI, (const uint16_t*)kI, wI, idx, teacher, grad, topk, loss,
                     (uint16_t*)dq, dw, dk);
  return hipGetLastError();
}

}  // namespace

int indexer_kl_max_topk() { return kMaxTopk; }

hipError_t launch_indexer_kl(const void* qI, const void* kI, const float* wI, const int32_t* idx,
                             const float* teacher, const float* grad, bool bf16, int T, int S, int H_I,
                             int D_I, int topk, float* loss, void* dq, float* dw, float* dk,
                             hipStream_t st) {
  hipLaunchKernelGGL(zero_kernel, dim3(1024), dim3(256), 0, st, dk, (int64_t)S * D_I);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  if (!bf16) {
    const size_t shm = (size_t)(topk + 16) * sizeof(float);
    e = hipFuncSetAttribute((const void*)indexer_kl_f32_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(indexer_kl_f32_kernel, dim3(T), dim3(kNT), shm, st, (const float*)qI,
                       (const float*)kI, wI, idx, teacher, grad, H_I, D_I, topk, loss, (float*)dq, dw, dk);
    return hipGetLastError();
  }
  switch (H_I * 1000 + D_I) {
    case 16064: return launch_kl<1, 64>(qI, kI, wI, idx, teacher, grad, T, topk, loss, dq, dw, dk, st);
    case 16128: return launch_kl<1, 128>(qI, kI, wI, idx, teacher, grad, T, topk, loss, dq, dw, dk, st);
    case 32064: return launch_kl<2, 64>(qI, kI, wI, idx, teacher, grad, T, topk, loss, dq, dw, dk, st);
    case 32128: return launch_kl<2, 128>(qI, kI, wI, idx, teacher, grad, T, topk, loss, dq, dw, dk, st);
    case 64064: return launch_kl<4, 64>(qI, kI, wI, idx, teacher, grad, T, topk, loss, dq, dw, dk, st);
    default: return launch_kl<4, 128>(qI, kI, wI, idx, teacher, grad, T, topk, loss, dq, dw, dk, st);
  }
}

}  // namespace sa
