// Sparse decode attention over the selected tokens, split-K with an fp32
// softmax and a log-sum-exp merge.
//
// Sources: reproduction card, "Layout" (full versus top-C sparse attention) and
// "Key finding" (the method attends to the C selected tokens only); research-map
// summary of AsyncSpade, "Approach" (the selection is consumed by the inference
// step).  Reading taken: the attention query is the actual current query, the
// prediction only chooses the tokens.
//
// Grid: (split, unit).  A workgroup of 4 wavefronts gathers up to
// 4 * 8 * KPW selected K and V rows of one unit (each row read once and used by
// all G query heads of the group), computes the G x tokens logits, the block
// softmax statistics (max in the log2 domain, sum) and the weighted V sum, and
// writes one partial (acc[G][D], m[G], l[G]).  The merge kernel combines the
// partials of each (sequence, query head).
#include "asp_internal.h"

namespace asp {

constexpr int ATT_THREADS = 256;
constexpr int ATT_WAVES = ATT_THREADS / 64;
constexpr int ATT_NL = 8;  // row loads in flight per lane for K and for V

int attend_tokens_per_block(int D, int kv) {
  const int row_bytes = D * (kv == 0 ? 2 : 4);
  const int kpw = 64 / (row_bytes / 16);
  return ATT_WAVES * ATT_NL * kpw;
}

int attend_num_splits(const Shape& s) {
  const int tpb = attend_tokens_per_block(s.D, s.kv);
  return (s.C + tpb - 1) / tpb;
}

size_t attend_partials_bytes(const Shape& s) {
  const size_t units = (size_t)s.B * s.Hkv;
  return units * attend_num_splits(s) * s.G * (s.D + 2) * sizeof(float);
}

template <typename KV>
__device__ __forceinline__ void unpack_row16(const uint4& r, float* x) {
  if constexpr (sizeof(KV) == 2) {
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z);
    x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
  } else {
    x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
  }
}

template <typename KV, int D, int G>
__global__ void __launch_bounds__(ATT_THREADS) attend_kernel(const float* __restrict__ q, const KV* __restrict__ k,
                                                             const KV* __restrict__ v,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ n_sel,
                                                             float* __restrict__ part_acc,
                                                             float* __restrict__ part_ml, int Hq, int Hkv, int T_cap,
                                                             int C, int nsplit) {
  constexpr int EPL = 16 / (int)sizeof(KV);
  constexpr int LPK = D / EPL;
  constexpr int KPW = 64 / LPK;
  constexpr int TPW = ATT_NL * KPW;
  constexpr int TPB = ATT_WAVES * TPW;
  __shared__ float sm_m[ATT_WAVES][G];
  __shared__ float sm_l[ATT_WAVES][G];
  __shared__ float sm_acc[ATT_WAVES][G][D];

  const int split = blockIdx.x, unit = blockIdx.y;
  const int b = unit / Hkv, g = unit % Hkv;
  const int n = clampi(n_sel[unit], 0, C);
  const int tok0 = split * TPB;
  if (tok0 >= n) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kl = lane / LPK;

  // Query slice, pre-scaled so that exp2 of a logit difference is the softmax
  // weight: log2(e) / sqrt(D).
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  float qr[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((size_t)b * Hq + (size_t)g * G + h) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[h][e] = qh[e] * scale;
  }

  const int32_t* ib = idx + (size_t)unit * C;
  int tk[ATT_NL];
  bool ok[ATT_NL];
#pragma unroll
  for (int i = 0; i < ATT_NL; ++i) {
    const int t = tok0 + wave * TPW + i * KPW + kl;
    const int id = t < n ? ib[t] : -1;
    ok[i] = id >= 0 && id < T_cap;
    tk[i] = ok[i] ? id : 0;
  }
  const KV* kb = k + (size_t)unit * T_cap * D + sub * EPL;
  const KV* vb = v + (size_t)unit * T_cap * D + sub * EPL;
  uint4 kr[ATT_NL], vr[ATT_NL];
#pragma unroll
  for (int i = 0; i < ATT_NL; ++i)
    kr[i] = ok[i] ? *reinterpret_cast<const uint4*>(kb + (size_t)tk[i] * D) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < ATT_NL; ++i)
    vr[i] = ok[i] ? *reinterpret_cast<const uint4*>(vb + (size_t)tk[i] * D) : make_uint4(0, 0, 0, 0);

  // Logits (log2 domain); every lane of a key's lane group holds the same value.
  float lg[G][ATT_NL];
#pragma unroll
  for (int i = 0; i < ATT_NL; ++i) {
    float x[EPL];
    unpack_row16<KV>(kr[i], x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc = fmaf(qr[h][e], x[e], acc);
      acc = group_sum<LPK>(acc);
      lg[h][i] = ok[i] ? acc : -INFINITY;
    }
  }
  // Block maximum per head.
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = lg[h][0];
#pragma unroll
    for (int i = 1; i < ATT_NL; ++i) x = fmaxf(x, lg[h][i]);
    x = group_max<64>(x);
    if (lane == 0) sm_m[wave][h] = x;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < ATT_WAVES; ++w) x = fmaxf(x, sm_m[w][h]);
    m[h] = x;
  }
  // Weights, their sum and the weighted V rows.
  float acc[G][EPL];
  float l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < ATT_NL; ++i) {
    float x[EPL];
    unpack_row16<KV>(vr[i], x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = ok[i] ? exp2f(lg[h][i] - m[h]) : 0.0f;
      l[h] += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
    }
  }
  // Reduce over the key lane groups of the wave (lanes with the same `sub`).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
  }
  if (kl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][h][sub * EPL + e] = acc[h][e];
      if (sub == 0) sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)unit * nsplit + split) * G;
  for (int e = threadIdx.x; e < G * D; e += ATT_THREADS) {
    const int h = e / D, d = e % D;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) s += sm_acc[w][h][d];
    part_acc[(pbase + h) * D + d] = s;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) s += sm_l[w][h];
    part_ml[(pbase + h) * 2 + 0] = m[h];
    part_ml[(pbase + h) * 2 + 1] = s;
  }
}

// One workgroup per (sequence, query head): log-sum-exp merge of the partials.
// The first wavefront reads the m/l pairs of all splits (independent loads,
// splits strided over its lanes) and forms the maximum, the split weights and
// the normaliser with cross-lane reductions; each output coordinate then reads
// its partial sums with independent loads.
constexpr int MERGE_MAX_SPLITS = 256;

__global__ void __launch_bounds__(128) merge_kernel(const float* __restrict__ part_acc,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ n_sel, float* __restrict__ out,
                                                    int Hq, int Hkv, int G, int D, int C, int nsplit, int tpb) {
  constexpr int PER = MERGE_MAX_SPLITS / 64;
  __shared__ float sw[MERGE_MAX_SPLITS];
  __shared__ float s_inv_l;
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / G, hh = h % G;
  const int unit = b * Hkv + g;
  const int n = clampi(n_sel[unit], 0, C);
  const int ns = min((n + tpb - 1) / tpb, MERGE_MAX_SPLITS);
  const int t = threadIdx.x;
  if (t < 64) {
    float m[PER], l[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int sp = t + 64 * r;
      m[r] = -INFINITY;
      l[r] = 0.0f;
      if (sp < ns) {
        const size_t p = ((size_t)unit * nsplit + sp) * G + hh;
        m[r] = part_ml[p * 2];
        l[r] = part_ml[p * 2 + 1];
      }
    }
    float mx = m[0];
#pragma unroll
    for (int r = 1; r < PER; ++r) mx = fmaxf(mx, m[r]);
    const float M = group_max<64>(mx);
    float lw = 0.0f;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int sp = t + 64 * r;
      // splits whose tokens were all skipped carry m = -inf and l = 0
      const float w = (sp < ns && m[r] != -INFINITY) ? exp2f(m[r] - M) : 0.0f;
      if (sp < ns) sw[sp] = w;
      lw = fmaf(l[r], w, lw);
    }
    const float L = group_sum<64>(lw);
    if (t == 0) s_inv_l = L > 0.0f ? 1.0f / L : 0.0f;
  }
  __syncthreads();
  const float inv_l = s_inv_l;
  for (int d = t; d < D; d += blockDim.x) {
    float o = 0.0f;
    const float* pa = part_acc + (((size_t)unit * nsplit) * G + hh) * D + d;
    for (int s = 0; s < ns; ++s) o = fmaf(pa[(size_t)s * G * D], sw[s], o);
    out[(size_t)bh * D + d] = o * inv_l;
  }
}

template <typename KV, int D>
static hipError_t launch_attend_d(const Shape& s, const float* q, const void* k, const void* v, const int32_t* idx,
                                  const int32_t* n_sel, float* part_acc, float* part_ml, hipStream_t st) {
  const int nsplit = attend_num_splits(s);
  const dim3 grid(nsplit, s.B * s.Hkv);
  const KV* kk = static_cast<const KV*>(k);
  const KV* vv = static_cast<const KV*>(v);
#define ASP_ATT_LAUNCH(GG)                                                                                   \
  hipLaunchKernelGGL((attend_kernel<KV, D, GG>), grid, dim3(ATT_THREADS), 0, st, q, kk, vv, idx, n_sel, part_acc, \
                     part_ml, s.Hq, s.Hkv, s.T_cap, s.C, nsplit)
  switch (s.G) {
    case 1: ASP_ATT_LAUNCH(1); break;
    case 2: ASP_ATT_LAUNCH(2); break;
    case 4: ASP_ATT_LAUNCH(4); break;
    case 8: ASP_ATT_LAUNCH(8); break;
    default: return hipErrorInvalidValue;
  }
#undef ASP_ATT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attend(const Shape& s, const float* q, const void* k, const void* v, const int32_t* idx,
                         const int32_t* n_sel, float* out, void* partials, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int nsplit = attend_num_splits(s);
  float* part_acc = static_cast<float*>(partials);
  float* part_ml = part_acc + (size_t)s.B * s.Hkv * nsplit * s.G * s.D;
  hipError_t e;
  if (s.kv == 0)
    e = s.D == 64 ? launch_attend_d<uint16_t, 64>(s, q, k, v, idx, n_sel, part_acc, part_ml, st)
                  : launch_attend_d<uint16_t, 128>(s, q, k, v, idx, n_sel, part_acc, part_ml, st);
  else
    e = s.D == 64 ? launch_attend_d<float, 64>(s, q, k, v, idx, n_sel, part_acc, part_ml, st)
                  : launch_attend_d<float, 128>(s, q, k, v, idx, n_sel, part_acc, part_ml, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(s.B * s.Hq), dim3(128), 0, st, part_acc, part_ml, n_sel, out, s.Hq, s.Hkv,
                     s.G, s.D, s.C, nsplit, attend_tokens_per_block(s.D, s.kv));
  return hipGetLastError();
}

}  // namespace asp
