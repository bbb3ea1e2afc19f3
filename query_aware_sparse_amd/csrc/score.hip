// Token-level key scoring: score[b][g][i] = max over the G query heads of
// KV head g of q_pred[b][h] . K[b][g][i].
//
// Sources: atlas.scime.ai research-map summary of AsyncSpade, "Approach"
// (token-level KV selection driven by the predicted query); arXiv 2510.07486
// abstract (token-level instead of coarse page-level selection; decoding is
// memory bound because the KV cache grows linearly).  The max over the GQA
// group is the reading taken for grouped-query attention, which the pages do
// not discuss.
//
// This pass streams the whole K cache once and is bound by HBM bandwidth.  The
// KV layout is head-major ([B][Hkv][T_cap][D]), so a unit's keys are one
// contiguous stream.  A wavefront issues 16-byte loads: one key row is LPK
// consecutive lanes, KPW keys per wave-wide load, U loads in flight per lane
// before any arithmetic.  The group's query slice stays in registers.
#include "asp_internal.h"

namespace asp {

constexpr int SCORE_THREADS = 256;
constexpr int SCORE_KEYS_PER_BLOCK = 2048;

template <typename KV>
__device__ __forceinline__ void unpack16(const uint4& r, float* x) {
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
__global__ void __launch_bounds__(SCORE_THREADS) score_valu_kernel(const float* __restrict__ q_pred,
                                                                   const KV* __restrict__ k,
                                                                   const int32_t* __restrict__ seq_lens,
                                                                   float* __restrict__ scores, int Hq, int Hkv,
                                                                   int T_cap) {
  constexpr int EPL = 16 / (int)sizeof(KV);  // elements per 16-byte load
  constexpr int LPK = D / EPL;               // lanes per key row
  constexpr int KPW = 64 / LPK;              // keys per wave-wide load
  constexpr int U = 4;                       // loads in flight per lane
  constexpr int WAVES = SCORE_THREADS / 64;

  const int unit = blockIdx.y;
  const int b = unit / Hkv, g = unit % Hkv;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int k0 = blockIdx.x * SCORE_KEYS_PER_BLOCK;
  if (k0 >= T) return;
  const int k1 = min(k0 + SCORE_KEYS_PER_BLOCK, T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kl = lane / LPK;

  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q_pred + ((size_t)b * Hq + (size_t)g * G + h) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[h][e] = qh[e];
  }
  const KV* kb = k + (size_t)unit * T_cap * D + sub * EPL;
  float* sb = scores + (size_t)unit * T_cap;

  for (int base = k0 + wave * KPW * U; base < k1; base += WAVES * KPW * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPW + kl;
      raw[u] = key < k1 ? *reinterpret_cast<const uint4*>(kb + (size_t)key * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[EPL];
      unpack16<KV>(raw[u], x);
      float best = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(q[h][e], x[e], acc);
        acc = group_sum<LPK>(acc);
        best = h == 0 ? acc : fmaxf(best, acc);
      }
      const int key = base + u * KPW + kl;
      if (sub == 0 && key < k1) sb[key] = best;
    }
  }
}

template <typename KV, int D>
static hipError_t launch_score_d(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                 float* scores, hipStream_t st) {
  const dim3 grid((s.T_cap + SCORE_KEYS_PER_BLOCK - 1) / SCORE_KEYS_PER_BLOCK, s.B * s.Hkv);
  const KV* kk = static_cast<const KV*>(k);
  switch (s.G) {
    case 1: hipLaunchKernelGGL((score_valu_kernel<KV, D, 1>), grid, dim3(SCORE_THREADS), 0, st, q_pred, kk, seq_lens, scores, s.Hq, s.Hkv, s.T_cap); break;
    case 2: hipLaunchKernelGGL((score_valu_kernel<KV, D, 2>), grid, dim3(SCORE_THREADS), 0, st, q_pred, kk, seq_lens, scores, s.Hq, s.Hkv, s.T_cap); break;
    case 4: hipLaunchKernelGGL((score_valu_kernel<KV, D, 4>), grid, dim3(SCORE_THREADS), 0, st, q_pred, kk, seq_lens, scores, s.Hq, s.Hkv, s.T_cap); break;
    case 8: hipLaunchKernelGGL((score_valu_kernel<KV, D, 8>), grid, dim3(SCORE_THREADS), 0, st, q_pred, kk, seq_lens, scores, s.Hq, s.Hkv, s.T_cap); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens, float* scores,
                        hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  if (s.kv == 0) {
    return s.D == 64 ? launch_score_d<uint16_t, 64>(s, q_pred, k, seq_lens, scores, st)
                     : launch_score_d<uint16_t, 128>(s, q_pred, k, seq_lens, scores, st);
  }
  return s.D == 64 ? launch_score_d<float, 64>(s, q_pred, k, seq_lens, scores, st)
                   : launch_score_d<float, 128>(s, q_pred, k, seq_lens, scores, st);
}

}  // namespace asp
