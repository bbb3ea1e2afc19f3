// Attention block (device function) of the attention launch: sparse decode
// attention over the selected tokens, split-K with an fp32 softmax and a
// log-sum-exp merge.
//
// Sources: reproduction card, "Layout" (full versus top-C sparse attention) and
// "Key finding" (the method attends to the C selected tokens only); research-map
// summary of AsyncSpade, "Approach" (the selection is consumed by the inference
// step).  Reading taken: the attention query is the actual current query, the
// prediction only chooses the tokens.  Optionally the newest R tokens of each
// sequence are attended beside the selection (a selected index among them
// counts once); the pages are silent on tokens newer than the selection.
//
// Grid: (split, unit).  A workgroup of 4 wavefronts gathers up to
// 4 * 8 * KPW selected K and V rows of one unit (each row read once and used by
// all G query heads of the group), computes the G x tokens logits, the block
// softmax statistics (max in the log2 domain, sum) and the weighted V sum, and
// writes one partial (acc[G][D], m[G], l[G]).  The merge kernel combines the
// partials of each (sequence, query head).
#pragma once

#include "asp_internal.h"

namespace asp {

constexpr int ATT_THREADS = 256;
constexpr int ATT_WAVES = ATT_THREADS / 64;
constexpr int ATT_NL = 8;  // row loads in flight per lane for K and for V

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

// LDS of one attention block: per-wave maxima, sums and accumulators.
template <int D, int G>
constexpr size_t attend_lds_bytes() {
  return (size_t)ATT_WAVES * G * (D + 2) * sizeof(float);
}

// Token list of a unit: its n selected entries, then the newest r tokens
// [lo, lo + r) of the sequence (r = min(R, seq_len); none when R == 0).
struct AttendList {
  int n, r, lo;
};
__device__ __forceinline__ AttendList attend_list(const int32_t* __restrict__ n_sel,
                                                  const int32_t* __restrict__ seq_lens, int unit, int Hkv, int C,
                                                  int R, int T_cap) {
  AttendList a;
  a.n = clampi(n_sel[unit], 0, C);
  const int T = R > 0 ? clampi(seq_lens[unit / Hkv], 0, T_cap) : 0;
  a.r = min(R, T);
  a.lo = T - a.r;
  return a;
}

// Attention block (split, unit); smem holds attend_lds_bytes<D, G>().
// RECENT: the newest-token window is on (R > 0); without it the token list is
// the selection alone.
template <typename KV, int D, int G, bool RECENT>
__device__ __forceinline__ void attend_block(const float* __restrict__ q, const KV* __restrict__ k,
                                             const KV* __restrict__ v, const int32_t* __restrict__ seq_lens,
                                             const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel,
                                             float* __restrict__ part_acc, float* __restrict__ part_ml, int Hq,
                                             int Hkv, int T_cap, int C, int R, int nsplit, int split, int unit,
                                             unsigned char* smem) {
  constexpr int EPL = 16 / (int)sizeof(KV);
  constexpr int LPK = D / EPL;
  constexpr int KPW = 64 / LPK;
  constexpr int TPW = ATT_NL * KPW;
  constexpr int TPB = ATT_WAVES * TPW;
  float (*sm_m)[G] = reinterpret_cast<float (*)[G]>(smem);
  float (*sm_l)[G] = reinterpret_cast<float (*)[G]>(smem + (size_t)ATT_WAVES * G * sizeof(float));
  float (*sm_acc)[G][D] = reinterpret_cast<float (*)[G][D]>(smem + (size_t)2 * ATT_WAVES * G * sizeof(float));

  const int b = unit / Hkv, g = unit % Hkv;
  const AttendList al = attend_list(n_sel, seq_lens, unit, Hkv, C, RECENT ? R : 0, T_cap);
  const int tok0 = split * TPB;
  if (tok0 >= al.n + al.r) return;
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
    int id = -1;
    bool in_list = false;
    if constexpr (RECENT) {
      if (t < al.n) {  // a selected entry inside the recent range is attended there
        id = ib[t];
        in_list = id >= 0 && id < T_cap && !(id >= al.lo && id < al.lo + al.r);
      } else if (t < al.n + al.r) {
        id = al.lo + (t - al.n);
        in_list = true;
      }
    } else {
      id = t < al.n ? ib[t] : -1;
      in_list = id >= 0 && id < T_cap;
    }
    ok[i] = in_list;
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

}  // namespace asp
