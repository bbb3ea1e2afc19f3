// Launches of the sparse attention and its merge; the attention block body is
// in attend_block.h.
#include "attend_block.h"

namespace asp {

int attend_tokens_per_block(int D, int kv) {
  const int row_bytes = D * (kv == 0 ? 2 : 4);
  const int kpw = 64 / (row_bytes / 16);
  return ATT_WAVES * ATT_NL * kpw;
}

int attend_num_splits(const Shape& s) {
  const int tpb = attend_tokens_per_block(s.D, s.kv);
  return (s.C + s.R + tpb - 1) / tpb;
}

size_t attend_partials_bytes(const Shape& s) {
  const size_t units = (size_t)s.B * s.Hkv;
  return units * attend_num_splits(s) * s.G * (s.D + 2) * sizeof(float);
}

template <typename KV, int D, int G, bool RECENT>
__global__ void __launch_bounds__(ATT_THREADS) attend_kernel(const float* __restrict__ q, const KV* __restrict__ k,
                                                             const KV* __restrict__ v,
                                                             const int32_t* __restrict__ seq_lens,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ n_sel,
                                                             float* __restrict__ part_acc,
                                                             float* __restrict__ part_ml, int Hq, int Hkv, int T_cap,
                                                             int C, int R, int nsplit) {
  __shared__ __align__(16) unsigned char smem[attend_lds_bytes<D, G>()];
  attend_block<KV, D, G, RECENT>(q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, Hq, Hkv, T_cap, C, R, nsplit,
                                 blockIdx.x, blockIdx.y, smem);
}

// One workgroup per (sequence, query head): log-sum-exp merge of the partials.
// The first wavefront reads the m/l pairs of all splits (independent loads,
// splits strided over its lanes) and forms the maximum, the split weights and
// the normaliser with cross-lane reductions; each output coordinate then reads
// its partial sums with independent loads.
constexpr int MERGE_MAX_SPLITS = 256;

__global__ void __launch_bounds__(128) merge_kernel(const float* __restrict__ part_acc,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ seq_lens,
                                                    const int32_t* __restrict__ n_sel, float* __restrict__ out,
                                                    int Hq, int Hkv, int G, int D, int T_cap, int C, int R,
                                                    int nsplit, int tpb) {
  constexpr int PER = MERGE_MAX_SPLITS / 64;
  __shared__ float sw[MERGE_MAX_SPLITS];
  __shared__ float s_inv_l;
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / G, hh = h % G;
  const int unit = b * Hkv + g;
  const AttendList al = attend_list(n_sel, seq_lens, unit, Hkv, C, R, T_cap);
  const int ns = min((al.n + al.r + tpb - 1) / tpb, MERGE_MAX_SPLITS);
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
static hipError_t launch_attend_d(const Shape& s, const float* q, const void* k, const void* v,
                                  const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel, float* part_acc,
                                  float* part_ml, hipStream_t st) {
  const int nsplit = attend_num_splits(s);
  const dim3 grid(nsplit, s.B * s.Hkv);
  const KV* kk = static_cast<const KV*>(k);
  const KV* vv = static_cast<const KV*>(v);
#define ASP_ATT_LAUNCH(GG)                                                                                     \
  do {                                                                                                             \
    if (s.R > 0)                                                                                                   \
      hipLaunchKernelGGL((attend_kernel<KV, D, GG, true>), grid, dim3(ATT_THREADS), 0, st, q, kk, vv, seq_lens,     \
                         idx, n_sel, part_acc, part_ml, s.Hq, s.Hkv, s.T_cap, s.C, s.R, nsplit);                    \
    else                                                                                                           \
      hipLaunchKernelGGL((attend_kernel<KV, D, GG, false>), grid, dim3(ATT_THREADS), 0, st, q, kk, vv, seq_lens,    \
                         idx, n_sel, part_acc, part_ml, s.Hq, s.Hkv, s.T_cap, s.C, 0, nsplit);                      \
  } while (0)
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

hipError_t launch_attend(const Shape& s, const float* q, const void* k, const void* v, const int32_t* seq_lens,
                         const int32_t* idx, const int32_t* n_sel, float* out, void* partials, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int nsplit = attend_num_splits(s);
  float* part_acc = static_cast<float*>(partials);
  float* part_ml = part_acc + (size_t)s.B * s.Hkv * nsplit * s.G * s.D;
  hipError_t e;
  if (s.kv == 0)
    e = s.D == 64 ? launch_attend_d<uint16_t, 64>(s, q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, st)
                  : launch_attend_d<uint16_t, 128>(s, q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, st);
  else
    e = s.D == 64 ? launch_attend_d<float, 64>(s, q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, st)
                  : launch_attend_d<float, 128>(s, q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, st);
  if (e != hipSuccess) return e;
  return launch_merge(s, seq_lens, n_sel, out, partials, st);
}

hipError_t launch_merge(const Shape& s, const int32_t* seq_lens, const int32_t* n_sel, float* out,
                        const void* partials, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int nsplit = attend_num_splits(s);
  const float* part_acc = static_cast<const float*>(partials);
  const float* part_ml = part_acc + (size_t)s.B * s.Hkv * nsplit * s.G * s.D;
  hipLaunchKernelGGL(merge_kernel, dim3(s.B * s.Hq), dim3(128), 0, st, part_acc, part_ml, seq_lens, n_sel, out,
                     s.Hq, s.Hkv, s.G, s.D, s.T_cap, s.C, s.R, nsplit, attend_tokens_per_block(s.D, s.kv));
  return hipGetLastError();
}

}  // namespace asp
