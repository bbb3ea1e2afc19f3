// Launches of the sparse attention and its merge.  bf16 K/V: the matrix-core
// block of attend_mfma.h, a few splits per unit (about ATTM_TARGET_BLOCKS
// blocks in all, at least ATTM_WAVES chunks per split), the merge only when a
// unit is split.  fp32 K/V: the VALU block of attend_block.h, one split per
// attend_tokens_per_block() tokens, then the merge.
#include "attend_block.h"
#include "attend_mfma.h"

namespace asp {

// Random 256-byte row gathers reach the read ceiling with some 256 blocks of
// 512 threads in flight (fewer leave the per-CU request rate as the bound).
constexpr int ATTM_TARGET_BLOCKS = 256;

int attend_tokens_per_block(int D, int kv) {
  const int row_bytes = D * (kv == 0 ? 2 : 4);
  const int kpw = 64 / (row_bytes / 16);
  return ATT_WAVES * ATT_NL * kpw;
}

// List positions per split of the bf16 path (a multiple of the chunk).
static int attm_per(const Shape& s, int nsplit) {
  const int total = s.C + s.R;
  const int per = (total + nsplit - 1) / nsplit;
  return (per + ATTM_CHUNK - 1) / ATTM_CHUNK * ATTM_CHUNK;
}

int attend_num_splits(const Shape& s) {
  const int total = s.C + s.R;
  if (s.kv == 0) {
    const int units = s.B * s.Hkv;
    const int want = units > 0 ? (ATTM_TARGET_BLOCKS + units - 1) / units : 1;
    const int cap = (total + ATTM_WAVES * ATTM_CHUNK - 1) / (ATTM_WAVES * ATTM_CHUNK);
    int ns = want < cap ? want : cap;
    if (ns < 1) ns = 1;
    // splits that the rounding of `per` leaves empty are not launched
    return (total + attm_per(s, ns) - 1) / attm_per(s, ns);
  }
  const int tpb = attend_tokens_per_block(s.D, s.kv);
  return (total + tpb - 1) / tpb;
}

// Positions of the list handled by one split (one attention block).
static int attend_split_positions(const Shape& s) {
  return s.kv == 0 ? attm_per(s, attend_num_splits(s)) : attend_tokens_per_block(s.D, s.kv);
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

template <int D, int G, bool RECENT>
__global__ void __launch_bounds__(ATTM_THREADS) attend_mfma_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel,
    float* __restrict__ out, float* __restrict__ part_acc, float* __restrict__ part_ml, int Hq, int Hkv, int T_cap,
    int C, int R, int nsplit, int per) {
  __shared__ __align__(16) unsigned char smem[attm_lds_bytes<D, G>()];
  attend_mfma_block<D, G, RECENT>(q, k, v, seq_lens, idx, n_sel, out, part_acc, part_ml, Hq, Hkv, T_cap, C, R,
                                  nsplit, per, blockIdx.x, blockIdx.y, smem);
}

// One workgroup per (sequence, query head): log-sum-exp merge of the partials.
// Thread d combines output coordinate d.  The splits are read in batches of
// MERGE_BATCH, each thread issuing the batch's (max, sum) pairs and its own
// partial sums together (one memory round trip per batch), with a running
// maximum across batches.
constexpr int MERGE_MAX_SPLITS = 256;
constexpr int MERGE_BATCH = 8;

__global__ void __launch_bounds__(128) merge_kernel(const float* __restrict__ part_acc,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ seq_lens,
                                                    const int32_t* __restrict__ n_sel, float* __restrict__ out,
                                                    int Hq, int Hkv, int G, int D, int T_cap, int C, int R,
                                                    int nsplit, int per) {
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int g = h / G, hh = h % G;
  const int unit = b * Hkv + g;
  const int d = threadIdx.x;
  if (d >= D) return;
  const AttendList al = attend_list(n_sel, seq_lens, unit, Hkv, C, R, T_cap);
  const int ns = min(min((al.n + al.r + per - 1) / per, nsplit), MERGE_MAX_SPLITS);
  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += MERGE_BATCH) {
    float m[MERGE_BATCH], l[MERGE_BATCH], a[MERGE_BATCH];
#pragma unroll
    for (int i = 0; i < MERGE_BATCH; ++i) {
      const int sp = s0 + i;
      m[i] = -INFINITY;
      l[i] = 0.0f;
      a[i] = 0.0f;
      if (sp < ns) {
        const size_t p = ((size_t)unit * nsplit + sp) * G + hh;
        m[i] = part_ml[p * 2];
        l[i] = part_ml[p * 2 + 1];
        a[i] = part_acc[p * D + d];
      }
    }
    float bm = m[0];
#pragma unroll
    for (int i = 1; i < MERGE_BATCH; ++i) bm = fmaxf(bm, m[i]);
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) continue;  // splits whose tokens were all skipped carry m = -inf and l = 0
    const float sc = M == -INFINITY ? 0.0f : exp2f(M - Mn);
    L *= sc;
    O *= sc;
#pragma unroll
    for (int i = 0; i < MERGE_BATCH; ++i) {
      const float w = m[i] == -INFINITY ? 0.0f : exp2f(m[i] - Mn);
      L = fmaf(w, l[i], L);
      O = fmaf(w, a[i], O);
    }
    M = Mn;
  }
  out[(size_t)bh * D + d] = L > 0.0f ? O / L : 0.0f;
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

template <int D>
static hipError_t launch_attend_mfma(const Shape& s, const float* q, const void* k, const void* v,
                                     const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel, float* out,
                                     float* part_acc, float* part_ml, hipStream_t st) {
  const int nsplit = attend_num_splits(s);
  const int per = attm_per(s, nsplit);
  const dim3 grid(nsplit, s.B * s.Hkv);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
#define ASP_ATTM_LAUNCH(GG)                                                                                       \
  do {                                                                                                            \
    if (s.R > 0)                                                                                                  \
      hipLaunchKernelGGL((attend_mfma_kernel<D, GG, true>), grid, dim3(ATTM_THREADS), 0, st, q, kk, vv, seq_lens, \
                         idx, n_sel, out, part_acc, part_ml, s.Hq, s.Hkv, s.T_cap, s.C, s.R, nsplit, per);        \
    else                                                                                                          \
      hipLaunchKernelGGL((attend_mfma_kernel<D, GG, false>), grid, dim3(ATTM_THREADS), 0, st, q, kk, vv,          \
                         seq_lens, idx, n_sel, out, part_acc, part_ml, s.Hq, s.Hkv, s.T_cap, s.C, 0, nsplit, per); \
  } while (0)
  switch (s.G) {
    case 1: ASP_ATTM_LAUNCH(1); break;
    case 2: ASP_ATTM_LAUNCH(2); break;
    case 4: ASP_ATTM_LAUNCH(4); break;
    case 8: ASP_ATTM_LAUNCH(8); break;
    default: return hipErrorInvalidValue;
  }
#undef ASP_ATTM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attend(const Shape& s, const float* q, const void* k, const void* v, const int32_t* seq_lens,
                         const int32_t* idx, const int32_t* n_sel, float* out, void* partials, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int nsplit = attend_num_splits(s);
  float* part_acc = static_cast<float*>(partials);
  float* part_ml = part_acc + (size_t)s.B * s.Hkv * nsplit * s.G * s.D;
  hipError_t e;
  if (s.kv == 0) {
    e = s.D == 64 ? launch_attend_mfma<64>(s, q, k, v, seq_lens, idx, n_sel, out, part_acc, part_ml, st)
                  : launch_attend_mfma<128>(s, q, k, v, seq_lens, idx, n_sel, out, part_acc, part_ml, st);
    if (e != hipSuccess || nsplit == 1) return e;  // one split: the blocks wrote out
  } else {
    e = s.D == 64 ? launch_attend_d<float, 64>(s, q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, st)
                  : launch_attend_d<float, 128>(s, q, k, v, seq_lens, idx, n_sel, part_acc, part_ml, st);
    if (e != hipSuccess) return e;
  }
  return launch_merge(s, seq_lens, n_sel, out, partials, st);
}

hipError_t launch_merge(const Shape& s, const int32_t* seq_lens, const int32_t* n_sel, float* out,
                        const void* partials, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int nsplit = attend_num_splits(s);
  const float* part_acc = static_cast<const float*>(partials);
  const float* part_ml = part_acc + (size_t)s.B * s.Hkv * nsplit * s.G * s.D;
  hipLaunchKernelGGL(merge_kernel, dim3(s.B * s.Hq), dim3(128), 0, st, part_acc, part_ml, seq_lens, n_sel, out,
                     s.Hq, s.Hkv, s.G, s.D, s.T_cap, s.C, s.R, nsplit, attend_split_positions(s));
  return hipGetLastError();
}

}  // namespace asp
