// Page-level selection, the baseline the pages compare AsyncSpade against
// (research-map summary, "Problem" and "Baselines"; arXiv abstract: Quest,
// which selects whole pages of the KV cache with the current query).  The page
// score is Quest's published criticality estimate (Tang et al., ICML 2024,
// method section): every page of P consecutive tokens keeps the element-wise
// minimum and maximum of its keys, and a query q scores the page with
// sum_d max(q_d * min_d, q_d * max_d), the largest q . k over that box.  For
// grouped-query attention a KV head takes the largest bound of its query heads,
// as its token scores take the largest dot product.
//
// Three launches:
//  - page_summary_kernel: one pass over K writing kmin/kmax rows in the KV
//    dtype (exact copies of key elements);
//  - page_score_kernel: one pass over the summaries, a page score row per unit
//    (f32), plus the page count of every sequence for the selection;
//  - the token-level top-C selection (select.hip) run on the page rows with a
//    budget of C / P pages, then page_tokens_kernel, which lists the selected
//    pages' tokens in ascending order as asp_sparse_decode reads them.
//
// Thread layout of the two streaming kernels: a page row of D elements is read
// as 16-byte chunks, TPP = D * esize / 16 consecutive lanes per row (8, 16 or
// 32), so a wave reads whole rows and the row-sum of the score is a reduction
// inside a DPP row or a half-wave.
#include "page.h"

namespace asp {
namespace {

constexpr int PAGE_THREADS = 256;
constexpr int PAGE_SCORE_ROUNDS = 8;  // page rows per lane group of a score block

template <int D, int KV>
struct RowChunks {
  static constexpr int esize = KV == 0 ? 2 : 4;
  static constexpr int ept = 16 / esize;  // elements per 16-byte chunk
  static constexpr int tpp = D * esize / 16;  // lanes per row
  static constexpr int ppb = PAGE_THREADS / tpp;  // rows per block pass
  static constexpr size_t row_bytes = (size_t)D * esize;
};

template <int KV>
__device__ __forceinline__ void widen16(const uint4 w, float* x) {
  if constexpr (KV == 0) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(a[i]);
      x[2 * i + 1] = bf16_hi(a[i]);
    }
  } else {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
}

// Inverse of widen16 for values that are exact in the KV dtype.
template <int KV>
__device__ __forceinline__ uint4 narrow16(const float* x) {
  if constexpr (KV == 0) {
    uint32_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xffff0000u);
    return make_uint4(a[0], a[1], a[2], a[3]);
  } else {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
  }
}

__device__ __forceinline__ int pages_of(const int32_t* seq_lens, int b, int T_cap, int P) {
  const int T = clampi(seq_lens[b], 0, T_cap);
  return (T + P - 1) / P;
}

// grid (ceil(NP / ppb), units); each lane group folds one page's rows.
template <int D, int KV>
__global__ __launch_bounds__(PAGE_THREADS) void page_summary_kernel(const unsigned char* __restrict__ k,
                                                                    const int32_t* __restrict__ seq_lens,
                                                                    unsigned char* __restrict__ kmin,
                                                                    unsigned char* __restrict__ kmax, int Hkv,
                                                                    int T_cap, int P, int NP) {
  using RC = RowChunks<D, KV>;
  const int u = blockIdx.y, b = u / Hkv;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int p = blockIdx.x * RC::ppb + (int)threadIdx.x / RC::tpp;
  const int c = (int)threadIdx.x % RC::tpp;
  if (p >= (T + P - 1) / P) return;
  const int first = p * P, last = min(first + P, T);
  const unsigned char* row = k + ((size_t)u * T_cap + first) * RC::row_bytes + (size_t)c * 16;
  float mn[RC::ept], mx[RC::ept];
  widen16<KV>(*reinterpret_cast<const uint4*>(row), mn);
#pragma unroll
  for (int e = 0; e < RC::ept; ++e) mx[e] = mn[e];
  int i = first + 1;
  for (; i + 4 <= last; i += 4) {  // four rows in flight
    uint4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = *reinterpret_cast<const uint4*>(row + (size_t)(i - first + j) * RC::row_bytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x[RC::ept];
      widen16<KV>(w[j], x);
#pragma unroll
      for (int e = 0; e < RC::ept; ++e) {
        mn[e] = fminf(mn[e], x[e]);
        mx[e] = fmaxf(mx[e], x[e]);
      }
    }
  }
  for (; i < last; ++i) {
    float x[RC::ept];
    widen16<KV>(*reinterpret_cast<const uint4*>(row + (size_t)(i - first) * RC::row_bytes), x);
#pragma unroll
    for (int e = 0; e < RC::ept; ++e) {
      mn[e] = fminf(mn[e], x[e]);
      mx[e] = fmaxf(mx[e], x[e]);
    }
  }
  const size_t out = ((size_t)u * NP + p) * RC::row_bytes + (size_t)c * 16;
  *reinterpret_cast<uint4*>(kmin + out) = narrow16<KV>(mn);
  *reinterpret_cast<uint4*>(kmax + out) = narrow16<KV>(mx);
}

// grid (ceil(NP / (ppb * ROUNDS)), units).  counts (nullable) receives every
// sequence's page count (written by the first block of the sequence's first
// KV head).
template <int D, int KV, int G>
__global__ __launch_bounds__(PAGE_THREADS) void page_score_kernel(const float* __restrict__ q,
                                                                  const unsigned char* __restrict__ kmin,
                                                                  const unsigned char* __restrict__ kmax,
                                                                  const int32_t* __restrict__ seq_lens,
                                                                  float* __restrict__ scores,
                                                                  int32_t* __restrict__ counts, int Hq, int Hkv,
                                                                  int T_cap, int P, int NP) {
  using RC = RowChunks<D, KV>;
  const int u = blockIdx.y, b = u / Hkv, g = u % Hkv;
  const int n_pages = pages_of(seq_lens, b, T_cap, P);
  if (counts != nullptr && g == 0 && blockIdx.x == 0 && threadIdx.x == 0) counts[b] = n_pages;
  const int c = (int)threadIdx.x % RC::tpp;
  const int p0 = blockIdx.x * RC::ppb * PAGE_SCORE_ROUNDS + (int)threadIdx.x / RC::tpp;
  if (p0 >= n_pages) return;
  float qv[G][RC::ept];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((size_t)b * Hq + (size_t)g * G + h) * D + c * RC::ept;
#pragma unroll
    for (int e = 0; e < RC::ept; ++e) qv[h][e] = qh[e];
  }
  const int p_end = min(n_pages, p0 + RC::ppb * PAGE_SCORE_ROUNDS);
  const size_t base = (size_t)u * NP * RC::row_bytes + (size_t)c * 16;
  for (int p = p0; p < p_end; p += RC::ppb) {
    const size_t off = base + (size_t)p * RC::row_bytes;
    float lo[RC::ept], hi[RC::ept];
    widen16<KV>(*reinterpret_cast<const uint4*>(kmin + off), lo);
    widen16<KV>(*reinterpret_cast<const uint4*>(kmax + off), hi);
    float best = 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < RC::ept; ++e) acc += fmaxf(qv[h][e] * lo[e], qv[h][e] * hi[e]);
      acc = group_sum<RC::tpp>(acc);
      best = h == 0 ? acc : fmaxf(best, acc);
    }
    if (c == 0) scores[(size_t)u * NP + p] = best;
  }
}

// One block per unit: the tokens of the n selected pages (ascending page
// indices from the selection, -1 after them), in order, then -1 up to C.  Only
// the sequence's last page can be partial, and it is the last one listed.
__global__ __launch_bounds__(PAGE_THREADS) void page_tokens_kernel(const int32_t* __restrict__ pidx,
                                                                   const int32_t* __restrict__ pn,
                                                                   const int32_t* __restrict__ seq_lens,
                                                                   int32_t* __restrict__ idx,
                                                                   int32_t* __restrict__ n_sel, int Hkv, int T_cap,
                                                                   int P, int K, int C) {
  const int u = blockIdx.x, b = u / Hkv;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int last_page = (T + P - 1) / P - 1;
  const int n = clampi(pn[u], 0, K);
  const int32_t* pages = pidx + (size_t)u * K;
  int total = n * P;
  if (n > 0 && pages[n - 1] == last_page) total -= (last_page + 1) * P - T;
  int32_t* out = idx + (size_t)u * C;
  for (int j = threadIdx.x; j < C; j += PAGE_THREADS) out[j] = j < total ? pages[j / P] * P + j % P : -1;
  if (threadIdx.x == 0) n_sel[u] = total;
}

template <int D, int KV>
hipError_t summary_for(const Shape& s, int P, int NP, const void* k, const int32_t* seq_lens, void* kmin, void* kmax,
                       hipStream_t st) {
  using RC = RowChunks<D, KV>;
  dim3 grid((NP + RC::ppb - 1) / RC::ppb, s.B * s.Hkv);
  hipLaunchKernelGGL((page_summary_kernel<D, KV>), grid, dim3(PAGE_THREADS), 0, st,
                     static_cast<const unsigned char*>(k), seq_lens, static_cast<unsigned char*>(kmin),
                     static_cast<unsigned char*>(kmax), s.Hkv, s.T_cap, P, NP);
  return hipGetLastError();
}

template <int D, int KV, int G>
hipError_t score_for(const Shape& s, int P, int NP, const float* q, const void* kmin, const void* kmax,
                     const int32_t* seq_lens, float* scores, int32_t* counts, hipStream_t st) {
  using RC = RowChunks<D, KV>;
  const int per_block = RC::ppb * PAGE_SCORE_ROUNDS;
  dim3 grid((NP + per_block - 1) / per_block, s.B * s.Hkv);
  hipLaunchKernelGGL((page_score_kernel<D, KV, G>), grid, dim3(PAGE_THREADS), 0, st, q,
                     static_cast<const unsigned char*>(kmin), static_cast<const unsigned char*>(kmax), seq_lens,
                     scores, counts, s.Hq, s.Hkv, s.T_cap, P, NP);
  return hipGetLastError();
}

template <int D, int KV>
hipError_t score_for_g(const Shape& s, int P, int NP, const float* q, const void* kmin, const void* kmax,
                       const int32_t* seq_lens, float* scores, int32_t* counts, hipStream_t st) {
  switch (s.G) {
    case 1: return score_for<D, KV, 1>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st);
    case 2: return score_for<D, KV, 2>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st);
    case 4: return score_for<D, KV, 4>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st);
    default: return score_for<D, KV, 8>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The selection's view of the page rows: one "token" per page, C / P of them kept.
Shape page_shape(const Shape& s, int P) {
  Shape ps = s;
  ps.T_cap = page_count(s.T_cap, P);
  ps.C = s.C / P;
  return ps;
}

struct PageWs {
  float* scores;    // [units][NP]
  int32_t* counts;  // [B] pages per sequence
  int32_t* pidx;    // [units][K] selected pages
  int32_t* pn;      // [units]
  void* sel;        // select_ws_bytes(page_shape, true)
};

PageWs page_carve(const Shape& s, int P, void* ws) {
  const size_t units = (size_t)s.B * s.Hkv, NP = (size_t)page_count(s.T_cap, P), K = (size_t)(s.C / P);
  unsigned char* p = static_cast<unsigned char*>(ws);
  PageWs w;
  w.scores = reinterpret_cast<float*>(p);
  p += align256(units * NP * 4);
  w.counts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)s.B * 4);
  w.pidx = reinterpret_cast<int32_t*>(p);
  p += align256(units * K * 4);
  w.pn = reinterpret_cast<int32_t*>(p);
  p += align256(units * 4);
  w.sel = p;
  return w;
}

}  // namespace

int page_count(int T_cap, int P) { return (T_cap + P - 1) / P; }

hipError_t launch_page_summary(const Shape& s, int P, const void* k, const int32_t* seq_lens, void* kmin, void* kmax,
                               hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int NP = page_count(s.T_cap, P);
  if (s.D == 64)
    return s.kv == 0 ? summary_for<64, 0>(s, P, NP, k, seq_lens, kmin, kmax, st)
                     : summary_for<64, 1>(s, P, NP, k, seq_lens, kmin, kmax, st);
  return s.kv == 0 ? summary_for<128, 0>(s, P, NP, k, seq_lens, kmin, kmax, st)
                   : summary_for<128, 1>(s, P, NP, k, seq_lens, kmin, kmax, st);
}

hipError_t launch_page_scores(const Shape& s, int P, const float* q, const void* kmin, const void* kmax,
                              const int32_t* seq_lens, float* scores, int32_t* counts, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const int NP = page_count(s.T_cap, P);
  if (s.D == 64)
    return s.kv == 0 ? score_for_g<64, 0>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st)
                     : score_for_g<64, 1>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st);
  return s.kv == 0 ? score_for_g<128, 0>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st)
                   : score_for_g<128, 1>(s, P, NP, q, kmin, kmax, seq_lens, scores, counts, st);
}

size_t page_select_ws_bytes(const Shape& s, int P) {
  const size_t units = (size_t)s.B * s.Hkv, NP = (size_t)page_count(s.T_cap, P), K = (size_t)(s.C / P);
  return align256(units * NP * 4) + align256((size_t)s.B * 4) + align256(units * K * 4) + align256(units * 4) +
         align256(select_ws_bytes(page_shape(s, P), true));
}

hipError_t launch_page_select(const Shape& s, int P, const float* q, const void* kmin, const void* kmax,
                              const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const PageWs w = page_carve(s, P, ws);
  hipError_t e = launch_page_scores(s, P, q, kmin, kmax, seq_lens, w.scores, w.counts, st);
  if (e != hipSuccess) return e;
  e = launch_select(page_shape(s, P), w.scores, nullptr, w.counts, w.pidx, w.pn, nullptr, nullptr, w.sel, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(page_tokens_kernel, dim3(s.B * s.Hkv), dim3(PAGE_THREADS), 0, st, w.pidx, w.pn, seq_lens, idx,
                     n_sel, s.Hkv, s.T_cap, P, s.C / P, s.C);
  return hipGetLastError();
}

}  // namespace asp
