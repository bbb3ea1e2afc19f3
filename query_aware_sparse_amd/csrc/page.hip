// Page-level selection, the baseline the pages compare AsyncSpade against
// (research-map summary, "Problem" and the baselines of "Experimental setup";
// arXiv abstract: Quest, which selects whole pages of the KV cache with the
// current query).  The page
// score is Quest's published criticality estimate (Tang et al., ICML 2024,
// method section): every page of P consecutive tokens keeps the element-wise
// minimum and maximum of its keys, and a query q scores the page with
// sum_d max(q_d * min_d, q_d * max_d), the largest q . k over that box.  For
// grouped-query attention a KV head takes the largest bound of its query heads,
// as its token scores take the largest dot product.
//
// Launches:
//  - page_summary_kernel: one pass over K writing kmin/kmax rows in the KV
//    dtype (exact copies of key elements), once per cache;
//  - page_score_kernel: one pass over the summaries, a page score row per unit
//    (f32), plus the page count of every sequence;
//  - page_topk_kernel: one workgroup per unit keeps the top C / P pages and
//    writes their tokens in ascending order, as asp_sparse_decode reads them;
//    rows of more than PAGE_TOPK_MAX pages take the token-level selection
//    (select.hip) on the page rows instead, then page_tokens_kernel.
//
// The larger of q_d * min_d and q_d * max_d is q_d * max_d when q_d >= 0 and
// q_d * min_d otherwise, so each term is one select and one fused multiply-add.
//
// Thread layout of the two streaming kernels: a page row of D elements is read
// as 16-byte chunks, TPP = D * esize / 16 consecutive lanes per row (8, 16 or
// 32), so a wave reads whole rows and the row-sum of the score is a reduction
// inside a DPP row or a half-wave.
#include "block_scan.h"
#include "page.h"

namespace asp {
namespace {

constexpr int PAGE_THREADS = 256;
constexpr int PAGE_SCORE_ROUNDS = 8;  // page rows per lane group of a score block
constexpr int PAGE_SCORE_BATCH = 2;   // of which loaded before any is reduced
constexpr int PAGE_TOPK_THREADS = 1024;
constexpr int PAGE_TOPK_MAX = 16384;  // pages per unit whose keys one workgroup holds in LDS

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
  // With eight query heads the group's queries sit in LDS and each head's chunk
  // is read there per row (registers for all eight would halve the waves in
  // flight); fewer heads keep theirs in registers.
  constexpr bool Q_LDS = G >= 8;
  __shared__ __align__(16) float q_s[Q_LDS ? G * D : 1];
  if constexpr (Q_LDS) {
    const float* qg = q + ((size_t)b * Hq + (size_t)g * G) * D;
    for (int i = threadIdx.x; i < G * D; i += PAGE_THREADS) q_s[i] = qg[i];
    __syncthreads();
  }
  if (p0 >= n_pages) return;
  float qv[Q_LDS ? 1 : G][RC::ept];
  if constexpr (!Q_LDS) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* qh = q + ((size_t)b * Hq + (size_t)g * G + h) * D + c * RC::ept;
#pragma unroll
      for (int e = 0; e < RC::ept; ++e) qv[h][e] = qh[e];
    }
  }
  const int p_end = min(n_pages, p0 + RC::ppb * PAGE_SCORE_ROUNDS);
  const size_t base = (size_t)u * NP * RC::row_bytes + (size_t)c * 16;
  for (int r0 = 0; r0 < PAGE_SCORE_ROUNDS; r0 += PAGE_SCORE_BATCH) {
    uint4 wlo[PAGE_SCORE_BATCH], whi[PAGE_SCORE_BATCH];  // a batch of rows in flight
#pragma unroll
    for (int j = 0; j < PAGE_SCORE_BATCH; ++j) {
      const int p = p0 + (r0 + j) * RC::ppb;
      wlo[j] = whi[j] = make_uint4(0u, 0u, 0u, 0u);
      if (p < p_end) {
        const size_t off = base + (size_t)p * RC::row_bytes;
        wlo[j] = *reinterpret_cast<const uint4*>(kmin + off);
        whi[j] = *reinterpret_cast<const uint4*>(kmax + off);
      }
    }
#pragma unroll
    for (int j = 0; j < PAGE_SCORE_BATCH; ++j) {
      const int p = p0 + (r0 + j) * RC::ppb;
      if (p >= p_end) break;  // the same for the whole lane group
      float lo[RC::ept], hi[RC::ept];
      widen16<KV>(wlo[j], lo);
      widen16<KV>(whi[j], hi);
      float best = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.0f;
        if constexpr (Q_LDS) {
          float qh[RC::ept];
          const float4* src = reinterpret_cast<const float4*>(q_s + h * D + c * RC::ept);
#pragma unroll
          for (int e4 = 0; e4 < RC::ept / 4; ++e4) {
            const float4 x = src[e4];
            qh[4 * e4] = x.x;
            qh[4 * e4 + 1] = x.y;
            qh[4 * e4 + 2] = x.z;
            qh[4 * e4 + 3] = x.w;
          }
#pragma unroll
          for (int e = 0; e < RC::ept; ++e) acc = fmaf(qh[e], qh[e] < 0.0f ? lo[e] : hi[e], acc);
        } else {
#pragma unroll
          for (int e = 0; e < RC::ept; ++e) acc = fmaf(qv[h][e], qv[h][e] < 0.0f ? lo[e] : hi[e], acc);
        }
        acc = group_sum<RC::tpp>(acc);
        best = h == 0 ? acc : fmaxf(best, acc);
      }
      if (c == 0) scores[(size_t)u * NP + p] = best;
    }
  }
}

// One workgroup per unit (n pages <= PAGE_TOPK_MAX): the top K pages of the
// unit's score row, as their tokens in ascending order.  The pages' order keys
// sit in LDS; the K-th key comes from three radix digits (11, 11, 10 bits),
// then two bitmaps (keys above it, keys equal to it) are compacted in page
// order, ties taking the lowest pages.  The chosen pages are listed in LDS,
// and the workgroup then writes their tokens in order.
template <int NT>
__global__ __launch_bounds__(NT) void page_topk_kernel(const float* __restrict__ scores,
                                                       const int32_t* __restrict__ seq_lens,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ n_sel,
                                                       int Hkv, int T_cap, int P, int NP, int K, int C) {
  __shared__ uint32_t key[PAGE_TOPK_MAX];
  __shared__ uint32_t hist[HIST_BINS];
  __shared__ uint32_t bm_gt[PAGE_TOPK_MAX / 32], bm_eq[PAGE_TOPK_MAX / 32];
  __shared__ uint32_t scratch[NT / 64];
  __shared__ uint32_t sh[4];
  __shared__ int last_taken;
  const int u = blockIdx.x, b = u / Hkv, tid = threadIdx.x;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int n = min((T + P - 1) / P, NP);
  const int k_eff = min(K, n);
  int32_t* out = idx + (size_t)u * C;
  if (k_eff == n) {  // every page: the tokens [0, T), T <= K * P = C
    for (int j = tid; j < C; j += NT) out[j] = j < T ? j : -1;
    if (tid == 0) n_sel[u] = T;
    return;
  }
  const float* row = scores + (size_t)u * NP;
  for (int i = tid; i < n; i += NT) key[i] = order_key(row[i]);
  uint32_t prefix = 0u, pmask = 0u, need = (uint32_t)k_eff;
  const int shifts[3] = {HIST_SHIFT, 10, 0};
  const uint32_t dmasks[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  for (int pass = 0; pass < 3; ++pass) {
    for (int j = tid; j < HIST_BINS; j += NT) hist[j] = 0u;
    __syncthreads();
    const int sft = shifts[pass];
    const uint32_t dm = dmasks[pass];
    for (int i = tid; i < n; i += NT) {
      const uint32_t k = key[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> sft) & dm], 1u);
    }
    __syncthreads();
    pick_digits<NT>(hist, need, 0u, scratch, sh);
    __syncthreads();
    const uint32_t d = sh[0] & dm;
    need -= sh[1];
    prefix |= d << sft;
    pmask |= dm << sft;
    const bool done = hist[d] == need;  // every remaining key of this digit is taken
    __syncthreads();
    if (done) break;
  }
  const int nwords = (n + 31) / 32;
  for (int j = tid; j < nwords; j += NT) {
    bm_gt[j] = 0u;
    bm_eq[j] = 0u;
  }
  if (tid == 0) last_taken = 0;
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const uint32_t mk = key[i] & pmask, bit = 1u << (i & 31);
    if (mk > prefix) atomicOr(&bm_gt[i >> 5], bit);
    else if (mk == prefix) atomicOr(&bm_eq[i >> 5], bit);
  }
  __syncthreads();
  // NT bitmap words per round, in page order
  uint32_t written = 0u, eq_seen = 0u;
  for (int w0 = 0; w0 < nwords; w0 += NT) {
    const int wi = w0 + tid;
    uint32_t eqw = wi < nwords ? bm_eq[wi] : 0u;
    const uint32_t gtw = wi < nwords ? bm_gt[wi] : 0u;
    uint32_t eq_tot;
    const uint32_t eb = eq_seen + block_excl_n<NT>((uint32_t)__popc(eqw), scratch, &eq_tot);
    uint32_t take = 0u;  // the lowest set bits of eqw while fewer than `need` ties are taken
    for (uint32_t k = eb; eqw != 0u && k < need; ++k) {
      const uint32_t low = eqw & (0u - eqw);
      take |= low;
      eqw ^= low;
    }
    eq_seen += eq_tot;
    uint32_t wv = gtw | take, tot;
    uint32_t at = written + block_excl_n<NT>((uint32_t)__popc(wv), scratch, &tot);
    if (wi == (n - 1) >> 5 && ((wv >> ((n - 1) & 31)) & 1u)) last_taken = 1;
    while (wv != 0u) {  // the chosen pages in page order, over the keys (no longer read)
      key[at++] = (uint32_t)(wi * 32 + __ffs((int)wv) - 1);
      wv &= wv - 1u;
    }
    written += tot;
  }
  __syncthreads();
  // Token lists, written by the whole workgroup in order (the partial last
  // page, if chosen, is the last listed, so its missing tokens are the tail).
  const int total = k_eff * P - (last_taken ? n * P - T : 0);
  for (int j = tid; j < C; j += NT) out[j] = j < total ? (int)key[j / P] * P + j % P : -1;
  if (tid == 0) n_sel[u] = total;
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
  const int NP = page_count(s.T_cap, P);
  hipError_t e = launch_page_scores(s, P, q, kmin, kmax, seq_lens, w.scores, w.counts, st);
  if (e != hipSuccess) return e;
  if (NP <= PAGE_TOPK_MAX) {
    hipLaunchKernelGGL(page_topk_kernel<PAGE_TOPK_THREADS>, dim3(s.B * s.Hkv), dim3(PAGE_TOPK_THREADS), 0, st,
                       w.scores, seq_lens, idx, n_sel, s.Hkv, s.T_cap, P, NP, s.C / P, s.C);
    return hipGetLastError();
  }
  // Longer rows: the token-level selection on the page rows, then the token lists.
  e = launch_select(page_shape(s, P), w.scores, nullptr, w.counts, w.pidx, w.pn, nullptr, nullptr, w.sel, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(page_tokens_kernel, dim3(s.B * s.Hkv), dim3(PAGE_THREADS), 0, st, w.pidx, w.pn, seq_lens, idx,
                     n_sel, s.Hkv, s.T_cap, P, s.C / P, s.C);
  return hipGetLastError();
}

}  // namespace asp
