// Overlap of two token selections per unit: the number of token indices that
// both selections contain.  The diagnostic behind the temporal-locality and
// prediction-recall measurements (reproduction card, "What reproduces":
// overlap of the top-k sets inside a recent 16-query window, and the share of
// the true next-step top-k that the ridge-predicted query recovers).
//
// One 1024-thread workgroup per unit: selection A (ascending, as written by
// the select launches) is staged in LDS, and every valid entry of B is looked
// up by binary search; a block reduction sums the hits.
#include "asp_internal.h"

namespace asp {

constexpr int OVL_THREADS = 1024;
constexpr int OVL_MAX_C = 32768;  // selection A staged in LDS (128 KiB)

__global__ void __launch_bounds__(OVL_THREADS) overlap_kernel(const int32_t* __restrict__ idx_a,
                                                              const int32_t* __restrict__ n_a,
                                                              const int32_t* __restrict__ idx_b,
                                                              const int32_t* __restrict__ n_b,
                                                              int32_t* __restrict__ out, int C, int T_cap) {
  __shared__ int32_t sa[OVL_MAX_C];
  __shared__ uint32_t part[OVL_THREADS / 64];
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int na = clampi(n_a[unit], 0, C), nb = clampi(n_b[unit], 0, C);
  const int32_t* a = idx_a + (size_t)unit * C;
  const int32_t* bl = idx_b + (size_t)unit * C;
  for (int i = tid; i < na; i += OVL_THREADS) sa[i] = a[i];
  __syncthreads();
  uint32_t hits = 0u;
  for (int j = tid; j < nb; j += OVL_THREADS) {
    const int32_t x = bl[j];
    if (x < 0 || x >= T_cap) continue;
    int lo = 0, hi = na;  // first position with sa[pos] >= x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sa[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    hits += (lo < na && sa[lo] == x) ? 1u : 0u;
  }
  // Block sum: a butterfly over the wave, then the 16 wave sums.
  uint32_t v = hits;
  v += (uint32_t)__shfl_xor((int)v, 1);
  v += (uint32_t)__shfl_xor((int)v, 2);
  v += (uint32_t)__shfl_xor((int)v, 4);
  v += (uint32_t)__shfl_xor((int)v, 8);
  v += (uint32_t)__shfl_xor((int)v, 16);
  v += (uint32_t)__shfl_xor((int)v, 32);
  if ((tid & 63) == 0) part[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) {
    uint32_t s = 0u;
    for (int w = 0; w < OVL_THREADS / 64; ++w) s += part[w];
    out[unit] = (int32_t)s;
  }
}

int overlap_max_c() { return OVL_MAX_C; }

hipError_t launch_overlap(const Shape& s, const int32_t* idx_a, const int32_t* n_a, const int32_t* idx_b,
                          const int32_t* n_b, int32_t* out, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  if (s.C > OVL_MAX_C) return hipErrorInvalidValue;
  hipLaunchKernelGGL(overlap_kernel, dim3(s.B * s.Hkv), dim3(OVL_THREADS), 0, st, idx_a, n_a, idx_b, n_b, out, s.C,
                     s.T_cap);
  return hipGetLastError();
}

}  // namespace asp
