// Block-wide scans and radix-digit picks shared by the selection kernels
// (select.hip, page.hip).  Device code only.
#pragma once

#include "asp_internal.h"

namespace asp {

// Inclusive scan over the 64 lanes of a wavefront with DPP: Hillis-Steele
// inside each 16-lane row (row_shr 1, 2, 4, 8; lanes shifted in from outside
// the row read 0), then the row totals are carried with row_bcast:15 (into
// rows 1 and 3) and row_bcast:31 (into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false); // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false); // row_bcast:31
  return x;
}

// Exclusive scan over a workgroup of NT threads; *total receives the sum.  Two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_n(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_scan(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = scratch[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// Digit of a 2048-bin histogram that holds the need-th key from the top, by NT
// threads: thread t owns the bins [2048 - PB(t+1), 2048 - PB t) (PB = 2048 / NT)
// and walks them from the highest.  For rank need_a, sh[0] = digit and sh[1] =
// the keys in higher bins; for need_b (0: none), sh[2] and sh[3].  A rank past
// the histogram's total leaves its slots as they were.  Barriers: those of
// block_excl_n.
template <int NT>
__device__ __forceinline__ void pick_digits(const uint32_t* hist, uint32_t need_a, uint32_t need_b,
                                            uint32_t* scratch, uint32_t* sh) {
  constexpr int PB = HIST_BINS / NT;
  const int top = HIST_BINS - 1 - PB * (int)threadIdx.x;
  uint32_t c[PB], sum = 0u;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    c[j] = hist[top - j];
    sum += c[j];
  }
  uint32_t tot;
  uint32_t acc = block_excl_n<NT>(sum, scratch, &tot);
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    if (acc < need_a && need_a <= acc + c[j]) {
      sh[0] = (uint32_t)(top - j);
      sh[1] = acc;
    }
    if (acc < need_b && need_b <= acc + c[j]) {
      sh[2] = (uint32_t)(top - j);
      sh[3] = acc;
    }
    acc += c[j];
  }
}

}  // namespace asp
