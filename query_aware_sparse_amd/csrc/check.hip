// Check of the arguments that live in device memory (sequence lengths, the
// query ring, a selection).  The host validates every other argument before
// anything is enqueued; the kernels clamp these into range, so a bad value
// gives unspecified results but no out-of-bounds access.  This launch tells
// a caller whether its values are the ones the library's own producers leave
// (asp_push_query for the ring, asp_select_topc / asp_step for a selection).
// It reads its inputs only; the values it checks never index memory.
#include "../../include/asp.h"
#include "asp_internal.h"

namespace asp {

constexpr int CHECK_THREADS = 256;

// One workgroup per unit; the workgroups of KV head 0 also check their
// sequence's length and ring.  The violated conditions are OR-ed into *status.
__global__ void __launch_bounds__(CHECK_THREADS) check_kernel(const int32_t* __restrict__ seq_lens,
                                                              const int32_t* __restrict__ hist_newest,
                                                              const int32_t* __restrict__ hist_len,
                                                              const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ n_sel,
                                                              uint32_t* __restrict__ status, int Hkv, int T_cap,
                                                              int C, int W) {
  __shared__ uint32_t block_bad;
  const int unit = blockIdx.x, b = unit / Hkv, g = unit % Hkv, tid = threadIdx.x;
  if (tid == 0) block_bad = 0u;
  __syncthreads();
  uint32_t bad = 0u;
  const int t_raw = seq_lens[b];
  if (g == 0 && tid == 0) {
    if (t_raw < 0 || t_raw > T_cap) bad |= ASP_CHECK_SEQ_LEN;
    if (hist_len != nullptr) {
      const int n = hist_len[b];
      if (n < 0 || n > W) {
        bad |= ASP_CHECK_HIST_LEN;
      } else if (n > 0) {
        const int s = hist_newest[b];
        if (s < 0 || s >= W) bad |= ASP_CHECK_HIST_NEWEST;
      }
    }
  }
  if (idx != nullptr) {
    const int T = clampi(t_raw, 0, T_cap);
    const int n_raw = n_sel[unit];
    if (tid == 0 && (n_raw < 0 || n_raw > min(C, T))) bad |= ASP_CHECK_N_SEL;
    const int n = clampi(n_raw, 0, C);
    const int32_t* row = idx + (size_t)unit * C;
    for (int j = tid; j < C; j += CHECK_THREADS) {
      const int32_t x = row[j];
      if (j < n) {
        if (x < 0 || x >= T || (j + 1 < n && row[j + 1] <= x)) bad |= ASP_CHECK_IDX;
      } else if (x != -1) {
        bad |= ASP_CHECK_IDX_PAD;
      }
    }
  }
  if (bad != 0u) atomicOr(&block_bad, bad);
  __syncthreads();
  if (tid == 0 && block_bad != 0u) atomicOr(status, block_bad);
}

hipError_t launch_check(const Shape& s, const int32_t* seq_lens, const int32_t* hist_newest, const int32_t* hist_len,
                        const int32_t* idx, const int32_t* n_sel, uint32_t* status, hipStream_t st) {
  hipError_t e = launch_clear_u32(status, 1, st);
  const int units = s.B * s.Hkv;
  if (e != hipSuccess || units == 0) return e;
  hipLaunchKernelGGL(check_kernel, dim3(units), dim3(CHECK_THREADS), 0, st, seq_lens, hist_newest, hist_len, idx,
                     n_sel, status, s.Hkv, s.T_cap, s.C, s.W);
  return hipGetLastError();
}

}  // namespace asp
