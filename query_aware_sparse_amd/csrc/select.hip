// Exact top-C token selection per (sequence, KV head), ties to the lower index,
// output in ascending index order.
//
// Sources: reproduction card, "Key finding" (C = 2k selected tokens per step);
// research-map summary of AsyncSpade, "Key results" (2k selected tokens).
// Readings for cases the pages never mention: NaN ranks as -infinity, -0 ties
// with +0, and the lower index wins a tie.
//
// One 1024-thread workgroup per unit.  Scores become order-preserving 32-bit
// keys; an MSD radix select (digits of 11, 11 and 10 bits, histograms in LDS)
// narrows down the exact C_eff-th key tau and how many of the keys equal to
// tau are still needed; a final ordered compaction (per-thread contiguous
// segments plus one block-wide scan per chunk) writes every key above tau and
// the first needed keys equal to tau, in index order.  Up to 32768 keys are
// kept in LDS for every pass; longer rows are read from L2 on each pass and
// staged through LDS in 32768-key chunks for the compaction.
#include "asp_internal.h"

namespace asp {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int KEYBUF = 32768;
constexpr int KEYBUF_PADDED = KEYBUF + KEYBUF / 32;
constexpr int NBINS = HIST_BINS;

// One padding word every 32 keys keeps a thread's contiguous segment on
// distinct LDS banks from its neighbours' segments.
__device__ __forceinline__ int padded(int i) { return i + (i >> 5); }

// Inclusive scan over the 1024 threads of the block; *total receives the sum.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t x = scratch[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + before;
}

__global__ void __launch_bounds__(SEL_THREADS) select_kernel(const float* __restrict__ scores,
                                                             const uint32_t* __restrict__ coarse,
                                                             const int32_t* __restrict__ seq_lens,
                                                             int32_t* __restrict__ idx, int32_t* __restrict__ n_sel,
                                                             int32_t* __restrict__ adv_newest,
                                                             int32_t* __restrict__ adv_len, int Hkv, int T_cap,
                                                             int C, int W) {
  __shared__ uint32_t keys[KEYBUF_PADDED];
  __shared__ uint32_t hist[NBINS];
  __shared__ uint32_t scratch[SEL_WAVES];
  __shared__ uint32_t sh_digit, sh_above;

  const int unit = blockIdx.x;
  const int b = unit / Hkv;
  const int tid = threadIdx.x;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int c_eff = C < T ? C : T;
  int32_t* out = idx + (size_t)unit * C;
  const float* row = scores + (size_t)unit * T_cap;

  // Ring advance of a fused step: the predictor launch of the same step has
  // read newest/len for every head and written the new query one slot ahead.
  if (adv_newest != nullptr && unit % Hkv == 0 && tid == 0) {
    int o = adv_newest[b] % W;
    if (o < 0) o += W;
    adv_newest[b] = o + 1 == W ? 0 : o + 1;
    adv_len[b] = min(clampi(adv_len[b], 0, W) + 1, W);
  }
  for (int j = c_eff + tid; j < C; j += SEL_THREADS) out[j] = -1;
  if (tid == 0) n_sel[unit] = c_eff;
  if (c_eff == T) {  // everything is selected (includes the empty row)
    for (int j = tid; j < T; j += SEL_THREADS) out[j] = j;
    return;
  }

  const bool resident = T <= KEYBUF;
  if (resident) {
    for (int i = tid; i < T; i += SEL_THREADS) keys[padded(i)] = order_key(row[i]);
  }

  // Radix select of the C_eff-th largest key: after each pass, `prefix` holds
  // the key bits fixed so far (under `pmask`) and `need` how many keys equal
  // to the prefix must still be taken.
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)c_eff;
  const int shifts[3] = {21, 10, 0};
  const uint32_t dmask[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dm = dmask[pass];
    if (pass == 0 && coarse != nullptr) {  // first digit already binned by the score launch
      const uint32_t* ch = coarse + (size_t)unit * NBINS;
      for (int j = tid; j < NBINS; j += SEL_THREADS) hist[j] = ch[j];
      __syncthreads();
    } else {
      for (int j = tid; j < NBINS; j += SEL_THREADS) hist[j] = 0;
      __syncthreads();
      for (int i = tid; i < T; i += SEL_THREADS) {
        const uint32_t key = resident ? keys[padded(i)] : order_key(row[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1u);
      }
      __syncthreads();
    }
    // Find digit d with (#keys with digit > d) < need <= (#keys with digit >= d).
    // Thread t owns bins 2047-2t and 2046-2t, so a prefix scan over threads is
    // a suffix scan over bins.
    const int hi = NBINS - 1 - 2 * tid, lo = hi - 1;
    const uint32_t chi = hist[hi], clo = hist[lo];
    uint32_t total;
    const uint32_t incl = block_scan(chi + clo, scratch, &total);
    const uint32_t excl = incl - chi - clo;
    if (excl < need && need <= excl + chi) {
      sh_digit = (uint32_t)hi;
      sh_above = excl;
    } else if (excl + chi < need && need <= incl) {
      sh_digit = (uint32_t)lo;
      sh_above = excl + chi;
    }
    __syncthreads();
    const uint32_t d = sh_digit;
    need -= sh_above;
    prefix |= d << sh;
    pmask |= dm << sh;
    const bool whole_bin = hist[d] == need;  // every key of this bin is taken: stop refining
    __syncthreads();
    if (whole_bin) break;
  }

  // Ordered compaction, one chunk of up to KEYBUF keys at a time.
  uint32_t written = 0, eq_seen = 0;
  for (int c0 = 0; c0 < T; c0 += KEYBUF) {
    const int n = min(KEYBUF, T - c0);
    if (!resident) {
      __syncthreads();
      for (int i = tid; i < n; i += SEL_THREADS) keys[padded(i)] = order_key(row[c0 + i]);
    }
    __syncthreads();
    const int seg = (n + SEL_THREADS - 1) / SEL_THREADS;
    const int s0 = min(tid * seg, n), s1 = min(s0 + seg, n);
    uint32_t gt = 0, eq = 0;
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = keys[padded(i)] & pmask;
      gt += key > prefix;
      eq += key == prefix;
    }
    // Counts per chunk are at most 32768, so both fit a 16-bit half.
    uint32_t tot;
    const uint32_t incl = block_scan((gt << 16) | eq, scratch, &tot);
    const uint32_t excl = incl - ((gt << 16) | eq);
    const uint32_t gt_before = excl >> 16, eq_before = excl & 0xffffu;
    const uint32_t gt_tot = tot >> 16, eq_tot = tot & 0xffffu;
    const uint32_t taken_eq_before = min(eq_seen + eq_before, need) - min(eq_seen, need);
    uint32_t pos = written + gt_before + taken_eq_before;
    uint32_t eq_rank = eq_seen + eq_before;
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = keys[padded(i)] & pmask;
      // pos < c_eff always holds when the counts are right; the test keeps a
      // miscount from ever writing past the row.
      if (key > prefix) {
        if (pos < (uint32_t)c_eff) out[pos] = c0 + i;
        ++pos;
      } else if (key == prefix) {
        if (eq_rank < need) {
          if (pos < (uint32_t)c_eff) out[pos] = c0 + i;
          ++pos;
        }
        ++eq_rank;
      }
    }
    written += gt_tot + (min(eq_seen + eq_tot, need) - min(eq_seen, need));
    eq_seen += eq_tot;
  }
}

hipError_t launch_select(const Shape& s, const float* scores, const uint32_t* hist, const int32_t* seq_lens,
                         int32_t* idx, int32_t* n_sel, int32_t* adv_newest, int32_t* adv_len, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3(s.B * s.Hkv), dim3(SEL_THREADS), 0, st, scores, hist, seq_lens, idx, n_sel,
                     adv_newest, adv_len, s.Hkv, s.T_cap, s.C, s.W > 0 ? s.W : 1);
  return hipGetLastError();
}

}  // namespace asp
