// Exact top-C token selection per (sequence, KV head), ties to the lower index,
// output in ascending index order.
//
// Sources: reproduction card, "Key finding" (C = 2k selected tokens per step);
// research-map summary of AsyncSpade, "Key results" (2k selected tokens).
// Readings for cases the pages never mention: NaN ranks as -infinity, -0 ties
// with +0, and the lower index wins a tie.
//
// One 1024-thread workgroup per unit.  Scores become order-preserving 32-bit
// keys; an MSD radix select (digits of 11, 11 and 10 bits) finds the exact
// C_eff-th key tau and how many keys equal to tau are still needed; an ordered
// compaction then writes every key above tau and the first needed keys equal
// to tau, in index order.
//  * The first digit's histogram comes from the score launch when given (it
//    was binned while the keys streamed), so the boundary bin is known before
//    the row is read; while the row is staged in LDS, the keys of that bin
//    (their number is the bin count) are copied to a short candidate list and
//    the remaining digits are resolved on that list alone.
//  * Rows up to 32768 keys stay in LDS for every pass; longer rows are read
//    from L2 on each pass and staged through LDS in 32768-key chunks for the
//    compaction.
//  * Compaction: each thread owns a contiguous segment (at most 32 keys, kept
//    in registers), one block-wide scan per chunk gives every thread its
//    output offset.
#include "asp_internal.h"

namespace asp {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int KEYBUF = 32768;                   // keys staged in LDS
constexpr int KEYBUF_PADDED = KEYBUF + KEYBUF / 32;
constexpr int SEG_MAX = KEYBUF / SEL_THREADS;   // keys per thread in a compaction chunk
constexpr int CAND_MAX = 3072;                  // boundary-bin candidates kept in LDS
constexpr int NBINS = HIST_BINS;
constexpr int LOAD_BATCH = 8;                   // global loads in flight per thread

// One padding word every 32 keys keeps a thread's contiguous segment on
// distinct LDS banks from its neighbours' segments.
__device__ __forceinline__ int padded(int i) { return i + (i >> 5); }

// Wave-aggregated append to the candidate list: one LDS atomic per wave.  A
// count beyond CAND_MAX (only possible with an inconsistent coarse histogram)
// is detected after the sweep.  Must be reached by every lane of the wave.
__device__ __forceinline__ void push_cand(uint32_t* cand, uint32_t* n_cand, bool pred, uint32_t key) {
  const unsigned long long mask = __ballot(pred);
  if (mask == 0ull) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n_cand, (uint32_t)__popcll(mask));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  if (pred) {
    const uint32_t p = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (p < (uint32_t)CAND_MAX) cand[p] = key;
  }
}

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

// Inclusive scan over the 1024 threads of the block; *total receives the sum.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan(v);
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

// Exclusive prefix over the block of a value whose two 16-bit halves are each
// at most 32 per thread (the compaction's per-thread counts): every bit plane
// is a ballot, so no cross-lane data movement is needed inside a wave.
__device__ __forceinline__ uint32_t block_excl_small(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t ex = 0u, wt = 0u;
#pragma unroll
  for (int half = 0; half < 32; half += 16) {
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const unsigned long long m = __ballot((v >> (half + b)) & 1u);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      ex += below << (half + b);
      wt += (uint32_t)__popcll(m) << (half + b);
    }
  }
  if (lane == 0) scratch[wave] = wt;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t x = scratch[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return ex + before;
}

// Given hist[] filled for the current digit, find the digit d with
// (#keys with digit > d) < need <= (#keys with digit >= d); narrow
// prefix/pmask and need.  Returns true when every key of bin d is taken.
__device__ __forceinline__ bool pick_digit(const uint32_t* hist, uint32_t* scratch, uint32_t* sh, int shift,
                                           uint32_t dmask, uint32_t& prefix, uint32_t& pmask, uint32_t& need) {
  const int tid = threadIdx.x;
  // Thread t owns bins 2047-2t and 2046-2t: a prefix scan over threads is a
  // suffix scan over bins.
  const int hi = NBINS - 1 - 2 * tid, lo = hi - 1;
  const uint32_t chi = hist[hi], clo = hist[lo];
  uint32_t total;
  const uint32_t incl = block_scan(chi + clo, scratch, &total);
  const uint32_t excl = incl - chi - clo;
  if (excl < need && need <= excl + chi) {
    sh[0] = (uint32_t)hi;
    sh[1] = excl;
  } else if (excl + chi < need && need <= incl) {
    sh[0] = (uint32_t)lo;
    sh[1] = excl + chi;
  }
  __syncthreads();
  const uint32_t d = sh[0];
  need -= sh[1];
  prefix |= d << shift;
  pmask |= dmask << shift;
  const bool whole = hist[d] == need;
  __syncthreads();
  return whole;
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
  __shared__ uint32_t cand[CAND_MAX];
  __shared__ uint32_t scratch[SEL_WAVES];
  __shared__ uint32_t sh[2];
  __shared__ uint32_t n_cand;

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

  // After each digit: `prefix` holds the key bits fixed so far (under
  // `pmask`), `need` how many keys equal to the prefix must still be taken.
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)c_eff;
  bool done = false;       // every key equal to the prefix is taken
  bool have_d0 = false;    // first digit resolved
  bool collect = false;    // the candidate list holds every key matching the prefix
  if (tid == 0) n_cand = 0;

  // Resident rows: issue every load of the row first (16-byte loads when the
  // row is 16-byte aligned), so that the coarse pick below runs while they fly.
  // (T_cap % 4 == 0 keeps the rounded-up float4 count inside every row.)
  const bool vec4 = resident && (T_cap & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0u;
  constexpr int V4 = KEYBUF / 4 / SEL_THREADS;  // float4 per thread for a full row
  float4 rv[V4];
  if (vec4) {
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const int nf = (T + 3) / 4;  // 4 * nf <= T_cap
#pragma unroll
    for (int u = 0; u < V4; ++u) {
      const int f = u * SEL_THREADS + tid;
      rv[u] = f < nf ? row4[f] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }

  if (coarse != nullptr) {
    // First digit from the score launch's histogram, resolved by wave 0 alone:
    // lane l sums bins [2048 - 32(l+1), 2048 - 32l); a wave scan of those sums
    // (highest bins first) locates the lane whose range crosses `need`, which
    // then walks its bins from the top.
    if (tid < 64) {
      const uint32_t* ch = coarse + (size_t)unit * NBINS + (NBINS - 32 * (tid + 1));
      uint32_t bins[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 x = reinterpret_cast<const uint4*>(ch)[q];
        bins[4 * q] = x.x;
        bins[4 * q + 1] = x.y;
        bins[4 * q + 2] = x.z;
        bins[4 * q + 3] = x.w;
      }
      uint32_t lsum = 0u;
#pragma unroll
      for (int q = 0; q < 32; ++q) lsum += bins[q];
      const uint32_t incl = wave_scan(lsum);
      const uint32_t excl = incl - lsum;
      if (excl < need && need <= incl) {
        uint32_t acc = excl;
        int d = 0;
        uint32_t above = 0u, cnt = 0u;
#pragma unroll
        for (int q = 31; q >= 0; --q) {  // bins from the highest down
          const uint32_t c = bins[q];
          if (d == 0 && acc + c >= need) {
            d = NBINS - 32 * (tid + 1) + q + 1;  // +1: 0 means "not found yet"
            above = acc;
            cnt = c;
          }
          acc += c;
        }
        sh[0] = (uint32_t)(d - 1);
        sh[1] = above;
        hist[0] = cnt;  // count of the boundary bin
      }
    }
    __syncthreads();
    const uint32_t d0 = sh[0];
    need -= sh[1];
    prefix = d0 << 21;
    pmask = 0x7ffu << 21;
    const uint32_t bin_count = hist[0];
    done = bin_count == need;
    have_d0 = true;
    __syncthreads();
    // A candidate list pays off only for rows that stay in global memory; a
    // resident row is refined straight from registers / LDS.
    collect = !resident && !done && bin_count <= (uint32_t)CAND_MAX;
  }

  if (vec4) {
#pragma unroll
    for (int u = 0; u < V4; ++u) {
      const int i0 = 4 * (u * SEL_THREADS + tid);
      const float vals[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const uint32_t key = order_key(vals[e]);
        if (i < T) keys[padded(i)] = key;
        if (collect) push_cand(cand, &n_cand, i < T && (key & pmask) == prefix, key);
      }
    }
  } else if (resident) {
    for (int base = 0; base < T; base += SEL_THREADS * LOAD_BATCH) {
      float v[LOAD_BATCH];
#pragma unroll
      for (int u = 0; u < LOAD_BATCH; ++u) {
        const int i = base + u * SEL_THREADS + tid;
        v[u] = i < T ? row[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < LOAD_BATCH; ++u) {
        const int i = base + u * SEL_THREADS + tid;
        const uint32_t key = order_key(v[u]);
        if (i < T) keys[padded(i)] = key;
        if (collect) push_cand(cand, &n_cand, i < T && (key & pmask) == prefix, key);
      }
    }
  } else if (collect) {
    for (int base = 0; base < T; base += SEL_THREADS * LOAD_BATCH) {
      float v[LOAD_BATCH];
#pragma unroll
      for (int u = 0; u < LOAD_BATCH; ++u) {
        const int i = base + u * SEL_THREADS + tid;
        v[u] = i < T ? row[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < LOAD_BATCH; ++u) {
        const int i = base + u * SEL_THREADS + tid;
        const uint32_t key = order_key(v[u]);
        push_cand(cand, &n_cand, i < T && (key & pmask) == prefix, key);
      }
    }
  }
  __syncthreads();

  if (collect && n_cand > (uint32_t)CAND_MAX) collect = false;
  // Remaining digits: histogram over the candidate list when it holds exactly
  // the keys matching the prefix, else over the whole row.
  const int shifts[3] = {21, 10, 0};
  const uint32_t dmask[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  for (int pass = have_d0 ? 1 : 0; pass < 3 && !done; ++pass) {
    for (int j = tid; j < NBINS; j += SEL_THREADS) hist[j] = 0;
    __syncthreads();
    const int s = shifts[pass];
    const uint32_t dm = dmask[pass];
    if (collect) {
      const int nc = (int)n_cand;
      for (int i = tid; i < nc; i += SEL_THREADS) {
        const uint32_t key = cand[i];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> s) & dm], 1u);
      }
    } else if (vec4) {  // the row is still in registers
#pragma unroll
      for (int u = 0; u < V4; ++u) {
        const int i0 = 4 * (u * SEL_THREADS + tid);
        const float vals[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = order_key(vals[e]);
          if (i0 + e < T && (key & pmask) == prefix) atomicAdd(&hist[(key >> s) & dm], 1u);
        }
      }
    } else if (resident) {
      for (int base = 0; base < T; base += SEL_THREADS * LOAD_BATCH) {
        uint32_t kv[LOAD_BATCH];
#pragma unroll
        for (int u = 0; u < LOAD_BATCH; ++u) {
          const int i = base + u * SEL_THREADS + tid;
          kv[u] = i < T ? keys[padded(i)] : 0u;
        }
#pragma unroll
        for (int u = 0; u < LOAD_BATCH; ++u) {
          const int i = base + u * SEL_THREADS + tid;
          if (i < T && (kv[u] & pmask) == prefix) atomicAdd(&hist[(kv[u] >> s) & dm], 1u);
        }
      }
    } else {
      for (int base = 0; base < T; base += SEL_THREADS * LOAD_BATCH) {
        float v[LOAD_BATCH];
#pragma unroll
        for (int u = 0; u < LOAD_BATCH; ++u) {
          const int i = base + u * SEL_THREADS + tid;
          v[u] = i < T ? row[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < LOAD_BATCH; ++u) {
          const int i = base + u * SEL_THREADS + tid;
          const uint32_t key = order_key(v[u]);
          if (i < T && (key & pmask) == prefix) atomicAdd(&hist[(key >> s) & dm], 1u);
        }
      }
    }
    __syncthreads();
    done = pick_digit(hist, scratch, sh, s, dm, prefix, pmask, need);
    if (pass == 0) {
      // Standalone call: the first digit was just found; the refinement can
      // still run on candidates, gathered by one more sweep.
      collect = !resident && !done && hist[prefix >> 21] <= (uint32_t)CAND_MAX;
      if (collect) {
        if (tid == 0) n_cand = 0;
        __syncthreads();
        for (int base = 0; base < T; base += SEL_THREADS * LOAD_BATCH) {
          uint32_t kv[LOAD_BATCH];
#pragma unroll
          for (int u = 0; u < LOAD_BATCH; ++u) {
            const int i = base + u * SEL_THREADS + tid;
            kv[u] = i < T ? (resident ? keys[padded(i)] : order_key(row[i])) : 0u;
          }
#pragma unroll
          for (int u = 0; u < LOAD_BATCH; ++u) {
            const int i = base + u * SEL_THREADS + tid;
            push_cand(cand, &n_cand, i < T && (kv[u] & pmask) == prefix, kv[u]);
          }
        }
        __syncthreads();
        if (n_cand > (uint32_t)CAND_MAX) collect = false;
      }
    }
  }

  // Ordered compaction, one chunk of up to KEYBUF keys at a time.
  uint32_t written = 0, eq_seen = 0;
  for (int c0 = 0; c0 < T; c0 += KEYBUF) {
    const int n = min(KEYBUF, T - c0);
    if (!resident) {
      __syncthreads();
      for (int base = 0; base < n; base += SEL_THREADS * LOAD_BATCH) {
        float v[LOAD_BATCH];
#pragma unroll
        for (int u = 0; u < LOAD_BATCH; ++u) {
          const int i = base + u * SEL_THREADS + tid;
          v[u] = i < n ? row[c0 + i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < LOAD_BATCH; ++u) {
          const int i = base + u * SEL_THREADS + tid;
          if (i < n) keys[padded(i)] = order_key(v[u]);
        }
      }
    }
    __syncthreads();
    const int seg = (n + SEL_THREADS - 1) / SEL_THREADS;  // <= SEG_MAX
    const int s0 = min(tid * seg, n), len = min(s0 + seg, n) - s0;
    // Bit i of gtm / eqm: key s0+i of this thread's segment is above / equal
    // to the prefix.
    uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
    for (int i = 0; i < SEG_MAX; ++i) {
      const uint32_t kv = i < len ? keys[padded(s0 + i)] & pmask : 0u;
      gtm |= (i < len && kv > prefix) ? (1u << i) : 0u;
      eqm |= (i < len && kv == prefix) ? (1u << i) : 0u;
    }
    const uint32_t gt = (uint32_t)__popc(gtm), eq = (uint32_t)__popc(eqm);
    // Counts per chunk are at most 32768, so both fit a 16-bit half.
    uint32_t tot;
    const uint32_t excl = block_excl_small((gt << 16) | eq, scratch, &tot);
    const uint32_t gt_before = excl >> 16, eq_before = excl & 0xffffu;
    const uint32_t gt_tot = tot >> 16, eq_tot = tot & 0xffffu;
    // Keys equal to the prefix are taken in index order until `need` are taken:
    // this thread takes the lowest `take` bits of eqm.  Both counts are formed
    // as differences of clamped prefix sums (no conditional subtraction: a
    // select around `need - before_eq` was once folded into a wrong pos).
    const uint32_t before_eq = eq_seen + eq_before;
    const uint32_t taken_before = min(before_eq, need);
    uint32_t take = min(before_eq + eq, need) - taken_before;
    uint32_t selm = gtm;
    for (uint32_t m = eqm; take > 0u; --take) {
      const uint32_t low = m & (0u - m);
      selm |= low;
      m ^= low;
    }
    // pos < c_eff always holds when the counts are right; the test keeps a
    // miscount from ever writing past the row.
    uint32_t pos = written + gt_before + (taken_before - min(eq_seen, need));
    while (selm != 0u) {
      const int i = __ffs((int)selm) - 1;
      selm &= selm - 1u;
      if (pos < (uint32_t)c_eff) out[pos] = c0 + s0 + i;
      ++pos;
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
