// Exact top-C token selection per (sequence, KV head), ties to the lower index,
// output in ascending index order.
//
// Sources: reproduction card, "Key finding" (C = 2k selected tokens per step);
// research-map summary of AsyncSpade, "Key results" (2k selected tokens).
// Readings for cases the pages never mention: NaN ranks as -infinity, -0 ties
// with +0, and the lower index wins a tie.
//
// Scores become order-preserving 32-bit keys (order_key).  The first 11 bits
// of the C_eff-th largest key (the boundary bin) come from a coarse histogram
// of the row: the score launch bins every key while it streams, or, for a
// standalone call, one workgroup per row builds it here.  Two launches follow.
//  * Classify: 8192 keys per 1024-thread workgroup, so a batch of long rows
//    fills every CU.  Each wave owns a region of 512 consecutive keys (eight
//    coalesced loads of 64 keys); a ballot per load gives 64 bits of the
//    region's "above the boundary bin" bitmap directly, and the keys inside
//    the bin are appended to the region's candidate list (low 21 key bits +
//    position in the region).
//  * Finish: one workgroup per row gathers the candidate lists (usually a few
//    percent of the row) in index order, resolves the remaining 21 key bits by
//    two radix digits over them alone, marks the chosen candidates in the
//    bitmap and compacts the bitmap in index order: every output position is
//    a prefix count of set bits.
#include "asp_internal.h"

namespace asp {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int KEYS_PER_LANE = 8;
constexpr int REGION = 64 * KEYS_PER_LANE;  // keys of one wave: one candidate list
constexpr int REGION_WORDS = REGION / 32;   // bitmap words of one region
constexpr int SEG = SEL_WAVES * REGION;     // keys of one classify workgroup
constexpr int NBINS = HIST_BINS;
constexpr int CAND_CAP = 8192;              // candidates staged in LDS by the finish
constexpr int MAX_REGIONS = (1 << 22) / REGION;  // t_cap <= 2^22
constexpr int BM_CHUNK = SEL_THREADS;       // bitmap words compacted per round

int select_regions(int T_cap) { return (T_cap + REGION - 1) / REGION; }

namespace {
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

// Workspace of one selection, carved from one allocation (256-byte aligned parts).
struct SelectWs {
  uint32_t* hist;    // [units][NBINS] (standalone calls only)
  uint32_t* meta;    // [units][2]: boundary bin d0, keys still needed from it
  uint32_t* counts;  // [units][regions]: candidates per region
  uint32_t* bitmap;  // [units][regions * REGION_WORDS]: keys above the bin
  uint32_t* cand;    // [units][regions * REGION]: candidate lists
};

size_t select_ws_bytes(const Shape& s, bool with_hist) {
  const size_t units = (size_t)s.B * s.Hkv, nr = (size_t)select_regions(s.T_cap);
  size_t b = with_hist ? align256(units * NBINS * 4) : 0;
  b += align256(units * 2 * 4);
  b += align256(units * nr * 4);
  b += align256(units * nr * REGION_WORDS * 4);
  b += align256(units * nr * REGION * 4);
  return b;
}

static SelectWs carve(const Shape& s, void* ws, bool with_hist) {
  const size_t units = (size_t)s.B * s.Hkv, nr = (size_t)select_regions(s.T_cap);
  unsigned char* p = static_cast<unsigned char*>(ws);
  SelectWs w;
  w.hist = nullptr;
  if (with_hist) {
    w.hist = reinterpret_cast<uint32_t*>(p);
    p += align256(units * NBINS * 4);
  }
  w.meta = reinterpret_cast<uint32_t*>(p);
  p += align256(units * 2 * 4);
  w.counts = reinterpret_cast<uint32_t*>(p);
  p += align256(units * nr * 4);
  w.bitmap = reinterpret_cast<uint32_t*>(p);
  p += align256(units * nr * REGION_WORDS * 4);
  w.cand = reinterpret_cast<uint32_t*>(p);
  return w;
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

// Exclusive scan over the block; *total receives the sum.  Two barriers.
__device__ __forceinline__ uint32_t block_excl(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_scan(v);
  if (lane == 63) scratch[wave] = incl;
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
  return before + incl - v;
}

__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Boundary bin of a coarse histogram, by one wave: lane l sums bins
// [2048 - 32(l+1), 2048 - 32l); a wave scan of those sums (highest bins first)
// locates the lane whose range crosses `need`, which walks its bins from the
// top.  That lane writes sh[0] = bin and sh[1] = number of keys in higher bins.
__device__ __forceinline__ void coarse_pick(const uint32_t* __restrict__ row_hist, uint32_t need, uint32_t* sh) {
  const int lane = threadIdx.x & 63;
  const uint4* ch = reinterpret_cast<const uint4*>(row_hist + (NBINS - 32 * (lane + 1)));
  uint32_t bins[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 x = ch[q];
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
    uint32_t above = 0u;
#pragma unroll
    for (int q = 31; q >= 0; --q) {  // bins from the highest down
      const uint32_t c = bins[q];
      if (d == 0 && acc + c >= need) {
        d = NBINS - 32 * (lane + 1) + q + 1;  // +1: 0 means "not found yet"
        above = acc;
      }
      acc += c;
    }
    sh[0] = (uint32_t)(d - 1);
    sh[1] = above;
  }
}

// Coarse histogram of whole rows (standalone selection): one workgroup per unit.
__global__ void __launch_bounds__(SEL_THREADS) select_hist_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ seq_lens,
                                                                  uint32_t* __restrict__ hist, int Hkv, int T_cap) {
  __shared__ uint32_t h[NBINS];
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int T = clampi(seq_lens[unit / Hkv], 0, T_cap);
  const float* row = scores + (size_t)unit * T_cap;
  for (int j = tid; j < NBINS; j += SEL_THREADS) h[j] = 0u;
  __syncthreads();
  for (int base = 0; base < T; base += SEL_THREADS * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * SEL_THREADS + tid;
      v[u] = i < T ? row[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u * SEL_THREADS + tid < T) atomicAdd(&h[order_key(v[u]) >> HIST_SHIFT], 1u);
  }
  __syncthreads();
  for (int j = tid; j < NBINS; j += SEL_THREADS) hist[(size_t)unit * NBINS + j] = h[j];
}

// Classify: grid (segments, units).
__global__ void __launch_bounds__(SEL_THREADS) select_classify_kernel(const float* __restrict__ scores,
                                                                      const uint32_t* __restrict__ coarse,
                                                                      const int32_t* __restrict__ seq_lens,
                                                                      SelectWs ws, int Hkv, int T_cap, int C,
                                                                      int n_regions) {
  __shared__ uint32_t sh[2];
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = clampi(seq_lens[unit / Hkv], 0, T_cap);
  const int c_eff = C < T ? C : T;
  if (c_eff == T || seg * SEG >= T) return;  // uniform over the workgroup
  const int wbase = seg * SEG + wave * REGION;
  const float* row = scores + (size_t)unit * T_cap;

  float v[KEYS_PER_LANE];
#pragma unroll
  for (int j = 0; j < KEYS_PER_LANE; ++j) {
    const int p = wbase + 64 * j + lane;
    v[j] = p < T ? row[p] : 0.0f;
  }
  if (tid < 64) coarse_pick(coarse + (size_t)unit * NBINS, (uint32_t)c_eff, sh);
  __syncthreads();
  const uint32_t d0 = sh[0] & 0x7ffu;  // in range even for an inconsistent histogram
  if (seg == 0 && tid == 0) {
    ws.meta[(size_t)unit * 2] = d0;
    ws.meta[(size_t)unit * 2 + 1] = (uint32_t)c_eff - sh[1];
  }
  if (wbase >= T) return;  // a region past the row end is never read

  const size_t region = (size_t)unit * n_regions + wbase / REGION;
  uint32_t* cand = ws.cand + region * REGION;
  uint32_t n = 0u, word = 0u;
#pragma unroll
  for (int j = 0; j < KEYS_PER_LANE; ++j) {
    const int p = wbase + 64 * j + lane;
    const uint32_t key = order_key(v[j]);
    const uint32_t dg = key >> HIST_SHIFT;
    const unsigned long long am = __ballot(p < T && dg > d0);
    const unsigned long long em = __ballot(p < T && dg == d0);
    if (p < T && dg == d0) cand[n + lanes_below(em)] = ((key & 0x1fffffu) << 11) | (uint32_t)(64 * j + lane);
    n += (uint32_t)__popcll(em);
    // Lanes 2j and 2j+1 keep the two halves of this load's bitmap.
    word = lane == 2 * j ? (uint32_t)am : word;
    word = lane == 2 * j + 1 ? (uint32_t)(am >> 32) : word;
  }
  if (lane < REGION_WORDS) ws.bitmap[region * REGION_WORDS + lane] = word;
  if (lane == 0) ws.counts[region] = n;
}

// Finish: one workgroup per unit.
__global__ void __launch_bounds__(SEL_THREADS) select_finish_kernel(const int32_t* __restrict__ seq_lens,
                                                                    SelectWs ws, int32_t* __restrict__ idx,
                                                                    int32_t* __restrict__ n_sel,
                                                                    int32_t* __restrict__ adv_newest,
                                                                    int32_t* __restrict__ adv_len, int Hkv,
                                                                    int T_cap, int C, int W, int n_regions) {
  __shared__ uint32_t woff[MAX_REGIONS + 1];
  __shared__ uint32_t ckey[CAND_CAP];
  __shared__ uint32_t cidx[CAND_CAP];
  __shared__ uint32_t hist[NBINS];
  __shared__ uint32_t bm[BM_CHUNK];
  __shared__ uint32_t scratch[SEL_WAVES];
  __shared__ uint32_t sh[2];

  const int unit = blockIdx.x, b = unit / Hkv, tid = threadIdx.x;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int c_eff = C < T ? C : T;
  int32_t* out = idx + (size_t)unit * C;

  // Ring advance of a step run on one stream: the predictor launch of the same
  // step has read newest/len for every head and written the new query one slot
  // ahead.
  if (adv_newest != nullptr && unit % Hkv == 0 && tid == 0) ring_advance(adv_newest, adv_len, b, W);
  for (int j = c_eff + tid; j < C; j += SEL_THREADS) out[j] = -1;
  if (tid == 0) n_sel[unit] = c_eff;
  if (c_eff == T) {  // everything is selected (includes the empty row)
    for (int j = tid; j < T; j += SEL_THREADS) out[j] = j;
    return;
  }

  const int nreg = (T + REGION - 1) / REGION;
  const int nwords = (T + 31) / 32;
  const uint32_t* counts = ws.counts + (size_t)unit * n_regions;
  const uint32_t* bitmap = ws.bitmap + (size_t)unit * n_regions * REGION_WORDS;
  const uint32_t* cand = ws.cand + (size_t)unit * n_regions * REGION;
  // Independent loads first: the first bitmap chunk and the boundary digit.
  const uint32_t bw0 = tid < nwords ? bitmap[tid] : 0u;
  const uint32_t d0 = ws.meta[(size_t)unit * 2] & 0x7ffu;
  const uint32_t need0 = ws.meta[(size_t)unit * 2 + 1];

  // Region offsets in the concatenated (index-ordered) candidate list: thread
  // t owns regions [t*m, t*m + m).
  const int m = (nreg + SEL_THREADS - 1) / SEL_THREADS;
  const int r0 = min(tid * m, nreg), r1 = min(r0 + m, nreg);
  uint32_t local = 0u;
  for (int r = r0; r < r1; ++r) {
    const uint32_t c = min(counts[r], (uint32_t)REGION);  // a region holds at most REGION candidates
    woff[r] = local;
    local += c;
  }
  uint32_t n_cand;
  const uint32_t before = block_excl(local, scratch, &n_cand);
  for (int r = r0; r < r1; ++r) woff[r] += before;
  __syncthreads();

  // Candidate p of the list: its region is the last one starting at or before p
  // (regions that start exactly at p and are empty come before it).
  auto fetch = [&](uint32_t p, uint32_t& key, uint32_t& pos) {
    int lo = 0, hi = nreg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (woff[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const uint32_t e = cand[(size_t)lo * REGION + (p - woff[lo])];
    key = (d0 << HIST_SHIFT) | (e >> 11);
    pos = (uint32_t)lo * REGION + (e & 0x7ffu);
  };
  const bool staged = n_cand <= (uint32_t)CAND_CAP;
  if (staged) {
    for (uint32_t p = tid; p < n_cand; p += SEL_THREADS) {
      uint32_t key, pos;
      fetch(p, key, pos);
      ckey[p] = key;
      cidx[p] = pos;
    }
    __syncthreads();
  }
  auto get = [&](uint32_t p, uint32_t& key, uint32_t& pos) {
    if (staged) {
      key = ckey[p];
      pos = cidx[p];
    } else {
      fetch(p, key, pos);
    }
  };

  // Remaining two digits of the C_eff-th key over the candidates.
  uint32_t prefix = d0 << HIST_SHIFT, pmask = 0x7ffu << HIST_SHIFT, need = need0;
  bool done = n_cand == need;
  const int shifts[2] = {10, 0};
  const uint32_t dmasks[2] = {0x7ffu, 0x3ffu};
  for (int pass = 0; pass < 2 && !done; ++pass) {
    for (int j = tid; j < NBINS; j += SEL_THREADS) hist[j] = 0u;
    __syncthreads();
    const int s = shifts[pass];
    const uint32_t dm = dmasks[pass];
    for (uint32_t p = tid; p < n_cand; p += SEL_THREADS) {
      uint32_t key, pos;
      get(p, key, pos);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> s) & dm], 1u);
    }
    __syncthreads();
    // Digit d with (#keys above d) < need <= (#keys at or above d): thread t
    // owns bins 2047-2t and 2046-2t, so a prefix over threads is a suffix over bins.
    const int hb = NBINS - 1 - 2 * tid, lb = hb - 1;
    const uint32_t chi = hist[hb], clo = hist[lb];
    uint32_t tot;
    const uint32_t ex = block_excl(chi + clo, scratch, &tot);
    if (ex < need && need <= ex + chi) {
      sh[0] = (uint32_t)hb;
      sh[1] = ex;
    } else if (ex + chi < need && need <= ex + chi + clo) {
      sh[0] = (uint32_t)lb;
      sh[1] = ex + chi;
    }
    __syncthreads();
    const uint32_t d = sh[0] & dm;
    need -= sh[1];
    prefix |= d << s;
    pmask |= dm << s;
    done = hist[d] == need;
    __syncthreads();
  }

  // Candidates in list order: above the prefix, or equal to it and among the
  // first `need` such.  Thread t owns items [t*mc, t*mc + mc).
  const uint32_t mc = (n_cand + SEL_THREADS - 1) / SEL_THREADS;
  const uint32_t i0 = min((uint32_t)tid * mc, n_cand), i1 = min(i0 + mc, n_cand);
  uint32_t eq_local = 0u;
  for (uint32_t p = i0; p < i1; ++p) {
    uint32_t key, pos;
    get(p, key, pos);
    eq_local += (key & pmask) == prefix ? 1u : 0u;
  }
  uint32_t eq_total;
  const uint32_t eq_before = block_excl(eq_local, scratch, &eq_total);

  // Compaction of the bitmap, BM_CHUNK words (32 keys each) per round.
  uint32_t written = 0u;
  for (int w0 = 0; w0 < nwords; w0 += BM_CHUNK) {
    const int wi = w0 + tid;
    bm[tid] = w0 == 0 ? bw0 : (wi < nwords ? bitmap[wi] : 0u);
    __syncthreads();
    uint32_t eb = eq_before;
    for (uint32_t p = i0; p < i1; ++p) {
      uint32_t key, pos;
      get(p, key, pos);
      const uint32_t mk = key & pmask;
      bool take = mk > prefix;
      if (mk == prefix) take = eb++ < need;
      const int wd = (int)(pos >> 5) - w0;
      if (take && wd >= 0 && wd < BM_CHUNK) atomicOr(&bm[wd], 1u << (pos & 31u));
    }
    __syncthreads();
    uint32_t wv = bm[tid];
    uint32_t tot;
    uint32_t at = written + block_excl((uint32_t)__popc(wv), scratch, &tot);
    while (wv != 0u) {
      const int bit = __ffs((int)wv) - 1;
      wv &= wv - 1u;
      if (at < (uint32_t)c_eff) out[at] = (w0 + tid) * 32 + bit;
      ++at;
    }
    written += tot;
  }
}

hipError_t launch_select(const Shape& s, const float* scores, const uint32_t* hist, const int32_t* seq_lens,
                         int32_t* idx, int32_t* n_sel, int32_t* adv_newest, int32_t* adv_len, void* ws,
                         hipStream_t st, hipEvent_t done) {
  if (s.B == 0) return done ? hipEventRecord(done, st) : hipSuccess;
  const int units = s.B * s.Hkv, nr = select_regions(s.T_cap);
  SelectWs w = carve(s, ws, hist == nullptr);
  if (hist == nullptr) {
    hipLaunchKernelGGL(select_hist_kernel, dim3(units), dim3(SEL_THREADS), 0, st, scores, seq_lens, w.hist, s.Hkv,
                       s.T_cap);
    hist = w.hist;
  }
  const int segs = (s.T_cap + SEG - 1) / SEG;
  hipLaunchKernelGGL(select_classify_kernel, dim3(segs, units), dim3(SEL_THREADS), 0, st, scores, hist, seq_lens, w,
                     s.Hkv, s.T_cap, s.C, nr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_recording(select_finish_kernel, dim3(units), dim3(SEL_THREADS), st, done, seq_lens, w, idx, n_sel,
                          adv_newest, adv_len, s.Hkv, s.T_cap, s.C, s.W > 0 ? s.W : 1, nr);
}

}  // namespace asp
