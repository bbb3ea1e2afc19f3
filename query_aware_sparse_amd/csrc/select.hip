// Exact top-C token selection per (sequence, KV head), ties to the lower index,
// output in ascending index order.
//
// Sources: reproduction card, "Key finding" (C = 2k selected tokens per step);
// research-map summary of AsyncSpade, "Key results" (2k selected tokens).
// Readings for cases the pages never mention: NaN ranks as -infinity, -0 ties
// with +0, and the lower index wins a tie.
//
// Scores become order-preserving 32-bit keys (order_key).  Two routes:
//  - from score rows (asp_select_topc), described here;
//  - from the keys a score launch kept above a threshold hint (the step and
//    asp_select_candidates): select_cand_kernel, further below.
// Score-row route.  The first 11 bits of the C_eff-th largest key (the boundary
// bin) come from a coarse histogram of the row: the score launch bins every key
// while it streams, or, for a standalone call, one workgroup per row builds it
// here.  Two launches follow.
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
#include "block_scan.h"

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
constexpr int CAND_BATCH = 8;               // 16-byte candidate loads in flight per thread
static_assert(CAND_REGION % (2 * CAND_BATCH) == 0, "batches stay inside a candidate region");

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

// Selection from candidates (the rows' keys at or above a threshold hint, in
// per-wave regions of CAND_REGION keys, written by the score launch): one
// workgroup of CAND_SEL_THREADS per unit.  The first launch takes every unit: it advances the ring,
// flags a unit whose candidates are fewer than C_eff (its keys are then all
// kept by a rescoring launch) and selects the others; the second launch
// selects the flagged units.  The C_eff-th key comes from three radix digits
// (11, 11, 10 bits) over the candidates; the output is compacted in index
// order through two LDS bitmaps per chunk of the row, one for the keys above
// the C_eff-th key and one for those equal to it, of which the lowest indices
// are taken.  The next hint is the lower edge of the fine bin (top 22 bits of
// the key, two digits) that holds the 1.5 C_eff-th candidate key; when fewer
// than 1.5 C_eff keys were kept, the current hint moves down by the shortfall
// at the density of the kept keys in its coarse bin (at most two coarse bins).
// CAP: candidates staged in LDS (0: none, every pass reads them from memory).
// The LDS a workgroup holds is taken from the concurrent score launches, so
// the first launch sizes CAP to the budget and the second one, which usually
// finds no unit flagged, stages nothing.
constexpr int CAND_SEL_THREADS = 1024;
template <int CAP>
__global__ void __launch_bounds__(CAND_SEL_THREADS) select_cand_kernel(const int32_t* __restrict__ seq_lens,
                                                                       CandWs cw, int32_t* __restrict__ idx,
                                                                       int32_t* __restrict__ n_sel,
                                                                       int32_t* __restrict__ adv_newest,
                                                                       int32_t* __restrict__ adv_len, int Hkv,
                                                                       int T_cap, int C, int W, int first) {
  constexpr int NT = CAND_SEL_THREADS;
  constexpr int CHUNK = NT;  // bitmap words (32 keys each) compacted per round
  __shared__ uint32_t ckey[CAP > 0 ? CAP : 1];
  __shared__ uint32_t cidx[CAP > 0 ? CAP : 1];
  __shared__ uint32_t hist[NBINS];
  __shared__ uint32_t bm_gt[CHUNK];
  __shared__ uint32_t bm_eq[CHUNK];
  __shared__ uint32_t scratch[NT / 64];
  __shared__ uint32_t sh[4];

  const int unit = blockIdx.x, b = unit / Hkv, tid = threadIdx.x;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int c_eff = C < T ? C : T;
  int32_t* out = idx + (size_t)unit * C;

  if (first) {
    if (adv_newest != nullptr && unit % Hkv == 0 && tid == 0) ring_advance(adv_newest, adv_len, b, W);
  } else if (cw.flag[unit] == 0u) {
    return;  // selected by the first launch (uniform over the workgroup)
  }
  if (c_eff == T) {  // everything is selected (includes the empty row)
    for (int j = c_eff + tid; j < C; j += NT) out[j] = -1;
    for (int j = tid; j < T; j += NT) out[j] = j;
    if (tid == 0) {
      n_sel[unit] = c_eff;
      cw.flag[unit] = 0u;
      cw.hint[unit] = 0u;
    }
    return;
  }
  const uint32_t hint_cur = cw.hint[unit];

  // Candidate count; thread t owns the regions [t*m, t*m + m) of the row.
  const int nr = cand_regions(T);
  const size_t rbase = (size_t)unit * cand_regions(T_cap);
  const int m = (nr + NT - 1) / NT;
  const int r0 = min(tid * m, nr), r1 = min(r0 + m, nr);
  uint32_t local = 0u;
  for (int r = r0; r < r1; ++r) local += min(cw.rcount[rbase + r], (uint32_t)CAND_REGION);
  uint32_t n;
  const uint32_t before = block_excl_n<NT>(local, scratch, &n);
  if (first) {
    const bool short_row = n < (uint32_t)c_eff;
    if (tid == 0) cw.flag[unit] = short_row ? 1u : 0u;
    if (short_row) return;  // rescored with every key kept, then selected by the second launch
  }
  for (int j = c_eff + tid; j < C; j += NT) out[j] = -1;
  if (tid == 0) {
    n_sel[unit] = c_eff;
    sh[0] = 0u;
    sh[1] = 0u;
    sh[2] = 0xffffffffu;
    sh[3] = 0u;
  }

  // f(key, index) for the candidates of this thread's regions, read with
  // batches of independent 16-byte loads (two slots each) so that a region's
  // slots arrive in a few round trips rather than one per slot.
  auto for_own = [&](auto&& f) {
    for (int r = r0; r < r1; ++r) {
      const uint32_t c = min(cw.rcount[rbase + r], (uint32_t)CAND_REGION);
      const uint4* e = reinterpret_cast<const uint4*>(cw.cand + (rbase + r) * CAND_REGION);
      for (uint32_t i0 = 0; i0 < c; i0 += 2 * CAND_BATCH) {
        uint4 x[CAND_BATCH];
#pragma unroll
        for (int j = 0; j < CAND_BATCH; ++j)
          x[j] = i0 + 2 * j < c ? e[i0 / 2 + j] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < CAND_BATCH; ++j) {
          if (i0 + 2 * j < c) f(x[j].x, x[j].y);
          if (i0 + 2 * j + 1 < c) f(x[j].z, x[j].w);
        }
      }
    }
  };
  const bool staged = CAP > 0 && n <= (uint32_t)CAP;
  if (staged) {
    uint32_t at = before;
    for_own([&](uint32_t key, uint32_t pos) {
      ckey[at] = key;
      cidx[at] = pos;
      ++at;
    });
  }
  // f(key, index) for every candidate, each visited by one thread.
  auto for_each = [&](auto&& f) {
    if (staged) {
      for (uint32_t p = tid; p < n; p += NT) f(ckey[p], cidx[p]);
    } else {
      for_own(f);
    }
  };

  // The C_eff-th key, digit by digit: after the loop the keys above `prefix`
  // (under pmask) are taken, with `need` more of those equal to it.
  uint32_t prefix = 0u, pmask = 0u, need = (uint32_t)c_eff;
  const uint32_t need2 = 3u * (uint32_t)c_eff / 2u;  // the hint's target: 1.5 C_eff kept keys
  uint32_t hint_next = 0u;
  bool refine_hint = false;  // the need2-th key's coarse bin is known: refine it by one digit
  const int shifts[3] = {HIST_SHIFT, 10, 0};
  const uint32_t dmasks[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  bool done = false;
  for (int pass = 0; pass < 3 && !done; ++pass) {
    for (int j = tid; j < NBINS; j += NT) hist[j] = 0u;
    __syncthreads();
    const int sft = shifts[pass];
    const uint32_t dm = dmasks[pass];
    for_each([&](uint32_t key, uint32_t) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sft) & dm], 1u);
    });
    __syncthreads();
    // pass 0 also locates the coarse bin of the need2-th candidate key
    pick_digits<NT>(hist, need, pass == 0 ? need2 : 0u, scratch, sh);
    __syncthreads();
    const uint32_t d = sh[0] & dm;
    need -= sh[1];
    prefix |= d << sft;
    pmask |= dm << sft;
    if (pass == 0) {
      if (sh[2] != 0xffffffffu) {
        hint_next = (sh[2] & 0x7ffu) << HIST_SHIFT;
        refine_hint = true;
      } else if (first) {
        // Fewer than need2 keys kept: move the hint down by the key range
        // that the shortfall (plus a quarter) would take at the density of
        // the kept keys in the hint's own coarse bin; at most two coarse bins.
        const uint32_t hb_cur = hint_cur >> HIST_SHIFT;
        const uint64_t span = ((uint64_t)(hb_cur + 1u) << HIST_SHIFT) - hint_cur;  // kept part of that bin
        const uint64_t c_lo = hist[hb_cur];
        const uint64_t cap = 2ull << HIST_SHIFT;
        const uint64_t down = c_lo ? min(span * (uint64_t)(need2 - n) * 5u / (4u * c_lo) + 1u, cap) : cap;
        hint_next = (uint32_t)((uint64_t)hint_cur > down ? (uint64_t)hint_cur - down : 0u) & ~0x3ffu;
      }  // else every key was kept and fewer than need2 exist: keep them all
    }
    done = hist[d] == need;
    __syncthreads();
  }

  // The hint's second digit: bits 20..10 of the need2-th candidate key, from
  // the keys of its coarse bin (one more histogram pass over the candidates).
  if (refine_hint) {
    const uint32_t need_h = need2 - sh[3];
    for (int j = tid; j < NBINS; j += NT) hist[j] = 0u;
    __syncthreads();
    for_each([&](uint32_t key, uint32_t) {
      if ((key >> HIST_SHIFT) == (hint_next >> HIST_SHIFT)) atomicAdd(&hist[(key >> 10) & 0x7ffu], 1u);
    });
    __syncthreads();
    pick_digits<NT>(hist, need_h, 0u, scratch, sh);
    __syncthreads();
    hint_next |= (sh[0] & 0x7ffu) << 10;
    __syncthreads();
  }

  // Output in ascending index order, CHUNK words (32 keys each) per round.
  const int nwords = (T + 31) / 32;
  uint32_t written = 0u, eq_seen = 0u;
  for (int w0 = 0; w0 < nwords; w0 += CHUNK) {
    bm_gt[tid] = 0u;
    bm_eq[tid] = 0u;
    __syncthreads();
    for_each([&](uint32_t key, uint32_t pos) {
      const int wd = (int)(pos >> 5) - w0;
      if (wd < 0 || wd >= CHUNK) return;
      const uint32_t mk = key & pmask, bit = 1u << (pos & 31u);
      if (mk > prefix) atomicOr(&bm_gt[wd], bit);
      else if (mk == prefix) atomicOr(&bm_eq[wd], bit);
    });
    __syncthreads();
    uint32_t eqw = bm_eq[tid];
    const uint32_t gtw = bm_gt[tid];
    uint32_t eq_tot;
    const uint32_t eb = eq_seen + block_excl_n<NT>((uint32_t)__popc(eqw), scratch, &eq_tot);
    uint32_t take = 0u;  // the lowest set bits of eqw while fewer than `need` ties are taken
    for (uint32_t k = eb; eqw != 0u && k < need; ++k) {
      const uint32_t low = eqw & (0u - eqw);
      take |= low;
      eqw ^= low;
    }
    eq_seen += eq_tot;
    uint32_t wv = gtw | take;
    uint32_t tot;
    uint32_t at = written + block_excl_n<NT>((uint32_t)__popc(wv), scratch, &tot);
    while (wv != 0u) {
      const int bit = __ffs((int)wv) - 1;
      wv &= wv - 1u;
      if (at < (uint32_t)c_eff) out[at] = (w0 + tid) * 32 + bit;
      ++at;
    }
    written += tot;
  }
  if (tid == 0) cw.hint[unit] = hint_next;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    cached[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cached[dev];
}

hipError_t launch_select_candidates(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                    const CandWs& cw, int32_t* idx, int32_t* n_sel, int32_t* adv_newest,
                                    int32_t* adv_len, hipStream_t st, hipEvent_t done) {
  if (s.B == 0) return done ? hipEventRecord(done, st) : hipSuccess;
  const int units = s.B * s.Hkv, W = s.W > 0 ? s.W : 1;
  // LDS of the first launch.  With few units (at most one workgroup per two
  // CUs) each workgroup takes a CU's whole LDS, which keeps the concurrent
  // score blocks off that CU: measured faster than sharing the CU with them
  // (64 units: 101.6 against 103.3 us per step; 128 units: 209.5 against
  // 210.3 us).  With more units that would take every CU from the score
  // launch (256 units: 240 against 228 us), so the stage is sized for about
  // 3 C candidates (a selection keeps some 2 C, the rest is room for the drift
  // of the scores between steps).
  const int want = 2 * units <= device_cus() ? 16384 : 3 * s.C;
#define ASP_SEL_FIRST(CAPV)                                                                                 \
  hipLaunchKernelGGL(select_cand_kernel<CAPV>, dim3(units), dim3(CAND_SEL_THREADS), 0, st, seq_lens, cw, idx, \
                     n_sel, adv_newest, adv_len, s.Hkv, s.T_cap, s.C, W, 1)
  switch ((want + 2047) / 2048) {  // LDS in steps of 2048 candidates (16 KiB), at most 16384
    case 0:
    case 1: ASP_SEL_FIRST(2048); break;
    case 2: ASP_SEL_FIRST(4096); break;
    case 3: ASP_SEL_FIRST(6144); break;
    case 4: ASP_SEL_FIRST(8192); break;
    case 5: ASP_SEL_FIRST(10240); break;
    case 6: ASP_SEL_FIRST(12288); break;
    case 7: ASP_SEL_FIRST(14336); break;
    default: ASP_SEL_FIRST(16384); break;
  }
#undef ASP_SEL_FIRST
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_score_candidates(s, q_pred, k, seq_lens, cw, true, st);
  if (e != hipSuccess) return e;
  return launch_recording(select_cand_kernel<0>, dim3(units), dim3(CAND_SEL_THREADS), st, done, seq_lens, cw, idx,
                          n_sel, adv_newest, adv_len, s.Hkv, s.T_cap, s.C, W, 0);
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
