// Score blocks (device functions) of the score launch.
// Token-level key scoring: score[b][g][i] = max over the G query heads of
// KV head g of q_pred[b][h] . K[b][g][i].
//
// Sources: atlas.scime.ai research-map summary of AsyncSpade, "Approach"
// (token-level KV selection driven by the predicted query); arXiv 2510.07486
// abstract (token-level instead of coarse page-level selection; decoding is
// memory bound because the KV cache grows linearly).  The max over the GQA
// group is the reading taken for grouped-query attention, which the pages do
// not discuss.
//
// This pass streams the whole K cache once and is bound by HBM bandwidth.  The
// KV layout is head-major ([B][Hkv][T_cap][D]), so a unit's keys are one
// contiguous stream.
//
// bf16 keys: the G x D query block times a 16-key tile is one
// v_mfma_f32_16x16x32_bf16 per 32 coordinates, with the keys as the B operand
// (lane l: key l%16, coordinates 8*(l/16)..+7 of each 32-wide step) and the
// query heads as rows of the A operand.  Keys arrive with fully coalesced
// non-temporal 16-byte loads (each wave-wide load covers whole key rows; four
// 16-key tiles in flight per wave) and are transposed into the MFMA layout
// through two per-wave, XOR-swizzled LDS slots: loading 64-byte column slices
// of 16 rows straight into the operand layout costs ~15% of the bandwidth on
// this part.  Two slots instead of one per tile in flight keep the block at
// 40 KiB of LDS, so four blocks (16 waves) share a CU; blocks of 512 keys keep
// the tail of the launch short.  The
// predicted query is fp32; it enters as two bf16 terms, hi = rne(q) and
// lo = rne(q - hi), so the product keeps ~17 significant bits of q (relative
// error <= 2^-18 per term) and accumulates in fp32.
// fp32 keys: a VALU dot product (LPK lanes per key, DPP reduction).
//
// A block writes either every score (optionally also binning them by the top
// 11 bits of the order-preserving key: an LDS histogram, then one global
// atomic per non-empty bin, the first radix pass of the top-C select done
// while the keys stream), or candidates: the (order key, index) pairs of the
// keys at or above the unit's threshold hint, compacted per wave (ballot,
// LDS staging) into the wave's region of CAND_REGION slots.  Writing only the
// candidates spares the DRAM writes of the score rows, which otherwise cut into
// the read stream.
#pragma once

#include "asp_internal.h"

namespace asp {

constexpr int SCORE_THREADS = 256;
constexpr int SCORE_WAVES = SCORE_THREADS / 64;
constexpr int SCORE_KEYS_PER_BLOCK = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

constexpr int SCORE_MFMA_U = 4;     // 16-key tiles loaded per wave and iteration
constexpr int SCORE_MFMA_SLOTS = 2;  // LDS transpose slots per wave (double buffer)

// Every wave of a block sees SCORE_KEYS_PER_BLOCK / SCORE_WAVES keys (whole
// iterations of its loop): its candidate region.
static_assert(SCORE_KEYS_PER_BLOCK % (SCORE_WAVES * 16 * SCORE_MFMA_U) == 0, "whole mfma iterations per wave");
static_assert(SCORE_KEYS_PER_BLOCK / SCORE_WAVES == CAND_REGION, "one candidate region per wave");
static_assert(SCORE_KEYS_PER_BLOCK == CAND_BLOCK_KEYS, "candidate regions follow the score blocks");

// What a score block writes.
enum ScoreOut : int {
  OUT_SCORES = 0,       // every score (HIST: and the coarse histogram)
  OUT_ABOVE_HINT = 1,   // candidates: the keys at or above the unit's hint
  OUT_ALL_FLAGGED = 2,  // candidates: every key, for units flagged for rescoring
};

constexpr size_t CAND_STAGE_BYTES = (size_t)SCORE_WAVES * CAND_REGION * sizeof(uint2);

// LDS of one bf16 score block: the per-wave transpose slots, then the
// histogram or the candidate staging.
template <int D, bool HIST, int OUT>
constexpr size_t score_mfma_lds_bytes() {
  return (size_t)SCORE_WAVES * SCORE_MFMA_SLOTS * 16 * (D * 2 / 16) * 16 + (HIST ? HIST_BINS * 4 : 0) +
         (OUT != OUT_SCORES ? CAND_STAGE_BYTES : 0);
}

// Candidate region `region`: the wave's staged (key, index) pairs, then their count.
__device__ __forceinline__ void flush_candidates(const CandWs& cw, size_t region, const uint2* stage, uint32_t kept,
                                                 int lane) {
  // the staging writes of every lane of the wave are visible to all of them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint2* dst = cw.cand + region * CAND_REGION;
  for (uint32_t i = (uint32_t)lane; i < kept; i += 64) dst[i] = stage[i];
  if (lane == 0) cw.rcount[region] = kept;
}

// Score block (bx, unit) for bf16 keys; smem holds score_mfma_lds_bytes<D, HIST, OUT>().
template <int D, int G, bool HIST, int OUT>
__device__ __forceinline__ void score_mfma_block(const float* __restrict__ q_pred, const uint16_t* __restrict__ k,
                                                 const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                                                 uint32_t* __restrict__ hist, const CandWs& cw, int Hq, int Hkv,
                                                 int T_cap, int bx, int unit, unsigned char* smem) {
  static_assert(!(HIST && OUT != OUT_SCORES), "the histogram goes with the score rows");
  constexpr int S = D / 32;          // MFMA steps over the coordinates
  constexpr int CH = D * 2 / 16;     // 16-byte chunks per key row
  constexpr int RPI = 64 / CH;       // key rows per wave-wide load
  constexpr int NI = 16 / RPI;       // loads per 16-key tile
  constexpr int U = SCORE_MFMA_U;
  constexpr int TB = SCORE_MFMA_SLOTS;
  u32x4 (*tile)[TB][16][CH] = reinterpret_cast<u32x4 (*)[TB][16][CH]>(smem);
  uint32_t* lhist = reinterpret_cast<uint32_t*>(smem + (size_t)SCORE_WAVES * TB * 16 * CH * 16);

  const int b = unit / Hkv, g = unit % Hkv;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int k0 = bx * SCORE_KEYS_PER_BLOCK;
  if (k0 >= T) return;
  const uint32_t hint = OUT == OUT_ABOVE_HINT ? cw.hint[unit] : 0u;
  const int k1 = min(k0 + SCORE_KEYS_PER_BLOCK, T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint2* stage = reinterpret_cast<uint2*>(smem + (size_t)SCORE_WAVES * TB * 16 * CH * 16) + wave * CAND_REGION;
  uint32_t kept = 0u;  // candidates staged by this wave (uniform)
  const int j = lane & 15, c = lane >> 4;          // MFMA roles: key column j, coordinate group c
  const int lrow = lane / CH, lchunk = lane % CH;  // load roles: row in the load, 16-byte chunk

  if constexpr (HIST) {
    for (int i = threadIdx.x; i < HIST_BINS; i += SCORE_THREADS) lhist[i] = 0u;
    __syncthreads();
  }

  // A operand: row j = query head j of the group (zero rows past G), step s
  // covers coordinates 32s + 8c .. 32s + 8c + 7.
  bf16x8 ahi[S], alo[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
    if (j < G) {
      const float* qh = q_pred + ((size_t)b * Hq + (size_t)g * G + j) * D + 32 * s + 8 * c;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = qh[e], x1 = qh[e + 1];
        const uint32_t h0 = bf16_rne_bits(x0), h1 = bf16_rne_bits(x1);
        const uint32_t l0 = bf16_rne_bits(x0 - __uint_as_float(h0 << 16));
        const uint32_t l1 = bf16_rne_bits(x1 - __uint_as_float(h1 << 16));
        hi[e / 2] = h0 | (h1 << 16);
        lo[e / 2] = l0 | (l1 << 16);
      }
    }
    ahi[s] = __builtin_bit_cast(bf16x8, hi);
    alo[s] = __builtin_bit_cast(bf16x8, lo);
  }

  const u32x4* kb = reinterpret_cast<const u32x4*>(k + (size_t)unit * T_cap * D);
  float* sb = scores + (size_t)unit * T_cap;

  // Candidate route: the kept-key bookkeeping of an iteration's tiles (ballot,
  // LDS staging) runs after the next iteration's loads are issued, so that it
  // never delays them.
  float pend[U];
  int pend_base = -1;
  auto keep_pending = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = pend_base + u * 16 + j;
      const uint32_t ok = order_key(pend[u]);
      const bool take = c == 0 && key < k1 && ok >= hint;
      const unsigned long long bal = __ballot(take);
      if (take) stage[kept + lanes_below(bal)] = make_uint2(ok, (uint32_t)key);
      kept += (uint32_t)__popcll(bal);
    }
  };
  for (int base = k0 + wave * 16 * U; base < k1; base += SCORE_WAVES * 16 * U) {
    // Coalesced non-temporal loads: each wave-wide load is RPI whole key rows.
    u32x4 gld[U][NI];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int key = base + u * 16 + RPI * i + lrow;
        gld[u][i] = key < k1 ? __builtin_nontemporal_load(kb + (size_t)key * CH + lchunk) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (OUT != OUT_SCORES) {
      if (pend_base >= 0) keep_pending();
    }
    // Transpose through LDS, one 16-key tile at a time through two slots:
    // tile u+1 is written while the MFMAs read tile u.  Chunk q of tile row r
    // is stored at q ^ (r % CH), which keeps both the row-wise writes and the
    // column-wise reads spread over all banks.
    auto put = [&](int u) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = RPI * i + lrow;
        tile[wave][u % TB][r][lchunk ^ (r % CH)] = gld[u][i];
      }
    };
    put(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u + 1 < U) put(u + 1);
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const bf16x8 bk = __builtin_bit_cast(bf16x8, tile[wave][u % TB][j][(4 * s + c) ^ (j % CH)]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[s], bk, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[s], bk, acc, 0, 0, 0);
      }
      // lane (c, j) holds heads 4c .. 4c+3 of key base + 16u + j
      float m = acc[0];
      if constexpr (G >= 2) m = fmaxf(m, acc[1]);
      if constexpr (G >= 4) m = fmaxf(fmaxf(m, acc[2]), acc[3]);
      if constexpr (G == 8) m = fmaxf(m, __shfl_xor(m, 16));
      const int key = base + u * 16 + j;
      if constexpr (OUT == OUT_SCORES) {
        if (c == 0 && key < k1) {
          sb[key] = m;  // a plain store: the select launches read the row back soon after
          if constexpr (HIST) atomicAdd(&lhist[order_key(m) >> HIST_SHIFT], 1u);
        }
      } else {
        pend[u] = m;
      }
      // Slot u % TB is written again two tiles later (or next iteration).
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    pend_base = base;
  }
  if constexpr (OUT != OUT_SCORES) {
    if (pend_base >= 0) keep_pending();
    const int nreg = cand_regions(T_cap);
    flush_candidates(cw, (size_t)unit * nreg + (size_t)bx * SCORE_WAVES + wave, stage, kept, lane);
  }
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = hist + (size_t)unit * HIST_BINS;
    for (int i = threadIdx.x; i < HIST_BINS; i += SCORE_THREADS) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
}

// LDS of one fp32 score block: the histogram or the candidate staging.
template <bool HIST, int OUT>
constexpr size_t score_valu_lds_bytes() {
  return HIST ? HIST_BINS * 4 : (OUT != OUT_SCORES ? CAND_STAGE_BYTES : 4);
}

// Score block (bx, unit) for fp32 keys; smem holds score_valu_lds_bytes<HIST, OUT>().
template <int D, int G, bool HIST, int OUT>
__device__ __forceinline__ void score_valu_block(const float* __restrict__ q_pred, const float* __restrict__ k,
                                                 const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                                                 uint32_t* __restrict__ hist, const CandWs& cw, int Hq, int Hkv,
                                                 int T_cap, int bx, int unit, unsigned char* smem) {
  static_assert(!(HIST && OUT != OUT_SCORES), "the histogram goes with the score rows");
  constexpr int EPL = 4;           // fp32 elements per 16-byte load
  constexpr int LPK = D / EPL;     // lanes per key row
  constexpr int KPW = 64 / LPK;    // keys per wave-wide load
  constexpr int U = 4;             // loads in flight per lane
  static_assert(SCORE_KEYS_PER_BLOCK % (SCORE_WAVES * KPW * U) == 0, "whole iterations per wave");
  uint32_t* lhist = reinterpret_cast<uint32_t*>(smem);

  const int b = unit / Hkv, g = unit % Hkv;
  const int T = clampi(seq_lens[b], 0, T_cap);
  const int k0 = bx * SCORE_KEYS_PER_BLOCK;
  if (k0 >= T) return;
  const uint32_t hint = OUT == OUT_ABOVE_HINT ? cw.hint[unit] : 0u;
  const int k1 = min(k0 + SCORE_KEYS_PER_BLOCK, T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kl = lane / LPK;
  uint2* stage = reinterpret_cast<uint2*>(smem) + wave * CAND_REGION;
  uint32_t kept = 0u;  // candidates staged by this wave (uniform)
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < HIST_BINS; i += SCORE_THREADS) lhist[i] = 0u;
    __syncthreads();
  }

  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q_pred + ((size_t)b * Hq + (size_t)g * G + h) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[h][e] = qh[e];
  }
  const float* kb = k + (size_t)unit * T_cap * D + sub * EPL;
  float* sb = scores + (size_t)unit * T_cap;

  for (int base = k0 + wave * KPW * U; base < k1; base += SCORE_WAVES * KPW * U) {
    float4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPW + kl;
      raw[u] = key < k1 ? *reinterpret_cast<const float4*>(kb + (size_t)key * D) : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float x[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      float best = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(q[h][e], x[e], acc);
        acc = group_sum<LPK>(acc);
        best = h == 0 ? acc : fmaxf(best, acc);
      }
      const int key = base + u * KPW + kl;
      if constexpr (OUT == OUT_SCORES) {
        if (sub == 0 && key < k1) {
          sb[key] = best;
          if constexpr (HIST) atomicAdd(&lhist[order_key(best) >> HIST_SHIFT], 1u);
        }
      } else {
        const uint32_t ok = order_key(best);
        const bool take = sub == 0 && key < k1 && ok >= hint;
        const unsigned long long bal = __ballot(take);
        if (take) stage[kept + lanes_below(bal)] = make_uint2(ok, (uint32_t)key);
        kept += (uint32_t)__popcll(bal);
      }
    }
  }
  if constexpr (OUT != OUT_SCORES) {
    const int nreg = cand_regions(T_cap);
    flush_candidates(cw, (size_t)unit * nreg + (size_t)bx * SCORE_WAVES + wave, stage, kept, lane);
  }
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = hist + (size_t)unit * HIST_BINS;
    for (int i = threadIdx.x; i < HIST_BINS; i += SCORE_THREADS) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
}

}  // namespace asp
