// Attention block (device function) for bf16 K/V: sparse decode attention over
// the selected tokens with both products on the matrix cores.
//
// Sources: reproduction card, "Layout" (full versus top-C sparse attention) and
// "Key finding" (the method attends to the C selected tokens only); research-map
// summary of AsyncSpade, "Approach" (the selection is consumed by the inference
// step).  As for the fp32 path (attend_block.h): the attention query is the
// actual current query; optionally the newest R tokens are attended beside
// the selection, a selected index among them counting once.
//
// Grid: (split, unit), ATTM_THREADS threads.  A unit's token list (its
// selection, then its newest tokens) is cut into `nsplit` contiguous ranges of
// `per` positions; the eight waves of a block take the range's 16-token chunks
// in turn, keep a running (max, sum, weighted V) per query head in log2
// units, and gather the next chunk's rows while the current one is computed.
// The waves are combined through LDS; with one split the block writes the
// normalised output, otherwise an unnormalised partial that the merge launch
// combines.
//
// Per 16-token chunk a wave computes on the matrix cores:
//  - logits S^T = K Q^T (v_mfma_f32_16x16x32_bf16): the A operand is the
//    gathered K tile (lane l: token l%16, coordinates 8(l/16)..+7 of each
//    32-wide step, a 16-byte row slice), the B operand the query (lane l:
//    head l%16), as two bf16 terms hi = rne(q'), lo = rne(q' - hi) of
//    q' = q log2(e) / sqrt(D).  Lane l then holds, for head l%16, the logits
//    of tokens 4(l/16) .. 4(l/16) + 3;
//  - O += P V (v_mfma_f32_16x16x16_bf16): these four weights per lane are
//    exactly an A operand (head l%16, tokens 4(l/16)..+3), again as hi + lo
//    bf16 terms; the B operand of the column block (blk, p) holds
//    V[4(l/16) + e][64 blk + 4(l%16) + p]: each lane gathers 8 bytes (four
//    columns) of its four tokens' rows, 16 lanes covering 128 contiguous bytes
//    of a row, and packs element p of each.
// Heads beyond G are zero rows of the query and are never written.
#pragma once

#include "asp_internal.h"
#include "attend_block.h"

namespace asp {

constexpr int ATTM_THREADS = 512;
constexpr int ATTM_WAVES = ATTM_THREADS / 64;
constexpr int ATTM_CHUNK = 16;
constexpr int ATTM_DEPTH = 2;  // chunks whose row gathers are in flight per wave

typedef __bf16 attm_bf16x8 __attribute__((ext_vector_type(8)));
typedef short attm_i16x4 __attribute__((ext_vector_type(4)));
typedef float attm_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int attm_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t attm_bf16_bits(float x) {  // round to nearest even
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// LDS of one block: per wave and head the running max and sum, and the
// weighted V sums.
template <int D, int G>
constexpr size_t attm_lds_bytes() {
  return (size_t)ATTM_WAVES * G * (D + 2) * sizeof(float);
}

// Registers of one chunk in flight.
template <int D>
struct AttmChunk {
  attm_u32x4 k[D / 32];  // K tile, step s
  uint2 v[4][D / 64];    // V token slot e (token 4(l/16) + e), column block blk
  uint32_t valid;        // bit e: token slot e is in the list
};

// A lane's list position in a chunk, looked up but not yet checked: `raw` is
// the selection entry (listed) or the newest-token index, or -1 past the list.
struct AttmTok {
  int raw;
  bool listed;
};

// Lanes l, l + 16, l + 32, l + 48 look up position p0 + (l & 15) of the chunk starting at
// p0 (positions below p_end).  The index load is issued here and its value is
// first used by attm_load: a chunk's lookup is issued before the previous
// chunk's row gathers, and loads complete in issue order for the wait counter,
// so waiting for the lookup does not wait for those gathers.
template <bool RECENT>
__device__ __forceinline__ AttmTok attm_lookup(const int32_t* __restrict__ ib, const AttendList& al, int p0,
                                               int p_end, int lane) {
  const int p = p0 + (lane & 15);
  AttmTok t;
  t.listed = p < p_end && p < al.n;
  t.raw = t.listed ? ib[p] : ((RECENT && p < p_end && p < al.n + al.r) ? al.lo + (p - al.n) : -1);
  return t;
}

// The token of a looked-up position, or -1 when its selection entry is
// skipped (outside [0, t_cap), or inside the newest-token range, where it is
// attended once as a newest token).
template <bool RECENT>
__device__ __forceinline__ int attm_token(const AttmTok& t, const AttendList& al, int T_cap) {
  if (!t.listed) return t.raw;
  bool ok = t.raw >= 0 && t.raw < T_cap;
  if constexpr (RECENT) ok = ok && !(t.raw >= al.lo && t.raw < al.lo + al.r);
  return ok ? t.raw : -1;
}

// Issues the row gathers of a looked-up chunk; the tokens are passed between
// lanes.
template <int D, bool RECENT>
__device__ __forceinline__ void attm_load(AttmChunk<D>& ch, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, const AttmTok& look,
                                          const AttendList& al, int T_cap, int lane) {
  const int tok = attm_token<RECENT>(look, al, T_cap);
  const int c = lane >> 4, n = lane & 15;
  const int tk = __shfl(tok, n);
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    ch.k[s] = tk >= 0 ? *reinterpret_cast<const attm_u32x4*>(kb + (size_t)tk * D + 32 * s + 8 * c)
                      : attm_u32x4{0u, 0u, 0u, 0u};
  uint32_t valid = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tv = __shfl(tok, 4 * c + e);
    valid |= tv >= 0 ? 1u << e : 0u;
#pragma unroll
    for (int blk = 0; blk < D / 64; ++blk)
      ch.v[e][blk] = tv >= 0 ? *reinterpret_cast<const uint2*>(vb + (size_t)tv * D + 64 * blk + 4 * n)
                             : make_uint2(0u, 0u);
  }
  ch.valid = valid;
}

// One chunk: logits, the online softmax update and the weighted V sums.
template <int D>
__device__ __forceinline__ void attm_compute(const AttmChunk<D>& ch, const attm_bf16x8 (&qhi)[D / 32],
                                             const attm_bf16x8 (&qlo)[D / 32], attm_f32x4 (&o)[D / 16],
                                             float& m_run, float& l_run, int lane) {
  attm_f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const attm_bf16x8 a = __builtin_bit_cast(attm_bf16x8, ch.k[s]);
    st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[s], st, 0, 0, 0);
    st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[s], st, 0, 0, 0);
  }
  float x[4];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = (ch.valid >> e) & 1u ? st[e] : -INFINITY;
    mx = fmaxf(mx, x[e]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  // m_new = -inf: nothing attended yet for this head; keep everything as is
  const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
  m_run = m_new;
  float p[4], ps = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = x[e] == -INFINITY ? 0.0f : exp2f(x[e] - m_new);
    ps += p[e];
  }
  l_run = l_run * alpha + ps;
  // rows of the accumulators are heads 4(l/16) + i: their scale factors
  const int c = lane >> 4;
  float a_i[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_i[i] = __shfl(alpha, 4 * c + i);
  // P as hi + lo bf16 terms (A operand: head l%16, tokens 4(l/16) + e)
  uint2 phi, plo;
  {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = attm_bf16_bits(p[e]);
      l[e] = attm_bf16_bits(p[e] - __uint_as_float(h[e] << 16));
    }
    phi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    plo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
  const attm_i16x4 pa_hi = __builtin_bit_cast(attm_i16x4, phi);
  const attm_i16x4 pa_lo = __builtin_bit_cast(attm_i16x4, plo);
#pragma unroll
  for (int blk = 0; blk < D / 64; ++blk) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      // element pp of each token slot's four columns
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pp < 2 ? ch.v[e][blk].x : ch.v[e][blk].y;
      const uint2 bv = (pp & 1) ? make_uint2((w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u))
                                : make_uint2((w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16));
      attm_f32x4& acc = o[blk * 4 + pp];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= a_i[i];
      const attm_i16x4 b = __builtin_bit_cast(attm_i16x4, bv);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, b, acc, 0, 0, 0);
    }
  }
}

// Attention block (split, unit) for bf16 K/V; smem holds attm_lds_bytes<D, G>().
// per: list positions of one split (a multiple of ATTM_CHUNK).  out_direct:
// nsplit == 1, the block writes out[b][h] itself.
template <int D, int G, bool RECENT>
__device__ __forceinline__ void attend_mfma_block(const float* __restrict__ q, const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  const int32_t* __restrict__ seq_lens,
                                                  const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel,
                                                  float* __restrict__ out, float* __restrict__ part_acc,
                                                  float* __restrict__ part_ml, int Hq, int Hkv, int T_cap, int C,
                                                  int R, int nsplit, int per, int split, int unit,
                                                  unsigned char* smem) {
  static_assert(D % 64 == 0 && G <= 16, "head_dim a multiple of 64, at most 16 heads per KV head");
  float (*sm_m)[G] = reinterpret_cast<float (*)[G]>(smem);
  float (*sm_l)[G] = reinterpret_cast<float (*)[G]>(smem + (size_t)ATTM_WAVES * G * sizeof(float));
  float (*sm_o)[G][D] = reinterpret_cast<float (*)[G][D]>(smem + (size_t)2 * ATTM_WAVES * G * sizeof(float));

  const int b = unit / Hkv, g = unit % Hkv;
  const AttendList al = attend_list(n_sel, seq_lens, unit, Hkv, C, RECENT ? R : 0, T_cap);
  const int total = al.n + al.r;
  const int p_begin = split * per;
  if (nsplit > 1 && p_begin >= total) return;  // an empty split writes no partial (the merge skips it)
  const int p_end = min(p_begin + per, total);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, n = lane & 15;

  // B operand of the logits: head n's query, scaled so that exp2 of a logit
  // difference is the softmax weight, as two bf16 terms.
  attm_bf16x8 qhi[D / 32], qlo[D / 32];
  {
    const float scale = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      attm_u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
      if (n < G) {
        const float* qh = q + ((size_t)b * Hq + (size_t)g * G + n) * D + 32 * s + 8 * c;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = qh[e] * scale, x1 = qh[e + 1] * scale;
          const uint32_t h0 = attm_bf16_bits(x0), h1 = attm_bf16_bits(x1);
          const uint32_t l0 = attm_bf16_bits(x0 - __uint_as_float(h0 << 16));
          const uint32_t l1 = attm_bf16_bits(x1 - __uint_as_float(h1 << 16));
          hi[e / 2] = h0 | (h1 << 16);
          lo[e / 2] = l0 | (l1 << 16);
        }
      }
      qhi[s] = __builtin_bit_cast(attm_bf16x8, hi);
      qlo[s] = __builtin_bit_cast(attm_bf16x8, lo);
    }
  }

  const int32_t* ib = idx + (size_t)unit * C;
  const uint16_t* kb = k + (size_t)unit * T_cap * D;
  const uint16_t* vb = v + (size_t)unit * T_cap * D;
  attm_f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = attm_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  // The wave's chunks j = 0, 1, ...: positions p_begin + 16 (wave + 8 j).
  // Chunk j lives in buffer j % ATTM_DEPTH.  While it is computed, the row
  // gathers of the next ATTM_DEPTH - 1 chunks and the lookup of the one after
  // are in flight.
  constexpr int STRIDE = ATTM_WAVES * ATTM_CHUNK;
  constexpr int NB = ATTM_DEPTH;
  const int first = p_begin + wave * ATTM_CHUNK;
  AttmChunk<D> buf[NB];
  AttmTok look[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) look[u] = attm_lookup<RECENT>(ib, al, first + u * STRIDE, p_end, lane);
#pragma unroll
  for (int u = 0; u + 1 < NB; ++u)
    if (first + u * STRIDE < p_end) attm_load<D, RECENT>(buf[u], kb, vb, look[u], al, T_cap, lane);
  for (int j0 = 0; first + j0 * STRIDE < p_end; j0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u;
      if (first + j * STRIDE >= p_end) break;
      constexpr int LAST = NB - 1;
      // the slot of chunk j + NB - 1 held chunk j - 1, already computed
      const int pl = first + (j + LAST) * STRIDE;
      const AttmTok nxt = attm_lookup<RECENT>(ib, al, pl + STRIDE, p_end, lane);  // chunk j + NB
      if (pl < p_end) attm_load<D, RECENT>(buf[(u + LAST) % NB], kb, vb, look[(u + LAST) % NB], al, T_cap, lane);
      look[u] = nxt;  // chunk j's lookup was used when its rows were gathered
      attm_compute<D>(buf[u], qhi, qlo, o, m_run, l_run, lane);
    }
  }
  // The head's sum over the lanes that hold its tokens.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (c == 0 && n < G) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_run;
  }
  // accumulator rows are heads 4c + i, columns 64 blk + 4n + pp
#pragma unroll
  for (int blk = 0; blk < D / 64; ++blk) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * c + i;
        if (h < G) sm_o[wave][h][64 * blk + 4 * n + pp] = o[blk * 4 + pp][i];
      }
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)unit * nsplit + split) * G;
  for (int e = threadIdx.x; e < G * D; e += ATTM_THREADS) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < ATTM_WAVES; ++w) M = fmaxf(M, sm_m[w][h]);
    float acc = 0.0f, L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < ATTM_WAVES; ++w) {
        const float mw = sm_m[w][h];
        const float wt = mw == -INFINITY ? 0.0f : exp2f(mw - M);
        acc = fmaf(wt, sm_o[w][h][d], acc);
        L = fmaf(wt, sm_l[w][h], L);
      }
    }
    if (nsplit == 1) {
      out[((size_t)b * Hq + (size_t)g * G + h) * D + d] = L > 0.0f ? acc / L : 0.0f;
    } else {
      part_acc[(pbase + h) * D + d] = acc;
      if (d == 0) {
        part_ml[(pbase + h) * 2 + 0] = M;
        part_ml[(pbase + h) * 2 + 1] = L;
      }
    }
  }
}

}  // namespace asp
