// Internal declarations shared by the HIP translation units of libasp.so.
// Nothing here is part of the public C ABI (include/asp.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace asp {

// Validated problem shape, as the kernels see it.
struct Shape {
  int B, Hq, Hkv, G, D, T_cap, kv;  // kv: 0 = bf16, 1 = fp32
  int W, C;
  double lambda;
  int R;  // newest tokens attended beside the selection
};

// Attention split size: tokens handled by one workgroup of the split-K
// attention kernel (depends on the KV row size: 4 waves x 16 loads x keys per load).
int attend_tokens_per_block(int D, int kv);
int attend_num_splits(const Shape& s);
size_t attend_partials_bytes(const Shape& s);

hipError_t launch_push(const Shape& s, const float* q_cur, float* q_hist, int32_t* newest, int32_t* len,
                       hipStream_t st);
// Predictor.  With q_cur == nullptr it predicts from the ring as it stands.
// With q_cur != nullptr it predicts from the ring after pushing q_cur (lag 0 is
// q_cur, the ring supplies the older lags) and writes q_cur into each head's
// next ring slot, but leaves newest/len unchanged: a later launch of the same
// step advances them (ring_advance, in the last select launch), once every
// predictor workgroup has read them.
// `done` (nullable) is recorded when the launch completes.
hipError_t launch_predict(const Shape& s, float* q_hist, const int32_t* newest, const int32_t* len,
                          const float* q_cur, float* q_pred, hipStream_t st,
                          hipEvent_t done = nullptr);
// Scores; hist (nullable) accumulates the coarse histogram of every unit and
// must be zero on entry.  `done` (nullable) is recorded when the launch completes.
hipError_t launch_score(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                        float* scores, uint32_t* hist, hipStream_t st, hipEvent_t done = nullptr);
// Zero fill of n words (a kernel, so that it can also stand in a captured graph).
hipError_t launch_clear_u32(uint32_t* p, size_t n, hipStream_t st);
// Top-C selection; hist (nullable) is the coarse histogram built by the score
// launch (when null, one is built in ws first).  adv_newest/adv_len (nullable)
// advance the query ring by one slot.  ws: select_ws_bytes(s, hist == nullptr).
size_t select_ws_bytes(const Shape& s, bool with_hist);
hipError_t launch_select(const Shape& s, const float* scores, const uint32_t* hist, const int32_t* seq_lens,
                         int32_t* idx, int32_t* n_sel, int32_t* adv_newest, int32_t* adv_len, void* ws,
                         hipStream_t st, hipEvent_t done = nullptr);
// Candidate path of the selection (the pipelined step, asp_score_candidates
// and asp_select_candidates).  Each unit carries a threshold hint, an order
// key: the score launch keeps every key at or above it as a (key, index)
// candidate, in per-wave regions of CAND_REGION consecutive keys, and writes
// no score rows.  The select launches pick the exact top C_eff from the
// candidates; a unit left with fewer than C_eff candidates is rescored with
// every key kept, so the result never depends on the hint.  Each selection
// stores the next hint: a bin edge of the key that keeps about 1.5 C_eff
// candidates of the scores it saw.
constexpr int CAND_REGION = 128;       // keys of one wave of a score block
constexpr int CAND_BLOCK_KEYS = 512;   // keys of one score block (four waves)
struct CandWs {
  uint32_t* hint;    // [units] threshold hint (order key)
  uint32_t* flag;    // [units] 1: the unit is rescored with every key kept
  uint32_t* rcount;  // [units][regions] candidates per region
  uint2* cand;       // [units][regions][CAND_REGION] (order key, index)
};
__host__ __device__ inline int cand_regions(int T_cap) {  // regions per unit
  return (T_cap + CAND_BLOCK_KEYS - 1) / CAND_BLOCK_KEYS * (CAND_BLOCK_KEYS / CAND_REGION);
}
size_t cand_ws_bytes(const Shape& s);
CandWs cand_carve(const Shape& s, void* ws);  // hint at offset 0
// fallback == false: keep the keys at or above each unit's hint.
// fallback == true: keep every key of the units flagged by the first select
// launch (the other units' blocks return at once).
hipError_t launch_score_candidates(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                   const CandWs& cw, bool fallback, hipStream_t st, hipEvent_t done = nullptr);
// Exact top-C_eff from the candidates (first launch), the rescoring of the
// flagged units, and their selection (last launch); new hints.
// adv_newest/adv_len (nullable) advance the query ring by one slot.
hipError_t launch_select_candidates(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                    const CandWs& cw, int32_t* idx, int32_t* n_sel, int32_t* adv_newest,
                                    int32_t* adv_len, hipStream_t st, hipEvent_t done = nullptr);
// Device-argument check (check.hip): clears *status, then ORs ASP_CHECK_* bits into it.
hipError_t launch_check(const Shape& s, const int32_t* seq_lens, const int32_t* hist_newest, const int32_t* hist_len,
                        const int32_t* idx, const int32_t* n_sel, uint32_t* status, hipStream_t st);
// Per unit, the number of indices that two ascending selections share
// (s.C <= overlap_max_c()).
int overlap_max_c();
hipError_t launch_overlap(const Shape& s, const int32_t* idx_a, const int32_t* n_a, const int32_t* idx_b,
                          const int32_t* n_b, int32_t* out, hipStream_t st);
// Sparse attention over the selection and the newest s.R tokens: split-K
// partials into `partials`, then the merge into out.  seq_lens may be null
// when s.R == 0.
hipError_t launch_attend(const Shape& s, const float* q, const void* k, const void* v, const int32_t* seq_lens,
                         const int32_t* idx, const int32_t* n_sel, float* out, void* partials, hipStream_t st);
// The merge alone (partials written by the attention blocks).
hipError_t launch_merge(const Shape& s, const int32_t* seq_lens, const int32_t* n_sel, float* out,
                        const void* partials, hipStream_t st);

// Whether `st` is being captured into a graph.
inline bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

// The id of the capture `st` takes part in, 0 when it is not being captured.
inline unsigned long long capture_id(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  if (hipStreamGetCaptureInfo(st, &cs, &id) != hipSuccess || cs != hipStreamCaptureStatusActive) return 0;
  return id;
}

// Launch that records `done` (nullable) when the kernel completes.  The event
// rides on the kernel's own completion signal (hipExtLaunchKernelGGL), so it
// costs no extra queue packet.  While `st` is being captured into a graph the
// launch is a plain one followed by an event record, the form stream capture
// defines.
template <typename... KArgs, typename... Args>
hipError_t launch_recording(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st, hipEvent_t done,
                            Args... args) {
  if (done != nullptr && !capturing(st)) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, nullptr, done, 0, args...);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && done != nullptr) e = hipEventRecord(done, st);
  return e;
}

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Number of set bits of m below this lane.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Cross-lane moves inside a 16-lane DPP row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Sum over aligned groups of N lanes (N in {1, 2, 4, 8, 16, 32, 64}); every lane
// of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f<DPP_QUAD_XOR1>(x);
  if constexpr (N >= 4) x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (N >= 8) x += dpp_f<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_f<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_f<DPP_QUAD_XOR1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_f<DPP_QUAD_XOR2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f<DPP_ROW_MIRROR>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

}  // namespace asp

namespace asp {

// Monotone map from float to uint32: a > b (as numbers) iff key(a) > key(b);
// NaN maps to the key of -inf and -0 to the key of +0.  Shared by the score
// kernel's coarse histogram and the select kernel, which must agree bit for bit.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Coarse histogram over the top 11 bits of order_key, per unit.
constexpr int HIST_BINS = 2048;
constexpr int HIST_SHIFT = 21;

// One slot forward in sequence b's query ring: newest moves to the slot the
// predictor of this step wrote (modulo W), the length grows up to W.
__device__ __forceinline__ void ring_advance(int32_t* newest, int32_t* len, int b, int W) {
  int o = newest[b] % W;
  if (o < 0) o += W;
  newest[b] = o + 1 == W ? 0 : o + 1;
  len[b] = min(clampi(len[b], 0, W) + 1, W);
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffffll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

}  // namespace asp
