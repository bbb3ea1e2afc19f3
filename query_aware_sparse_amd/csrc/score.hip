// Launches of the score pass; the block bodies are in score_block.h.
#include "score_block.h"

namespace asp {

template <int D, int G, bool HIST>
__global__ void __launch_bounds__(SCORE_THREADS) score_mfma_kernel(const float* __restrict__ q_pred,
                                                                   const uint16_t* __restrict__ k,
                                                                   const int32_t* __restrict__ seq_lens,
                                                                   float* __restrict__ scores,
                                                                   uint32_t* __restrict__ hist, int Hq, int Hkv,
                                                                   int T_cap) {
  __shared__ __align__(16) unsigned char smem[score_mfma_lds_bytes<D, HIST>()];
  score_mfma_block<D, G, HIST>(q_pred, k, seq_lens, scores, hist, Hq, Hkv, T_cap, blockIdx.x, blockIdx.y, smem);
}

template <int D, int G, bool HIST>
__global__ void __launch_bounds__(SCORE_THREADS) score_valu_kernel(const float* __restrict__ q_pred,
                                                                   const float* __restrict__ k,
                                                                   const int32_t* __restrict__ seq_lens,
                                                                   float* __restrict__ scores,
                                                                   uint32_t* __restrict__ hist, int Hq, int Hkv,
                                                                   int T_cap) {
  __shared__ __align__(16) unsigned char smem[score_valu_lds_bytes<HIST>()];
  score_valu_block<D, G, HIST>(q_pred, k, seq_lens, scores, hist, Hq, Hkv, T_cap, blockIdx.x, blockIdx.y, smem);
}

template <int D, bool HIST>
static hipError_t launch_score_dh(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                  float* scores, uint32_t* hist, hipStream_t st, hipEvent_t done) {
  const dim3 grid((s.T_cap + SCORE_KEYS_PER_BLOCK - 1) / SCORE_KEYS_PER_BLOCK, s.B * s.Hkv);
  const dim3 block(SCORE_THREADS);
#define ASP_SCORE_LAUNCH(GG)                                                                                    \
  (s.kv == 0 ? launch_recording(score_mfma_kernel<D, GG, HIST>, grid, block, st, done, q_pred,                   \
                                static_cast<const uint16_t*>(k), seq_lens, scores, hist, s.Hq, s.Hkv, s.T_cap)   \
             : launch_recording(score_valu_kernel<D, GG, HIST>, grid, block, st, done, q_pred,                   \
                                static_cast<const float*>(k), seq_lens, scores, hist, s.Hq, s.Hkv, s.T_cap))
  hipError_t e;
  switch (s.G) {
    case 1: e = ASP_SCORE_LAUNCH(1); break;
    case 2: e = ASP_SCORE_LAUNCH(2); break;
    case 4: e = ASP_SCORE_LAUNCH(4); break;
    case 8: e = ASP_SCORE_LAUNCH(8); break;
    default: return hipErrorInvalidValue;
  }
#undef ASP_SCORE_LAUNCH
  return e;
}

__global__ void __launch_bounds__(256) clear_u32_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_clear_u32(uint32_t* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(clear_u32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_score(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens, float* scores,
                        uint32_t* hist, hipStream_t st, hipEvent_t done) {
  if (s.B == 0) return done ? hipEventRecord(done, st) : hipSuccess;
  if (hist != nullptr)
    return s.D == 64 ? launch_score_dh<64, true>(s, q_pred, k, seq_lens, scores, hist, st, done)
                     : launch_score_dh<128, true>(s, q_pred, k, seq_lens, scores, hist, st, done);
  return s.D == 64 ? launch_score_dh<64, false>(s, q_pred, k, seq_lens, scores, nullptr, st, done)
                   : launch_score_dh<128, false>(s, q_pred, k, seq_lens, scores, nullptr, st, done);
}

}  // namespace asp
