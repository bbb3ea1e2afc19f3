// Launches of the score pass; the block bodies are in score_block.h.
#include "score_block.h"

namespace asp {

template <int D, int G, bool HIST, int OUT>
__device__ __forceinline__ void score_mfma_grid(const float* __restrict__ q_pred, const uint16_t* __restrict__ k,
                                                const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                                                uint32_t* __restrict__ hist, const CandWs& cw, int Hq, int Hkv,
                                                int T_cap, unsigned char* smem) {
  // The rescoring launch follows every selection and usually finds no unit
  // flagged: its workgroups (a few per unit) then leave at once; those of a
  // flagged unit loop over its key blocks.
  if constexpr (OUT == OUT_ALL_FLAGGED) {
    if (cw.flag[blockIdx.y] == 0u) return;
    const int nblk = (T_cap + SCORE_KEYS_PER_BLOCK - 1) / SCORE_KEYS_PER_BLOCK;
    for (int bx = blockIdx.x; bx < nblk; bx += gridDim.x)
      score_mfma_block<D, G, HIST, OUT>(q_pred, k, seq_lens, scores, hist, cw, Hq, Hkv, T_cap, bx, blockIdx.y, smem);
    return;
  }
  // Otherwise one key block per workgroup: a loop here slows the launch inside the step.
  score_mfma_block<D, G, HIST, OUT>(q_pred, k, seq_lens, scores, hist, cw, Hq, Hkv, T_cap, blockIdx.x, blockIdx.y, smem);
}

// Streaming launches (G >= 2, score rows or kept keys) are held to 128
// registers per lane, four waves per SIMD: with fewer waves resident the
// launch loses more to the kernels that share its CUs inside a step than it
// gains alone.  The rescoring launch and G = 1 would spill under that cap and
// run without it.
template <int D, int G, bool HIST, int OUT>
constexpr bool score_regs_capped() {
  return G >= 2 && OUT != OUT_ALL_FLAGGED;
}

template <int D, int G, bool HIST, int OUT>
__global__ void __launch_bounds__(SCORE_THREADS) __attribute__((amdgpu_waves_per_eu(4, 8)))
score_mfma_kernel(const float* __restrict__ q_pred, const uint16_t* __restrict__ k,
                  const int32_t* __restrict__ seq_lens, float* __restrict__ scores, uint32_t* __restrict__ hist,
                  CandWs cw, int Hq, int Hkv, int T_cap) {
  __shared__ __align__(16) unsigned char smem[score_mfma_lds_bytes<D, HIST, OUT>()];
  score_mfma_grid<D, G, HIST, OUT>(q_pred, k, seq_lens, scores, hist, cw, Hq, Hkv, T_cap, smem);
}

template <int D, int G, bool HIST, int OUT>
__global__ void __launch_bounds__(SCORE_THREADS)
score_mfma_kernel_uncapped(const float* __restrict__ q_pred, const uint16_t* __restrict__ k,
                           const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                           uint32_t* __restrict__ hist, CandWs cw, int Hq, int Hkv, int T_cap) {
  __shared__ __align__(16) unsigned char smem[score_mfma_lds_bytes<D, HIST, OUT>()];
  score_mfma_grid<D, G, HIST, OUT>(q_pred, k, seq_lens, scores, hist, cw, Hq, Hkv, T_cap, smem);
}

template <int D, int G, bool HIST, int OUT>
static hipError_t launch_mfma(dim3 grid, dim3 block, hipStream_t st, hipEvent_t done, const float* q_pred,
                              const uint16_t* k, const int32_t* seq_lens, float* scores, uint32_t* hist,
                              const CandWs& cw, int Hq, int Hkv, int T_cap) {
  if constexpr (score_regs_capped<D, G, HIST, OUT>())
    return launch_recording(score_mfma_kernel<D, G, HIST, OUT>, grid, block, st, done, q_pred, k, seq_lens, scores,
                            hist, cw, Hq, Hkv, T_cap);
  else
    return launch_recording(score_mfma_kernel_uncapped<D, G, HIST, OUT>, grid, block, st, done, q_pred, k, seq_lens,
                            scores, hist, cw, Hq, Hkv, T_cap);
}

template <int D, int G, bool HIST, int OUT>
__global__ void __launch_bounds__(SCORE_THREADS) score_valu_kernel(const float* __restrict__ q_pred,
                                                                   const float* __restrict__ k,
                                                                   const int32_t* __restrict__ seq_lens,
                                                                   float* __restrict__ scores,
                                                                   uint32_t* __restrict__ hist, CandWs cw, int Hq,
                                                                   int Hkv, int T_cap) {
  __shared__ __align__(16) unsigned char smem[score_valu_lds_bytes<HIST, OUT>()];
  if constexpr (OUT == OUT_ALL_FLAGGED) {
    if (cw.flag[blockIdx.y] == 0u) return;
    const int nblk = (T_cap + SCORE_KEYS_PER_BLOCK - 1) / SCORE_KEYS_PER_BLOCK;
    for (int bx = blockIdx.x; bx < nblk; bx += gridDim.x)
      score_valu_block<D, G, HIST, OUT>(q_pred, k, seq_lens, scores, hist, cw, Hq, Hkv, T_cap, bx, blockIdx.y, smem);
    return;
  }
  score_valu_block<D, G, HIST, OUT>(q_pred, k, seq_lens, scores, hist, cw, Hq, Hkv, T_cap, blockIdx.x, blockIdx.y, smem);
}

// Workgroups per unit of the rescoring launch.
constexpr int RESCORE_BLOCKS_PER_UNIT = 4;

template <int D, bool HIST, int OUT>
static hipError_t launch_score_dh(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                  float* scores, uint32_t* hist, const CandWs& cw, hipStream_t st, hipEvent_t done) {
  const int nblk = (s.T_cap + SCORE_KEYS_PER_BLOCK - 1) / SCORE_KEYS_PER_BLOCK;
  const int gx = OUT == OUT_ALL_FLAGGED && nblk > RESCORE_BLOCKS_PER_UNIT ? RESCORE_BLOCKS_PER_UNIT : nblk;
  const dim3 grid(gx, s.B * s.Hkv);
  const dim3 block(SCORE_THREADS);
#define ASP_SCORE_LAUNCH(GG)                                                                                      \
  (s.kv == 0 ? launch_mfma<D, GG, HIST, OUT>(grid, block, st, done, q_pred, static_cast<const uint16_t*>(k),      \
                                             seq_lens, scores, hist, cw, s.Hq, s.Hkv, s.T_cap)                    \
             : launch_recording(score_valu_kernel<D, GG, HIST, OUT>, grid, block, st, done, q_pred,                \
                                static_cast<const float*>(k), seq_lens, scores, hist, cw, s.Hq, s.Hkv, s.T_cap))
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
  const CandWs none{};
  if (hist != nullptr)
    return s.D == 64 ? launch_score_dh<64, true, OUT_SCORES>(s, q_pred, k, seq_lens, scores, hist, none, st, done)
                     : launch_score_dh<128, true, OUT_SCORES>(s, q_pred, k, seq_lens, scores, hist, none, st, done);
  return s.D == 64 ? launch_score_dh<64, false, OUT_SCORES>(s, q_pred, k, seq_lens, scores, nullptr, none, st, done)
                   : launch_score_dh<128, false, OUT_SCORES>(s, q_pred, k, seq_lens, scores, nullptr, none, st, done);
}

hipError_t launch_score_candidates(const Shape& s, const float* q_pred, const void* k, const int32_t* seq_lens,
                                   const CandWs& cw, bool fallback, hipStream_t st, hipEvent_t done) {
  if (s.B == 0) return done ? hipEventRecord(done, st) : hipSuccess;
  if (fallback)
    return s.D == 64 ? launch_score_dh<64, false, OUT_ALL_FLAGGED>(s, q_pred, k, seq_lens, nullptr, nullptr, cw, st,
                                                                    done)
                     : launch_score_dh<128, false, OUT_ALL_FLAGGED>(s, q_pred, k, seq_lens, nullptr, nullptr, cw, st,
                                                                     done);
  return s.D == 64
             ? launch_score_dh<64, false, OUT_ABOVE_HINT>(s, q_pred, k, seq_lens, nullptr, nullptr, cw, st, done)
             : launch_score_dh<128, false, OUT_ABOVE_HINT>(s, q_pred, k, seq_lens, nullptr, nullptr, cw, st, done);
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

size_t cand_ws_bytes(const Shape& s) {
  const size_t units = (size_t)s.B * s.Hkv, nr = (size_t)cand_regions(s.T_cap);
  return align256(units * 4) + align256(units * 4) + align256(units * nr * 4) +
         align256(units * nr * CAND_REGION * sizeof(uint2));
}

CandWs cand_carve(const Shape& s, void* ws) {
  const size_t units = (size_t)s.B * s.Hkv, nr = (size_t)cand_regions(s.T_cap);
  unsigned char* p = static_cast<unsigned char*>(ws);
  CandWs w;
  w.hint = reinterpret_cast<uint32_t*>(p);
  p += align256(units * 4);
  w.flag = reinterpret_cast<uint32_t*>(p);
  p += align256(units * 4);
  w.rcount = reinterpret_cast<uint32_t*>(p);
  p += align256(units * nr * 4);
  w.cand = reinterpret_cast<uint2*>(p);
  return w;
}

}  // namespace asp
