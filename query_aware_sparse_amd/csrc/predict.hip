// Query-history push and next-query prediction (softmax-normalised ridge
// regression with multi-window average pooling).
//
// Sources: atlas.scime.ai research-map summary of AsyncSpade, "Approach" (the
// next query is predicted from a short window of recent queries by a ridge
// regression with softmax-normalised weights, pooled over several windows);
// arXiv 2510.07486 abstract (a light-weight, training-free temporal-regressive
// module, one formulation for every head and layer); reproduction card
// "What reproduces" table (linear one-step-ahead ridge prediction, a recent
// window of 16 queries).  The pages print no equations; the reading
// implemented is the one documented on asp_predict_query in include/asp.h.
//
// One 64-lane wavefront per (sequence, query head):
//  1. the lags q_t .. q_{t-P} (P = largest window - 1) are staged in LDS;
//  2. their Gram matrix is accumulated in fp64 with v_mfma_f64_16x16x4 (fp32
//     inputs widen exactly, so the products are exact);
//  3. the ridge system of the largest window is factorised as L D L^T in
//     registers (lane i holds row i, columns are broadcast with readlane, the
//     pivots inverted by v_rcp_f64 plus Newton steps); every smaller window's
//     system is a leading block, so the same factor and the same forward
//     substitution serve all windows;
//  4. the back substitutions of all windows run side by side, then each
//     window's softmax runs across lanes, and the window predictions are
//     pooled as one weighted sum of the lags.
#include "asp_internal.h"

namespace asp {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// One workgroup per sequence: copy its Hq queries into the next ring slot, then
// advance the slot and the length (after every thread has read the old slot).
__global__ void __launch_bounds__(256) push_kernel(const float* __restrict__ q_cur, float* __restrict__ q_hist,
                                                   int32_t* __restrict__ newest, int32_t* __restrict__ len,
                                                   int Hq, int W, int D) {
  const int b = blockIdx.x;
  int old = newest[b] % W;
  if (old < 0) old += W;
  const int slot = old + 1 == W ? 0 : old + 1;
  const int n = clampi(len[b], 0, W);
  const float4* src = reinterpret_cast<const float4*>(q_cur + (size_t)b * Hq * D);
  const int d4 = D / 4;
  for (int e = threadIdx.x; e < Hq * d4; e += blockDim.x) {
    const int h = e / d4, c = e % d4;
    float4* dst = reinterpret_cast<float4*>(q_hist + (((size_t)b * Hq + h) * W + slot) * D);
    dst[c] = src[e];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    newest[b] = slot;
    len[b] = n + 1 > W ? W : n + 1;
  }
}

hipError_t launch_push(const Shape& s, const float* q_cur, float* q_hist, int32_t* newest, int32_t* len,
                       hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  hipLaunchKernelGGL(push_kernel, dim3(s.B), dim3(256), 0, st, q_cur, q_hist, newest, len, s.Hq, s.W, s.D);
  return hipGetLastError();
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(v & 0xffffffffll), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
// Reductions over the lanes 0 .. 16*ROWS-1 that hold values (other lanes must
// hold the identity); DPP inside each 16-lane row, shuffles across rows.
template <int ROWS>
__device__ __forceinline__ double lanes_max_f64(double x) {
  x = fmax(x, dpp_f64<DPP_QUAD_XOR1>(x));
  x = fmax(x, dpp_f64<DPP_QUAD_XOR2>(x));
  x = fmax(x, dpp_f64<DPP_ROW_HALF_MIRROR>(x));
  x = fmax(x, dpp_f64<DPP_ROW_MIRROR>(x));
  if constexpr (ROWS > 1) x = fmax(x, __shfl_xor(x, 16));
  if constexpr (ROWS > 2) x = fmax(x, __shfl_xor(x, 32));
  return x;
}
template <int ROWS>
__device__ __forceinline__ double lanes_sum_f64(double x) {
  x += dpp_f64<DPP_QUAD_XOR1>(x);
  x += dpp_f64<DPP_QUAD_XOR2>(x);
  x += dpp_f64<DPP_ROW_HALF_MIRROR>(x);
  x += dpp_f64<DPP_ROW_MIRROR>(x);
  if constexpr (ROWS > 1) x += __shfl_xor(x, 16);
  if constexpr (ROWS > 2) x += __shfl_xor(x, 32);
  return x;
}

constexpr int PRED_THREADS = 64;
constexpr int XS = 128 + 1;  // LDS row stride of the staged lags (floats); +1 avoids bank conflicts

// Stage lag rows 0..P of one head into LDS (rows P+1 .. 16*NT-1 are zeroed).
// Lag j is q_cur for j == 0 when qc is given, else ring slot (on - j + shift)
// mod W.  Every lane issues all of its 16-byte loads of a tile before storing.
template <int DD>
__device__ __forceinline__ void stage_lags(float* X, const float* ring, const float* qc, int P, int NT, int on,
                                           int shift, int W, int t) {
  constexpr int C4 = DD / 4;                   // float4 per row
  constexpr int PER = 16 * C4 / PRED_THREADS;  // float4 per lane per 16-row tile
  for (int ti = 0; ti < NT; ++ti) {
    float4 v[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int idx = it * PRED_THREADS + t;
      const int j = ti * 16 + idx / C4, c4 = idx % C4;
      float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (j <= P) {
        const float* src;
        if (qc != nullptr && j == 0) {
          src = qc;
        } else {
          int slot = on - j + shift;  // in [-(W-1), W-1]
          if (slot < 0) slot += W;
          src = ring + (size_t)slot * DD;
        }
        x = reinterpret_cast<const float4*>(src)[c4];
      }
      v[it] = x;
    }
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int idx = it * PRED_THREADS + t;
      float* dst = X + (ti * 16 + idx / C4) * XS + 4 * (idx % C4);
      dst[0] = v[it].x;
      dst[1] = v[it].y;
      dst[2] = v[it].z;
      dst[3] = v[it].w;
    }
  }
}

// Solves the ridge systems of every window from the Gram matrix M of lags
// 0..P (row stride NR) and returns, in lane t < P, the pooled weight of lag t:
// (1 / #windows) * sum over windows w with t < p_w of softmax(beta_w)[t].
//  A[i][j] = M[i+1][j+1] + lambda [i == j] (lags 1..P), r_i = M[0][i+1].
// A = L diag(dd) L^T with L unit lower triangular (no square roots); lane i
// holds row i, column k is broadcast with readlane, each pivot is inverted by
// v_rcp_f64 and two Newton steps.  Every window's system is a leading block of
// A, so the factor and the forward substitution are shared; the back
// substitutions of all windows run side by side.
// EXACT: P == PB and the window set is {P+1, (P+1)/2, (P+1)/4} minus windows
// below 2, so every loop bound is a compile-time constant and no lane needs a
// guard (entries above the diagonal may collect garbage: they are never read).
template <int PB, int NR, bool EXACT>
__device__ __forceinline__ double pooled_weights(double* M, double lambda, int P, int nw, const int* wset, int t) {
  double a[PB];
#pragma unroll
  for (int j = 0; j < PB; ++j)
    a[j] = ((EXACT || (t < P && j < P)) && t < PB) ? M[(t + 1) * NR + (j + 1)] + (j == t ? lambda : 0.0) : 0.0;
  double y = (t < P && t < PB) ? M[t + 1] : 0.0;
  double invd = 0.0;  // 1 / dd_t in lane t
#pragma unroll
  for (int k = 0; k < PB; ++k) {
    if (EXACT || k < P) {
      const double dk = readlane_f64(a[k], k);
      double rk = __builtin_amdgcn_rcp(dk);
      rk = fma(rk, fma(-dk, rk, 1.0), rk);  // Newton steps: ~2^-22 -> full precision
      rk = fma(rk, fma(-dk, rk, 1.0), rk);
      invd = t == k ? rk : invd;
      const double w = t > k ? a[k] * rk : 0.0;  // L[t][k] below the diagonal
#pragma unroll
      for (int j = k + 1; j < PB; ++j) {
        if (EXACT || j < P) {
          const double ljk = readlane_f64(w, j);  // L[j][k]
          a[j] = fma(-a[k], ljk, a[j]);           // A[t][j] -= A[t][k] L[j][k]
        }
      }
      a[k] = t > k ? w : a[k];
    }
  }
  // Forward substitution L z = r (unit diagonal), then y = z / dd.
#pragma unroll
  for (int k = 0; k < PB; ++k) {
    if (EXACT || k < P) {
      const double zk = readlane_f64(y, k);
      y = t > k ? fma(-a[k], zk, y) : y;
    }
  }
  y *= invd;
  // Transpose L through LDS so that lane k holds column k: lt[i] = L[i][k].
  __syncthreads();
  if (t < P) {
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (j < t) M[t * NR + j] = a[j];
  }
  __syncthreads();
  double lt[PB];
#pragma unroll
  for (int i = 0; i < PB; ++i) lt[i] = ((EXACT || i < P) && i > t) ? M[i * NR + t] : 0.0;

  // Window sizes p_w = w - 1 (zero for an absent window).
  int pw[3];
  if constexpr (EXACT) {
    pw[0] = PB;
    pw[1] = (PB + 1) / 2 >= 2 ? (PB + 1) / 2 - 1 : 0;
    pw[2] = (PB + 1) / 4 >= 2 ? (PB + 1) / 4 - 1 : 0;
  } else {
#pragma unroll
    for (int w = 0; w < 3; ++w) pw[w] = w < nw ? wset[w] - 1 : 0;
  }
  // L^T beta = y (unit diagonal) on each window's leading block.
  double z[3], beta[3];
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    z[w] = t < pw[w] ? y : 0.0;
    beta[w] = 0.0;
  }
#pragma unroll
  for (int i = PB - 1; i >= 0; --i) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      if (i < pw[w]) {
        const double bi = readlane_f64(z[w], i);
        beta[w] = t == i ? bi : beta[w];
        z[w] = t < i ? fma(-lt[i], bi, z[w]) : z[w];
      }
    }
  }
  // Softmax over each window's lag weights (lane t carries lag t+1, whose
  // one-step-ahead partner is lag t), pooled over the windows.
  constexpr int ROWS = (PB + 15) / 16;  // lanes t < P <= PB hold the weights
  int nwin = 0;
  double c = 0.0;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (pw[w] > 0) {
      const bool in = t < pw[w];
      const double m = lanes_max_f64<ROWS>(in ? beta[w] : -INFINITY);
      const double e = in ? exp(beta[w] - m) : 0.0;
      const double sum = lanes_sum_f64<ROWS>(e);
      c += e / sum;
      ++nwin;
    }
  }
  return c / nwin;
}

// PB: a bound on P = (largest window) - 1; PB + 1 is a multiple of 4 and at most 64.
// DD: head_dim (64 or 128), a compile-time bound so that the Gram loop unrolls.
template <int PB, int DD>
__global__ void __launch_bounds__(PRED_THREADS) predict_kernel(float* __restrict__ q_hist,
                                                               const int32_t* __restrict__ newest,
                                                               const int32_t* __restrict__ len,
                                                               const float* __restrict__ q_cur,
                                                               float* __restrict__ q_pred,
                                                               int Hq,
                                                               int W, double lambda) {
  constexpr int D = DD;
  constexpr int NR = ((PB + 1 + 15) / 16) * 16;  // lag rows staged (whole 16-row MFMA tiles)
  __shared__ float X[NR * XS];
  __shared__ double M[NR * NR];  // Gram of lags 0..P; later reused for L
  __shared__ double cw[NR];      // pooled weight of each lag

  const int t = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  float* ring = q_hist + (size_t)bh * W * D;
  float* out = q_pred + (size_t)bh * D;

  int on = newest[b] % W;
  if (on < 0) on += W;
  const int old_n = clampi(len[b], 0, W);
  const bool push = q_cur != nullptr;
  const float* qc = push ? q_cur + (size_t)bh * D : nullptr;
  const int n = push ? min(old_n + 1, W) : old_n;
  // Lag j lives in ring slot (on - j) without a push, (on - j + 1) with one
  // (lag 0 then being q_cur itself).
  const int shift = push ? 1 : 0;
  if (push) {
    // The next slot held lag W-1 of the ring before the push, which no window
    // reads (the largest window uses lags 0..W-1 counted after the push).
    const int slot = on + 1 == W ? 0 : on + 1;
    for (int d = t; d < D; d += PRED_THREADS) ring[(size_t)slot * D + d] = qc[d];
  }

  if (n == 0) {
    for (int d = t; d < D; d += PRED_THREADS) out[d] = 0.0f;
    return;
  }
  int wset[3] = {0, 0, 0};
  int nw = 0;
  {
    const int cand[3] = {W, W / 2, W / 4};
#pragma unroll
    for (int c = 0; c < 3; ++c)
      if (cand[c] >= 2 && cand[c] <= n) wset[nw++] = cand[c];
  }
  if (nw == 0) {  // a single query held: predict it unchanged
    for (int d = t; d < D; d += PRED_THREADS) {
      int slot = on;
      out[d] = push ? qc[d] : ring[(size_t)slot * D + d];
    }
    return;
  }
  const int P = wset[0] - 1;
  const int NT = (P + 1 + 15) / 16;

  // 1. Stage lags 0..P (rows up to the tile boundary are zero).
  stage_lags<DD>(X, ring, qc, P, NT, on, shift, W, t);
  __syncthreads();

  // 2. Gram matrix M[a][c] = <lag a, lag c>, fp64 MFMA over 16x16 tiles.  The
  // contraction index k = 4s + lane/16 walks all D coordinates.
  const int lr = t & 15, lk = t >> 4;
  for (int ti = 0; ti < NT; ++ti) {
    for (int tj = ti; tj < NT; ++tj) {
      // Four independent accumulation chains (coordinates 16m + 4q + lk for
      // chain q) keep the MFMA pipeline busy; they are summed at the end.
      f64x4 acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f64x4{0.0, 0.0, 0.0, 0.0};
      const float* xa = X + (ti * 16 + lr) * XS + lk;
      const float* xb = X + (tj * 16 + lr) * XS + lk;
#pragma unroll
      for (int m = 0; m < D / 16; ++m) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[16 * m + 4 * q], (double)xb[16 * m + 4 * q],
                                                        acc[q], 0, 0, 0);
      }
      const f64x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      // lane t, register r holds tile element (t/16 + 4r, t%16)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti * 16 + lk + 4 * r, j = tj * 16 + lr;
        M[i * NR + j] = sum[r];
        M[j * NR + i] = sum[r];
      }
    }
  }
  __syncthreads();

  // 3-4. Ridge solves of every window and the pooled lag weights.
  double c;
  if (P == PB)  // the ring is full: sizes and window set are compile-time
    c = pooled_weights<PB, NR, true>(M, lambda, P, nw, wset, t);
  else
    c = pooled_weights<PB, NR, false>(M, lambda, P, nw, wset, t);
  if (t < NR) cw[t] = t < P ? c : 0.0;
  __syncthreads();
  for (int d = t; d < D; d += PRED_THREADS) {
    double acc = 0.0;
    for (int j = 0; j < P; ++j) acc = fma(cw[j], (double)X[j * XS + d], acc);
    out[d] = (float)acc;
  }
}

hipError_t launch_predict(const Shape& s, float* q_hist, const int32_t* newest, const int32_t* len,
                          const float* q_cur, float* q_pred, hipStream_t st, hipEvent_t done) {
  if (s.B == 0) return done ? hipEventRecord(done, st) : hipSuccess;
  const dim3 grid(s.B * s.Hq), block(PRED_THREADS);
  const int P = s.W - 1;
#define ASP_PRED_LAUNCH(PB)                                                                                  \
  (s.D == 64 ? launch_recording(predict_kernel<PB, 64>, grid, block, st, done, q_hist, newest, len, q_cur, q_pred,  \
                                s.Hq, s.W, s.lambda)                                                            \
             : launch_recording(predict_kernel<PB, 128>, grid, block, st, done, q_hist, newest, len, q_cur, q_pred, \
                                s.Hq, s.W, s.lambda))
  hipError_t e;
  if (P <= 3) e = ASP_PRED_LAUNCH(3);
  else if (P <= 7) e = ASP_PRED_LAUNCH(7);
  else if (P <= 15) e = ASP_PRED_LAUNCH(15);
  else if (P <= 31) e = ASP_PRED_LAUNCH(31);
  else e = ASP_PRED_LAUNCH(63);
#undef ASP_PRED_LAUNCH
  return e;
}

}  // namespace asp
