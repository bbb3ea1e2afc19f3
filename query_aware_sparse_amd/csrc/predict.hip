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
//  3. the ridge system of the largest window is factorised by a register
//     Cholesky (lane i holds row i, columns are broadcast with readlane); every
//     smaller window's system is a leading block, so the same factor and the
//     same forward substitution serve all windows;
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

__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmax(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

constexpr int PRED_THREADS = 64;
constexpr int XS = 128 + 1;  // LDS row stride of the staged lags (floats); +1 avoids bank conflicts

// PB: a bound on P = (largest window) - 1; PB + 1 is a multiple of 4 and at most 64.
template <int PB>
__global__ void __launch_bounds__(PRED_THREADS) predict_kernel(float* __restrict__ q_hist,
                                                               const int32_t* __restrict__ newest,
                                                               const int32_t* __restrict__ len,
                                                               const float* __restrict__ q_cur,
                                                               float* __restrict__ q_pred,
                                                               uint32_t* __restrict__ hist_zero, int Hq, int Hkv,
                                                               int W, int D, double lambda) {
  constexpr int NR = ((PB + 1 + 15) / 16) * 16;  // lag rows staged (whole 16-row MFMA tiles)
  __shared__ float X[NR * XS];
  __shared__ double M[NR * NR];  // Gram of lags 0..P; later reused for L
  __shared__ double cw[NR];      // pooled weight of each lag

  const int t = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  float* ring = q_hist + (size_t)bh * W * D;
  float* out = q_pred + (size_t)bh * D;

  if (hist_zero != nullptr) {  // the G heads of a KV head clear its histogram row together
    const int G = Hq / Hkv, h = bh % Hq;
    uint32_t* row = hist_zero + ((size_t)b * Hkv + h / G) * HIST_BINS;
    const int per = HIST_BINS / G, j0 = (h % G) * per;
    for (int j = j0 + t; j < j0 + per; j += PRED_THREADS) row[j] = 0u;
  }

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
  for (int e = t; e < NT * 16 * D; e += PRED_THREADS) {
    const int j = e / D, d = e % D;
    float v = 0.0f;
    if (j <= P) {
      if (push && j == 0) {
        v = qc[d];
      } else {
        int slot = (on - j + shift) % W;
        if (slot < 0) slot += W;
        v = ring[(size_t)slot * D + d];
      }
    }
    X[j * XS + d] = v;
  }
  __syncthreads();

  // 2. Gram matrix M[a][c] = <lag a, lag c>, fp64 MFMA over 16x16 tiles.  The
  // contraction index k = 4s + lane/16 walks all D coordinates.
  const int lr = t & 15, lk = t >> 4;
  for (int ti = 0; ti < NT; ++ti) {
    for (int tj = ti; tj < NT; ++tj) {
      f64x4 acc = {0.0, 0.0, 0.0, 0.0};
      const float* xa = X + (ti * 16 + lr) * XS + lk;
      const float* xb = X + (tj * 16 + lr) * XS + lk;
      for (int s = 0; s < D / 4; ++s)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[4 * s], (double)xb[4 * s], acc, 0, 0, 0);
      // lane t, register r holds tile element (t/16 + 4r, t%16)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti * 16 + lk + 4 * r, j = tj * 16 + lr;
        M[i * NR + j] = acc[r];
        M[j * NR + i] = acc[r];
      }
    }
  }
  __syncthreads();

  // 3. Ridge system of the largest window over lags 1..P:
  //    A[i][j] = M[i+1][j+1] + lambda [i == j],  r_i = M[0][i+1]; lane i owns row i.
  double a[PB];
#pragma unroll
  for (int j = 0; j < PB; ++j)
    a[j] = (t < P && j < P) ? M[(t + 1) * NR + (j + 1)] + (j == t ? lambda : 0.0) : 0.0;
  double y = t < P ? M[t + 1] : 0.0;
  double invd = 0.0;
  // Cholesky A = L L^T (right-looking; column k is broadcast lane by lane).
#pragma unroll
  for (int k = 0; k < PB; ++k) {
    if (k < P) {
      const double dk = sqrt(readlane_f64(a[k], k));
      const double ik = 1.0 / dk;
      if (t == k) {
        a[k] = dk;
        invd = ik;
      } else if (t > k) {
        a[k] *= ik;
      }
#pragma unroll
      for (int j = k + 1; j < PB; ++j) {
        if (j < P) {
          const double ljk = readlane_f64(a[k], j);
          if (t >= j) a[j] = fma(-a[k], ljk, a[j]);
        }
      }
    }
  }
  // Forward substitution L y = r (shared by every window).
#pragma unroll
  for (int k = 0; k < PB; ++k) {
    if (k < P) {
      if (t == k) y *= invd;
      const double yk = readlane_f64(y, k);
      if (t > k) y = fma(-a[k], yk, y);
    }
  }
  // Transpose L through LDS so that lane k holds column k: lt[i] = L[i][k].
  __syncthreads();
  if (t < P) {
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (j <= t) M[t * NR + j] = a[j];
  }
  __syncthreads();
  double lt[PB];
#pragma unroll
  for (int i = 0; i < PB; ++i) lt[i] = (i < P && i > t) ? M[i * NR + t] : 0.0;

  // 4. Back substitutions L_p^T beta = y_p of every window, side by side.
  int pw[3];
  double z[3], beta[3];
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    pw[w] = w < nw ? wset[w] - 1 : 0;
    z[w] = t < pw[w] ? y : 0.0;
    beta[w] = 0.0;
  }
#pragma unroll
  for (int i = PB - 1; i >= 0; --i) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      if (i < pw[w]) {
        if (t == i) beta[w] = z[w] * invd;
        const double bi = readlane_f64(beta[w], i);
        if (t < i) z[w] = fma(-lt[i], bi, z[w]);
      }
    }
  }
  // Softmax over each window's lag weights; lane t carries lag t+1, whose
  // one-step-ahead partner is lag t.  Pool: weight / number of windows.
  double c = 0.0;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (w < nw) {
      const bool in = t < pw[w];
      const double m = wave_max_f64(in ? beta[w] : -INFINITY);
      const double e = in ? exp(beta[w] - m) : 0.0;
      const double sum = wave_sum_f64(e);
      c += e / sum;
    }
  }
  if (t < NR) cw[t] = t < P ? c / nw : 0.0;
  __syncthreads();
  for (int d = t; d < D; d += PRED_THREADS) {
    double acc = 0.0;
    for (int j = 0; j < P; ++j) acc = fma(cw[j], (double)X[j * XS + d], acc);
    out[d] = (float)acc;
  }
}

hipError_t launch_predict(const Shape& s, float* q_hist, const int32_t* newest, const int32_t* len,
                          const float* q_cur, float* q_pred, uint32_t* hist_zero, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const dim3 grid(s.B * s.Hq), block(PRED_THREADS);
  const int P = s.W - 1;
#define ASP_PRED_LAUNCH(PB)                                                                                      \
  hipLaunchKernelGGL(predict_kernel<PB>, grid, block, 0, st, q_hist, newest, len, q_cur, q_pred, hist_zero, s.Hq, \
                     s.Hkv, s.W, s.D, s.lambda)
  if (P <= 3) ASP_PRED_LAUNCH(3);
  else if (P <= 7) ASP_PRED_LAUNCH(7);
  else if (P <= 15) ASP_PRED_LAUNCH(15);
  else if (P <= 31) ASP_PRED_LAUNCH(31);
  else ASP_PRED_LAUNCH(63);
#undef ASP_PRED_LAUNCH
  return hipGetLastError();
}

}  // namespace asp
