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
// Work per (sequence, query head) is tiny (a 16x16 Gram matrix at W = 16), so
// one 64-lane wavefront handles one head: the Gram matrix is accumulated in
// fp64 (products of fp32 values are exact in fp64), factorised once by
// Cholesky and reused by every window, because the system of a smaller window
// is the leading block of the largest one.
#include "asp_internal.h"

namespace asp {

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

// LDS layout of the predictor (dynamic shared memory, sized per launch):
//   X     [W][D + 1] float   lag rows, X[j] = q_{t-j}; +1 pad breaks bank conflicts
//   M     [W][W]     double  Gram of lags 0..P (only the upper triangle filled)
//   A     [W][W]     double  ridge system, factorised in place (lower triangle)
//   y     [W]        double  forward-substitution result, shared by all windows
//   z     [W]        double  back-substitution scratch
//   coef  [W]        double  beta, then alpha of the current window
constexpr int PRED_THREADS = 64;

size_t predict_lds_bytes(int W, int D) {
  size_t x = (size_t)W * (D + 1) * sizeof(float);
  x = (x + 7) & ~(size_t)7;
  return x + sizeof(double) * ((size_t)W * W * 2 + 3 * (size_t)W);
}

__global__ void __launch_bounds__(PRED_THREADS) predict_kernel(const float* __restrict__ q_hist,
                                                               const int32_t* __restrict__ newest,
                                                               const int32_t* __restrict__ len,
                                                               float* __restrict__ q_pred, int Hq, int W, int D,
                                                               double lambda) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int t = threadIdx.x;
  const int xs = D + 1;
  float* X = reinterpret_cast<float*>(smem);
  size_t xbytes = ((size_t)W * xs * sizeof(float) + 7) & ~(size_t)7;
  double* M = reinterpret_cast<double*>(smem + xbytes);
  double* A = M + W * W;
  double* y = A + W * W;
  double* z = y + W;
  double* coef = z + W;

  const int n = clampi(len[b], 0, W);
  int nw_slot = newest[b] % W;
  if (nw_slot < 0) nw_slot += W;
  float* out = q_pred + (size_t)bh * D;
  const float* ring = q_hist + (size_t)bh * W * D;

  if (n == 0) {  // no history: predict zero
    for (int d = t; d < D; d += PRED_THREADS) out[d] = 0.0f;
    return;
  }
  // Window set {W, W/2, W/4} restricted to 2 <= w <= n, largest first.
  int wset[3];
  int nw = 0;
  {
    const int cand[3] = {W, W / 2, W / 4};
    for (int c = 0; c < 3; ++c)
      if (cand[c] >= 2 && cand[c] <= n) wset[nw++] = cand[c];
  }
  if (nw == 0) {  // a single query held: predict it unchanged
    const float* q0 = ring + (size_t)nw_slot * D;
    for (int d = t; d < D; d += PRED_THREADS) out[d] = q0[d];
    return;
  }
  const int P = wset[0] - 1;  // lags used by the largest window

  // Stage lags 0..P (newest first) in LDS.
  for (int e = t; e < (P + 1) * D; e += PRED_THREADS) {
    const int j = e / D, d = e % D;
    int slot = nw_slot - j;
    if (slot < 0) slot += W;
    X[j * xs + d] = ring[(size_t)slot * D + d];
  }
  __syncthreads();

  // Gram entries M[a][c] = <q_{t-a}, q_{t-c}> for 0 <= a <= c <= P, fp64.
  for (int a = 0; a <= P; ++a) {
    for (int c = a + t; c <= P; c += PRED_THREADS) {
      const float* xa = X + a * xs;
      const float* xc = X + c * xs;
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc = fma((double)xa[d], (double)xc[d], acc);
      M[a * W + c] = acc;
    }
  }
  __syncthreads();

  // Ridge system of the largest window: A = G_P + lambda I (lags 1..P), r = M[0][1..P].
  for (int e = t; e < P * P; e += PRED_THREADS) {
    const int i = e / P, j = e % P;
    if (j <= i) A[i * W + j] = M[(j + 1) * W + (i + 1)] + (i == j ? lambda : 0.0);
  }
  for (int i = t; i < P; i += PRED_THREADS) y[i] = M[0 * W + (i + 1)];
  __syncthreads();

  // Cholesky A = L L^T in place (lower triangle), right-looking, one row per lane.
  for (int k = 0; k < P; ++k) {
    if (t == 0) A[k * W + k] = sqrt(A[k * W + k]);
    __syncthreads();
    const double dkk = A[k * W + k];
    for (int i = k + 1 + t; i < P; i += PRED_THREADS) A[i * W + k] /= dkk;
    __syncthreads();
    for (int i = k + 1 + t; i < P; i += PRED_THREADS) {
      const double lik = A[i * W + k];
      for (int j = k + 1; j <= i; ++j) A[i * W + j] = fma(-lik, A[j * W + k], A[i * W + j]);
    }
    __syncthreads();
  }
  // Forward substitution L y = r (column oriented); y's leading entries serve
  // every smaller window unchanged.
  for (int i = 0; i < P; ++i) {
    if (t == 0) y[i] = y[i] / A[i * W + i];
    __syncthreads();
    const double yi = y[i];
    for (int k = i + 1 + t; k < P; k += PRED_THREADS) y[k] = fma(-A[k * W + i], yi, y[k]);
    __syncthreads();
  }

  double acc[128 / PRED_THREADS] = {0.0, 0.0};
  for (int wi = 0; wi < nw; ++wi) {
    const int p = wset[wi] - 1;
    // Back substitution L_p^T beta = y_p on the leading p x p block.
    for (int i = t; i < p; i += PRED_THREADS) z[i] = y[i];
    __syncthreads();
    for (int i = p - 1; i >= 0; --i) {
      if (t == 0) coef[i] = z[i] / A[i * W + i];
      __syncthreads();
      const double bi = coef[i];
      for (int k = t; k < i; k += PRED_THREADS) z[k] = fma(-A[i * W + k], bi, z[k]);
      __syncthreads();
    }
    // Softmax over the p lag weights (max subtracted first).
    if (t == 0) {
      double m = coef[0];
      for (int j = 1; j < p; ++j) m = fmax(m, coef[j]);
      double sum = 0.0;
      for (int j = 0; j < p; ++j) {
        const double e = exp(coef[j] - m);
        coef[j] = e;
        sum += e;
      }
      const double inv = 1.0 / sum;
      for (int j = 0; j < p; ++j) coef[j] *= inv;
    }
    __syncthreads();
    // One step ahead: weight j (j = 1..p) multiplies q_{t+1-j} = X[j-1].
    for (int r = 0, d = t; d < D; ++r, d += PRED_THREADS) {
      double s = 0.0;
      for (int j = 0; j < p; ++j) s = fma(coef[j], (double)X[j * xs + d], s);
      acc[r] += s;
    }
    __syncthreads();
  }
  const double inv_nw = 1.0 / nw;
  for (int r = 0, d = t; d < D; ++r, d += PRED_THREADS) out[d] = (float)(acc[r] * inv_nw);
}

hipError_t launch_predict(const Shape& s, const float* q_hist, const int32_t* newest, const int32_t* len,
                          float* q_pred, hipStream_t st) {
  if (s.B == 0) return hipSuccess;
  const size_t lds = predict_lds_bytes(s.W, s.D);
  hipLaunchKernelGGL(predict_kernel, dim3(s.B * s.Hq), dim3(PRED_THREADS), lds, st, q_hist, newest, len, q_pred,
                     s.Hq, s.W, s.D, s.lambda);
  return hipGetLastError();
}

}  // namespace asp
