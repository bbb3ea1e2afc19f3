/*
 * asp_oracle.c -- plain, slow CPU oracle for the AsyncSpade sparse decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the HIP library is
 * checked against.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it.  It shares no code, header, table or helper with the HIP
 * library under query_aware_sparse_amd/, and it never calls that library.
 *
 * Everything is computed in fp64 from the fp32 / bf16 inputs (each widened
 * exactly), in the plainest order the definitions allow: no blocking, fusion or
 * reuse across windows.  OpenMP only runs independent (sequence, head) units on
 * different threads; the arithmetic inside one unit is serial.
 *
 * Sources (the pages that describe the method):
 *   [card]     Hugging Face dataset card "Reproduction: AsyncSpade -- Efficient
 *              Test-Time Scaling with Asynchronous Sparse Decoding"
 *              (debajyotidasgupta/asyncspade-repro-artifacts).
 *   [summary]  atlas.scime.ai research-map page "AsyncSpade: Efficient Test-Time
 *              Scaling with Asynchronous Sparse Decoding" (AI-written summary).
 *   [abstract] arXiv 2510.07486 abstract, as shown on fugumt.com and
 *              searcharxiv.org.
 *
 * None of the pages prints the predictor's equations (the card names an
 * Algorithm 1 and Eqs. 1-11 of the paper without reproducing them), so every
 * step of oracle_predict_one below states the reading it implements.
 *
 * Parity pins: every function here is pinned by tests that do not call this
 * file's arithmetic again (closed forms, a least-squares route, brute-force
 * ranks, a library attention routine).  No function is parity-unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_KV_BF16 0
#define ORACLE_KV_F32 1

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double kv_at(const void* base, int kv_dtype, size_t i) {
  if (kv_dtype == ORACLE_KV_BF16) return bf16_bits_to_double(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Dense linear solve: Gaussian elimination with partial pivoting.            */
/* A is n x n row-major and is overwritten; rhs is overwritten; x receives    */
/* the solution.  Returns 0 on success, -1 on a zero pivot.                   */
/* ------------------------------------------------------------------------- */
static int solve_dense(int n, double* A, double* rhs, double* x) {
  for (int col = 0; col < n; ++col) {
    int piv = col;
    double best = fabs(A[col * n + col]);
    for (int r = col + 1; r < n; ++r) {
      double v = fabs(A[r * n + col]);
      if (v > best) { best = v; piv = r; }
    }
    if (best == 0.0) return -1;
    if (piv != col) {
      for (int c = 0; c < n; ++c) {
        double t = A[col * n + c]; A[col * n + c] = A[piv * n + c]; A[piv * n + c] = t;
      }
      double t = rhs[col]; rhs[col] = rhs[piv]; rhs[piv] = t;
    }
    for (int r = col + 1; r < n; ++r) {
      double f = A[r * n + col] / A[col * n + col];
      if (f == 0.0) continue;
      for (int c = col; c < n; ++c) A[r * n + c] -= f * A[col * n + c];
      rhs[r] -= f * rhs[col];
    }
  }
  for (int r = n - 1; r >= 0; --r) {
    double s = rhs[r];
    for (int c = r + 1; c < n; ++c) s -= A[r * n + c] * x[c];
    x[r] = s / A[r * n + r];
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Next-query predictor for one (sequence, query head).                        */
/*                                                                             */
/* [summary] "Approach" and [abstract]: the next query state is predicted,     */
/* without training, from a short window of the most recent queries, by a     */
/* ridge regression whose weights are normalised with a softmax, and the       */
/* predictions of several windows are averaged ("multi-window average          */
/* pooling").  [card] "What reproduces" table: the prediction is a linear,     */
/* one-step-ahead ridge prediction over a recent window of 16 queries.         */
/*                                                                             */
/* Readings adopted where the pages are silent:                                */
/*  - window set: {W, W/2, W/4}, keeping only windows w with 2 <= w <= n,      */
/*    where n is the number of queries held; no window left -> q_hat = q_t,    */
/*    and n = 0 -> q_hat = 0.                                                  */
/*  - model: q_t ~ sum_{j=1..p} beta_j q_{t-j} with p = w-1 scalar lag        */
/*    coefficients shared by all D coordinates (the coordinates are the       */
/*    regression samples); ridge solution beta = (G + lambda I)^-1 r with      */
/*    G_jk = <q_{t-j}, q_{t-k}>, r_j = <q_{t-j}, q_t>, lambda added unscaled.  */
/*  - softmax normalisation: alpha = softmax(beta), temperature 1.            */
/*  - one step ahead: q_hat^(w) = sum_j alpha_j q_{t+1-j} (lag j of q_{t+1}).  */
/*  - pooling: q_hat = mean over the window set of q_hat^(w).                 */
/*                                                                             */
/* lags: n rows of D values, row j = q_{t-j} (row 0 is the newest query).      */
/* Outputs: q_pred[D]; windows[3] and *n_windows; beta[3*W] and alpha[3*W]     */
/* (row i holds window i's p coefficients, unused entries zero).  Any output  */
/* pointer except q_pred may be NULL.  Returns 0, or -1 on a singular system. */
/* ------------------------------------------------------------------------- */
int oracle_predict_one(int n, int D, int W, double lambda, const double* lags,
                       double* q_pred, int* windows, int* n_windows,
                       double* beta, double* alpha) {
  int wset[3];
  int nw = 0;
  const int cand[3] = {W, W / 2, W / 4};
  for (int c = 0; c < 3; ++c)
    if (cand[c] >= 2 && cand[c] <= n) wset[nw++] = cand[c];
  if (windows) for (int c = 0; c < 3; ++c) windows[c] = c < nw ? wset[c] : 0;
  if (n_windows) *n_windows = nw;
  if (beta) memset(beta, 0, sizeof(double) * 3 * (size_t)W);
  if (alpha) memset(alpha, 0, sizeof(double) * 3 * (size_t)W);

  for (int d = 0; d < D; ++d) q_pred[d] = 0.0;
  if (n <= 0) return 0;
  if (nw == 0) {
    for (int d = 0; d < D; ++d) q_pred[d] = lags[d];
    return 0;
  }

  int rc = 0;
  for (int wi = 0; wi < nw; ++wi) {
    const int p = wset[wi] - 1;
    double* A = (double*)malloc(sizeof(double) * (size_t)p * p);
    double* r = (double*)malloc(sizeof(double) * (size_t)p);
    double* b = (double*)malloc(sizeof(double) * (size_t)p);
    double* a = (double*)malloc(sizeof(double) * (size_t)p);
    /* Normal equations of the ridge problem over lags 1..p. */
    for (int j = 1; j <= p; ++j) {
      for (int k = 1; k <= p; ++k) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += lags[(size_t)j * D + d] * lags[(size_t)k * D + d];
        A[(j - 1) * p + (k - 1)] = s + (j == k ? lambda : 0.0);
      }
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += lags[(size_t)j * D + d] * lags[d];
      r[j - 1] = s;
    }
    if (solve_dense(p, A, r, b) != 0) rc = -1;
    /* Softmax over the p lag coefficients (max subtracted first). */
    double m = b[0];
    for (int j = 1; j < p; ++j) if (b[j] > m) m = b[j];
    double z = 0.0;
    for (int j = 0; j < p; ++j) { a[j] = exp(b[j] - m); z += a[j]; }
    for (int j = 0; j < p; ++j) a[j] /= z;
    if (beta) for (int j = 0; j < p; ++j) beta[wi * W + j] = b[j];
    if (alpha) for (int j = 0; j < p; ++j) alpha[wi * W + j] = a[j];
    /* One step ahead: coefficient j multiplies q_{t+1-j}, i.e. lag row j-1. */
    for (int d = 0; d < D; ++d) {
      double s = 0.0;
      for (int j = 1; j <= p; ++j) s += a[j - 1] * lags[(size_t)(j - 1) * D + d];
      q_pred[d] += s / nw;
    }
    free(A); free(r); free(b); free(a);
  }
  return rc;
}

/* Ring layout of the query history: q_hist[B][Hq][W][D] fp32, newest[b] is the
 * slot of q_t, len[b] the number of valid queries; lag j sits in slot
 * (newest - j) mod W.  Out-of-range newest / len are reduced into range. */
static int ring_slot(int newest, int j, int W) {
  int s = (newest - j) % W;
  return s < 0 ? s + W : s;
}

int oracle_predict(int B, int Hq, int W, int D, const float* q_hist, const int* newest,
                   const int* len, double lambda, double* q_pred) {
  int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (long u = 0; u < (long)B * Hq; ++u) {
    const int b = (int)(u / Hq);
    int n = len[b];
    if (n < 0) n = 0;
    if (n > W) n = W;
    double* lags = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    for (int j = 0; j < n; ++j) {
      const float* row = q_hist + ((size_t)u * W + ring_slot(newest[b], j, W)) * D;
      for (int d = 0; d < D; ++d) lags[(size_t)j * D + d] = (double)row[d];
    }
    int r = oracle_predict_one(n, D, W, lambda, lags, q_pred + (size_t)u * D, NULL, NULL, NULL, NULL);
    if (r < rc) rc = r;
    free(lags);
  }
  return rc;
}

/* History push: the actual query q_t of every head enters the ring one slot
 * after the current newest; the count of valid queries saturates at W.
 * ([summary] summary paragraph: the window slides over the most recent
 * queries.) */
void oracle_push(int B, int Hq, int W, int D, const float* q_cur, float* q_hist, int* newest, int* len) {
  for (int b = 0; b < B; ++b) {
    const int slot = ring_slot(newest[b], -1, W);
    for (int h = 0; h < Hq; ++h)
      memcpy(q_hist + (((size_t)b * Hq + h) * W + slot) * D, q_cur + ((size_t)b * Hq + h) * D,
             sizeof(float) * D);
    newest[b] = slot;
    int n = len[b] < 0 ? 0 : len[b];
    len[b] = n + 1 > W ? W : n + 1;
  }
}

/* ------------------------------------------------------------------------- */
/* Token-level key scoring.  [summary] "Approach" / [abstract]: selection is   */
/* made per token (not per page) by comparing every cached key with the        */
/* (predicted) query.  Reading adopted for grouped-query attention, on which  */
/* the pages are silent: a KV head's score for key i is the largest raw dot    */
/* product q_hat[h] . K[i] over the query heads h that share that KV head      */
/* (no 1/sqrt(D): a positive scale does not change a ranking).                 */
/* Layout: q_pred[B][Hq][D] fp32, K[B][Hkv][T_cap][D], scores[B][Hkv][T_cap];  */
/* entries i >= seq_lens[b] are set to NaN.                                    */
/* ------------------------------------------------------------------------- */
void oracle_score(int B, int Hq, int Hkv, int D, int T_cap, int kv_dtype, const float* q_pred,
                  const void* k, const int* seq_lens, double* scores) {
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < (long)B * Hkv; ++u) {
    const int b = (int)(u / Hkv), g = (int)(u % Hkv);
    int T = seq_lens[b];
    if (T < 0) T = 0;
    if (T > T_cap) T = T_cap;
    for (int i = 0; i < T_cap; ++i) {
      double best = NAN;
      if (i < T) {
        for (int hh = 0; hh < G; ++hh) {
          const float* q = q_pred + ((size_t)b * Hq + (size_t)g * G + hh) * D;
          double s = 0.0;
          for (int d = 0; d < D; ++d) s += (double)q[d] * kv_at(k, kv_dtype, ((size_t)u * T_cap + i) * D + d);
          if (hh == 0 || s > best) best = s;
        }
      }
      scores[(size_t)u * T_cap + i] = best;
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Top-C selection per (sequence, KV head).  [card] "Key finding" and          */
/* [summary] "Key results": C tokens (2k in the paper) are kept per step.      */
/* Definition implemented: C_eff = min(C, T_b); order the tokens i < T_b by    */
/* score descending, then index ascending (a lower index wins a tie); keep the */
/* first C_eff; write them in ascending index order, pad with -1.              */
/* Readings for values the pages never mention: NaN ranks as -infinity, and   */
/* -0 equals +0 (plain numeric comparison).                                    */
/* ------------------------------------------------------------------------- */
typedef struct { double s; int i; } scored_token;

static int cmp_rank(const void* pa, const void* pb) {
  const scored_token* a = (const scored_token*)pa;
  const scored_token* b = (const scored_token*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

static int cmp_int(const void* pa, const void* pb) {
  const int a = *(const int*)pa, b = *(const int*)pb;
  return (a > b) - (a < b);
}

void oracle_select(int B, int Hkv, int T_cap, int C, const double* scores, const int* seq_lens,
                   int* idx, int* n_sel) {
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < (long)B * Hkv; ++u) {
    const int b = (int)(u / Hkv);
    int T = seq_lens[b];
    if (T < 0) T = 0;
    if (T > T_cap) T = T_cap;
    const int c_eff = C < T ? C : T;
    scored_token* items = (scored_token*)malloc(sizeof(scored_token) * (size_t)(T > 0 ? T : 1));
    for (int i = 0; i < T; ++i) {
      double s = scores[(size_t)u * T_cap + i];
      items[i].s = isnan(s) ? -INFINITY : s;
      items[i].i = i;
    }
    qsort(items, (size_t)T, sizeof(scored_token), cmp_rank);
    int* out = idx + (size_t)u * C;
    for (int j = 0; j < c_eff; ++j) out[j] = items[j].i;
    qsort(out, (size_t)c_eff, sizeof(int), cmp_int);
    for (int j = c_eff; j < C; ++j) out[j] = -1;
    n_sel[u] = c_eff;
    free(items);
  }
}

/* ------------------------------------------------------------------------- */
/* Sparse decode attention.  [card] "Layout" (full vs top-C sparse attention)  */
/* and "Key finding" (the method attends to the selected tokens only);         */
/* [summary] "Approach": the selection made from the predicted query is used   */
/* by the inference step.  Reading: the attention query is the actual q_t;     */
/* for each query head h of KV head g = h / G,                                 */
/*   s_i = q_t[h] . K[g, i] / sqrt(D) over the selected i,                     */
/*   out[h] = sum_i exp(s_i - m) V[g, i] / sum_i exp(s_i - m),  m = max s_i;    */
/* an empty selection gives out[h] = 0.  idx[B][Hkv][C] (first n_sel[u]        */
/* entries used), q[B][Hq][D] fp32, K/V[B][Hkv][T_cap][D], out[B][Hq][D].       */
/* Returns 0, or -1 if an index lies outside [0, T_cap).                       */
/* ------------------------------------------------------------------------- */
int oracle_attend(int B, int Hq, int Hkv, int D, int T_cap, int kv_dtype, int C, const float* q,
                  const void* k, const void* v, const int* idx, const int* n_sel, double* out) {
  const int G = Hq / Hkv;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (long uh = 0; uh < (long)B * Hq; ++uh) {
    const int b = (int)(uh / Hq), h = (int)(uh % Hq);
    const long u = (long)b * Hkv + h / G;
    int n = n_sel[u];
    if (n < 0) n = 0;
    if (n > C) n = C;
    double* o = out + (size_t)uh * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n == 0) continue;
    const int* sel = idx + (size_t)u * C;
    int bad = 0;
    for (int j = 0; j < n; ++j) if (sel[j] < 0 || sel[j] >= T_cap) bad = 1;
    if (bad) { rc = -1; continue; }
    const float* qh = q + (size_t)uh * D;
    double* s = (double*)malloc(sizeof(double) * (size_t)(unsigned)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += (double)qh[d] * kv_at(k, kv_dtype, ((size_t)u * T_cap + sel[j]) * D + d);
      s[j] = acc * inv_sqrt_d;
      if (s[j] > m) m = s[j];
    }
    double z = 0.0;
    for (int j = 0; j < n; ++j) { s[j] = exp(s[j] - m); z += s[j]; }
    for (int j = 0; j < n; ++j)
      for (int d = 0; d < D; ++d) o[d] += s[j] * kv_at(v, kv_dtype, ((size_t)u * T_cap + sel[j]) * D + d);
    for (int d = 0; d < D; ++d) o[d] /= z;
    free(s);
  }
  return rc;
}

/* Overlap of two selections per unit: the number of distinct token indices in
 * [0, T_cap) present in both idx_a[u][0..n_a[u]) and idx_b[u][0..n_b[u]) (n
 * clamped to [0, C]).  Reproduction card, "What reproduces": the temporal
 * locality (overlap of top-k sets within a recent window) and the recall of the
 * predicted selection against the true one are both such set intersections.
 * A marker array per unit: 1 = in A, 2 = in A and already counted from B. */
void oracle_overlap(int units, int C, int T_cap, const int* idx_a, const int* n_a, const int* idx_b,
                    const int* n_b, int* out) {
#pragma omp parallel for schedule(dynamic)
  for (int u = 0; u < units; ++u) {
    unsigned char* mark = (unsigned char*)calloc((size_t)(unsigned)T_cap, 1);
    int na = n_a[u] < 0 ? 0 : (n_a[u] > C ? C : n_a[u]);
    int nb = n_b[u] < 0 ? 0 : (n_b[u] > C ? C : n_b[u]);
    const int* a = idx_a + (size_t)u * C;
    const int* b = idx_b + (size_t)u * C;
    for (int i = 0; i < na; ++i)
      if (a[i] >= 0 && a[i] < T_cap) mark[a[i]] = 1;
    int count = 0;
    for (int j = 0; j < nb; ++j) {
      if (b[j] < 0 || b[j] >= T_cap || mark[b[j]] != 1) continue;
      mark[b[j]] = 2;
      ++count;
    }
    out[u] = count;
    free(mark);
  }
}

/* ------------------------------------------------------------------------- */
/* Page-level selection, the baseline the pages compare against.  [summary]   */
/* "Problem" and "Experimental setup" (its baselines), [abstract]: Quest       */
/* selects whole pages of the KV cache with the current query.  The pages do   */
/* not define how a page is scored; the definition used is the one Quest       */
/* publishes (Tang et al., "Quest: Query-Aware Sparsity for Efficient          */
/* Long-Context LLM Inference",                                                */
/* ICML 2024, the criticality estimate of its method section): each page keeps */
/* the element-wise minimum and maximum of its keys, and a query q scores the  */
/* page by sum_d max(q_d * min_d, q_d * max_d), the largest value q . k can    */
/* take over the box [min, max], hence an upper bound on q . k for every key   */
/* of the page.  Readings for what Quest leaves open here:                     */
/*  - pages are runs of P consecutive tokens from token 0; a sequence's last   */
/*    page may be partial and then summarises only its valid tokens;          */
/*  - grouped-query attention: as for token scores, a KV head's page score is  */
/*    the largest bound over the query heads that share it;                    */
/*  - the token budget C buys C / P pages, ranked like tokens (score           */
/*    descending, lower page index first on ties).                             */
/* ------------------------------------------------------------------------- */

/* Page summaries.  K[B][Hkv][T_cap][D] -> kmin, kmax [B][Hkv][NP][D] (fp64,   */
/* exact copies of key elements), NP = ceil(T_cap / P); page p of sequence b   */
/* covers tokens [p*P, min(p*P + P, T_b)); pages with no token are NaN.        */
void oracle_page_summary(int B, int Hkv, int D, int T_cap, int kv_dtype, int P, const void* k, const int* seq_lens,
                         double* kmin, double* kmax) {
  const int NP = (T_cap + P - 1) / P;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < (long)B * Hkv; ++u) {
    const int b = (int)(u / Hkv);
    int T = seq_lens[b];
    if (T < 0) T = 0;
    if (T > T_cap) T = T_cap;
    for (int p = 0; p < NP; ++p) {
      double* mn = kmin + ((size_t)u * NP + p) * D;
      double* mx = kmax + ((size_t)u * NP + p) * D;
      const int first = p * P;
      int last = first + P;
      if (last > T) last = T;
      for (int d = 0; d < D; ++d) {
        mn[d] = NAN;
        mx[d] = NAN;
      }
      for (int i = first; i < last; ++i) {
        for (int d = 0; d < D; ++d) {
          const double x = kv_at(k, kv_dtype, ((size_t)u * T_cap + i) * D + d);
          if (i == first || x < mn[d]) mn[d] = x;
          if (i == first || x > mx[d]) mx[d] = x;
        }
      }
    }
  }
}

/* Page scores.  q[B][Hq][D] fp32, kmin/kmax [B][Hkv][NP][D] fp64,            */
/* n_pages[B] (pages with at least one token) -> scores[B][Hkv][NP]:           */
/*   scores[b][g][p] = max over h of g of sum_d max(q[h][d] * kmin[p][d],      */
/*                                                   q[h][d] * kmax[p][d])     */
/* for p < n_pages[b], NaN beyond.                                             */
void oracle_page_score(int B, int Hq, int Hkv, int D, int NP, const float* q, const double* kmin, const double* kmax,
                       const int* n_pages, double* scores) {
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < (long)B * Hkv; ++u) {
    const int b = (int)(u / Hkv), g = (int)(u % Hkv);
    int n = n_pages[b];
    if (n < 0) n = 0;
    if (n > NP) n = NP;
    for (int p = 0; p < NP; ++p) {
      double best = NAN;
      if (p < n) {
        const double* mn = kmin + ((size_t)u * NP + p) * D;
        const double* mx = kmax + ((size_t)u * NP + p) * D;
        for (int hh = 0; hh < G; ++hh) {
          const float* qh = q + ((size_t)b * Hq + (size_t)g * G + hh) * D;
          double s = 0.0;
          for (int d = 0; d < D; ++d) {
            const double lo = (double)qh[d] * mn[d], hi = (double)qh[d] * mx[d];
            s += lo > hi ? lo : hi;
          }
          if (hh == 0 || s > best) best = s;
        }
      }
      scores[(size_t)u * NP + p] = best;
    }
  }
}
