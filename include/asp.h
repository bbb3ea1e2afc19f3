/*
 * asp.h -- C ABI of libasp.so, the MI355X (gfx950) AsyncSpade sparse decode step.
 *
 * The step predicts each query head's next query from a ring of its recent
 * queries, scores every cached key of each KV head against the prediction,
 * keeps the top-C tokens per (sequence, KV head), and runs decode attention
 * with the actual query over only those tokens.  Selection for the next step
 * can run on a second HIP stream while this step's attention runs.  The
 * page-level selection the pages compare against (asp_page_*) is provided
 * beside it as a baseline.
 *
 * Sources: [card] the Hugging Face dataset card "Reproduction: AsyncSpade --
 * Efficient Test-Time Scaling with Asynchronous Sparse Decoding"; [summary] the
 * atlas.scime.ai research-map page on AsyncSpade; [abstract] the arXiv
 * 2510.07486 abstract.  Where the pages leave a step open, the reading taken is
 * stated at the entry point that implements it.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major in the layout given.  K, V, q_cur and q_hist must be 16-byte
 *    aligned (16-byte vector loads), every other array 4-byte aligned; a
 *    misaligned pointer is rejected with ASP_ERR_INVALID_ARG.  A workspace
 *    must be 16-byte aligned, else ASP_ERR_WORKSPACE.
 *  - A "unit" is one (sequence b, KV head g); G = n_q_heads / n_kv_heads query
 *    heads h = g*G .. g*G+G-1 share KV head g.
 *  - The library allocates no device memory, keeps no state of its own and
 *    never waits on the host: work is enqueued on the given stream(s) and the
 *    call returns.  The one exception is asp_sparse_decode_static, whose
 *    scratch is a device array built into the library (its address is looked
 *    up once per device).  The two-stream asp_step needs a caller-owned
 *    asp_context (a stream and three events, made by asp_context_create and
 *    released by asp_context_destroy).  Calls are re-entrant and may run concurrently
 *    from several host threads; two calls that write the same buffers, share
 *    a workspace or share a context must be ordered by the caller.
 *  - Every entry point except asp_step and asp_context_join enqueues kernel
 *    launches only (no memset or copy node, no event), so a sequence of them
 *    can be captured into a HIP graph on one stream and replayed; so can
 *    asp_step, on one stream or on two under the rules given with it.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued.  Values that live in device memory (seq_lens,
 *    hist_newest, hist_len, idx, n_sel) cannot be checked on the host: the
 *    kernels clamp them into range (a length to [0, t_cap], a ring slot modulo
 *    W, a count to [0, W] or [0, C]; an index outside [0, t_cap) is skipped),
 *    so a bad value gives unspecified results but never an out-of-bounds access.
 *  - ASP_ERR_HIP is returned when a kernel launch or an event/stream call fails.
 *  - No C++ exception crosses this interface.
 */
#ifndef ASP_H
#define ASP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ASP_OK = 0,
  ASP_ERR_INVALID_ARG = 1, /* a dimension, config value or pointer is invalid */
  ASP_ERR_UNSUPPORTED = 2, /* valid in principle, not implemented (e.g. head_dim 96) */
  ASP_ERR_WORKSPACE = 3,   /* ws is NULL, not 16-byte aligned, or ws_bytes < asp_workspace_size(...) */
  ASP_ERR_HIP = 4,         /* a HIP launch / event / stream call failed */
  ASP_ERR_HOST_MEMORY = 5, /* a host allocation failed (asp_context_create) */
  ASP_ERR_SCRATCH = 6      /* more scratch than ASP_STATIC_SCRATCH_BYTES (asp_sparse_decode_static) */
} asp_status;

typedef enum { ASP_KV_BF16 = 0, ASP_KV_F32 = 1 } asp_kv_dtype;

/* Problem shape.  batch >= 0 (0 is a no-op); n_q_heads % n_kv_heads == 0 with
 * G in {1, 2, 4, 8}; head_dim in {64, 128}; 1 <= t_cap <= 4194304 (the
 * allocated token stride of K and V); kv_dtype an asp_kv_dtype. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t t_cap;
  int32_t kv_dtype;
} asp_dims;

/* Method configuration.  window W: ring length, a multiple of 4 in [4, 64];
 * top_c C: tokens kept per unit, 1 <= C <= t_cap; lambda: ridge penalty,
 * finite and > 0; recent R: the attention also attends each sequence's
 * newest R tokens [seq_len - R, seq_len) beside the selection (0 = off;
 * 0 <= R <= t_cap).  C + R may span at most 256 attention blocks (32768
 * tokens for bf16 and head_dim 128), else ASP_ERR_UNSUPPORTED. */
typedef struct {
  int32_t window;
  int32_t top_c;
  double lambda;
  int32_t recent;
} asp_cfg;

typedef enum {
  ASP_OP_PUSH = 0,
  ASP_OP_PREDICT = 1,
  ASP_OP_SCORE = 2,
  ASP_OP_SELECT = 3,
  ASP_OP_DECODE = 4,
  ASP_OP_STEP = 5,
  ASP_OP_CANDIDATES = 6
} asp_op;

/* Bytes of device workspace the entry point for `op` needs (0 if none), or 0
 * when dims/cfg are invalid.  Host only. */
size_t asp_workspace_size(const asp_dims* dims, const asp_cfg* cfg, asp_op op);

/* Static English text for a status code.  Host only; never NULL. */
const char* asp_status_string(asp_status status);

/* Ring push (the window of recent queries slides by one; [summary], summary
 * paragraph).  q_cur[B][Hq][D] fp32 is written into slot
 * (hist_newest[b] + 1) mod W of q_hist[B][Hq][W][D] fp32; hist_newest[b]
 * becomes that slot and hist_len[b] becomes min(hist_len[b] + 1, W).  Lag j
 * of sequence b is slot (hist_newest[b] - j) mod W.  An empty ring is
 * hist_len = 0 with any hist_newest. */
asp_status asp_push_query(const asp_dims* dims, const asp_cfg* cfg, const float* q_cur, float* q_hist,
                          int32_t* hist_newest, int32_t* hist_len, hipStream_t stream);

/* Next-query prediction ([summary] "Approach"; [abstract], first component;
 * [card] "What reproduces": linear one-step-ahead ridge prediction over a
 * recent window).  For every (b, h), from the n = hist_len[b] queries in the
 * ring (q_t newest):
 *   windows: w in {W, W/2, W/4} with 2 <= w <= n;
 *   per window, p = w - 1 scalar lag weights beta solve the ridge problem
 *     q_t ~ sum_{j=1..p} beta_j q_{t-j} over the D coordinates, i.e.
 *     (Gram(q_{t-1..t-p}) + lambda I) beta = (<q_{t-j}, q_t>)_j;
 *   alpha = softmax(beta); q_hat_w = sum_j alpha_j q_{t+1-j};
 *   q_pred = mean over the windows of q_hat_w;
 *   no window (n = 1): q_pred = q_t; n = 0: q_pred = 0.
 * The Gram matrix and the solve are computed in fp64 (one L D L^T
 * factorisation serves all windows: a smaller window's system is a leading
 * block).
 * Output q_pred[B][Hq][D] fp32. */
asp_status asp_predict_query(const asp_dims* dims, const asp_cfg* cfg, const float* q_hist,
                             const int32_t* hist_newest, const int32_t* hist_len, float* q_pred,
                             hipStream_t stream);

/* Token-level key scoring ([summary] "Approach"; [abstract]: token-level, not
 * page-level, selection).  For i < seq_lens[b]:
 *   scores[b][g][i] = max over the G query heads h of g of q_pred[b][h] . K[b][g][i]
 * accumulated in fp32 (no 1/sqrt(D): a ranking is scale-free).  Entries at
 * i >= seq_lens[b] are not written.  q_pred[B][Hq][D] fp32,
 * k[B][Hkv][t_cap][D] in dims->kv_dtype, scores[B][Hkv][t_cap] fp32.
 * hist: NULL, or [B][Hkv][ASP_HIST_BINS] uint32, 16-byte aligned, which the
 * call overwrites with each unit's coarse histogram: bin j counts the scores
 * i < seq_lens[b] whose order key (the scores' monotone map to uint32 that
 * asp_select_topc ranks by) has j as its top 11 bits.  Passing it on to
 * asp_select_topc saves that call a pass over the scores.
 * Keys must be finite.  For bf16 keys the fp32 predicted query enters the
 * products as a pair of bf16 terms (hi + lo), so an infinite key element can
 * give NaN (ranked as -inf) where the exact product is infinite; a non-finite
 * key gives an unspecified score for its token (and an unspecified, still
 * well-formed, selection downstream), never an access outside the arguments. */
#define ASP_HIST_BINS 2048
asp_status asp_score_keys(const asp_dims* dims, const float* q_pred, const void* k, const int32_t* seq_lens,
                          float* scores, uint32_t* hist, hipStream_t stream);

/* Exact top-C selection per unit ([card] "Key finding": C = 2k tokens; [summary]
 * "Key results").  C_eff = min(C, seq_lens[b]); the C_eff tokens i < seq_lens[b]
 * that come first when ordered by score descending, then index ascending (ties
 * go to the lower index; NaN ranks as -inf; -0 ties with +0), are written to
 * idx[b][g][0..C_eff) in ascending index order, idx[b][g][C_eff..C) = -1, and
 * n_sel[b][g] = C_eff.  scores[B][Hkv][t_cap] fp32, idx[B][Hkv][C] int32,
 * n_sel[B][Hkv] int32.  hist: NULL, or the coarse histograms of these scores
 * as asp_score_keys writes them (16-byte aligned); with NULL the call builds
 * them first.  A histogram that does not match the scores gives an
 * unspecified selection (never an access outside the arguments).
 * ws/ws_bytes: asp_workspace_size(ASP_OP_SELECT) bytes of device scratch
 * (about 4.2 bytes per key slot plus 8 KiB per unit; its contents need no
 * initialisation and are not kept between calls). */
asp_status asp_select_topc(const asp_dims* dims, const asp_cfg* cfg, const float* scores, const uint32_t* hist,
                           const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* The same selection by the route asp_step takes ([card] "Key finding"; the
 * candidate route is a property of this implementation, not of the pages).
 * asp_score_candidates runs the score pass of asp_score_keys but writes no
 * score rows: per unit it keeps, as candidates, the keys whose order key is at
 * or above the unit's threshold hint.  asp_select_candidates then selects the
 * exact top C_eff among them; a unit left with fewer than C_eff candidates is
 * first rescored with every key kept.  idx and n_sel therefore equal, bit for
 * bit, those of asp_score_keys followed by asp_select_topc, whatever the hints
 * hold.  Each selection stores the unit's next hint: the lower edge of the bin
 * of the top 22 bits of the order key that holds the (3*C_eff/2)-th kept key, or,
 * when fewer keys were kept, the current hint moved down by the key range the
 * shortfall would take at the density of the kept keys just above it.  Scores
 * close to those of the previous step thus cost one pass over the keys plus
 * about 1.5*C_eff candidate writes per unit.
 * ws/ws_bytes: asp_workspace_size(ASP_OP_CANDIDATES) bytes, 16-byte aligned
 * (about 8 bytes per key slot).  Its first 4*batch*n_kv_heads bytes are the
 * hints ([B][Hkv] uint32), carried from one selection to the next; any value
 * is valid (a zeroed workspace keeps every key on its first use).
 * asp_score_candidates: q_pred, k and seq_lens as in asp_score_keys.
 * asp_select_candidates: selects from what the last asp_score_candidates call
 * on this workspace kept; q_pred, k and seq_lens must be that call's (a
 * rescoring reads them); idx and n_sel as in asp_select_topc.  Two calls that
 * share a workspace must be ordered by the caller. */
asp_status asp_score_candidates(const asp_dims* dims, const asp_cfg* cfg, const float* q_pred, const void* k,
                                const int32_t* seq_lens, void* ws, size_t ws_bytes, hipStream_t stream);
asp_status asp_select_candidates(const asp_dims* dims, const asp_cfg* cfg, const float* q_pred, const void* k,
                                 const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Overlap of two selections per unit, the diagnostic of the temporal locality
 * and prediction recall claims ([card] "What reproduces (and what does not)":
 * the overlap of top-k sets within a recent 16-query window, and the share of
 * the true next-step top-k selection that the ridge-predicted query recovers).
 * overlap[b][g] = the number of indices i in [0, t_cap) that appear both in
 * idx_a[b][g][0..n_sel_a[b][g]) and in idx_b[b][g][0..n_sel_b[b][g]).  Both
 * lists must be strictly ascending, as asp_select_topc and asp_step write
 * them (other orders give unspecified counts); the n_sel values are clamped
 * to [0, top_c].  idx_* [B][Hkv][top_c] int32, n_sel_* and overlap [B][Hkv]
 * int32.  ASP_ERR_UNSUPPORTED when top_c > 32768. */
asp_status asp_selection_overlap(const asp_dims* dims, const asp_cfg* cfg, const int32_t* idx_a,
                                 const int32_t* n_sel_a, const int32_t* idx_b, const int32_t* n_sel_b,
                                 int32_t* overlap, hipStream_t stream);

/* Check of the arguments that live in device memory, which the host-side
 * validation cannot see (no passage of the pages: part of this interface's
 * error convention).  The other entry points clamp such values (see the
 * conventions above); this call reports whether they are what the library's
 * own producers leave.  It enqueues a clear of *status and one check launch
 * (kernel launches only, so it may be captured), reads its inputs only, and
 * ORs into *status (one uint32 in device memory, 4-byte aligned) the bits of
 * every violated condition, 0 when all hold:
 *   ASP_CHECK_SEQ_LEN      seq_lens[b] outside [0, t_cap];
 *   ASP_CHECK_HIST_LEN     hist_len[b] outside [0, window];
 *   ASP_CHECK_HIST_NEWEST  hist_len[b] > 0 and hist_newest[b] outside [0, window);
 *   ASP_CHECK_N_SEL        n_sel[b][g] outside [0, min(top_c, seq_lens[b])];
 *   ASP_CHECK_IDX          an entry idx[b][g][j], j < n_sel[b][g] (clamped to
 *                          [0, top_c]), outside [0, seq_lens[b]) or not below
 *                          the next such entry (the list is strictly ascending);
 *   ASP_CHECK_IDX_PAD      an entry at or beyond n_sel[b][g] that is not -1
 *                          (no entry point reads those entries).
 * seq_lens[B] int32 is required; hist_newest/hist_len ([B] int32) and
 * idx/n_sel ([B][Hkv][top_c], [B][Hkv] int32) are optional pairs (both NULL
 * skips those checks; one of a pair NULL is ASP_ERR_INVALID_ARG).  The status
 * word is valid once the stream reaches the end of the call's work. */
#define ASP_CHECK_SEQ_LEN 0x01u
#define ASP_CHECK_HIST_LEN 0x02u
#define ASP_CHECK_HIST_NEWEST 0x04u
#define ASP_CHECK_N_SEL 0x08u
#define ASP_CHECK_IDX 0x10u
#define ASP_CHECK_IDX_PAD 0x20u
asp_status asp_check_device_args(const asp_dims* dims, const asp_cfg* cfg, const int32_t* seq_lens,
                                 const int32_t* hist_newest, const int32_t* hist_len, const int32_t* idx,
                                 const int32_t* n_sel, uint32_t* status, hipStream_t stream);

/* Sparse decode attention over the selected tokens ([card] "Layout" and "Key
 * finding": attention over the top-C tokens only).  For every (b, h), with
 * g = h / G, n = n_sel[b][g] clamped to [0, C], T = seq_lens[b] clamped to
 * [0, t_cap] and r = min(cfg->recent, T), the attended list S holds the
 * entries idx[b][g][j], j < n, that lie in [0, t_cap) and outside [T - r, T)
 * (as listed: asp_select_topc writes distinct ones), then every token of
 * [T - r, T) once:
 *   out[b][h] = sum_{i in S} exp(s_i - m) V[b][g][i] / sum_{i in S} exp(s_i - m),
 *   s_i = q[b][h] . K[b][g][i] / sqrt(D), m = max s_i;
 * out = 0 when S is empty.  Accumulation is fp32 (online softmax over split-K partials merged
 * by log-sum-exp).  q[B][Hq][D] fp32, k/v [B][Hkv][t_cap][D] in
 * dims->kv_dtype, seq_lens[B] int32 (may be NULL when cfg->recent is 0),
 * out[B][Hq][D] fp32.  ws/ws_bytes: asp_workspace_size(ASP_OP_DECODE) bytes. */
asp_status asp_sparse_decode(const asp_dims* dims, const asp_cfg* cfg, const float* q, const void* k, const void* v,
                             const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel, float* out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* asp_sparse_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same attention and merge, with the split-K partials in a
 * scratch buffer built into the library instead of a caller's workspace.
 * Arguments, results and errors as asp_sparse_decode, minus ws/ws_bytes; the
 * call allocates nothing (no hipMalloc, no allocating library routine).
 * The scratch is ASP_STATIC_SCRATCH_BYTES of device memory per GPU, held from
 * the library's load until the process ends; a shape whose partials
 * (asp_workspace_size(ASP_OP_DECODE) bytes) exceed it gives ASP_ERR_SCRATCH
 * before anything is enqueued.  Its contents need no initialisation (every
 * partial is written before it is read) and are left behind by each call.
 * Every call on one GPU uses that GPU's single copy: two calls whose work
 * overlaps on a device (different streams, different host threads, not
 * ordered by the caller) race and give unspecified outputs.  The first call
 * on a device looks the buffer's address up with that device current. */
#define ASP_STATIC_SCRATCH_BYTES (8u << 20)
asp_status asp_sparse_decode_static(const asp_dims* dims, const asp_cfg* cfg, const float* q, const void* k,
                                    const void* v, const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel,
                                    float* out, hipStream_t stream);

/* Page-level selection, the baseline the pages compare against ([summary]
 * "Problem" and "Experimental setup", its baselines; [abstract]: Quest, which
 * selects pages of the KV cache with the current query, on the decode critical
 * path).  The pages do not define how a page is scored; the score is the
 * criticality estimate that Quest publishes (Tang et al., ICML 2024, method
 * section):
 *   pages: runs of P = page_size consecutive tokens from token 0,
 *     NP = ceil(t_cap / P) page rows per unit; page p of sequence b holds the
 *     tokens [p*P, min(p*P + P, T)), T = seq_lens[b] clamped to [0, t_cap], so
 *     the sequence has ceil(T / P) pages and only its last may be partial;
 *   summary: kmin[b][g][p][d] and kmax[b][g][p][d], the minimum and maximum
 *     over the page's tokens of K[b][g][i][d] (exact elements, in
 *     dims->kv_dtype);
 *   score: max over the G query heads h of g of
 *     sum_d max(q[b][h][d] * kmin[b][g][p][d], q[b][h][d] * kmax[b][g][p][d]),
 *     the largest value of q[h] . k over the page's min/max box (an upper
 *     bound on the dot product of every key of the page), accumulated in fp32;
 *   selection: with a budget of C = cfg->top_c tokens, the K = C / P pages
 *     that come first by score descending, then page index ascending (the
 *     order of asp_select_topc); their tokens are written in ascending order
 *     to idx[b][g][0..n), n = n_sel[b][g] (at most C; fewer when the
 *     sequence has fewer than K pages or its partial last page is chosen),
 *     and idx[b][g][n..C) = -1, ready for asp_sparse_decode.
 * Keys must be finite (a NaN key gives unspecified summaries).
 * 1 <= page_size <= t_cap, else ASP_ERR_INVALID_ARG; asp_page_select also
 * needs top_c % page_size == 0.
 * kmin, kmax: [B][Hkv][NP][D] in dims->kv_dtype, 16-byte aligned,
 * asp_page_summary_size() bytes each (0 when dims or page_size are invalid);
 * rows of pages without tokens are not written.  q[B][Hq][D] fp32,
 * k[B][Hkv][t_cap][D], seq_lens[B] int32, scores[B][Hkv][NP] fp32 (rows past
 * a sequence's pages not written), idx[B][Hkv][C] and n_sel[B][Hkv] int32.
 * asp_page_select: ws/ws_bytes: asp_page_select_workspace_size() bytes,
 * 16-byte aligned (0 when the arguments are invalid); contents need no
 * initialisation and are not kept. */
size_t asp_page_summary_size(const asp_dims* dims, int32_t page_size);
asp_status asp_page_summary(const asp_dims* dims, int32_t page_size, const void* k, const int32_t* seq_lens,
                            void* kmin, void* kmax, hipStream_t stream);
asp_status asp_page_scores(const asp_dims* dims, int32_t page_size, const float* q, const void* kmin,
                           const void* kmax, const int32_t* seq_lens, float* scores, hipStream_t stream);
size_t asp_page_select_workspace_size(const asp_dims* dims, const asp_cfg* cfg, int32_t page_size);
asp_status asp_page_select(const asp_dims* dims, const asp_cfg* cfg, int32_t page_size, const float* q,
                           const void* kmin, const void* kmax, const int32_t* seq_lens, int32_t* idx,
                           int32_t* n_sel, void* ws, size_t ws_bytes, hipStream_t stream);

/* Caller-owned state of the two-stream asp_step ([abstract], second
 * component; [summary] "Approach": selection runs beside the decoding loop):
 * one HIP stream (default priority) on which the score passes of successive
 * steps run back to back, and three events that order it with the caller's
 * streams.
 * asp_context_create makes one on `device` (0 <= device < the device count,
 * else ASP_ERR_INVALID_ARG) and stores it in *ctx (NULL on failure).  flags:
 * 0, or ASP_CTX_SCORE_ALL_CUS; other bits give ASP_ERR_INVALID_ARG.
 *  - 0: the score stream leaves the last 32-CU group of the device (one XCD of
 *    MI355X) to the latency-bound launches of the step (predictor, selection,
 *    attention merge), which would otherwise wait for CU slots behind the
 *    score blocks (a CU-masked stream; where the device has a single group or
 *    the mask is refused, an unmasked one).  A CU-masked stream synchronises
 *    with the legacy default stream.
 *  - ASP_CTX_SCORE_ALL_CUS: the score stream may use every CU.
 * A context serves one asp_step call at a time (calls that share it must be
 * ordered by the caller, e.g. made from one host thread); different contexts
 * are independent and may be used concurrently.  Its stream needs a hardware
 * queue of its own beside the caller's two streams: HIP gives a process four
 * unless GPU_MAX_HW_QUEUES says otherwise, and streams that share a queue run
 * in submission order.
 * asp_context_destroy waits for the context's stream to drain, then releases
 * the stream and the events (NULL is a no-op); ASP_ERR_HIP if a HIP call
 * failed (the rest is still released).  Returns ASP_ERR_HOST_MEMORY when the
 * host allocation fails, ASP_ERR_HIP when a stream or event cannot be made.
 * asp_context_join makes `stream` wait for every score pass enqueued on the
 * context so far (an event recorded on the context's stream, waited on by
 * `stream`; it enqueues nothing else).  A graph capture that contains
 * two-stream asp_step calls must, before it ends, join the context's stream
 * (this call, after the last such step) and the caller's sel_stream back into
 * the capture's origin stream.  ASP_ERR_INVALID_ARG for a NULL ctx. */
typedef struct asp_context_s asp_context;
#define ASP_CTX_SCORE_ALL_CUS 1u
asp_status asp_context_create(int32_t device, uint32_t flags, asp_context** ctx);
asp_status asp_context_destroy(asp_context* ctx);
asp_status asp_context_join(asp_context* ctx, hipStream_t stream);

/* One decode step of one layer ([abstract], second component; [summary]
 * "Approach": selection for the next step is taken off the decode critical
 * path and overlapped with the current step's attention).
 *
 * Pipelined mode (idx_cur != NULL): attention with the actual query q_cur over
 * the selection idx_cur/n_sel_cur (made by the previous step) and, with
 * cfg->recent > 0, the newest tokens (as asp_sparse_decode) writes out; and,
 * independently, q_cur is pushed into the ring, the next query is predicted,
 * keys are scored and the next step's selection is written to
 * idx_next/n_sel_next.
 *  - sel_stream NULL or equal to attn_stream: everything runs in that order on
 *    attn_stream (attention first); ctx and idx_cur_ready are ignored (may be
 *    NULL); idx_next_ready, when not NULL, is recorded when the selection is
 *    written.
 *  - otherwise (two streams): ctx (a context made on the current device) is
 *    required, and idx_cur_ready too unless attn_stream is being captured,
 *    else ASP_ERR_INVALID_ARG.
 *      attn_stream waits for idx_cur_ready, then pushes q_cur into the ring
 *      and predicts the next query, then runs the attention over idx_cur and
 *      its merge;
 *      the context's stream waits for the prediction and scores the keys;
 *      sel_stream waits for the scores, selects into idx_next/n_sel_next,
 *      advances the ring and records idx_next_ready (when not NULL).
 *    idx_cur_ready is the event recorded when the selection idx_cur was
 *    written (the idx_next_ready of the step that made it, which must also be
 *    the last step that used this workspace: in a decode loop each layer keeps
 *    its own workspace, idx/n_sel buffer pair and event pair).  The caller
 *    swaps idx/n_sel buffers and events between the steps of a layer; the
 *    selection of step t writes the buffer that step t-1's attention read,
 *    and is ordered after it through attn_stream.  When the call returns,
 *    `out` is complete in attn_stream's order; the selection and the ring
 *    are complete in sel_stream's order (idx_next_ready).
 * Graph capture: every mode may be captured with attn_stream as the origin
 * (the one-stream modes make kernel launches and at most one event record on
 * attn_stream).  With two streams, the call forks the context's stream and
 * sel_stream off attn_stream inside the capture, so sel_stream must not be
 * capturing into another graph (ASP_ERR_UNSUPPORTED), idx_cur_ready must be
 * NULL or an event recorded earlier in the same capture (a wait on an event
 * recorded outside it is refused by HIP), and the capture must end with
 * both forked streams joined back into attn_stream (asp_context_join, and a
 * wait on an event recorded on sel_stream).  With idx_cur_ready NULL, the
 * caller orders the step after the selection it reads (graphs replayed on one
 * stream run one after the other).
 * Bootstrap mode (idx_cur == NULL): everything runs on attn_stream: push,
 * predict, score, select into idx_next, then attention over idx_next; the
 * workspace's hints are reset first, so that this selection keeps every key.
 * Every mode selects by the candidate route of asp_score_candidates and
 * asp_select_candidates, so the selection equals that of asp_score_keys with
 * asp_select_topc; results do not depend on the stream arrangement (the
 * kernels are deterministic).  Keys must be finite, as for asp_score_keys.
 * Shapes as in the entry points above; ws/ws_bytes:
 * asp_workspace_size(ASP_OP_STEP) bytes, 16-byte aligned, used by all the
 * streams (disjoint regions), so it must not be shared with a concurrent step.
 * Its first 4*batch*n_kv_heads bytes are the per-unit threshold hints of the
 * candidate route, which each step updates for the next step of the layer. */
asp_status asp_step(asp_context* ctx, const asp_dims* dims, const asp_cfg* cfg, const float* q_cur,
                    float* q_hist, int32_t* hist_newest, int32_t* hist_len, const void* k, const void* v,
                    const int32_t* seq_lens, const int32_t* idx_cur, const int32_t* n_sel_cur,
                    int32_t* idx_next, int32_t* n_sel_next, float* out, void* ws, size_t ws_bytes,
                    hipStream_t attn_stream, hipStream_t sel_stream, hipEvent_t idx_cur_ready,
                    hipEvent_t idx_next_ready);

#ifdef __cplusplus
}
#endif

#endif /* ASP_H */
