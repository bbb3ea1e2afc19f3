// C ABI of libasp.so: host-side validation, workspace layout and the order in
// which the kernels are enqueued.  See include/asp.h for the contract of every
// entry point.
#include <math.h>

#include <mutex>
#include <new>

#include "../../include/asp.h"
#include "asp_internal.h"
#include "page.h"

using asp::Shape;

static_assert(ASP_HIST_BINS == asp::HIST_BINS, "the public histogram size is the kernels'");

namespace {

constexpr int32_t kMaxTCap = 1 << 22;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

asp_status check_dims(const asp_dims* d, Shape* s) {
  if (d == nullptr) return ASP_ERR_INVALID_ARG;
  if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->t_cap < 1 || d->t_cap > kMaxTCap)
    return ASP_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return ASP_ERR_INVALID_ARG;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ASP_ERR_UNSUPPORTED;
  if (d->head_dim < 1) return ASP_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return ASP_ERR_UNSUPPORTED;
  if (d->kv_dtype != ASP_KV_BF16 && d->kv_dtype != ASP_KV_F32) return ASP_ERR_INVALID_ARG;
  // Grid limits: units index gridDim.y of the streaming kernels.
  if ((int64_t)d->batch * d->n_kv_heads > 65535 || (int64_t)d->batch * d->n_q_heads > (1 << 24))
    return ASP_ERR_UNSUPPORTED;
  s->B = d->batch;
  s->Hq = d->n_q_heads;
  s->Hkv = d->n_kv_heads;
  s->G = G;
  s->D = d->head_dim;
  s->T_cap = d->t_cap;
  s->kv = d->kv_dtype == ASP_KV_BF16 ? 0 : 1;
  s->W = 0;
  s->C = 0;
  s->lambda = 0.0;
  s->R = 0;
  return ASP_OK;
}

asp_status check_cfg(const asp_cfg* c, Shape* s) {
  if (c == nullptr) return ASP_ERR_INVALID_ARG;
  if (c->window < 4 || c->window > 64 || c->window % 4 != 0) return ASP_ERR_INVALID_ARG;
  if (c->top_c < 1 || c->top_c > s->T_cap) return ASP_ERR_INVALID_ARG;
  if (!(c->lambda > 0.0) || !isfinite(c->lambda)) return ASP_ERR_INVALID_ARG;
  if (c->recent < 0 || c->recent > s->T_cap) return ASP_ERR_INVALID_ARG;
  const int tpb = asp::attend_tokens_per_block(s->D, s->kv);
  if (((int64_t)c->top_c + c->recent + tpb - 1) / tpb > 256)
    return ASP_ERR_UNSUPPORTED;  // more attention splits than the merge handles
  s->W = c->window;
  s->C = c->top_c;
  s->lambda = c->lambda;
  s->R = c->recent;
  return ASP_OK;
}

asp_status check_all(const asp_dims* d, const asp_cfg* c, Shape* s) {
  asp_status st = check_dims(d, s);
  if (st != ASP_OK) return st;
  return check_cfg(c, s);
}

struct StepLayout {
  size_t cand, q_pred, partials, total;
};

// Workspace of asp_step: the candidate workspace (threshold hints first, kept
// from one step of the layer to the next; candidate regions) and the predicted
// queries (selection streams), attention partials (attention stream).
StepLayout step_layout(const Shape& s) {
  StepLayout l;
  l.cand = 0;
  l.q_pred = align_up(l.cand + asp::cand_ws_bytes(s));
  l.partials = align_up(l.q_pred + (size_t)s.B * s.Hq * s.D * sizeof(float));
  l.total = align_up(l.partials + asp::attend_partials_bytes(s));
  return l;
}

size_t ws_bytes_for(const Shape& s, asp_op op) {
  switch (op) {
    case ASP_OP_SELECT: return align_up(asp::select_ws_bytes(s, true));
    case ASP_OP_DECODE: return align_up(asp::attend_partials_bytes(s));
    case ASP_OP_STEP: return step_layout(s).total;
    case ASP_OP_CANDIDATES: return align_up(asp::cand_ws_bytes(s));
    default: return 0;
  }
}

asp_status hip_status(hipError_t e) { return e == hipSuccess ? ASP_OK : ASP_ERR_HIP; }

// The kernels use 16-byte vector loads on K, V, queries and the ring.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define ASP_TRY_HIP(expr)                          \
  do {                                             \
    if ((expr) != hipSuccess) return ASP_ERR_HIP;  \
  } while (0)

}  // namespace

// Caller-owned state of the two-stream asp_step: the stream that runs the
// score passes and the two events that order the step's streams.  Created by
// asp_context_create on one device, used by one asp_step call at a time, and
// released by asp_context_destroy; the library keeps nothing else.
struct asp_context_s {
  int device;
  uint32_t flags;
  hipStream_t score;    // score passes of successive calls run back to back here
  hipEvent_t pred;      // recorded by the predictor launch (q_pred and the ring slot written)
  hipEvent_t scored;    // recorded by the score launch (candidates kept)
  hipEvent_t joined;    // recorded by asp_context_join on the score stream
};

namespace {

// The score stream's CU mask: every CU but those of the last 32-CU group.  On
// MI355X (256 CUs) the mask words map to the eight XCDs, so the score passes
// run on seven XCDs and leave the eighth to the latency-bound launches
// (predictor, select, merge), which otherwise wait for CU slots behind score
// blocks.  Falls back to an unmasked stream where the device has one group or
// the mask is refused.
hipError_t create_score_stream(int dev, bool masked, hipStream_t* st) {
  int ncu = 0;
  if (masked && hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      ncu % 32 == 0 && ncu / 32 >= 2 && ncu / 32 <= 32) {
    uint32_t mask[32] = {};
    const int words = ncu / 32;
    for (int w = 0; w + 1 < words; ++w) mask[w] = 0xffffffffu;
    if (hipExtStreamCreateWithCUMask(st, (uint32_t)words, mask) == hipSuccess) return hipSuccess;
    (void)hipGetLastError();  // refused: clear the error, fall back below
  }
  return hipStreamCreateWithFlags(st, hipStreamNonBlocking);
}

// Releases what a context holds (any member may be null).
void context_release(asp_context* c) {
  if (c->score) {
    (void)hipStreamSynchronize(c->score);
    (void)hipStreamDestroy(c->score);
  }
  if (c->pred) (void)hipEventDestroy(c->pred);
  if (c->scored) (void)hipEventDestroy(c->scored);
  if (c->joined) (void)hipEventDestroy(c->joined);
  delete c;
}

// Selection work of one step on one stream: the predictor pushes q_cur into
// every head's ring slot and predicts; the score launch keeps the candidates;
// the select launches pick from them (rescoring the units left short), and the
// first advances the ring.
asp_status run_selection(const Shape& s, const float* q_cur, float* q_hist, int32_t* newest, int32_t* len,
                         const void* k, const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, float* q_pred,
                         const asp::CandWs& cw, hipStream_t st, hipEvent_t done) {
  ASP_TRY_HIP(asp::launch_predict(s, q_hist, newest, len, q_cur, q_pred, st));
  ASP_TRY_HIP(asp::launch_score_candidates(s, q_pred, k, seq_lens, cw, false, st));
  ASP_TRY_HIP(asp::launch_select_candidates(s, q_pred, k, seq_lens, cw, idx, n_sel, newest, len, st, done));
  return ASP_OK;
}

// Candidate workspace checks shared by the candidate entry points.
asp_status check_cand_ws(const Shape& s, void* ws, size_t ws_bytes) {
  if (ws == nullptr || ws_bytes < asp::cand_ws_bytes(s) || !aligned16(ws)) return ASP_ERR_WORKSPACE;
  return ASP_OK;
}

constexpr int kMaxDevices = 64;

}  // namespace

// Scratch of asp_sparse_decode_static: the attention's split-K partials.  One
// copy per device, held while the library is loaded.  Host code never uses
// this name as an address (it is the host-side stand-in of the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[ASP_STATIC_SCRATCH_BYTES];

namespace {

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipErrorNotInitialized;
};
ScratchSlot g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call made with that device current.
asp_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ASP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ASP_ERR_UNSUPPORTED;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess || slot.ptr == nullptr) return ASP_ERR_HIP;
  *out = slot.ptr;
  return ASP_OK;
}

}  // namespace

extern "C" {

size_t asp_workspace_size(const asp_dims* dims, const asp_cfg* cfg, asp_op op) {
  Shape s;
  if (check_all(dims, cfg, &s) != ASP_OK) return 0;
  return ws_bytes_for(s, op);
}

const char* asp_status_string(asp_status status) {
  switch (status) {
    case ASP_OK: return "ok";
    case ASP_ERR_INVALID_ARG: return "invalid argument (dimension, configuration value or null pointer)";
    case ASP_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be 64 or 128, GQA group 1, 2, 4 or 8)";
    case ASP_ERR_WORKSPACE: return "workspace missing, not 16-byte aligned or smaller than asp_workspace_size()";
    case ASP_ERR_HIP: return "a HIP kernel launch, event or stream call failed";
    case ASP_ERR_HOST_MEMORY: return "host memory allocation failed";
    case ASP_ERR_SCRATCH:
      return "the shape needs more attention scratch than the built-in buffer (ASP_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

asp_status asp_push_query(const asp_dims* dims, const asp_cfg* cfg, const float* q_cur, float* q_hist,
                          int32_t* hist_newest, int32_t* hist_len, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q_cur || !q_hist || !hist_newest || !hist_len) return ASP_ERR_INVALID_ARG;
  if (!aligned16(q_cur) || !aligned16(q_hist) || !aligned4(hist_newest) || !aligned4(hist_len))
    return ASP_ERR_INVALID_ARG;
  return hip_status(asp::launch_push(s, q_cur, q_hist, hist_newest, hist_len, stream));
}

asp_status asp_predict_query(const asp_dims* dims, const asp_cfg* cfg, const float* q_hist,
                             const int32_t* hist_newest, const int32_t* hist_len, float* q_pred,
                             hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q_hist || !hist_newest || !hist_len || !q_pred) return ASP_ERR_INVALID_ARG;
  if (!aligned16(q_hist) || !aligned4(q_pred) || !aligned4(hist_newest) || !aligned4(hist_len))
    return ASP_ERR_INVALID_ARG;
  return hip_status(asp::launch_predict(s, const_cast<float*>(q_hist), hist_newest, hist_len, nullptr, q_pred,
                                        stream));
}

asp_status asp_score_keys(const asp_dims* dims, const float* q_pred, const void* k, const int32_t* seq_lens,
                          float* scores, uint32_t* hist, hipStream_t stream) {
  Shape s;
  asp_status st = check_dims(dims, &s);
  if (st != ASP_OK) return st;
  if (!q_pred || !k || !seq_lens || !scores) return ASP_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned4(q_pred) || !aligned4(seq_lens) || !aligned4(scores) || !aligned16(hist))
    return ASP_ERR_INVALID_ARG;
  if (hist != nullptr)  // the score launch adds to the histograms
    ASP_TRY_HIP(asp::launch_clear_u32(hist, (size_t)s.B * s.Hkv * asp::HIST_BINS, stream));
  return hip_status(asp::launch_score(s, q_pred, k, seq_lens, scores, hist, stream));
}

asp_status asp_select_topc(const asp_dims* dims, const asp_cfg* cfg, const float* scores, const uint32_t* hist,
                           const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!scores || !seq_lens || !idx || !n_sel) return ASP_ERR_INVALID_ARG;
  if (!aligned4(scores) || !aligned16(hist) || !aligned4(seq_lens) || !aligned4(idx) || !aligned4(n_sel))
    return ASP_ERR_INVALID_ARG;
  const size_t need = ws_bytes_for(s, ASP_OP_SELECT);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return ASP_ERR_WORKSPACE;
  return hip_status(asp::launch_select(s, scores, hist, seq_lens, idx, n_sel, nullptr, nullptr, ws, stream));
}

asp_status asp_score_candidates(const asp_dims* dims, const asp_cfg* cfg, const float* q_pred, const void* k,
                                const int32_t* seq_lens, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q_pred || !k || !seq_lens) return ASP_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned4(q_pred) || !aligned4(seq_lens)) return ASP_ERR_INVALID_ARG;
  st = check_cand_ws(s, ws, ws_bytes);
  if (st != ASP_OK) return st;
  return hip_status(asp::launch_score_candidates(s, q_pred, k, seq_lens, asp::cand_carve(s, ws), false, stream));
}

asp_status asp_select_candidates(const asp_dims* dims, const asp_cfg* cfg, const float* q_pred, const void* k,
                                 const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q_pred || !k || !seq_lens || !idx || !n_sel) return ASP_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned4(q_pred) || !aligned4(seq_lens) || !aligned4(idx) || !aligned4(n_sel))
    return ASP_ERR_INVALID_ARG;
  st = check_cand_ws(s, ws, ws_bytes);
  if (st != ASP_OK) return st;
  return hip_status(asp::launch_select_candidates(s, q_pred, k, seq_lens, asp::cand_carve(s, ws), idx, n_sel,
                                                  nullptr, nullptr, stream));
}

asp_status asp_selection_overlap(const asp_dims* dims, const asp_cfg* cfg, const int32_t* idx_a,
                                 const int32_t* n_sel_a, const int32_t* idx_b, const int32_t* n_sel_b,
                                 int32_t* overlap, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!idx_a || !n_sel_a || !idx_b || !n_sel_b || !overlap) return ASP_ERR_INVALID_ARG;
  if (!aligned4(idx_a) || !aligned4(n_sel_a) || !aligned4(idx_b) || !aligned4(n_sel_b) || !aligned4(overlap))
    return ASP_ERR_INVALID_ARG;
  if (s.C > asp::overlap_max_c()) return ASP_ERR_UNSUPPORTED;
  return hip_status(asp::launch_overlap(s, idx_a, n_sel_a, idx_b, n_sel_b, overlap, stream));
}

asp_status asp_check_device_args(const asp_dims* dims, const asp_cfg* cfg, const int32_t* seq_lens,
                                 const int32_t* hist_newest, const int32_t* hist_len, const int32_t* idx,
                                 const int32_t* n_sel, uint32_t* status, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!seq_lens || !status) return ASP_ERR_INVALID_ARG;
  if ((hist_newest == nullptr) != (hist_len == nullptr) || (idx == nullptr) != (n_sel == nullptr))
    return ASP_ERR_INVALID_ARG;
  if (!aligned4(seq_lens) || !aligned4(status) || !aligned4(hist_newest) || !aligned4(hist_len) || !aligned4(idx) ||
      !aligned4(n_sel))
    return ASP_ERR_INVALID_ARG;
  return hip_status(asp::launch_check(s, seq_lens, hist_newest, hist_len, idx, n_sel, status, stream));
}

asp_status asp_sparse_decode(const asp_dims* dims, const asp_cfg* cfg, const float* q, const void* k, const void* v,
                             const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel, float* out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q || !k || !v || !idx || !n_sel || !out) return ASP_ERR_INVALID_ARG;
  if (s.R > 0 && seq_lens == nullptr) return ASP_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned4(q) || !aligned4(out) || !aligned4(seq_lens) || !aligned4(idx) ||
      !aligned4(n_sel))
    return ASP_ERR_INVALID_ARG;
  const size_t need = ws_bytes_for(s, ASP_OP_DECODE);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return ASP_ERR_WORKSPACE;
  return hip_status(asp::launch_attend(s, q, k, v, seq_lens, idx, n_sel, out, ws, stream));
}

asp_status asp_sparse_decode_static(const asp_dims* dims, const asp_cfg* cfg, const float* q, const void* k,
                                    const void* v, const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel,
                                    float* out, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q || !k || !v || !idx || !n_sel || !out) return ASP_ERR_INVALID_ARG;
  if (s.R > 0 && seq_lens == nullptr) return ASP_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned4(q) || !aligned4(out) || !aligned4(seq_lens) || !aligned4(idx) ||
      !aligned4(n_sel))
    return ASP_ERR_INVALID_ARG;
  if (asp::attend_partials_bytes(s) > (size_t)ASP_STATIC_SCRATCH_BYTES) return ASP_ERR_SCRATCH;
  void* partials = nullptr;
  st = scratch_on_current_device(&partials);
  if (st != ASP_OK) return st;
  return hip_status(asp::launch_attend(s, q, k, v, seq_lens, idx, n_sel, out, partials, stream));
}

size_t asp_page_summary_size(const asp_dims* dims, int32_t page_size) {
  Shape s;
  if (check_dims(dims, &s) != ASP_OK || page_size < 1 || page_size > s.T_cap) return 0;
  return (size_t)s.B * s.Hkv * asp::page_count(s.T_cap, page_size) * s.D * (s.kv == 0 ? 2 : 4);
}

asp_status asp_page_summary(const asp_dims* dims, int32_t page_size, const void* k, const int32_t* seq_lens,
                            void* kmin, void* kmax, hipStream_t stream) {
  Shape s;
  asp_status st = check_dims(dims, &s);
  if (st != ASP_OK) return st;
  if (page_size < 1 || page_size > s.T_cap) return ASP_ERR_INVALID_ARG;
  if (!k || !seq_lens || !kmin || !kmax) return ASP_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(kmin) || !aligned16(kmax) || !aligned4(seq_lens)) return ASP_ERR_INVALID_ARG;
  return hip_status(asp::launch_page_summary(s, page_size, k, seq_lens, kmin, kmax, stream));
}

asp_status asp_page_scores(const asp_dims* dims, int32_t page_size, const float* q, const void* kmin,
                           const void* kmax, const int32_t* seq_lens, float* scores, hipStream_t stream) {
  Shape s;
  asp_status st = check_dims(dims, &s);
  if (st != ASP_OK) return st;
  if (page_size < 1 || page_size > s.T_cap) return ASP_ERR_INVALID_ARG;
  if (!q || !kmin || !kmax || !seq_lens || !scores) return ASP_ERR_INVALID_ARG;
  if (!aligned4(q) || !aligned16(kmin) || !aligned16(kmax) || !aligned4(seq_lens) || !aligned4(scores))
    return ASP_ERR_INVALID_ARG;
  return hip_status(asp::launch_page_scores(s, page_size, q, kmin, kmax, seq_lens, scores, nullptr, stream));
}

size_t asp_page_select_workspace_size(const asp_dims* dims, const asp_cfg* cfg, int32_t page_size) {
  Shape s;
  if (check_all(dims, cfg, &s) != ASP_OK || page_size < 1 || s.C % page_size != 0) return 0;
  return align_up(asp::page_select_ws_bytes(s, page_size));
}

asp_status asp_page_select(const asp_dims* dims, const asp_cfg* cfg, int32_t page_size, const float* q,
                           const void* kmin, const void* kmax, const int32_t* seq_lens, int32_t* idx,
                           int32_t* n_sel, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (page_size < 1 || s.C % page_size != 0) return ASP_ERR_INVALID_ARG;
  if (!q || !kmin || !kmax || !seq_lens || !idx || !n_sel) return ASP_ERR_INVALID_ARG;
  if (!aligned4(q) || !aligned16(kmin) || !aligned16(kmax) || !aligned4(seq_lens) || !aligned4(idx) ||
      !aligned4(n_sel))
    return ASP_ERR_INVALID_ARG;
  const size_t need = align_up(asp::page_select_ws_bytes(s, page_size));
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return ASP_ERR_WORKSPACE;
  return hip_status(asp::launch_page_select(s, page_size, q, kmin, kmax, seq_lens, idx, n_sel, ws, stream));
}

asp_status asp_context_create(int32_t device, uint32_t flags, asp_context** ctx) {
  if (ctx == nullptr) return ASP_ERR_INVALID_ARG;
  *ctx = nullptr;
  if ((flags & ~(uint32_t)ASP_CTX_SCORE_ALL_CUS) != 0) return ASP_ERR_INVALID_ARG;
  int n = 0, cur = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || hipGetDevice(&cur) != hipSuccess) return ASP_ERR_HIP;
  if (device < 0 || device >= n) return ASP_ERR_INVALID_ARG;
  asp_context* c = new (std::nothrow) asp_context{device, flags, nullptr, nullptr, nullptr, nullptr};
  if (c == nullptr) return ASP_ERR_HOST_MEMORY;
  hipError_t e = cur == device ? hipSuccess : hipSetDevice(device);
  if (e == hipSuccess) e = create_score_stream(device, (flags & ASP_CTX_SCORE_ALL_CUS) == 0, &c->score);
  const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->pred, ev_flags);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->scored, ev_flags);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->joined, ev_flags);
  if (cur != device) (void)hipSetDevice(cur);
  if (e != hipSuccess) {
    context_release(c);
    return ASP_ERR_HIP;
  }
  *ctx = c;
  return ASP_OK;
}

asp_status asp_context_destroy(asp_context* ctx) {
  if (ctx == nullptr) return ASP_OK;
  bool ok = hipStreamSynchronize(ctx->score) == hipSuccess;
  ok &= hipStreamDestroy(ctx->score) == hipSuccess;
  ok &= hipEventDestroy(ctx->pred) == hipSuccess;
  ok &= hipEventDestroy(ctx->scored) == hipSuccess;
  ok &= hipEventDestroy(ctx->joined) == hipSuccess;
  delete ctx;
  return ok ? ASP_OK : ASP_ERR_HIP;
}

asp_status asp_context_join(asp_context* ctx, hipStream_t stream) {
  if (ctx == nullptr) return ASP_ERR_INVALID_ARG;
  ASP_TRY_HIP(hipEventRecord(ctx->joined, ctx->score));
  ASP_TRY_HIP(hipStreamWaitEvent(stream, ctx->joined, 0));
  return ASP_OK;
}

asp_status asp_step(asp_context* ctx, const asp_dims* dims, const asp_cfg* cfg, const float* q_cur, float* q_hist,
                    int32_t* hist_newest, int32_t* hist_len, const void* k, const void* v,
                    const int32_t* seq_lens, const int32_t* idx_cur, const int32_t* n_sel_cur,
                    int32_t* idx_next, int32_t* n_sel_next, float* out, void* ws, size_t ws_bytes,
                    hipStream_t attn_stream, hipStream_t sel_stream, hipEvent_t idx_cur_ready,
                    hipEvent_t idx_next_ready) {
  Shape s;
  asp_status st = check_all(dims, cfg, &s);
  if (st != ASP_OK) return st;
  if (!q_cur || !q_hist || !hist_newest || !hist_len || !k || !v || !seq_lens || !idx_next || !n_sel_next || !out)
    return ASP_ERR_INVALID_ARG;
  if ((idx_cur == nullptr) != (n_sel_cur == nullptr)) return ASP_ERR_INVALID_ARG;
  if (!aligned16(q_cur) || !aligned16(q_hist) || !aligned16(k) || !aligned16(v) || !aligned4(out) ||
      !aligned4(hist_newest) || !aligned4(hist_len) || !aligned4(seq_lens) || !aligned4(idx_cur) ||
      !aligned4(n_sel_cur) || !aligned4(idx_next) || !aligned4(n_sel_next))
    return ASP_ERR_INVALID_ARG;
  if (!aligned16(ws)) return ASP_ERR_WORKSPACE;
  const bool pipelined = idx_cur != nullptr;
  const bool two_streams = pipelined && sel_stream != nullptr && sel_stream != attn_stream;
  if (two_streams) {
    // Under capture the caller may order the step itself (no idx_cur_ready).
    if (ctx == nullptr) return ASP_ERR_INVALID_ARG;
    if (idx_cur_ready == nullptr && !asp::capturing(attn_stream)) return ASP_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ASP_ERR_HIP;
    if (dev != ctx->device) return ASP_ERR_INVALID_ARG;  // the context's stream is on another device
    // Under capture the context's stream and sel_stream join the capture of
    // attn_stream through the step's own events; sel_stream must not be
    // capturing into another graph (or into one while attn_stream is not).
    const unsigned long long sel_cap = asp::capture_id(sel_stream);
    if (sel_cap != 0 && sel_cap != asp::capture_id(attn_stream)) return ASP_ERR_UNSUPPORTED;
  }
  const StepLayout lay = step_layout(s);
  if (ws == nullptr || ws_bytes < lay.total) return ASP_ERR_WORKSPACE;
  unsigned char* base = static_cast<unsigned char*>(ws);
  const asp::CandWs cw = asp::cand_carve(s, base + lay.cand);
  float* q_pred = reinterpret_cast<float*>(base + lay.q_pred);
  void* partials = base + lay.partials;

  if (!pipelined) {
    // A first step: whatever the workspace holds, every key is kept (hint 0)
    // rather than left to the rescoring launch.
    ASP_TRY_HIP(asp::launch_clear_u32(cw.hint, (size_t)s.B * s.Hkv, attn_stream));
    st = run_selection(s, q_cur, q_hist, hist_newest, hist_len, k, seq_lens, idx_next, n_sel_next, q_pred, cw,
                       attn_stream, nullptr);
    if (st != ASP_OK) return st;
    ASP_TRY_HIP(asp::launch_attend(s, q_cur, k, v, seq_lens, idx_next, n_sel_next, out, partials, attn_stream));
    if (idx_next_ready) ASP_TRY_HIP(hipEventRecord(idx_next_ready, attn_stream));
    return ASP_OK;
  }
  if (!two_streams) {
    ASP_TRY_HIP(asp::launch_attend(s, q_cur, k, v, seq_lens, idx_cur, n_sel_cur, out, partials, attn_stream));
    return run_selection(s, q_cur, q_hist, hist_newest, hist_len, k, seq_lens, idx_next, n_sel_next, q_pred, cw,
                         attn_stream, idx_next_ready);
  }
  // Two streams of the caller and the context's score stream:
  //  - attn_stream waits for idx_cur_ready (the selection it attends over is
  //    written, and the previous selection made with this workspace has
  //    finished with the candidates, the hints and the ring), then the
  //    predictor pushes q_cur into the ring and predicts (its launch records
  //    the context's `pred` event), then the attention over idx_cur and its
  //    merge run;
  //  - the score stream waits for `pred` and scores (the launch records
  //    `scored`);
  //  - sel_stream waits for `scored` and selects (its first launch advances
  //    the ring); the last launch records idx_next_ready.
  // Events recorded by a launch itself cost no extra queue packet.  A wait on
  // an event that has not completed costs the host ~14 us, so the step makes
  // two (pred, scored); idx_cur_ready has usually completed by the time the
  // layer's next step is issued.  The attention is issued before those two
  // waits: when the GPU is idle (the first steps of a run) it then starts
  // right after the predictor instead of after the host's waits, and the next
  // step's predictor, queued behind it, is not held back.
  if (idx_cur_ready != nullptr) ASP_TRY_HIP(hipStreamWaitEvent(attn_stream, idx_cur_ready, 0));
  ASP_TRY_HIP(asp::launch_predict(s, q_hist, hist_newest, hist_len, q_cur, q_pred, attn_stream, ctx->pred));
  ASP_TRY_HIP(asp::launch_attend(s, q_cur, k, v, seq_lens, idx_cur, n_sel_cur, out, partials, attn_stream));
  ASP_TRY_HIP(hipStreamWaitEvent(ctx->score, ctx->pred, 0));
  ASP_TRY_HIP(asp::launch_score_candidates(s, q_pred, k, seq_lens, cw, false, ctx->score, ctx->scored));
  ASP_TRY_HIP(hipStreamWaitEvent(sel_stream, ctx->scored, 0));
  ASP_TRY_HIP(asp::launch_select_candidates(s, q_pred, k, seq_lens, cw, idx_next, n_sel_next, hist_newest, hist_len,
                                            sel_stream, idx_next_ready));
  return ASP_OK;
}

}  // extern "C"
