// The C ABI used from C++ alone (no Python, no PyTorch).  A layer's pipelined
// decode steps run from identical inputs
//  - on one stream,
//  - on two streams with a context, serially,
//  - on two streams with a context each, in two host threads at once (each
//    thread its own copy of the layer's state, streams and events),
// and every step's attention output, selection and query ring must agree bit
// for bit across all of them.  Built by __graft_entry__.build(); run by
// tests/test_gpu_c_abi.py.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "asp.h"

namespace {

#define CHECK_HIP(x)                                                          \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
      return 2;                                                               \
    }                                                                         \
  } while (0)
#define CHECK_ASP(x)                                                          \
  do {                                                                        \
    asp_status s_ = (x);                                                      \
    if (s_ != ASP_OK) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, asp_status_string(s_));     \
      return 3;                                                               \
    }                                                                         \
  } while (0)

struct Lcg {  // deterministic inputs
  uint64_t s;
  float uniform() {  // [-1, 1)
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((s >> 40) & 0xffffff) / 8388608.0f - 1.0f;
  }
};

uint16_t to_bf16(float x) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

const asp_dims kDims = {4, 16, 4, 128, 4096, ASP_KV_BF16};
const asp_cfg kCfg = {8, 512, 1e-2, 0};
constexpr int kSteps = 6;

// What a step leaves behind: the attention output, the new selection and the ring.
struct Snapshot {
  std::vector<float> out, ring;
  std::vector<int32_t> idx, nsel;
  bool operator==(const Snapshot& o) const {
    return out == o.out && ring == o.ring && idx == o.idx && nsel == o.nsel;
  }
};

// Shared read-only inputs.
struct Inputs {
  void *k, *v;
  int32_t* lens;
  std::vector<float> qs;  // (W + kSteps) queries [B][Hq][D]
};

enum class Mode { one_stream, two_streams };

// One copy of a layer's state, its streams and events; run() makes the
// bootstrap step and kSteps pipelined steps and snapshots each.
struct Layer {
  float *q_hist = nullptr, *out = nullptr, *q = nullptr;
  int32_t *newest = nullptr, *len = nullptr, *idx[2] = {}, *nsel[2] = {};
  uint32_t* status = nullptr;  // asp_check_device_args' word
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t attn = nullptr, sel = nullptr;
  hipEvent_t ev[2] = {};
  std::vector<Snapshot> snaps;

  int init() {
    const int B = kDims.batch, Hq = kDims.n_q_heads, Hkv = kDims.n_kv_heads, D = kDims.head_dim;
    const int W = kCfg.window, C = kCfg.top_c;
    const size_t q_n = (size_t)B * Hq * D;
    CHECK_HIP(hipMalloc((void**)&q_hist, (size_t)B * Hq * W * D * 4));
    CHECK_HIP(hipMalloc((void**)&out, q_n * 4));
    CHECK_HIP(hipMalloc((void**)&q, q_n * 4));
    CHECK_HIP(hipMalloc((void**)&newest, B * 4));
    CHECK_HIP(hipMalloc((void**)&len, B * 4));
    CHECK_HIP(hipMalloc((void**)&status, 4));
    for (int i = 0; i < 2; ++i) {
      CHECK_HIP(hipMalloc((void**)&idx[i], (size_t)B * Hkv * C * 4));
      CHECK_HIP(hipMalloc((void**)&nsel[i], (size_t)B * Hkv * 4));
      CHECK_HIP(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming));
    }
    ws_bytes = asp_workspace_size(&kDims, &kCfg, ASP_OP_STEP);
    if (ws_bytes == 0) return 4;
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_HIP(hipMemset(q_hist, 0, (size_t)B * Hq * W * D * 4));
    CHECK_HIP(hipMemset(len, 0, B * 4));
    std::vector<int32_t> nw(B, W - 1);
    CHECK_HIP(hipMemcpy(newest, nw.data(), B * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipStreamCreateWithFlags(&attn, hipStreamNonBlocking));
    CHECK_HIP(hipStreamCreateWithFlags(&sel, hipStreamNonBlocking));
    return 0;
  }

  // Also checks that the lengths, the ring and the selection just written are
  // what the library's producers leave (no asp_check_device_args bit set).
  int snapshot(int buf, const int32_t* lens) {
    const int B = kDims.batch, Hq = kDims.n_q_heads, Hkv = kDims.n_kv_heads, D = kDims.head_dim;
    CHECK_ASP(asp_check_device_args(&kDims, &kCfg, lens, newest, len, idx[buf], nsel[buf], status, attn));
    uint32_t bits = 0;
    CHECK_HIP(hipMemcpyAsync(&bits, status, 4, hipMemcpyDeviceToHost, attn));
    CHECK_HIP(hipStreamSynchronize(attn));
    if (bits != 0u) {
      std::fprintf(stderr, "asp_check_device_args reported 0x%x\n", bits);
      return 5;
    }
    Snapshot s;
    s.out.resize((size_t)B * Hq * D);
    s.ring.resize((size_t)B * Hq * kCfg.window * D);
    s.idx.resize((size_t)B * Hkv * kCfg.top_c);
    s.nsel.resize((size_t)B * Hkv);
    CHECK_HIP(hipMemcpy(s.out.data(), out, s.out.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(s.ring.data(), q_hist, s.ring.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(s.idx.data(), idx[buf], s.idx.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(s.nsel.data(), nsel[buf], s.nsel.size() * 4, hipMemcpyDeviceToHost));
    snaps.push_back(std::move(s));
    return 0;
  }

  int sync() {
    CHECK_HIP(hipStreamSynchronize(attn));
    CHECK_HIP(hipStreamSynchronize(sel));
    return 0;
  }

  // The history, the bootstrap step, then kSteps pipelined steps; only this
  // layer's streams are synchronised, so that two threads can run at once.
  int run(const Inputs& in, Mode mode, asp_context* ctx) {
    const int W = kCfg.window;
    const size_t q_n = (size_t)kDims.batch * kDims.n_q_heads * kDims.head_dim;
    for (int t = 0; t < W - 1; ++t) {  // the copy and the push in one stream's order
      CHECK_HIP(hipMemcpyAsync(q, in.qs.data() + (size_t)t * q_n, q_n * 4, hipMemcpyHostToDevice, attn));
      CHECK_ASP(asp_push_query(&kDims, &kCfg, q, q_hist, newest, len, attn));
      CHECK_HIP(hipStreamSynchronize(attn));
    }
    CHECK_HIP(hipMemcpyAsync(q, in.qs.data() + (size_t)(W - 1) * q_n, q_n * 4, hipMemcpyHostToDevice, attn));
    CHECK_ASP(asp_step(nullptr, &kDims, &kCfg, q, q_hist, newest, len, in.k, in.v, in.lens, nullptr, nullptr,
                       idx[0], nsel[0], out, ws, ws_bytes, attn, nullptr, nullptr, ev[0]));
    if (int rc = sync()) return rc;
    if (int rc = snapshot(0, in.lens)) return rc;
    for (int s = 0; s < kSteps; ++s) {
      const int cur = s % 2, nxt = 1 - cur;
      CHECK_HIP(hipMemcpyAsync(q, in.qs.data() + (size_t)(W + s) * q_n, q_n * 4, hipMemcpyHostToDevice, attn));
      if (mode == Mode::one_stream)
        CHECK_ASP(asp_step(nullptr, &kDims, &kCfg, q, q_hist, newest, len, in.k, in.v, in.lens, idx[cur],
                           nsel[cur], idx[nxt], nsel[nxt], out, ws, ws_bytes, attn, nullptr, nullptr, nullptr));
      else
        CHECK_ASP(asp_step(ctx, &kDims, &kCfg, q, q_hist, newest, len, in.k, in.v, in.lens, idx[cur], nsel[cur],
                           idx[nxt], nsel[nxt], out, ws, ws_bytes, attn, sel, ev[cur], ev[nxt]));
      if (int rc = sync()) return rc;
      if (int rc = snapshot(nxt, in.lens)) return rc;
    }
    return 0;
  }
};

// Names the first field that differs between two snapshots.
void report(const Snapshot& a, const Snapshot& b) {
  std::printf("  out %s, idx %s, n_sel %s, ring %s\n", a.out == b.out ? "same" : "differs",
              a.idx == b.idx ? "same" : "differs", a.nsel == b.nsel ? "same" : "differs",
              a.ring == b.ring ? "same" : "differs");
}

}  // namespace

int main() {
  const int B = kDims.batch, Hq = kDims.n_q_heads, Hkv = kDims.n_kv_heads, D = kDims.head_dim, T = kDims.t_cap;
  const size_t kv_n = (size_t)B * Hkv * T * D, q_n = (size_t)B * Hq * D;

  Lcg r{12345};
  std::vector<uint16_t> kh(kv_n), vh(kv_n);
  for (auto& x : kh) x = to_bf16(r.uniform() * 2.0f);
  for (auto& x : vh) x = to_bf16(r.uniform());
  const int32_t lens_h[4] = {4096, 3000, 700, 1};
  Inputs in;
  in.qs.resize((size_t)(kCfg.window + kSteps) * q_n);
  for (auto& x : in.qs) x = r.uniform();
  CHECK_HIP(hipMalloc(&in.k, kv_n * 2));
  CHECK_HIP(hipMalloc(&in.v, kv_n * 2));
  CHECK_HIP(hipMalloc((void**)&in.lens, sizeof lens_h));
  CHECK_HIP(hipMemcpy(in.k, kh.data(), kv_n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(in.v, vh.data(), kv_n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(in.lens, lens_h, sizeof lens_h, hipMemcpyHostToDevice));

  // [0] one stream, [1] two streams serially, [2] and [3] two streams in two threads at once.
  Layer L[4];
  for (auto& l : L)
    if (int rc = l.init()) return rc;
  asp_context* ctx[3] = {};
  CHECK_ASP(asp_context_create(0, 0, &ctx[0]));
  CHECK_ASP(asp_context_create(0, 0, &ctx[1]));
  CHECK_ASP(asp_context_create(0, ASP_CTX_SCORE_ALL_CUS, &ctx[2]));

  if (int rc = L[0].run(in, Mode::one_stream, nullptr)) return rc;
  if (int rc = L[1].run(in, Mode::two_streams, ctx[0])) return rc;
  int rc2 = 0, rc3 = 0;
  std::thread t2([&] { rc2 = L[2].run(in, Mode::two_streams, ctx[1]); });
  std::thread t3([&] { rc3 = L[3].run(in, Mode::two_streams, ctx[2]); });
  t2.join();
  t3.join();
  if (rc2 || rc3) {
    std::printf("a thread failed: %d %d\n", rc2, rc3);
    return rc2 ? rc2 : rc3;
  }
  bool ok = true;
  for (int s = 0; s <= kSteps; ++s) {
    const Snapshot& ref = L[0].snaps[s];
    int sel_total = 0;
    for (int x : ref.nsel) sel_total += x;
    const char* what = s == 0 ? "bootstrap" : "step";
    const bool two = ref == L[1].snaps[s];
    const bool threads = ref == L[2].snaps[s] && ref == L[3].snaps[s];
    std::printf("%s %d: one stream and two streams %s; two threads with a context each %s (selected %d tokens)\n",
                what, s, two ? "agree" : "DIFFER", threads ? "agree" : "DIFFER", sel_total);
    if (!two) report(ref, L[1].snaps[s]);
    if (!threads) {
      report(ref, L[2].snaps[s]);
      report(ref, L[3].snaps[s]);
    }
    ok &= two && threads;
  }
  for (auto* c : ctx) CHECK_ASP(asp_context_destroy(c));
  if (!ok) return 1;
  std::printf("c-abi step check: ok\n");
  return 0;
}
