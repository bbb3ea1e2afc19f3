// The C ABI used from C++ alone (no Python, no PyTorch): a layer's pipelined
// decode steps run on one stream and on two streams from identical inputs, and
// every step's attention output, selection and query ring must agree bit for
// bit.  Built by __graft_entry__.build(); run by tests/test_gpu_c_abi.py.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "asp.h"

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

namespace {

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

struct Layer {
  float *q_hist, *out, *q;
  int32_t *newest, *len, *idx[2], *nsel[2];
  void* ws;
};

}  // namespace

int main() {
  const asp_dims d = {4, 16, 4, 128, 4096, ASP_KV_BF16};
  const asp_cfg c = {8, 512, 1e-2, 0};
  const int B = d.batch, Hq = d.n_q_heads, Hkv = d.n_kv_heads, D = d.head_dim, T = d.t_cap, C = c.top_c;
  const int W = c.window, steps = 6;
  const size_t kv_n = (size_t)B * Hkv * T * D, q_n = (size_t)B * Hq * D;

  Lcg r{12345};
  std::vector<uint16_t> kh(kv_n), vh(kv_n);
  for (auto& x : kh) x = to_bf16(r.uniform() * 2.0f);
  for (auto& x : vh) x = to_bf16(r.uniform());
  const int32_t lens_h[4] = {4096, 3000, 700, 1};
  std::vector<float> qs((size_t)(W + steps) * q_n);
  for (auto& x : qs) x = r.uniform();

  void *k, *v;
  int32_t* lens;
  CHECK_HIP(hipMalloc(&k, kv_n * 2));
  CHECK_HIP(hipMalloc(&v, kv_n * 2));
  CHECK_HIP(hipMalloc((void**)&lens, sizeof lens_h));
  CHECK_HIP(hipMemcpy(k, kh.data(), kv_n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, vh.data(), kv_n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(lens, lens_h, sizeof lens_h, hipMemcpyHostToDevice));
  const size_t ws_bytes = asp_workspace_size(&d, &c, ASP_OP_STEP);
  if (ws_bytes == 0) return 4;

  // Two copies of the layer's state: [0] one stream, [1] two streams.
  Layer L[2];
  for (auto& l : L) {
    CHECK_HIP(hipMalloc((void**)&l.q_hist, (size_t)B * Hq * W * D * 4));
    CHECK_HIP(hipMalloc((void**)&l.out, q_n * 4));
    CHECK_HIP(hipMalloc((void**)&l.q, q_n * 4));
    CHECK_HIP(hipMalloc((void**)&l.newest, B * 4));
    CHECK_HIP(hipMalloc((void**)&l.len, B * 4));
    for (int i = 0; i < 2; ++i) {
      CHECK_HIP(hipMalloc((void**)&l.idx[i], (size_t)B * Hkv * C * 4));
      CHECK_HIP(hipMalloc((void**)&l.nsel[i], (size_t)B * Hkv * 4));
    }
    CHECK_HIP(hipMalloc(&l.ws, ws_bytes));
    CHECK_HIP(hipMemset(l.q_hist, 0, (size_t)B * Hq * W * D * 4));
    CHECK_HIP(hipMemset(l.len, 0, B * 4));
    std::vector<int32_t> nw(B, W - 1);
    CHECK_HIP(hipMemcpy(l.newest, nw.data(), B * 4, hipMemcpyHostToDevice));
  }
  hipStream_t attn, sel;
  CHECK_HIP(hipStreamCreateWithFlags(&attn, hipStreamNonBlocking));
  CHECK_HIP(hipStreamCreateWithFlags(&sel, hipStreamNonBlocking));
  hipEvent_t q_ready, ev[2];
  CHECK_HIP(hipEventCreateWithFlags(&q_ready, hipEventDisableTiming));
  for (auto& e : ev) CHECK_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));

  // History, then the bootstrap step, identical for both copies.
  for (auto& l : L) {
    for (int t = 0; t < W - 1; ++t) {  // the copy and the push in one stream's order
      CHECK_HIP(hipMemcpyAsync(l.q, qs.data() + (size_t)t * q_n, q_n * 4, hipMemcpyHostToDevice, attn));
      CHECK_ASP(asp_push_query(&d, &c, l.q, l.q_hist, l.newest, l.len, attn));
      CHECK_HIP(hipStreamSynchronize(attn));
    }
    CHECK_HIP(hipMemcpyAsync(l.q, qs.data() + (size_t)(W - 1) * q_n, q_n * 4, hipMemcpyHostToDevice, attn));
    CHECK_ASP(asp_step(&d, &c, l.q, l.q_hist, l.newest, l.len, k, v, lens, nullptr, nullptr, l.idx[0], l.nsel[0],
                       l.out, l.ws, ws_bytes, attn, nullptr, nullptr, nullptr, &l == &L[1] ? ev[0] : nullptr));
    CHECK_HIP(hipStreamSynchronize(attn));
  }

  std::vector<float> o0(q_n), o1(q_n);
  std::vector<int32_t> i0((size_t)B * Hkv * C), i1((size_t)B * Hkv * C), n0(B * Hkv), n1(B * Hkv);
  std::vector<float> h0((size_t)B * Hq * W * D), h1((size_t)B * Hq * W * D);
  {  // the bootstrap steps agree too
    CHECK_HIP(hipMemcpy(o0.data(), L[0].out, q_n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(o1.data(), L[1].out, q_n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(i0.data(), L[0].idx[0], i0.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(i1.data(), L[1].idx[0], i1.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(n0.data(), L[0].nsel[0], n0.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(n1.data(), L[1].nsel[0], n1.size() * 4, hipMemcpyDeviceToHost));
    const bool same_out = std::memcmp(o0.data(), o1.data(), q_n * 4) == 0;
    const bool same_idx = std::memcmp(i0.data(), i1.data(), i0.size() * 4) == 0;
    const bool same_n = std::memcmp(n0.data(), n1.data(), n0.size() * 4) == 0;
    std::printf("bootstrap: %s\n", same_out && same_idx && same_n ? "agree" : "DIFFER");
    if (!(same_out && same_idx && same_n)) {
      std::printf("  out %s, idx %s, n_sel %s\n", same_out ? "same" : "differs", same_idx ? "same" : "differs",
                  same_n ? "same" : "differs");
      return 1;
    }
  }
  for (int s = 0; s < steps; ++s) {
    const int cur = s % 2, nxt = 1 - cur;
    const float* qsrc = qs.data() + (size_t)(W + s) * q_n;
    for (int m = 0; m < 2; ++m) {
      Layer& l = L[m];
      CHECK_HIP(hipMemcpyAsync(l.q, qsrc, q_n * 4, hipMemcpyHostToDevice, attn));
      if (m == 0)
        CHECK_ASP(asp_step(&d, &c, l.q, l.q_hist, l.newest, l.len, k, v, lens, l.idx[cur], l.nsel[cur], l.idx[nxt],
                           l.nsel[nxt], l.out, l.ws, ws_bytes, attn, nullptr, nullptr, nullptr, nullptr));
      else
        CHECK_ASP(asp_step(&d, &c, l.q, l.q_hist, l.newest, l.len, k, v, lens, l.idx[cur], l.nsel[cur], l.idx[nxt],
                           l.nsel[nxt], l.out, l.ws, ws_bytes, attn, sel, q_ready, ev[cur], ev[nxt]));
      CHECK_HIP(hipDeviceSynchronize());
    }
    CHECK_HIP(hipMemcpy(o0.data(), L[0].out, q_n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(o1.data(), L[1].out, q_n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(i0.data(), L[0].idx[nxt], i0.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(i1.data(), L[1].idx[nxt], i1.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(n0.data(), L[0].nsel[nxt], n0.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(n1.data(), L[1].nsel[nxt], n1.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h0.data(), L[0].q_hist, h0.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h1.data(), L[1].q_hist, h1.size() * 4, hipMemcpyDeviceToHost));
    const bool same_out = std::memcmp(o0.data(), o1.data(), q_n * 4) == 0;
    const bool same_idx = std::memcmp(i0.data(), i1.data(), i0.size() * 4) == 0;
    const bool same_n = std::memcmp(n0.data(), n1.data(), n0.size() * 4) == 0;
    const bool same_ring = std::memcmp(h0.data(), h1.data(), h0.size() * 4) == 0;
    const bool same = same_out && same_idx && same_n && same_ring;
    int sel_total = 0;
    for (int x : n0) sel_total += x;
    std::printf("step %d: one stream and two streams %s (selected %d tokens)\n", s, same ? "agree" : "DIFFER",
                sel_total);
    if (!same) {
      std::printf("  out %s, idx %s, n_sel %s, ring %s\n", same_out ? "same" : "differs",
                  same_idx ? "same" : "differs", same_n ? "same" : "differs", same_ring ? "same" : "differs");
      for (size_t i = 0; i < i0.size(); ++i)
        if (i0[i] != i1[i]) {
          std::printf("  first idx difference at unit %zu slot %zu: %d vs %d\n", i / C, i % C, i0[i], i1[i]);
          break;
        }
    }
    if (!same) return 1;
  }
  CHECK_ASP(asp_release_streams());
  std::printf("c-abi step check: ok\n");
  return 0;
}
