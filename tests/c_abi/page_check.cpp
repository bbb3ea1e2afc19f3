// The page-level (Quest) baseline through the C ABI from C++ alone (no Python,
// no PyTorch).  With one-token pages a page's min/max box is the key itself and
// its bound is the key's score, so on small-integer inputs (every product and
// sum exact in fp32) asp_page_select must equal asp_score_keys followed by
// asp_select_topc bit for bit.  With pages of 16 the token lists must be whole
// pages in ascending order, each sequence's partial last page cut at its length.
// Built by __graft_entry__.build(); run by tests/test_gpu_c_abi.py.
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

struct Lcg {
  uint64_t s;
  int small_int() {  // uniform in {-3..3}
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (int)((s >> 33) % 7u) - 3;
  }
};

uint16_t int_to_bf16(int x) {  // small integers are exact in bf16
  float f = (float)x;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

}  // namespace

int main() {
  const asp_dims d = {3, 16, 4, 128, 3000, ASP_KV_BF16};
  const int B = d.batch, Hq = d.n_q_heads, Hkv = d.n_kv_heads, D = d.head_dim, T = d.t_cap;
  const int32_t lens_h[3] = {3000, 1777, 5};
  const size_t kv_n = (size_t)B * Hkv * T * D, q_n = (size_t)B * Hq * D;
  Lcg r{777};
  std::vector<uint16_t> kh(kv_n);
  for (auto& x : kh) x = int_to_bf16(r.small_int());
  std::vector<float> qh(q_n);
  for (auto& x : qh) x = (float)r.small_int();

  void* k;
  float* q;
  int32_t* lens;
  CHECK_HIP(hipMalloc(&k, kv_n * 2));
  CHECK_HIP(hipMalloc((void**)&q, q_n * 4));
  CHECK_HIP(hipMalloc((void**)&lens, sizeof lens_h));
  CHECK_HIP(hipMemcpy(k, kh.data(), kv_n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(q, qh.data(), q_n * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(lens, lens_h, sizeof lens_h, hipMemcpyHostToDevice));
  hipStream_t st;
  CHECK_HIP(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
  int failures = 0;

  for (const int P : {1, 16}) {
    const asp_cfg c = {8, P == 1 ? 300 : 320, 1e-2, 0};
    const int C = c.top_c;
    const size_t sum_bytes = asp_page_summary_size(&d, P);
    const size_t ws_bytes = asp_page_select_workspace_size(&d, &c, P);
    if (sum_bytes == 0 || ws_bytes == 0) return 4;
    void *kmin, *kmax, *ws;
    int32_t *idx, *nsel;
    CHECK_HIP(hipMalloc(&kmin, sum_bytes));
    CHECK_HIP(hipMalloc(&kmax, sum_bytes));
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_HIP(hipMalloc((void**)&idx, (size_t)B * Hkv * C * 4));
    CHECK_HIP(hipMalloc((void**)&nsel, (size_t)B * Hkv * 4));
    CHECK_ASP(asp_page_summary(&d, P, k, lens, kmin, kmax, st));
    CHECK_ASP(asp_page_select(&d, &c, P, q, kmin, kmax, lens, idx, nsel, ws, ws_bytes, st));
    std::vector<int32_t> i_pg((size_t)B * Hkv * C), n_pg((size_t)B * Hkv);
    CHECK_HIP(hipMemcpyAsync(i_pg.data(), idx, i_pg.size() * 4, hipMemcpyDeviceToHost, st));
    CHECK_HIP(hipMemcpyAsync(n_pg.data(), nsel, n_pg.size() * 4, hipMemcpyDeviceToHost, st));
    CHECK_HIP(hipStreamSynchronize(st));

    if (P == 1) {  // the token-level route on the same inputs
      float* scores;
      void* ws_sel;
      const size_t sel_bytes = asp_workspace_size(&d, &c, ASP_OP_SELECT);
      CHECK_HIP(hipMalloc((void**)&scores, (size_t)B * Hkv * T * 4));
      CHECK_HIP(hipMalloc(&ws_sel, sel_bytes));
      CHECK_ASP(asp_score_keys(&d, q, k, lens, scores, nullptr, st));
      CHECK_ASP(asp_select_topc(&d, &c, scores, nullptr, lens, idx, nsel, ws_sel, sel_bytes, st));
      std::vector<int32_t> i_tk(i_pg.size()), n_tk(n_pg.size());
      CHECK_HIP(hipMemcpyAsync(i_tk.data(), idx, i_tk.size() * 4, hipMemcpyDeviceToHost, st));
      CHECK_HIP(hipMemcpyAsync(n_tk.data(), nsel, n_tk.size() * 4, hipMemcpyDeviceToHost, st));
      CHECK_HIP(hipStreamSynchronize(st));
      const bool same = i_tk == i_pg && n_tk == n_pg;
      std::printf("one-token pages and the token selection %s\n", same ? "agree" : "DIFFER");
      failures += !same;
      CHECK_HIP(hipFree(scores));
      CHECK_HIP(hipFree(ws_sel));
    } else {  // whole pages, ascending, cut at the sequence length
      bool ok = true;
      for (int u = 0; u < B * Hkv && ok; ++u) {
        const int Tb = lens_h[u / Hkv], n = n_pg[u];
        const int pages = (Tb + P - 1) / P, keep = pages < C / P ? pages : C / P;
        const int32_t* row = i_pg.data() + (size_t)u * C;
        int expect_n = 0, j = 0;
        for (int pg = 0; pg < keep && ok; ++pg) {
          const int first = row[j];
          ok = first >= 0 && first % P == 0 && (j == 0 || first > row[j - 1]);
          const int cnt = first + P <= Tb ? P : Tb - first;
          for (int t = 0; t < cnt && ok; ++t) ok = row[j + t] == first + t;
          j += cnt;
          expect_n += cnt;
        }
        ok = ok && n == expect_n;
        for (int t = n; t < C && ok; ++t) ok = row[t] == -1;
        if (!ok) std::printf("  unit %d: malformed token list (n_sel %d)\n", u, n);
      }
      std::printf("page token lists %s\n", ok ? "well-formed" : "MALFORMED");
      failures += !ok;
    }
    CHECK_HIP(hipFree(kmin));
    CHECK_HIP(hipFree(kmax));
    CHECK_HIP(hipFree(ws));
    CHECK_HIP(hipFree(idx));
    CHECK_HIP(hipFree(nsel));
  }
  CHECK_HIP(hipStreamDestroy(st));
  if (failures) return 1;
  std::printf("c-abi page check: ok\n");
  return 0;
}
