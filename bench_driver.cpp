// Timing driver of bench.py: the decode loop over layers in rotation, issued
// from C++ through the C ABI (include/asp.h) with no Python between the
// steps.  bench.py allocates every buffer, stream and event, fills the layers'
// state, calls bench_rotation() through ctypes and reads back the times and
// each layer's buffer parity and step count.  Built by __graft_entry__.build()
// into bench_driver.so beside this file.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdint>

#include "asp.h"

// One wave that spins until `ticks` of the constant-rate wall clock have
// passed (a bounded loop), holding the stream it runs on.
__global__ void hold_kernel(long long ticks) {
  const long long t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) {
  }
}

extern "C" {

// Holds `stream` for about `us` microseconds (a single-wave kernel), so that
// the host can queue the timed steps behind it and the GPU, not the host,
// then sets their pace (used for kernel traces, whose tracer slows the host).
// Returns 0, or -1 for a HIP error.
int bench_hold(hipStream_t stream, double us) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      khz <= 0)
    return -1;
  const long long ticks = (long long)(us * 1e-3 * khz);
  if (ticks <= 0) return 0;
  hipLaunchKernelGGL(hold_kernel, dim3(1), dim3(64), 0, stream, ticks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One layer of the rotation: its queries (qs[t] is the actual query of its
// step t, [B][Hq][D] fp32), ring, KV cache, selection buffer pair and event
// pair, output and step workspace.  cur: the buffer holding the selection the
// next step attends over; t: the index of the next step's query.
typedef struct {
  const float* qs;
  float* q_hist;
  int32_t* newest;
  int32_t* len;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  int32_t* idx[2];
  int32_t* nsel[2];
  hipEvent_t ev[2];
  float* out;
  void* ws;
  size_t ws_bytes;
  int32_t cur;
  int32_t t;
} bench_layer;

// Runs `warmup` untimed steps, then `steps` timed steps, step i on layer
// i mod n_layers (pipelined; two streams when sel != NULL and != attn, with
// ctx).  The timed region is bracketed by events on attn, after the selection
// stream is joined into it, and by the host clock; times[0] = GPU ms between
// the events, times[1] = wall ms (first record to the end of the final
// synchronisation), times[2] = host ms spent issuing the timed steps.
// hold_us > 0: attn is first held that long (bench_hold), after the warm-up
// and before the first event; the wall time then includes the hold.
// Returns 0, or the first failing asp_status / -1 for a HIP error.
int bench_rotation(asp_context* ctx, const asp_dims* dims, const asp_cfg* cfg, bench_layer* layers, int n_layers,
                   int warmup, int steps, hipStream_t attn, hipStream_t sel, double hold_us, double* times) {
  using clk = std::chrono::steady_clock;
  const size_t q_n = (size_t)dims->batch * dims->n_q_heads * dims->head_dim;
  hipEvent_t e0, e1, joined;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess ||
      hipEventCreateWithFlags(&joined, hipEventDisableTiming) != hipSuccess)
    return -1;
  auto step = [&](int i) -> int {
    bench_layer& l = layers[i % n_layers];
    const int cur = l.cur, nxt = 1 - cur;
    const asp_status st =
        asp_step(ctx, dims, cfg, l.qs + (size_t)l.t * q_n, l.q_hist, l.newest, l.len, l.k, l.v, l.seq_lens,
                 l.idx[cur], l.nsel[cur], l.idx[nxt], l.nsel[nxt], l.out, l.ws, l.ws_bytes, attn, sel, l.ev[cur],
                 l.ev[nxt]);
    l.cur = nxt;
    l.t += 1;
    return (int)st;
  };
  int rc = 0;
  for (int i = 0; i < warmup && rc == 0; ++i) rc = step(i);
  if (rc == 0 && hipDeviceSynchronize() != hipSuccess) rc = -1;
  if (rc == 0) {
    if (hold_us > 0.0) rc = bench_hold(attn, hold_us);
    const auto w0 = clk::now();
    if (hipEventRecord(e0, attn) != hipSuccess) rc = -1;
    for (int i = warmup; i < warmup + steps && rc == 0; ++i) rc = step(i);
    const auto issued = clk::now();
    if (rc == 0 && sel != nullptr && sel != attn &&
        (hipEventRecord(joined, sel) != hipSuccess || hipStreamWaitEvent(attn, joined, 0) != hipSuccess))
      rc = -1;
    if (rc == 0 && (hipEventRecord(e1, attn) != hipSuccess || hipDeviceSynchronize() != hipSuccess)) rc = -1;
    const auto w1 = clk::now();
    float ms = 0.0f;
    if (rc == 0 && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) rc = -1;
    times[0] = ms;
    times[1] = std::chrono::duration<double, std::milli>(w1 - w0).count();
    times[2] = std::chrono::duration<double, std::milli>(issued - w0).count();
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipEventDestroy(joined);
  return rc;
}

}  // extern "C"
