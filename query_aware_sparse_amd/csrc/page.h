// Internal declarations of the page-level (Quest) selection, shared by page.hip
// and the C ABI in api.hip.  Not part of the public interface.
#pragma once

#include "asp_internal.h"

namespace asp {

// Pages are runs of P tokens from token 0, NP = page_count(T_cap, P) rows per
// unit.  Summaries kmin/kmax are [units][NP][D] in the KV dtype; scores
// [units][NP] f32; counts (nullable) receives each sequence's page count.  The
// selection keeps s.C / P pages and writes their tokens (ascending) to idx, -1
// after them.
int page_count(int T_cap, int P);
hipError_t launch_page_summary(const Shape& s, int P, const void* k, const int32_t* seq_lens, void* kmin, void* kmax,
                               hipStream_t st);
hipError_t launch_page_scores(const Shape& s, int P, const float* q, const void* kmin, const void* kmax,
                              const int32_t* seq_lens, float* scores, int32_t* counts, hipStream_t st);
size_t page_select_ws_bytes(const Shape& s, int P);
hipError_t launch_page_select(const Shape& s, int P, const float* q, const void* kmin, const void* kmax,
                              const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws, hipStream_t st);

}  // namespace asp
