// kvsel_score dispatch: workspace sizing and the choice of score kernels.
//
// Window mode with R = G*W <= 128 query rows per KV head uses the streaming
// window kernels (score_window.hip); external queries and larger R use the
// general two-pass kernels (score_twopass.hip). The choice depends on the
// shapes alone, so the workspace is sized for the chosen kernels and a size
// query needs no device.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

size_t score_ws_bytes(const ScorePlan& p) {
  if (window_applicable(p)) {
    WindowLayout w;
    window_plan(p, &w);
    return w.bytes;
  }
  TwoPassLayout t;
  twopass_plan(p, &t);
  return t.bytes;
}

hipError_t score_launch(const ScorePlan& p, const void* q, const void* k, float* scores,
                        float* raw, void* ws, size_t, hipStream_t st) {
  if (p.chunk_m > 0) return hipErrorInvalidValue;   // chunked: score_chunked_launch
  if (window_applicable(p)) {
    WindowLayout w;
    window_plan(p, &w);
    return window_launch(p, w, q, k, scores, raw, ws, st);
  }
  TwoPassLayout t;
  twopass_plan(p, &t);
  return twopass_launch(p, t, q, k, nullptr, scores, raw, ws, st);
}

// KVzip's chunked scoring always runs on the general kernels.
hipError_t score_chunked_launch(const ScorePlan& p, const void* q, const void* k,
                                const void* k_self, float* scores, float* raw, void* ws,
                                hipStream_t st) {
  TwoPassLayout t;
  twopass_plan(p, &t);
  return twopass_launch(p, t, q, k, k_self, scores, raw, ws, st);
}

}  // namespace kvsel
