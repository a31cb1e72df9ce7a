// kvsel_score dispatch: workspace sizing and the choice of score kernels.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

size_t score_ws_bytes(const ScorePlan& p) {
  TwoPassLayout o;
  twopass_plan(p, &o);
  return o.bytes;
}

hipError_t score_launch(const ScorePlan& p, const void* q, const void* k, float* scores,
                        float* raw, void* ws, size_t, hipStream_t st) {
  TwoPassLayout o;
  twopass_plan(p, &o);
  return twopass_launch(p, o, q, k, scores, raw, ws, st);
}

}  // namespace kvsel
