// C ABI of libkvsel: argument checks, workspace sizing, dispatch.
// Every check runs before the first HIP call, so a rejected call touches
// neither the device nor the outputs (and works on a host without a GPU).
#include <cmath>
#include <cstdint>

#include "kvsel.h"
#include "kvsel_kernels.h"

namespace kvsel {
hipError_t score_launch(const ScorePlan& p, const void* q, const void* k, float* scores,
                        float* raw, void* ws, size_t ws_bytes, hipStream_t st);
hipError_t score_chunked_launch(const ScorePlan& p, const void* q, const void* k,
                                const void* k_self, float* scores, float* raw, void* ws,
                                hipStream_t st);
size_t score_ws_bytes(const ScorePlan& p);
bool select_groups_ok(int groups);
}  // namespace kvsel

using namespace kvsel;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

}  // namespace

namespace kvsel {

// Argument checks and plan of kvsel_select (shared with the entry point
// that takes its scratch from a static device array).
int32_t select_plan(bool two_stage, int32_t L, int32_t H_kv, int32_t n, int32_t W, int64_t budget,
                    int32_t adaptive, float score_norm, float eps, float alpha, SelectPlan* out) {
  if (L < 1 || H_kv < 1 || n < 1 || W < 0 || W >= n) return KVSEL_ERR_ARG;
  if (adaptive != 0 && adaptive != 1) return KVSEL_ERR_ARG;
  const int64_t n_cand = (int64_t)n - W;
  const int64_t groups = adaptive ? H_kv : 1;
  if (budget < groups * W || budget > groups * (int64_t)n) return KVSEL_ERR_ARG;
  if (two_stage) {
    if (!(alpha >= 0.f && alpha <= 1.f)) return KVSEL_ERR_ARG;
    if (!(score_norm > 0.f) || !std::isfinite(score_norm)) return KVSEL_ERR_ARG;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return KVSEL_ERR_ARG;
  }
  if (groups * n_cand > kMaxIndex || budget > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  if (adaptive && !select_groups_ok(H_kv)) return KVSEL_ERR_UNSUPPORTED;
  SelectPlan& p = *out;
  p.L = L; p.H = H_kv; p.n = n; p.W = W; p.n_cand = (int)n_cand;
  p.budget = budget;
  p.adaptive = adaptive != 0;
  p.two_stage = two_stage;
  p.score_norm = score_norm;
  p.eps = eps;
  p.k = budget - groups * W;
  p.k1 = p.two_stage ? (int64_t)std::floor((double)alpha * (double)p.k) : 0;
  p.segments = adaptive ? L : L * H_kv;
  p.seg_len = groups * n_cand;
  p.resident = false;
  return KVSEL_OK;
}

int32_t select_pointers_ok(const SelectPlan& p, const float* scores, const float* weight,
                           const int32_t* idx, const int32_t* head_offsets) {
  if (!scores || (p.budget > 0 && !idx) || (p.adaptive && !head_offsets)) return KVSEL_ERR_ARG;
  if (!aligned16(scores) || (weight && !aligned16(weight))) return KVSEL_ERR_ARG;
  return KVSEL_OK;
}

}  // namespace kvsel

extern "C" {

int32_t kvsel_abi_version(void) { return 2; }

const char* kvsel_status_str(int32_t status) {
  switch (status) {
    case KVSEL_OK: return "KVSEL_OK";
    case KVSEL_ERR_ARG: return "KVSEL_ERR_ARG: invalid argument";
    case KVSEL_ERR_UNSUPPORTED: return "KVSEL_ERR_UNSUPPORTED: request outside what this build covers";
    case KVSEL_ERR_WORKSPACE: return "KVSEL_ERR_WORKSPACE: workspace too small";
    case KVSEL_ERR_HIP: return "KVSEL_ERR_HIP: HIP launch failed";
    case KVSEL_ERR_SCRATCH: return "KVSEL_ERR_SCRATCH: request needs more than the static scratch";
    default: return "KVSEL: unknown status";
  }
}

int32_t kvsel_score(const void* q, const void* k, int32_t L, int32_t H_kv, int32_t G,
                    int32_t d, int32_t n, int32_t W, int32_t q_mode, int32_t agg, float scale,
                    int32_t pool, float* scores, float* raw, void* ws, size_t* ws_bytes,
                    void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || G < 1 || d < 1 || n < 1 || W < 1) return KVSEL_ERR_ARG;
  if (q_mode != KVSEL_Q_WINDOW && q_mode != KVSEL_Q_EXTERNAL) return KVSEL_ERR_ARG;
  if (agg != KVSEL_AGG_SUM && agg != KVSEL_AGG_MAX && agg != KVSEL_AGG_LOGIT_MAX)
    return KVSEL_ERR_ARG;
  if (agg == KVSEL_AGG_LOGIT_MAX && q_mode != KVSEL_Q_EXTERNAL) return KVSEL_ERR_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return KVSEL_ERR_ARG;
  if (pool < 1 || pool % 2 == 0) return KVSEL_ERR_ARG;
  if (q_mode == KVSEL_Q_WINDOW && W >= n) return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic) return KVSEL_ERR_UNSUPPORTED;
  if (pool > 65) return KVSEL_ERR_UNSUPPORTED;
  if ((int64_t)G * W > kMaxIndex || (int64_t)H_kv * n > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  // the kernels address one head's K, and one head's query rows, through
  // buffer resources with 31-bit byte offsets
  if ((int64_t)n * kRowBytesPublic > kMaxIndex || (int64_t)G * W * kRowBytesPublic > kMaxIndex)
    return KVSEL_ERR_UNSUPPORTED;
  ScorePlan p;
  p.L = L; p.H = H_kv; p.G = G; p.n = n; p.W = W;
  p.R = G * W;
  p.causal = q_mode == KVSEL_Q_WINDOW;
  p.n_cand = p.causal ? n - W : n;
  p.pool = pool;
  p.max_agg = agg != KVSEL_AGG_SUM;
  p.logit = agg == KVSEL_AGG_LOGIT_MAX;
  p.need_raw_tmp = raw == nullptr;
  p.scale = scale;
  const size_t need = score_ws_bytes(p);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  // scores == NULL: raw only (no pooling), for kvsel_select_pool
  if (!q || !k || (!scores && !raw)) return KVSEL_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || (scores && !aligned16(scores)) || !aligned16(ws) ||
      (raw && !aligned16(raw)))
    return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  const hipError_t e = score_launch(p, q, k, scores, raw, ws, *ws_bytes,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_score_chunked(const void* q, const void* k, const void* k_self, int32_t L,
                            int32_t H_kv, int32_t G, int32_t d, int32_t n, int32_t m,
                            int32_t n_prompt, float scale, int32_t pool, float* scores, float* raw,
                            void* ws, size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || G < 1 || d < 1 || n < 1 || m < 1 || n_prompt < 0) return KVSEL_ERR_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return KVSEL_ERR_ARG;
  if (pool < 1 || pool % 2 == 0) return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic || pool > 65) return KVSEL_ERR_UNSUPPORTED;
  const int64_t m_eff = m < n ? m : n;          // one chunk holds at most the whole cache
  const int64_t n_in = (int64_t)n_prompt + m_eff;
  const int64_t T = ((int64_t)n + m_eff - 1) / m_eff;
  const int64_t R = (int64_t)G * n_in;
  if (R > kMaxIndex || (int64_t)H_kv * n > kMaxIndex || L * T * H_kv > kMaxIndex)
    return KVSEL_ERR_UNSUPPORTED;
  // one head's keys, query rows and own keys each span < 2^31 bytes
  if ((int64_t)n * kRowBytesPublic > kMaxIndex || R * kRowBytesPublic > kMaxIndex)
    return KVSEL_ERR_UNSUPPORTED;
  ScorePlan p;
  p.L = L; p.H = H_kv; p.G = G; p.n = n; p.W = (int)n_in;
  p.R = (int)R;
  p.causal = false;
  p.n_cand = n;
  p.pool = pool;
  p.max_agg = true;
  p.need_raw_tmp = raw == nullptr;
  p.scale = scale;
  p.chunk_m = (int)m_eff;
  p.n_prompt = n_prompt;
  const size_t need = score_ws_bytes(p);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!q || !k || !k_self || !scores) return KVSEL_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(k_self) || !aligned16(scores) ||
      !aligned16(ws) || (raw && !aligned16(raw)))
    return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  const hipError_t e = score_chunked_launch(p, q, k, k_self, scores, raw, ws,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_value_weight(const void* v, const void* w_o, int32_t L, int32_t H_kv, int32_t G,
                           int32_t d, int32_t n, int32_t D, int32_t n_cand, int32_t group_mode,
                           float* weight, void* ws, size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || G < 1 || d < 1 || n < 1 || D < 1) return KVSEL_ERR_ARG;
  if (n_cand < 1 || n_cand > n) return KVSEL_ERR_ARG;
  if (group_mode != KVSEL_GROUP_MEAN_OF_NORMS && group_mode != KVSEL_GROUP_NORM_OF_SUM)
    return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic || D % 32 != 0) return KVSEL_ERR_UNSUPPORTED;
  if ((int64_t)H_kv * G * d > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  // w_o is read through buffer resources with 31-bit byte offsets
  if ((int64_t)D * H_kv * G * d * 2 > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  const size_t need = value_weight_ws_bytes(L, H_kv, D, group_mode);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!v || !w_o || !weight) return KVSEL_ERR_ARG;
  if (!aligned16(v) || !aligned16(w_o) || !aligned16(weight) || !aligned16(ws))
    return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  const hipError_t e = value_weight_launch(v, w_o, L, H_kv, G, n, D, n_cand, group_mode, weight,
                                           ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_value_l2_factor(const void* w_o, int32_t L, int32_t H_kv, int32_t G, int32_t d,
                              int32_t D, void* factor, void* stream) {
  if (!w_o || !factor) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || G < 1 || d < 1 || D < 1) return KVSEL_ERR_ARG;
  if (!aligned16(w_o) || !aligned16(factor)) return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic) return KVSEL_ERR_UNSUPPORTED;
  if ((int64_t)H_kv * G * d > kMaxIndex || (int64_t)L * H_kv * G > kMaxIndex)
    return KVSEL_ERR_UNSUPPORTED;
  const hipError_t e = value_l2_factor_launch(w_o, L, H_kv, G, D, factor,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_value_weight_l2(const void* v, const void* factor, int32_t L, int32_t H_kv,
                              int32_t G, int32_t d, int32_t n, int32_t n_cand, float* weight,
                              void* stream) {
  if (!v || !factor || !weight) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || G < 1 || d < 1 || n < 1) return KVSEL_ERR_ARG;
  if (n_cand < 1 || n_cand > n) return KVSEL_ERR_ARG;
  if (!aligned16(v) || !aligned16(factor) || !aligned16(weight)) return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic) return KVSEL_ERR_UNSUPPORTED;
  if ((int64_t)L * H_kv * G > kMaxIndex || (int64_t)H_kv * n > kMaxIndex)
    return KVSEL_ERR_UNSUPPORTED;
  const hipError_t e = value_weight_l2_launch(v, factor, L, H_kv, G, n, n_cand, weight,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_select(const float* scores, const float* weight, int32_t L, int32_t H_kv,
                     int32_t n, int32_t W, int64_t budget, int32_t adaptive, float score_norm,
                     float eps, float alpha, int32_t* idx, int32_t* head_offsets,
                     uint8_t* stage, void* ws, size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  SelectPlan p;
  const int32_t rc = select_plan(weight != nullptr, L, H_kv, n, W, budget, adaptive, score_norm,
                                 eps, alpha, &p);
  if (rc != KVSEL_OK) return rc;
  const size_t need = select_ws_bytes(p);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  const int32_t rp = select_pointers_ok(p, scores, weight, idx, head_offsets);
  if (rp != KVSEL_OK) return rp;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return KVSEL_ERR_ARG;
  const hipError_t e = select_launch(p, scores, weight, idx, head_offsets, stage, ws,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_select_pool(const float* raw, const float* weight, int32_t pool, int32_t L,
                          int32_t H_kv, int32_t n, int32_t W, int64_t budget, int32_t adaptive,
                          float score_norm, float eps, float alpha, int32_t* idx,
                          int32_t* head_offsets, uint8_t* stage, float* pooled, void* ws,
                          size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (pool < 1 || pool % 2 == 0) return KVSEL_ERR_ARG;
  SelectPlan p;
  const int32_t rc = select_plan(weight != nullptr, L, H_kv, n, W, budget, adaptive, score_norm,
                                 eps, alpha, &p);
  if (rc != KVSEL_OK) return rc;
  if (pool > 65) return KVSEL_ERR_UNSUPPORTED;
  // one head's raw row on chip when it fits; else the pooled scores go
  // through memory (`pooled`, or the workspace): written by the many-
  // workgroup selection's first pass (radius <= 3), or by the pool kernel
  // before the selection
  const int r = pool / 2;
  const bool on_chip = select_pools_on_chip(p, r);
  const size_t pooled_ws = on_chip || pooled ? 0 : al256((size_t)L * H_kv * p.n_cand * sizeof(float));
  const size_t need = pooled_ws + select_ws_bytes(p);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  const int32_t rp = select_pointers_ok(p, raw, weight, idx, head_offsets);
  if (rp != KVSEL_OK) return rp;
  if (pooled && !aligned16(pooled)) return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return KVSEL_ERR_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (on_chip) {
    p.pool_r = r;
    p.in_stride = n;
    p.pooled = pooled;
    e = select_launch(p, raw, weight, idx, head_offsets, stage, ws, st);
  } else {
    float* ps = pooled ? pooled : static_cast<float*>(ws);
    void* sws = static_cast<char*>(ws) + pooled_ws;
    if (select_pools_in_passes(p, r)) {   // pooled in the selection's first pass
      p.pool_r = r;
      p.in_stride = n;
      p.pooled = ps;
      e = select_launch(p, raw, weight, idx, head_offsets, stage, sws, st);
    } else {
      e = pool_launch(raw, L, H_kv, n, p.n_cand, r, ps, st);
      if (e == hipSuccess) e = select_launch(p, ps, weight, idx, head_offsets, stage, sws, st);
    }
  }
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_select_budgets(const float* scores, const float* weight, int32_t L, int32_t H_kv,
                             int32_t n, int32_t W, const int32_t* budgets, int64_t layer_stride,
                             float score_norm, float eps, float alpha, int32_t* idx,
                             int32_t* head_offsets, uint8_t* stage, void* ws, size_t* ws_bytes,
                             void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || n < 1 || W < 0 || W >= n) return KVSEL_ERR_ARG;
  if (layer_stride < 1 || layer_stride > (int64_t)H_kv * n) return KVSEL_ERR_ARG;
  if (weight) {
    if (!(alpha >= 0.f && alpha <= 1.f)) return KVSEL_ERR_ARG;
    if (!(score_norm > 0.f) || !std::isfinite(score_norm)) return KVSEL_ERR_ARG;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return KVSEL_ERR_ARG;
  }
  const int64_t n_cand = (int64_t)n - W;
  if ((int64_t)H_kv * n > kMaxIndex || layer_stride > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  SelectPlan p;
  p.L = L; p.H = H_kv; p.n = n; p.W = W; p.n_cand = (int)n_cand;
  p.budget = 0;           // per segment, from the budget vector
  p.adaptive = false;
  p.two_stage = weight != nullptr;
  p.score_norm = score_norm;
  p.eps = eps;
  p.k = 0;
  p.k1 = 0;
  p.segments = L * H_kv;
  p.seg_len = n_cand;
  p.resident = false;
  p.budgets = budgets;
  p.stride = layer_stride;
  p.alpha = alpha;
  const size_t need = select_ws_bytes(p);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!scores || !budgets || !idx || !head_offsets) return KVSEL_ERR_ARG;
  if (!aligned16(scores) || (weight && !aligned16(weight))) return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return KVSEL_ERR_ARG;
  const hipError_t e = select_launch(p, scores, weight, idx, head_offsets, stage, ws,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_head_score(const float* scores, int32_t L, int32_t H_kv, int32_t n_pos,
                         float* head_score, void* stream) {
  if (!scores || !head_score) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || n_pos < 1) return KVSEL_ERR_ARG;
  if ((int64_t)L * H_kv > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  const hipError_t e = head_score_launch(scores, L, H_kv, n_pos, head_score,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_head_budgets(const float* head_score, int32_t L, int32_t H_kv, int32_t keep,
                           int32_t n, int32_t W, int32_t* budgets, void* ws, size_t* ws_bytes,
                           void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || n < 1 || W < 0 || W > n) return KVSEL_ERR_ARG;
  const int64_t count = (int64_t)L * H_kv;
  if (count > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  if (keep < 0 || keep > count) return KVSEL_ERR_ARG;
  const size_t need = head_budgets_ws_bytes((int)count, keep);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!head_score || !budgets) return KVSEL_ERR_ARG;
  if (!aligned16(head_score) || !aligned16(ws)) return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  const hipError_t e = head_budgets_launch(head_score, (int)count, keep, n, W, budgets, ws,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_anchor_select(const float* scores, const float* rand, int32_t L, int32_t H_kv,
                            int32_t n, int32_t W, int32_t k, float rho, int32_t* anchors,
                            void* ws, size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || n < 1 || W < 0 || W >= n || k < W || k > n) return KVSEL_ERR_ARG;
  if (!(rho >= 0.f && rho <= 1.f)) return KVSEL_ERR_ARG;
  const int64_t n_cand = (int64_t)n - W;
  if (n_cand > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  // the two-stage selection with stage 2 keyed (score * 0 + 1) * draw
  SelectPlan p;
  p.L = L; p.H = H_kv; p.n = n; p.W = W; p.n_cand = (int)n_cand;
  p.budget = k;
  p.adaptive = false;
  p.two_stage = true;
  p.score_norm = 0.f;
  p.eps = 1.f;
  p.k = k - W;
  p.k1 = (int64_t)std::floor((double)rho * (double)p.k);
  p.segments = L * H_kv;
  p.seg_len = n_cand;
  p.resident = false;
  const size_t need = select_ws_bytes(p);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!scores || !rand || !anchors) return KVSEL_ERR_ARG;
  if (!aligned16(scores) || !aligned16(rand)) return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return KVSEL_ERR_ARG;
  const hipError_t e = select_launch(p, scores, rand, anchors, nullptr, nullptr, ws,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_anchor_assign(const void* x, const int32_t* anchors, int32_t L, int32_t H_kv,
                            int32_t d, int32_t n, int32_t k, int32_t* slot, float* gamma,
                            void* ws, size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || d < 1 || n < 1 || k < 1 || k > n) return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic || k > kMaxAnchorsPublic) return KVSEL_ERR_UNSUPPORTED;
  if ((int64_t)L * H_kv > 65535 || (int64_t)H_kv * n > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  const size_t need = anchor_ws_bytes(L, H_kv, k);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!x || !anchors || !slot || !gamma) return KVSEL_ERR_ARG;
  if (!aligned16(x) || !aligned16(ws)) return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  const hipError_t e = anchor_assign_launch(x, anchors, L, H_kv, n, k, slot, gamma, ws,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_compact(const void* k, const void* v, int32_t L, int32_t H_kv, int32_t d,
                      int32_t n, const int32_t* idx, const int32_t* head_offsets,
                      int64_t kept_per_layer, void* k_out, void* v_out, void* stream) {
  if (!k || !v || !idx || !k_out || !v_out) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || d < 1 || n < 1 || kept_per_layer < 1) return KVSEL_ERR_ARG;
  if (d % 8 != 0) return KVSEL_ERR_UNSUPPORTED;
  if (!head_offsets && kept_per_layer % H_kv != 0) return KVSEL_ERR_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return KVSEL_ERR_ARG;
  if (kept_per_layer > (int64_t)H_kv * n) return KVSEL_ERR_ARG;
  const hipError_t e = compact_launch(k, v, L, H_kv, d, n, idx, head_offsets, kept_per_layer,
                                      k_out, v_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

int32_t kvsel_decode_attention(const void* q, const void* k, const void* v, int32_t L,
                               int32_t H_kv, int32_t G, int32_t d, int64_t kept_per_layer,
                               const int32_t* head_offsets, float scale, float* out, void* ws,
                               size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVSEL_ERR_ARG;
  if (L < 1 || H_kv < 1 || G < 1 || d < 1 || kept_per_layer < 1) return KVSEL_ERR_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return KVSEL_ERR_ARG;
  if (!head_offsets && kept_per_layer % H_kv != 0) return KVSEL_ERR_ARG;
  if (d != kHeadDimPublic || G > 8 || H_kv > 1024) return KVSEL_ERR_UNSUPPORTED;
  if (kept_per_layer > kMaxIndex || (int64_t)L * H_kv * G > kMaxIndex) return KVSEL_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(L, H_kv, G, kept_per_layer, head_offsets != nullptr);
  if (!ws) {
    *ws_bytes = need;
    return KVSEL_OK;
  }
  if (!q || !k || !v || !out) return KVSEL_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws))
    return KVSEL_ERR_ARG;
  if (*ws_bytes < need) return KVSEL_ERR_WORKSPACE;
  const hipError_t e = decode_launch(q, k, v, L, H_kv, G, kept_per_layer, head_offsets, scale, out,
                                     ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

}  // extern "C"
