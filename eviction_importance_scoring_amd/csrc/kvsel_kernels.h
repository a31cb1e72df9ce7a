// Host-side interfaces between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvsel {

constexpr int kHeadDimPublic = 128;   // the head dimension the library accepts
constexpr int kRowBytesPublic = kHeadDimPublic * 2;   // one bf16 row

// ------------------------------------------------------------- scoring ----
struct ScorePlan {
  int L, H, G, n, W;      // W = queries per query head
  int R;                  // rows per KV head = G*W
  int n_cand;             // n-W (window) or n (external)
  int pool;
  bool causal;            // window mode
  bool max_agg;
  bool logit = false;     // max of the scaled logits, no softmax (external only)
  int chunk_m = 0;        // chunked scoring: cached keys per chunk (0: not chunked)
  int n_prompt = 0;       // chunked scoring: prompt tokens before each chunk
  bool need_raw_tmp;      // caller passed raw == NULL
  float scale;
};

struct TwoPassLayout {
  int row_blocks, splits, keys_per_split;
  int sp_stride;          // statistics slots per row (splits, or 2 when chunked)
  int Lv;                 // grid layers: L, or L * chunks
  size_t part_off, stat_off, raw_off, bytes;
};

void twopass_plan(const ScorePlan& p, TwoPassLayout* o);
hipError_t twopass_launch(const ScorePlan& p, const TwoPassLayout& o, const void* q,
                          const void* k, const void* k_self, float* scores, float* raw,
                          void* ws, hipStream_t st);

struct WindowLayout {
  int kpb, blocks;          // keys per workgroup, workgroups per head
  size_t part_off, stat_off, raw_off, bytes;
};

bool window_applicable(const ScorePlan& p);
void window_plan(const ScorePlan& p, WindowLayout* o);
hipError_t window_launch(const ScorePlan& p, const WindowLayout& o, const void* q, const void* k,
                         float* scores, float* raw, void* ws, hipStream_t st);

// ------------------------------------------------------------ selection ----
struct SelectPlan {
  int L, H, n, W, n_cand;
  int64_t budget;
  bool adaptive, two_stage;
  float score_norm, eps;
  int64_t k, k1;          // candidates kept (all stages), stage-1 share
  int segments;           // L*H (uniform) or L (adaptive)
  int64_t seg_len;        // n_cand or H*n_cand
  bool resident;          // segment fits in LDS
  const int32_t* budgets = nullptr;   // per-head budgets [L][H] (device), or null
  int64_t stride = 0;     // layer row of idx when budgets are given
  float alpha = 0.f;
  // Max-pooling in the selection: the scores are raw rows `in_stride`
  // floats apart, pooled with radius pool_r over each head's candidates.
  // On chip (resident segments of one head) the pooled scores go to
  // `pooled` if given; on the many-workgroup path they go to `pooled`.
  int pool_r = 0;
  int64_t in_stride = 0;  // 0: seg_len
  float* pooled = nullptr;
};

// Whether select_launch pools on chip for this plan (raw rows in, the
// pooled scores out only if asked).
bool select_pools_on_chip(const SelectPlan& p, int pool_r);
// Whether select_launch pools in the first pass of its many-workgroup path
// (raw rows in; the pooled scores go to SelectPlan::pooled, which is
// required). Otherwise the caller pools.
bool select_pools_in_passes(const SelectPlan& p, int pool_r);

// scores[lh][j] = max raw[lh][t] over |t - j| <= r, 0 <= t < n_cand (raw
// rows n apart); scores == nullptr: nothing.
hipError_t pool_launch(const float* raw, int L, int H, int n, int n_cand, int r, float* scores,
                       hipStream_t st);

size_t select_ws_bytes(const SelectPlan& p);
int32_t select_plan(bool two_stage, int32_t L, int32_t H_kv, int32_t n, int32_t W, int64_t budget,
                    int32_t adaptive, float score_norm, float eps, float alpha, SelectPlan* out);
int32_t select_pointers_ok(const SelectPlan& p, const float* scores, const float* weight,
                           const int32_t* idx, const int32_t* head_offsets);
hipError_t select_launch(const SelectPlan& p, const float* scores, const float* weight,
                         int32_t* idx, int32_t* head_offsets, uint8_t* stage, void* ws,
                         hipStream_t st);

// ----------------------------------------------------------- compaction ----
hipError_t compact_launch(const void* k, const void* v, int L, int H, int d, int n,
                          const int32_t* idx, const int32_t* head_offsets,
                          int64_t kept, void* k_out, void* v_out, hipStream_t st);

// --------------------------------------------------------- value weight ----
size_t value_weight_ws_bytes(int L, int H, int D, int group_mode);
hipError_t value_weight_launch(const void* v, const void* w_o, int L, int H, int G, int n,
                               int D, int n_cand, int group_mode, float* weight, void* ws,
                               hipStream_t st);
hipError_t value_l2_factor_launch(const void* w_o, int L, int H, int G, int D, void* factor,
                                  hipStream_t st);
hipError_t value_weight_l2_launch(const void* v, const void* factor, int L, int H, int G, int n,
                                  int n_cand, float* weight, hipStream_t st);

// ---------------------------------------------------------------- anchors ----
constexpr int kMaxAnchorsPublic = 2048;
size_t anchor_ws_bytes(int L, int H, int k);
hipError_t anchor_assign_launch(const void* x, const int32_t* anchors, int L, int H, int n, int k,
                                int32_t* slot, float* gamma, void* ws, hipStream_t st);

// ------------------------------------------------------------ head level ----
hipError_t head_score_launch(const float* scores, int L, int H, int n_pos, float* out,
                             hipStream_t st);
size_t head_budgets_ws_bytes(int count, int keep);
hipError_t head_budgets_launch(const float* head_score, int count, int keep, int n, int W,
                               int32_t* budgets, void* ws, hipStream_t st);

// -------------------------------------------------------------- decoding ----
size_t decode_ws_bytes(int L, int H, int G, int64_t kept, bool ragged);
hipError_t decode_launch(const void* q, const void* k, const void* v, int L, int H, int G,
                         int64_t kept, const int32_t* head_offsets, float scale, float* out,
                         void* ws, hipStream_t st);

}  // namespace kvsel
