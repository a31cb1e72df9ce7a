// Head-level importance and head-level eviction ([KVzip] §3.4, §3.6).
//
// k_head_score: the score of a head is the largest of its per-position
// scores, S_head = max_i S[l][h][i]. One workgroup per (layer, head) reads
// the head's row once (16-byte loads when the row allows them) and reduces
// in registers, then across the wave and the block.
//
// Head budgets: the `keep` heads with the largest head score over all
// layers and heads keep every entry (budget n) and the others a recent
// window (budget W), DuoAttention's structure that KVzip's context-
// independent eviction adopts. The top `keep` heads are found with the
// library's own selection (one segment of L*H candidates, equal scores to
// the lower flat index), then a fill and a scatter write the budgets, the
// input of kvsel_select_budgets.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kHeadThreads = 256;

__device__ __forceinline__ float hmax_wave(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// grid L*H, block 256
__global__ __launch_bounds__(kHeadThreads) void k_head_score(const float* __restrict__ scores,
                                                             int n_pos, int vec4,
                                                             float* __restrict__ out) {
  __shared__ float wm[kHeadThreads / 64];
  const size_t lh = blockIdx.x;
  const float* row = scores + lh * (size_t)n_pos;
  const int tid = threadIdx.x;
  float m = neg_inf();
  if (vec4) {   // n_pos % 4 == 0 and the rows 16-byte aligned
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
    const int n4 = n_pos >> 2;
    for (int i = tid; i < n4; i += kHeadThreads) {
      const f32x4 v = __builtin_nontemporal_load(r4 + i);
      m = fmaxf(m, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    }
  } else {
    for (int i = tid; i < n_pos; i += kHeadThreads) m = fmaxf(m, row[i]);
  }
  m = hmax_wave(m);
  if ((tid & 63) == 0) wm[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float b = wm[0];
#pragma unroll
    for (int w = 1; w < kHeadThreads / 64; ++w) b = fmaxf(b, wm[w]);
    out[lh] = b;
  }
}

// every budget to W
__global__ __launch_bounds__(kHeadThreads) void k_budget_fill(int count, int W,
                                                              int32_t* __restrict__ budgets) {
  const int i = blockIdx.x * kHeadThreads + threadIdx.x;
  if (i < count) budgets[i] = W;
}

// the kept heads (their flat indices from the selection) to n
__global__ __launch_bounds__(kHeadThreads) void k_budget_keep(const int32_t* __restrict__ idx,
                                                              int keep, int count, int n,
                                                              int32_t* __restrict__ budgets) {
  const int j = blockIdx.x * kHeadThreads + threadIdx.x;
  if (j < keep) {
    const int32_t h = idx[j];
    if (h >= 0 && h < count) budgets[h] = n;
  }
}

hipError_t head_score_launch(const float* scores, int L, int H, int n_pos, float* out,
                             hipStream_t st) {
  const long long blocks = (long long)L * H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int vec4 = (n_pos % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0) ? 1 : 0;
  hipLaunchKernelGGL(k_head_score, dim3((unsigned)blocks), dim3(kHeadThreads), 0, st, scores,
                     n_pos, vec4, out);
  return hipGetLastError();
}

static size_t al256h(size_t x) { return (x + 255) & ~size_t(255); }

// the selection over the flat head scores: one segment of L*H candidates,
// no window, k = keep
static SelectPlan head_plan(int count, int keep) {
  SelectPlan p;
  p.L = 1; p.H = 1; p.n = count; p.W = 0; p.n_cand = count;
  p.budget = keep;
  p.adaptive = false;
  p.two_stage = false;
  p.score_norm = 1.f;
  p.eps = 0.f;
  p.k = keep;
  p.k1 = 0;
  p.segments = 1;
  p.seg_len = count;
  p.resident = false;
  return p;
}

size_t head_budgets_ws_bytes(int count, int keep) {
  return al256h((size_t)(keep > 0 ? keep : 1) * sizeof(int32_t)) +
         select_ws_bytes(head_plan(count, keep));
}

hipError_t head_budgets_launch(const float* head_score, int count, int keep, int n, int W,
                               int32_t* budgets, void* ws, hipStream_t st) {
  int32_t* idx = static_cast<int32_t*>(ws);
  void* sel_ws = static_cast<char*>(ws) + al256h((size_t)(keep > 0 ? keep : 1) * sizeof(int32_t));
  const unsigned g = (unsigned)((count + kHeadThreads - 1) / kHeadThreads);
  hipLaunchKernelGGL(k_budget_fill, dim3(g), dim3(kHeadThreads), 0, st, count, W, budgets);
  if (keep > 0) {
    const hipError_t e = select_launch(head_plan(count, keep), head_score, nullptr, idx, nullptr,
                                       nullptr, sel_ws, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_budget_keep, dim3((unsigned)((keep + kHeadThreads - 1) / kHeadThreads)),
                       dim3(kHeadThreads), 0, st, idx, keep, count, n, budgets);
  }
  return hipGetLastError();
}

}  // namespace kvsel
