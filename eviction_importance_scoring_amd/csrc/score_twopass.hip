// Two-pass attention scoring: exact softmax weights aggregated per key.
//
// [CriticalKV] §3.3 Algorithm 2 steps 2-4 (window scores, then max-pool) and
// [KVzip] §3.2 (max over the group queries of the softmax weight). The row
// softmax runs over keys while the aggregate runs over queries ([KVzip] §3.4
// names this cross-dimension dependence), so the exact weight needs each
// row's normaliser over all keys before any column can be summed:
//   pass 1  per query row r: m_r = max_j x_rj, l_r = sum_j 2^(x_rj - m_r),
//           with x = log2(e) * scale * <q_r, k_j>; split over key ranges.
//   combine c_r = m_r + log2(l_r) over the key ranges (fixed order).
//   pass 2  per key j: sum_r 2^(x_rj - c_r)  or  2^(max_r (x_rj - c_r)).
//   pool    max over +-pool/2 neighbours inside the candidate range.
// Both passes run the Q K^T products on MFMA (32x32x16 bf16, fp32 accum).
// Pass 1 puts queries on lanes so the per-row max/sum stays in-lane; pass 2
// puts keys on lanes so the per-key sum/max over rows stays in-lane.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

// ---------------------------------------------------------------- pass 1 ----
// grid (row_blocks * splits, H, L), block 256: 4 waves x 32 query rows.
// Each wave streams 32-key tiles of its split; lane l owns query row
// rb*128 + wave*32 + l%32 and, per tile, 16 of the 32 keys (by lane half).
template <bool CAUSAL>
__global__ __launch_bounds__(256) void k_rowstats(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, int H, int R,
    int W, int n, float alpha, int splits, int keys_per_split,
    float2* __restrict__ part) {
  const int rb = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int h = blockIdx.y, l = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int row = rb * 128 + wave * 32 + col;
  const size_t lh = (size_t)l * H + h;
  const __bf16* qh = q + lh * (size_t)R * kHeadDim;
  const __bf16* kh = k + lh * (size_t)n * kHeadDim;

  bf16x8 b[8];
  if (row < R) load_half_row(qh + (size_t)row * kHeadDim, hf, b);
  else zero_ops(b);
  // last key this row sees
  const int vis = CAUSAL ? (n - W + (row % W)) : (n - 1);
  const int j0 = sp * keys_per_split;
  const int j1 = min(n, j0 + keys_per_split);

  float m = neg_inf(), s = 0.f;
  for (int kt = j0; kt < j1; kt += 32) {
    bf16x8 a[8];
    const int key = kt + col;
    if (key < n) load_half_row(kh + (size_t)key * kHeadDim, hf, a);
    else zero_ops(a);
    f32x16 acc = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) acc = mfma32(a[st], b[st], acc);
    float x[16];
    float tmax = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = kt + acc_row(i, lane);
      const bool ok = kj < j1 && kj <= vis;
      x[i] = ok ? acc[i] * alpha : neg_inf();
      tmax = fmaxf(tmax, x[i]);
    }
    const float mn = fmaxf(m, tmax);
    if (mn != neg_inf()) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t += fast_exp2(x[i] - mn);
      s = s * fast_exp2(m - mn) + t;
      m = mn;
    }
  }
  // the other lane half holds the other 16 keys of every tile
  const float m2 = __shfl_xor(m, 32), s2 = __shfl_xor(s, 32);
  lse_merge(m, s, m2, s2);
  if (hf == 0 && row < R) part[(lh * splits + sp) * (size_t)R + row] = make_float2(m, s);
}

// c_r = m_r + log2(l_r) over the splits, in split order.
__global__ __launch_bounds__(256) void k_combine(const float2* __restrict__ part,
                                                 int H, int R, int splits,
                                                 float* __restrict__ stat) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, l = blockIdx.z;
  if (r >= R) return;
  const size_t lh = (size_t)l * H + h;
  float m = neg_inf(), s = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const float2 p = part[(lh * splits + sp) * (size_t)R + r];
    lse_merge(m, s, p.x, p.y);
  }
  stat[lh * R + r] = m + __log2f(s);
}

// ---------------------------------------------------------------- pass 2 ----
// grid (ceil(n/128), H, L), block 256: 4 waves x 32 keys. Lane l owns key
// kb*128 + wave*32 + l%32 and loops over all R query rows in tiles of 32;
// per tile it holds 16 of the 32 rows (by lane half).
template <bool CAUSAL, bool MAXAGG>
__global__ __launch_bounds__(256) void k_colagg(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, int H, int R,
    int W, int n, float alpha, const float* __restrict__ stat,
    float* __restrict__ raw) {
  const int kb = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int key = kb * 128 + wave * 32 + col;
  const size_t lh = (size_t)l * H + h;
  const __bf16* qh = q + lh * (size_t)R * kHeadDim;
  const __bf16* kh = k + lh * (size_t)n * kHeadDim;
  const float* sh = stat + lh * R;

  bf16x8 b[8];
  if (key < n) load_half_row(kh + (size_t)key * kHeadDim, hf, b);
  else zero_ops(b);
  float agg = MAXAGG ? neg_inf() : 0.f;
  for (int rt = 0; rt < R; rt += 32) {
    bf16x8 a[8];
    const int qrow = rt + col;
    if (qrow < R) load_half_row(qh + (size_t)qrow * kHeadDim, hf, a);
    else zero_ops(a);
    f32x16 acc = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) acc = mfma32(a[st], b[st], acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rt + acc_row(i, lane);
      bool ok = r < R;
      if (CAUSAL) ok = ok && key <= n - W + (r % W);
      const float c = sh[min(r, R - 1)];
      const float x = acc[i] * alpha - c;
      if (MAXAGG) agg = ok ? fmaxf(agg, x) : agg;
      else agg += ok ? fast_exp2(x) : 0.f;
    }
  }
  const float o = __shfl_xor(agg, 32);
  if (MAXAGG) agg = fast_exp2(fmaxf(agg, o));
  else agg += o;
  if (hf == 0 && key < n) raw[lh * n + key] = agg;
}

// ------------------------------------------------------------------ pool ----
// scores[j] = max raw[t], |t - j| <= r, 0 <= t < n_cand.   grid (.., L*H)
__global__ __launch_bounds__(256) void k_pool(const float* __restrict__ raw, int n,
                                              int n_cand, int r,
                                              float* __restrict__ scores) {
  __shared__ float tile[256 + 2 * 32];
  const size_t lh = blockIdx.y;
  const int j0 = blockIdx.x * 256;
  const float* src = raw + lh * n;
  for (int t = threadIdx.x; t < 256 + 2 * r; t += 256) {
    const int j = j0 - r + t;
    tile[t] = (j >= 0 && j < n_cand) ? src[j] : 0.f;  // scores are >= 0
  }
  __syncthreads();
  const int j = j0 + threadIdx.x;
  if (j >= n_cand) return;
  float m = tile[threadIdx.x + r];
  for (int o = 1; o <= r; ++o) m = fmaxf(m, fmaxf(tile[threadIdx.x + r - o], tile[threadIdx.x + r + o]));
  scores[lh * n_cand + j] = m;
}

// ------------------------------------------------------------------ host ----

hipError_t combine_launch(const float2* part, int L, int H, int R, int splits, float* stat,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3((R + 255) / 256, H, L), dim3(256), 0, st, part, H, R,
                     splits, stat);
  return hipGetLastError();
}

hipError_t pool_launch(const float* raw, int L, int H, int n, int n_cand, int r, float* scores,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_pool, dim3((n_cand + 255) / 256, L * H), dim3(256), 0, st, raw, n,
                     n_cand, r, scores);
  return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void twopass_plan(const ScorePlan& p, TwoPassLayout* o) {
  const int row_blocks = (p.R + 127) / 128;
  const long long base = (long long)row_blocks * p.H * p.L;
  int splits = (int)((2048 + base - 1) / base);
  const int max_splits = (p.n + 255) / 256;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int kps = (p.n + splits - 1) / splits;
  kps = (kps + 31) / 32 * 32;
  splits = (p.n + kps - 1) / kps;
  o->row_blocks = row_blocks;
  o->splits = splits;
  o->keys_per_split = kps;
  const size_t LH = (size_t)p.L * p.H;
  o->part_off = 0;
  o->stat_off = align256(LH * splits * p.R * sizeof(float2));
  o->raw_off = o->stat_off + align256(LH * p.R * sizeof(float));
  o->bytes = o->raw_off + (p.need_raw_tmp ? align256(LH * p.n * sizeof(float)) : 0);
}

hipError_t twopass_launch(const ScorePlan& p, const TwoPassLayout& o, const void* q,
                          const void* k, float* scores, float* raw, void* ws,
                          hipStream_t st) {
  char* w = static_cast<char*>(ws);
  float2* part = reinterpret_cast<float2*>(w + o.part_off);
  float* stat = reinterpret_cast<float*>(w + o.stat_off);
  float* rawbuf = raw ? raw : reinterpret_cast<float*>(w + o.raw_off);
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const float alpha = p.scale * kLog2e;
  dim3 g1(o.row_blocks * o.splits, p.H, p.L);
  if (p.causal)
    hipLaunchKernelGGL(k_rowstats<true>, g1, dim3(256), 0, st, qb, kb, p.H, p.R, p.W, p.n,
                       alpha, o.splits, o.keys_per_split, part);
  else
    hipLaunchKernelGGL(k_rowstats<false>, g1, dim3(256), 0, st, qb, kb, p.H, p.R, p.W, p.n,
                       alpha, o.splits, o.keys_per_split, part);
  hipLaunchKernelGGL(k_combine, dim3((p.R + 255) / 256, p.H, p.L), dim3(256), 0, st, part,
                     p.H, p.R, o.splits, stat);
  dim3 g2((p.n + 127) / 128, p.H, p.L);
  if (p.causal) {
    if (p.max_agg)
      hipLaunchKernelGGL((k_colagg<true, true>), g2, dim3(256), 0, st, qb, kb, p.H, p.R, p.W,
                         p.n, alpha, stat, rawbuf);
    else
      hipLaunchKernelGGL((k_colagg<true, false>), g2, dim3(256), 0, st, qb, kb, p.H, p.R, p.W,
                         p.n, alpha, stat, rawbuf);
  } else {
    if (p.max_agg)
      hipLaunchKernelGGL((k_colagg<false, true>), g2, dim3(256), 0, st, qb, kb, p.H, p.R, p.W,
                         p.n, alpha, stat, rawbuf);
    else
      hipLaunchKernelGGL((k_colagg<false, false>), g2, dim3(256), 0, st, qb, kb, p.H, p.R, p.W,
                         p.n, alpha, stat, rawbuf);
  }
  hipLaunchKernelGGL(k_pool, dim3((p.n_cand + 255) / 256, p.L * p.H), dim3(256), 0, st,
                     rawbuf, p.n, p.n_cand, p.pool / 2, scores);
  return hipGetLastError();
}

}  // namespace kvsel
