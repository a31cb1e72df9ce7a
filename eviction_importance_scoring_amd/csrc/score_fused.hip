// Window scoring in one pass over K: [CriticalKV] §3.3 Algorithm 2 steps
// 2-4 (softmax(Q_hat K^T) of the last W queries, aggregated over the window
// queries and the G query heads, then max-pooled).
//
// The exact softmax weight of a key needs every row's normaliser over all n
// keys first ([KVzip] §3.4: softmax along keys, aggregate along queries). A
// two-pass scheme streams K twice; this kernel reads it once. Each
// workgroup owns 256 keys of one (layer, KV head) and all R = G*W <= 128
// query rows:
//   1. logits x = log2(e)*scale*<q, k> for its 256 x R tile on MFMA (K on
//      the A side straight from HBM, Q from LDS), causal mask applied;
//   2. per lane and row: m = max x, e = 2^(x - m) kept in registers, l = sum e;
//      rows merged over lanes and waves -> one (m, l) pair per row;
//   3. per-head barrier: the last workgroup of the head to arrive folds all
//      chunk pairs in chunk order into c_r = M_r + log2(L_r) and releases
//      the others;
//   4. weight of key j = sum_r e_rj 2^(m_lane,r - c_r): scaled in-lane,
//      then reduced over the 32 query lanes by a reduce-scatter that leaves
//      one key per lane;
//   5. max-pool inside the chunk plus a halo of pool/2 raw scores from each
//      neighbouring chunk (published after step 4, so never waited on early).
//
// Barrier safety: workgroups take tickets in the order they start, and the
// tickets enumerate the heads in order, so every workgroup of the oldest
// unfinished head is already running whenever any later one is. The host
// only uses this kernel when one head's workgroups fit on the GPU at once
// (with a 2x margin), so that head can always finish. All waits are
// bounded: on a timeout the kernel records an error, writes NaN scores for
// that head and still exits.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kFusedKeys = 256;          // keys per workgroup
constexpr int kQStride = kRowBytes + 16; // LDS row pitch of Q (bytes), padded
constexpr int kMaxPoolR = 8;             // pool <= 17
constexpr uint32_t kSpinLimit = 1u << 22;

struct FusedArgs {
  const __bf16* q;
  const __bf16* k;
  float* scores;
  float* raw;
  float2* part;        // [LH][C][R]   per-chunk (m, l) of every row
  float* stat;         // [LH][R]      c_r
  uint32_t* arrive;    // [LH]
  uint32_t* ready;     // [LH]
  float* halo;         // [LH][C][2*kMaxPoolR]
  uint32_t* halo_flag; // [LH][C]
  uint32_t* ticket;    // [1]
  uint32_t* err;       // [1]
  int R, W, n, n_cand, C, pr, items;
  float alpha;
};

__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until *flag != 0. Returns false on timeout.
__device__ bool wait_flag(const uint32_t* flag) {
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (ld_flag(flag) != 0u) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

template <int NT>
__global__ __launch_bounds__(256) void k_window_fused(FusedArgs a) {
  __shared__ __align__(16) unsigned char q_lds[NT * 32 * kQStride];
  __shared__ float2 wstat[4][NT * 32];
  __shared__ float craw[kFusedKeys + 2 * kMaxPoolR];
  __shared__ uint32_t s_item, s_flag;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  if (tid == 0) s_item = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int item = (int)s_item;
  if (item >= a.items) return;
  const int lh = item / a.C, c = item - lh * a.C;
  const int R = a.R, W = a.W, n = a.n;
  const __bf16* qh = a.q + (size_t)lh * R * kHeadDim;
  const __bf16* kh = a.k + (size_t)lh * n * kHeadDim;

  // ---- K operands of this wave's 64 keys (HBM -> registers, once)
  const int kbase = c * kFusedKeys + wave * 64;
  bf16x8 ka[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = kbase + mt * 32 + col;
    if (key < n) load_half_row(kh + (size_t)key * kHeadDim, hf, ka[mt]);
    else zero_ops(ka[mt]);
  }
  // ---- Q tile -> LDS (rows >= R zero)
  for (int t = tid; t < NT * 32 * 16; t += 256) {
    const int r = t >> 4, piece = t & 15;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < R) val = *reinterpret_cast<const u32x4*>(qh + (size_t)r * kHeadDim + piece * 8);
    *reinterpret_cast<u32x4*>(q_lds + r * kQStride + piece * 16) = val;
  }
  __syncthreads();

  // ---- 1. logits on MFMA: acc[mt][nt][i] = <k_key, q_row>, key on M, row on N
  f32x16 acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero16();
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 b = ld16(q_lds + (nt * 32 + col) * kQStride + hf * 128 + s * 16);
      acc[0][nt] = mfma32(ka[0][s], b, acc[0][nt]);
      acc[1][nt] = mfma32(ka[1][s], b, acc[1][nt]);
    }
  }

  // ---- 2. masked exps in place, per-lane (m, l) per row
  float mloc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = nt * 32 + col;
    const int last = (row < R) ? (n - W + row % W) : -1;   // last visible key
    float mx = neg_inf();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + mt * 32 + acc_row(i, lane);
        const float x = (key <= last) ? acc[mt][nt][i] * a.alpha : neg_inf();
        acc[mt][nt][i] = x;
        mx = fmaxf(mx, x);
      }
    const float ref = (mx == neg_inf()) ? 0.f : mx;
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(acc[mt][nt][i] - ref);
        acc[mt][nt][i] = e;
        sum += e;
      }
    mloc[nt] = mx;
    float m2 = __shfl_xor(mx, 32), s2 = __shfl_xor(sum, 32);
    float mw = mx, sw = sum;
    lse_merge(mw, sw, m2, s2);
    if (hf == 0) wstat[wave][row] = make_float2(mw, sw);
  }
  __syncthreads();
  float2* part_c = a.part + ((size_t)lh * a.C + c) * R;
  if (tid < R) {
    float m = neg_inf(), s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) lse_merge(m, s, wstat[w][tid].x, wstat[w][tid].y);
    part_c[tid] = make_float2(m, s);
  }

  // ---- 3. per-head barrier; the last arrival folds all chunks of the head
  fence_release();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.arrive + lh, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_flag = (old == (uint32_t)a.C - 1u) ? 1u : 0u;
  }
  __syncthreads();
  bool ok = true;
  if (s_flag) {
    fence_acquire();
    if (tid < R) {
      const float2* pp = a.part + (size_t)lh * a.C * R + tid;
      float m = neg_inf(), s = 0.f;
      int cc = 0;
      for (; cc + 8 <= a.C; cc += 8) {
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pp[(size_t)(cc + u) * R];
#pragma unroll
        for (int u = 0; u < 8; ++u) lse_merge(m, s, v[u].x, v[u].y);
      }
      for (; cc < a.C; ++cc) {
        const float2 v = pp[(size_t)cc * R];
        lse_merge(m, s, v.x, v.y);
      }
      a.stat[(size_t)lh * R + tid] = m + __log2f(s);
    }
    fence_release();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.ready + lh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if (tid == 0) s_flag = wait_flag(a.ready + lh) ? 2u : 3u;
    __syncthreads();
    ok = s_flag == 2u;
  }
  fence_acquire();
  if (!ok && tid == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 4. per-key weights: scale by 2^(m_lane - c_r), reduce over rows
  float fct[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = nt * 32 + col;
    const float cr = (row < R) ? a.stat[(size_t)lh * R + row] : 0.f;
    fct[nt] = (row < R && mloc[nt] != neg_inf()) ? fast_exp2(mloc[nt] - cr) : 0.f;
  }
  float v[32];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float t = acc[mt][0][i] * fct[0];
#pragma unroll
      for (int nt = 1; nt < NT; ++nt) t += acc[mt][nt][i] * fct[nt];
      v[mt * 16 + i] = t;
    }
  // reduce-scatter over the 32 lanes of this half: lane col keeps entry col
#pragma unroll
  for (int m = 16, cnt = 32; m >= 1; m >>= 1, cnt >>= 1) {
    const bool up = (col & m) != 0;
#pragma unroll
    for (int j = 0; j < cnt / 2; ++j) {
      const float send = up ? v[j] : v[j + cnt / 2];
      const float keep = up ? v[j + cnt / 2] : v[j];
      v[j] = keep + __shfl_xor(send, m);
    }
  }
  const int kloc = wave * 64 + (col >> 4) * 32 + acc_row(col & 15, lane);
  const int key = c * kFusedKeys + kloc;
  const float rawv = ok ? v[0] : __builtin_nanf("");
  craw[a.pr + kloc] = rawv;
  if (a.raw && key < n) a.raw[(size_t)lh * n + key] = rawv;
  __syncthreads();

  // ---- 5. halo exchange and max-pool over candidates [0, n_cand)
  const int pr = a.pr;
  float* halo_c = a.halo + ((size_t)lh * a.C + c) * (2 * kMaxPoolR);
  if (pr > 0) {
    if (tid < pr) halo_c[tid] = craw[pr + tid];
    else if (tid >= 64 && tid < 64 + pr) halo_c[kMaxPoolR + tid - 64] = craw[kFusedKeys + (tid - 64)];
    fence_release();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.halo_flag + (size_t)lh * a.C + c, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    const int c0 = c * kFusedKeys;
    const bool need_left = c > 0 && c0 - 1 < a.n_cand;
    const bool need_right = c + 1 < a.C && c0 + kFusedKeys < a.n_cand;
    if (tid == 0) {
      bool good = true;
      if (need_left) good = wait_flag(a.halo_flag + (size_t)lh * a.C + c - 1) && good;
      if (need_right) good = wait_flag(a.halo_flag + (size_t)lh * a.C + c + 1) && good;
      s_flag = good ? 1u : 0u;
      if (!good) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    fence_acquire();
    if (tid < pr) {
      craw[tid] = need_left ? a.halo[((size_t)lh * a.C + c - 1) * (2 * kMaxPoolR) + kMaxPoolR + tid] : 0.f;
      craw[pr + kFusedKeys + tid] =
          need_right ? a.halo[((size_t)lh * a.C + c + 1) * (2 * kMaxPoolR) + tid] : 0.f;
      if (!s_flag) craw[tid] = craw[pr + kFusedKeys + tid] = __builtin_nanf("");
    }
    __syncthreads();
  }
  const int j = c * kFusedKeys + tid;
  if (j < a.n_cand) {
    float m = craw[pr + tid];
    for (int o = 1; o <= pr; ++o) {
      if (j - o >= 0) m = fmaxf(m, craw[pr + tid - o]);
      if (j + o < a.n_cand) m = fmaxf(m, craw[pr + tid + o]);
    }
    a.scores[(size_t)lh * a.n_cand + j] = (ok && s_flag) || pr == 0 ? m : __builtin_nanf("");
  }
}

// Zero the barrier counters and flags of the workspace.
__global__ void k_fused_init(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

// ------------------------------------------------------------------ host ----

static size_t al(size_t x) { return (x + 255) & ~size_t(255); }

static int nt_for(int R) { return R <= 32 ? 1 : (R <= 64 ? 2 : 4); }

static int fused_capacity(int nt) {
  static int cached[5] = {0, 0, 0, 0, 0};
  if (cached[nt] == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const void* fn = nt == 1 ? (const void*)k_window_fused<1>
                   : nt == 2 ? (const void*)k_window_fused<2> : (const void*)k_window_fused<4>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess) return 0;
    cached[nt] = cus * per_cu;
  }
  return cached[nt];
}

bool fused_applicable(const ScorePlan& p, int* chunks) {
  if (!p.causal || p.max_agg || p.R > 128 || p.pool / 2 > kMaxPoolR) return false;
  const int C = (p.n + kFusedKeys - 1) / kFusedKeys;
  *chunks = C;
  const int cap = fused_capacity(nt_for(p.R));
  return cap > 0 && 2 * C <= cap;
}

void fused_plan(const ScorePlan& p, FusedLayout* o) {
  const int C = (p.n + kFusedKeys - 1) / kFusedKeys;
  const size_t LH = (size_t)p.L * p.H;
  o->chunks = C;
  size_t off = 0;
  o->flags_off = off;                                  // ticket, err, arrive, ready, halo_flag
  o->flag_words = 2 + 2 * LH + LH * C;
  off += al(o->flag_words * 4);
  o->part_off = off;  off += al(LH * C * p.R * sizeof(float2));
  o->stat_off = off;  off += al(LH * p.R * sizeof(float));
  o->halo_off = off;  off += al(LH * C * 2 * kMaxPoolR * sizeof(float));
  o->bytes = off;
}

hipError_t fused_launch(const ScorePlan& p, const FusedLayout& o, const void* q, const void* k,
                        float* scores, float* raw, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  uint32_t* flags = reinterpret_cast<uint32_t*>(w + o.flags_off);
  const size_t LH = (size_t)p.L * p.H;
  FusedArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.scores = scores;
  a.raw = raw;
  a.part = reinterpret_cast<float2*>(w + o.part_off);
  a.stat = reinterpret_cast<float*>(w + o.stat_off);
  a.ticket = flags;
  a.err = flags + 1;
  a.arrive = flags + 2;
  a.ready = flags + 2 + LH;
  a.halo_flag = flags + 2 + 2 * LH;
  a.halo = reinterpret_cast<float*>(w + o.halo_off);
  a.R = p.R;
  a.W = p.W;
  a.n = p.n;
  a.n_cand = p.n_cand;
  a.C = o.chunks;
  a.pr = p.pool / 2;
  a.items = (int)(LH * o.chunks);
  a.alpha = p.scale * kLog2e;
  const unsigned init_blocks = (unsigned)((o.flag_words + 255) / 256 < 1024 ? (o.flag_words + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_fused_init, dim3(init_blocks), dim3(256), 0, st, flags, o.flag_words);
  const int nt = nt_for(p.R);
  if (nt == 1)
    hipLaunchKernelGGL(k_window_fused<1>, dim3(a.items), dim3(256), 0, st, a);
  else if (nt == 2)
    hipLaunchKernelGGL(k_window_fused<2>, dim3(a.items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_window_fused<4>, dim3(a.items), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvsel
