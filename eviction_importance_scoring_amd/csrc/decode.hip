// One decoding step of attention over the compacted cache ([KVzip] §7.1:
// after eviction each KV head keeps its own number of rows, and a new
// token's attention runs over each head's kept rows with a variable-length
// kernel). The query of query head h*G+g attends over KV head h's kept
// rows: out = softmax_t(scale * <q, k_t>) . v_t; an empty head gives zeros.
//
// Work is split into items of up to dec_chunk(G) kept rows of one head
// (flash-decoding): every item computes, for the G query heads of its KV
// head, the item's max logit m, sum of exponentials l and unnormalised
// output o; a second kernel merges a head's items. Items of a layer are
// numbered head by head (prefix over ceil(len_h / chunk)), recomputed from
// the head offsets by each workgroup, so ragged heads need no host
// knowledge of their lengths.
//
// In an item (256 threads) a key row is spread over 16 lanes, 8 head-dim
// elements (one 16-byte load) each, so a wave reads 4 whole rows per load
// instruction; a logit is 4 bf16 dot2 instructions per query head and lane
// (fp32 accumulation) and a 16-lane sum by DPP. Two kernels:
//   k_decode_stream (G <= 4, 512-row items): a wave streams its 128 rows 4
//     at a time, the K and V rows of the next kDecDepth steps in flight,
//     with an online softmax per query head in every 16-lane slot (running
//     max, sum of exponentials, p * v over the lane's 8 elements)
//   k_decode_phased (G > 4, 256-row items): a wave's 64 K rows in flight,
//     the logits to LDS, V's rows in flight while the item's max and
//     exponentials are taken, then p * v (fewer registers a lane at large G)
// Exponentials are base 2 with the scale folded in (alpha = scale * log2
// e). Deterministic: fixed-order sums, no atomics.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kStreamChunk = 512;   // kept rows per work item, G <= 4
constexpr int kPhasedChunk = 256;   // kept rows per work item, G > 4
constexpr int kDecThreads = 256;    // 4 waves
constexpr int kDecDepth = 4;        // streaming: steps of 4 rows whose loads are in flight ahead
constexpr int kDecSteps = kStreamChunk / 16;   // streaming: steps a wave takes (4 rows each)
constexpr float kDecFloor = -1.0e30f;       // running max before any row

__host__ __device__ constexpr int dec_chunk(int G) { return G <= 4 ? kStreamChunk : kPhasedChunk; }
constexpr int kDecMaxG = 8;
constexpr int kDecMaxHeads = 1024;
constexpr int kDecRec = kHeadDim + 2;   // partial of one query head: o[128], m, l

// kept rows [start, start + len) of head h in layer l, from the effective
// offsets eo[0..H] that dec_prefix leaves in LDS
struct DecHead {
  int start, len;
};

__device__ __forceinline__ DecHead dec_head(const int* eo, int h) {
  return DecHead{eo[h], eo[h + 1] - eo[h]};
}

// Called by every thread of the block; wave 0 does the work.
// eo[h] (h <= H): the head offsets clamped into [0, kept] and raised to the
// largest earlier one, so the heads are disjoint ranges inside the layer
// whose lengths sum to at most kept (the grid and workspace are sized for
// that; valid offsets are unchanged). Uniform layout: eo[h] = h * (kept/H).
// pre[h] = work items (of `chunk` rows) of the layer's heads before h,
// pre[H] = all of them.
// Both are visible after the caller's barrier.
__device__ __forceinline__ void dec_prefix(const int32_t* offs, int l, int H, int kept, int chunk,
                                           int* eo, int* pre) {
  const int lane = threadIdx.x;
  if (threadIdx.x < 64) {
    const int32_t* o = offs ? offs + (size_t)l * (H + 1) : nullptr;
    int run = 0;
    for (int base = 0; base <= H; base += 64) {
      const int h = base + lane;
      int x = 0;
      if (h <= H) x = o ? min(max(o[h], 0), kept) : h * (kept / H);
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const int y = __shfl_up(x, s);
        if (lane >= s) x = max(x, y);
      }
      x = max(x, run);
      if (h <= H) eo[h] = x;
      run = __shfl(x, 63);
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  int carry = 0;
  for (int base = 0; base < H; base += 64) {
    const int h = base + lane;
    const int cnt = h < H ? (dec_head(eo, h).len + chunk - 1) / chunk : 0;
    int x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (h < H) pre[h + 1] = carry + x;
    carry += __shfl(x, 63);
  }
  if (lane == 0) pre[0] = 0;
}

// last head whose first item is <= i (pre non-decreasing, pre[0] = 0)
__device__ __forceinline__ int dec_find(const int* pre, int H, int i) {
  int lo = 0, hi = H - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// sum over the 16 lanes of a row (all 16 get it): quad swaps, then the
// half-row and row mirrors
__device__ __forceinline__ float sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
  return x;
}

// 8 bf16 (one 16-byte piece) as fp32
__device__ __forceinline__ void bf16x8_to_f32(u32x4 b, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(b[i] << 16);
    f[2 * i + 1] = __uint_as_float(b[i] & 0xFFFF0000u);
  }
}

// a.lo * b.lo + a.hi * b.hi + c over bf16 pairs, in fp32 (bf16 products
// are exact in fp32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// G <= 4: items of kStreamChunk rows. 1-D grid of L * items workgroups,
// block 256. part[l][item][g][kDecRec].
// Wave w takes the item's rows r0 + w * kStreamChunk / 4 + 4s + slot (s =
// 0 .. kDecSteps - 1), 4 rows a step (one per 16-lane slot), and streams
// them: the K and V rows of the next kDecDepth steps are in flight while a
// step is folded. Each slot keeps an online softmax per query head (max m,
// sum l, output o over its 8 head-dim elements), rescaled only when a
// wave's max moves; the slots of a wave merge by lane swaps, the waves
// through LDS, in a fixed order.
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_decode_stream(const __bf16* __restrict__ q,
                                                        const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, int H,
                                                        int kept, const int32_t* __restrict__ offs,
                                                        float alpha, int items,
                                                        float* __restrict__ part) {
  static_assert(G >= 1 && G <= kDecMaxG, "query heads per KV head");
  __shared__ int pre[kDecMaxHeads + 1];
  __shared__ int eo[kDecMaxHeads + 1];
  __shared__ float wml[4][G][2];              // per wave: m, l
  __shared__ float wout[4][G][kHeadDim];      // per wave: o at its own m
  const int l = blockIdx.x / items, it = blockIdx.x - l * items;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = lane >> 4, piece = lane & 15;

  dec_prefix(offs, l, H, kept, kStreamChunk, eo, pre);
  __syncthreads();
  if (it >= pre[H]) return;   // uniform: past the layer's items
  const int h = dec_find(pre, H, it);
  const DecHead hd = dec_head(eo, h);
  const int r0 = hd.start + (it - pre[h]) * kStreamChunk;
  const int r1 = min(hd.start + hd.len, r0 + kStreamChunk);   // r0 < r1

  // this lane's 8 head-dim elements of the G queries, as bf16 pairs
  u32x4 qp[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qp[g] = *reinterpret_cast<const u32x4*>(q + ((size_t)l * H * G + h * G + g) * kHeadDim + piece * 8);
  const size_t lrow = (size_t)l * kept;
  const int wr0 = r0 + wave * (kStreamChunk / 4) + slot;
  // rows past the item repeat its last row (in range; their weight is 0),
  // so every load is unconditional and none waits for another
  auto kv_load = [&](int s, u32x4& kk, u32x4& vv) {
    const int row = min(wr0 + 4 * s, r1 - 1);
    kk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + (lrow + row) * kHeadDim + piece * 8));
    vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + (lrow + row) * kHeadDim + piece * 8));
  };
  u32x4 kb[kDecDepth], vb[kDecDepth];
#pragma unroll
  for (int d = 0; d < kDecDepth; ++d) kv_load(d, kb[d], vb[d]);

  // m starts at a finite floor so that rows of no weight (x = -inf) give
  // p = 0 and a scale of 1 even before any live row
  float m[G], ls[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kDecFloor;
    ls[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < kDecSteps; ++s) {
    const int d = s % kDecDepth;
    const bool live = wr0 + 4 * s < r1;
    float x[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = bf16_dot2(qp[g][e], kb[d][e], dot);
      const float sdot = sum16(dot);   // every lane of the 16-lane row takes part
      x[g] = live ? sdot * alpha : neg_inf();
    }
    float vf[8];
    bf16x8_to_f32(vb[d], vf);
    if (s + kDecDepth < kDecSteps) kv_load(s + kDecDepth, kb[d], vb[d]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(m[g], x[g]);
      const float p = fast_exp2(x[g] - mn);
      if (__ballot(mn != m[g]) != 0) {   // some slot's max moved: rescale (1 elsewhere)
        const float sc = fast_exp2(m[g] - mn);
        ls[g] *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= sc;
        m[g] = mn;
      }
      ls[g] += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = __builtin_fmaf(p, vf[e], o[g][e]);
    }
  }
  // the wave's 4 slots (lanes 16 and 32 apart hold the same elements)
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      const float m2 = __shfl_xor(m[g], sh);
      const float mx = fmaxf(m[g], m2);
      const float a = fast_exp2(m[g] - mx), b = fast_exp2(m2 - mx);
      ls[g] = ls[g] * a + __shfl_xor(ls[g], sh) * b;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = o[g][e] * a + __shfl_xor(o[g][e], sh) * b;
      m[g] = mx;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wout[wave][g][piece * 8 + e] = o[g][e];
      if (piece == 0) {
        wml[wave][g][0] = m[g];
        wml[wave][g][1] = ls[g];
      }
    }
  }
  __syncthreads();
  // the 4 waves, in order
  float* rec = part + ((size_t)l * items + it) * G * kDecRec;
  for (int t = tid; t < G * kHeadDim; t += kDecThreads) {
    const int g = t / kHeadDim, dd = t - g * kHeadDim;
    const float mx = fmaxf(fmaxf(wml[0][g][0], wml[1][g][0]), fmaxf(wml[2][g][0], wml[3][g][0]));
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_fmaf(fast_exp2(wml[w][g][0] - mx), wout[w][g][dd], acc);
    rec[g * kDecRec + dd] = acc;
  }
  if (tid < G) {
    const int g = tid;
    const float mx = fmaxf(fmaxf(wml[0][g][0], wml[1][g][0]), fmaxf(wml[2][g][0], wml[3][g][0]));
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) lsum = __builtin_fmaf(fast_exp2(wml[w][g][0] - mx), wml[w][g][1], lsum);
    rec[g * kDecRec + kHeadDim] = mx;
    rec[g * kDecRec + kHeadDim + 1] = lsum;
  }
}

// G > 4: items of kPhasedChunk rows; wave w takes rows 64w .. 64w+63 in
// phases: all of its K rows in flight, the logits (to LDS), V's rows in
// flight while the item's max and exponentials are taken (one thread per
// key), then p * v in the K layout. Holds fewer registers a lane than the
// streaming kernel at large G (three waves per SIMD at G = 7 against two).
// 1-D grid of L * items workgroups, block 256. part[l][item][g][kDecRec].
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_decode_phased(const __bf16* __restrict__ q,
                                                        const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, int H,
                                                        int kept, const int32_t* __restrict__ offs,
                                                        float alpha, int items,
                                                        float* __restrict__ part) {
  __shared__ int pre[kDecMaxHeads + 1];
  __shared__ int eo[kDecMaxHeads + 1];
  __shared__ __align__(16) float pr[kPhasedChunk][kDecMaxG];   // logits, then exponentials
  __shared__ float red[2][4][kDecMaxG];
  __shared__ float osum[4][G][kHeadDim];
  const int l = blockIdx.x / items, it = blockIdx.x - l * items;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = lane >> 4, piece = lane & 15;

  dec_prefix(offs, l, H, kept, kPhasedChunk, eo, pre);
  __syncthreads();
  if (it >= pre[H]) return;   // uniform: past the layer's items
  const int h = dec_find(pre, H, it);
  const DecHead hd = dec_head(eo, h);
  const int r0 = hd.start + (it - pre[h]) * kPhasedChunk;
  const int r1 = min(hd.start + hd.len, r0 + kPhasedChunk);   // r0 < r1

  // this lane's 8 head-dim elements of the G queries, as bf16 pairs
  u32x4 qp[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qp[g] = *reinterpret_cast<const u32x4*>(q + ((size_t)l * H * G + h * G + g) * kHeadDim + piece * 8);
  const size_t lrow = (size_t)l * kept;
  // ---- logits: wave rows [64w, 64w + 64), 4 rows per step (one per slot)
  // rows past the item repeat its last row (in range; their weight is 0),
  // so every load is unconditional and none waits for another
  u32x4 kb[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int row = min(r0 + wave * 64 + s * 4 + slot, r1 - 1);
    kb[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + (lrow + row) * kHeadDim + piece * 8));
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = wave * 64 + s * 4 + slot;
    float mine = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = bf16_dot2(qp[g][e], kb[s][e], dot);
      dot = sum16(dot);
      if (piece == g) mine = dot;
    }
    if (piece < G) pr[j][piece] = r0 + j < r1 ? mine * alpha : neg_inf();
  }
  // V's loads fly while the chunk's exponentials are taken
  u32x4 vb[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int row = min(r0 + wave * 64 + s * 4 + slot, r1 - 1);
    vb[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + (lrow + row) * kHeadDim + piece * 8));
  }
  __syncthreads();
  // ---- the chunk's max and exponentials: thread t takes key t
  float x[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    x[g] = pr[tid][g];
    const float wm = wave_max(x[g]);
    if (lane == 0) red[0][wave][g] = wm;
  }
  __syncthreads();
  float m[G], ls[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = fmaxf(fmaxf(red[0][0][g], red[0][1][g]), fmaxf(red[0][2][g], red[0][3][g]));   // finite: r1 > r0
    const float p = fast_exp2(x[g] - m[g]);   // 0 for rows past the item
    pr[tid][g] = p;
    const float ws = wave_sum(p);
    if (lane == 0) red[1][wave][g] = ws;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) ls[g] = (red[1][0][g] + red[1][1][g]) + (red[1][2][g] + red[1][3][g]);
  // ---- p . v in the same layout as the logits
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = wave * 64 + s * 4 + slot;
    float vf[8];
    bf16x8_to_f32(vb[s], vf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = pr[j][g];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = __builtin_fmaf(p, vf[e], o[g][e]);
    }
  }
  // the 4 slots of the wave, then the 4 waves (fixed order)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = o[g][e] + __shfl_xor(o[g][e], 16);
      t += __shfl_xor(t, 32);
      o[g][e] = t;
    }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) osum[wave][g][piece * 8 + e] = o[g][e];
  }
  __syncthreads();
  float* rec = part + ((size_t)l * items + it) * G * kDecRec;
  for (int t = tid; t < G * kHeadDim; t += kDecThreads) {
    const int g = t / kHeadDim, d = t - g * kHeadDim;
    rec[g * kDecRec + d] = (osum[0][g][d] + osum[1][g][d]) + (osum[2][g][d] + osum[3][g][d]);
  }
  if (tid < G) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (tid == g) {
        rec[g * kDecRec + kHeadDim] = m[g];
        rec[g * kDecRec + kHeadDim + 1] = ls[g];
      }
  }
}

// grid L * H * G, block 128 (one thread per head-dim element): merge the
// items of one query head. The max over the items is a block reduction;
// then every thread weighs its element of each item (independent loads).
__global__ __launch_bounds__(kHeadDim) void k_decode_merge(int H, int G, int kept, int chunk,
                                                           const int32_t* __restrict__ offs,
                                                           int items, const float* __restrict__ part,
                                                           float* __restrict__ out) {
  __shared__ int pre[kDecMaxHeads + 1];
  __shared__ int eo[kDecMaxHeads + 1];
  __shared__ float wmax[kHeadDim / 64];
  const int g = blockIdx.x % G, lh = blockIdx.x / G;
  const int h = lh % H, l = lh / H;
  dec_prefix(offs, l, H, kept, chunk, eo, pre);
  __syncthreads();
  const int d = threadIdx.x;
  const int i0 = pre[h], i1 = pre[h + 1];
  float* dst = out + ((size_t)l * H * G + h * G + g) * kHeadDim + d;
  if (i0 == i1) {   // no kept rows
    *dst = 0.f;
    return;
  }
  const size_t stride = (size_t)G * kDecRec;
  const float* rec = part + ((size_t)l * items) * stride + g * kDecRec;
  float mx = neg_inf();
  for (int i = i0 + d; i < i1; i += kHeadDim) mx = fmaxf(mx, rec[(size_t)i * stride + kHeadDim]);
  mx = wave_max(mx);
  if ((d & 63) == 0) wmax[d >> 6] = mx;
  __syncthreads();
  mx = fmaxf(wmax[0], wmax[1]);
  float num = 0.f, den = 0.f;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) {
    const float* r = rec + (size_t)i * stride;
    const float w = fast_exp2(r[kHeadDim] - mx);
    num = __builtin_fmaf(w, r[d], num);
    den = __builtin_fmaf(w, r[kHeadDim + 1], den);
  }
  *dst = num / den;
}

static int decode_items(int H, int64_t kept, bool ragged, int chunk) {
  if (ragged) return (int)((kept + chunk - 1) / chunk) + H;
  const int64_t b = kept / H;
  return H * (int)((b + chunk - 1) / chunk);
}

size_t decode_ws_bytes(int L, int H, int G, int64_t kept, bool ragged) {
  return (size_t)L * decode_items(H, kept, ragged, dec_chunk(G)) * G * kDecRec * sizeof(float);
}

hipError_t decode_launch(const void* q, const void* k, const void* v, int L, int H, int G,
                         int64_t kept, const int32_t* head_offsets, float scale, float* out,
                         void* ws, hipStream_t st) {
  const int chunk = dec_chunk(G);
  const int items = decode_items(H, kept, head_offsets != nullptr, chunk);
  const long long blocks = (long long)L * items;
  if (blocks > 0x7fffffffLL || (long long)L * H * G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float alpha = scale * kLog2e;
  float* part = static_cast<float*>(ws);
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const __bf16* vb = static_cast<const __bf16*>(v);
  const int kp = (int)kept;
  switch (G) {
#define KVSEL_DEC(GG, KERNEL)                                                                      \
  case GG:                                                                                          \
    hipLaunchKernelGGL(KERNEL<GG>, dim3((unsigned)blocks), dim3(kDecThreads), 0, st, qb, kb, vb,   \
                       H, kp, head_offsets, alpha, items, part);                                   \
    break;
    KVSEL_DEC(1, k_decode_stream) KVSEL_DEC(2, k_decode_stream) KVSEL_DEC(3, k_decode_stream)
    KVSEL_DEC(4, k_decode_stream) KVSEL_DEC(5, k_decode_phased) KVSEL_DEC(6, k_decode_phased)
    KVSEL_DEC(7, k_decode_phased) KVSEL_DEC(8, k_decode_phased)
#undef KVSEL_DEC
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k_decode_merge, dim3((unsigned)(L * H * G)), dim3(kHeadDim), 0, st, H, G, kp,
                     chunk, head_offsets, items, part, out);
  return hipGetLastError();
}

}  // namespace kvsel
