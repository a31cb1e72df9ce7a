// Compaction of the kept K/V rows from the un-replicated cache ([KVzip] §4.2:
// eviction acts on the original H_kv heads, before GQA replication).
// Plain row copies; every kept row of K and V is read once and written once.
//
// The copy runs over the flat (packed row, 16-byte piece) items of a layer.
// A thread takes kItems items a block-width apart, so each access of a
// wave is one contiguous 1 KB run and every thread has 2 * kItems loads in
// flight (K and V) after its index loads. Data is streamed with
// non-temporal loads and stores: it is touched once here.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kItems = 4;
constexpr int kCompactThreads = 256;

// grid (ceil(kept * vecs / (kItems * 256)), L), block 256.
// VECS = 16-byte pieces per row when known at compile time (d = 128), else 0.
template <int VECS>
__global__ __launch_bounds__(256) void k_compact(const u32x4* __restrict__ k,
                                                 const u32x4* __restrict__ v, int H, int n,
                                                 int vecs_rt, const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ offs,
                                                 int64_t kept, int64_t per_head,
                                                 u32x4* __restrict__ ko, u32x4* __restrict__ vo) {
  const int vecs = VECS ? VECS : vecs_rt;
  const int l = blockIdx.y;
  const int64_t total = kept * vecs;
  const int64_t base = (int64_t)blockIdx.x * kItems * kCompactThreads + threadIdx.x;
  const int32_t* il = idx + (size_t)l * kept;
  const int32_t* o = offs ? offs + (size_t)l * (H + 1) : nullptr;
  // packed rows: only those before the last head's end (clamped into the
  // layer) are written; a budget-vector row may end well before `kept`
  int64_t lim = total;
  if (o) {
    const int64_t e = o[H];
    lim = (e < 0 ? 0 : (e > kept ? kept : e)) * vecs;
  }
  if (base >= lim) return;   // no barriers below

  int64_t row[kItems];
  int c[kItems];
  int32_t pos[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t item = base + (int64_t)j * kCompactThreads;
    row[j] = item / vecs;
    c[j] = (int)(item - row[j] * vecs);
    pos[j] = item < lim ? il[row[j]] : -1;
  }
  u32x4 kv[kItems], vv[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    int h;
    if (o) {   // head owning this packed row: last h with offs[h] <= row
      int lo = 0, hi = H - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (o[mid] <= row[j]) lo = mid; else hi = mid - 1;
      }
      h = lo;
    } else {
      h = (int)(row[j] / per_head);
    }
    kv[j] = vv[j] = u32x4{0u, 0u, 0u, 0u};
    if (pos[j] >= 0 && pos[j] < n) {
      const size_t src = (((size_t)l * H + h) * n + pos[j]) * vecs + c[j];
      kv[j] = __builtin_nontemporal_load(k + src);
      vv[j] = __builtin_nontemporal_load(v + src);
    }
  }
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t item = base + (int64_t)j * kCompactThreads;
    if (item < lim) {
      const size_t dst = (size_t)l * total + item;
      __builtin_nontemporal_store(kv[j], ko + dst);
      __builtin_nontemporal_store(vv[j], vo + dst);
    }
  }
}

hipError_t compact_launch(const void* k, const void* v, int L, int H, int d, int n,
                          const int32_t* idx, const int32_t* head_offsets, int64_t kept,
                          void* k_out, void* v_out, hipStream_t st) {
  const int vecs = d * 2 / 16;
  const int64_t total = kept * vecs;
  const int64_t per_block = (int64_t)kItems * kCompactThreads;
  const int64_t blocks = (total + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int64_t per_head = head_offsets ? 0 : kept / H;
  const dim3 grid((unsigned)blocks, L);
  const u32x4* kk = static_cast<const u32x4*>(k);
  const u32x4* vv = static_cast<const u32x4*>(v);
  u32x4* ko = static_cast<u32x4*>(k_out);
  u32x4* vo = static_cast<u32x4*>(v_out);
  if (vecs == kRowBytes / 16)
    hipLaunchKernelGGL(k_compact<kRowBytes / 16>, grid, dim3(kCompactThreads), 0, st, kk, vv, H,
                       n, vecs, idx, head_offsets, kept, per_head, ko, vo);
  else
    hipLaunchKernelGGL(k_compact<0>, grid, dim3(kCompactThreads), 0, st, kk, vv, H, n, vecs, idx,
                       head_offsets, kept, per_head, ko, vo);
  return hipGetLastError();
}

}  // namespace kvsel
