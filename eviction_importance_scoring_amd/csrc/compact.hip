// Compaction of the kept K/V rows from the un-replicated cache ([KVzip] §4.2:
// eviction acts on the original H_kv heads, before GQA replication).
// Plain 16-byte row copies; every kept row of K and V is read once and
// written once.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

// grid (ceil(kept*vecs/256), L), block 256; vecs = 16-byte pieces per row.
__global__ __launch_bounds__(256) void k_compact(const u32x4* __restrict__ k,
                                                 const u32x4* __restrict__ v, int H, int n,
                                                 int vecs, const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ offs,
                                                 int64_t kept, int64_t per_head,
                                                 u32x4* __restrict__ ko, u32x4* __restrict__ vo) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int l = blockIdx.y;
  const int64_t row = t / vecs;
  const int c = (int)(t - row * vecs);
  if (row >= kept) return;
  int h;
  if (offs) {  // head owning this packed row: last h with offs[h] <= row
    const int32_t* o = offs + (size_t)l * (H + 1);
    int lo = 0, hi = H - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (o[mid] <= row) lo = mid; else hi = mid - 1;
    }
    h = lo;
  } else {
    h = (int)(row / per_head);
  }
  const int32_t pos = idx[(size_t)l * kept + row];
  u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
  if (pos >= 0 && pos < n) {
    const size_t src = (((size_t)l * H + h) * n + pos) * vecs + c;
    kv = k[src];
    vv = v[src];
  }
  const size_t dst = ((size_t)l * kept + row) * vecs + c;
  ko[dst] = kv;
  vo[dst] = vv;
}

hipError_t compact_launch(const void* k, const void* v, int L, int H, int d, int n,
                          const int32_t* idx, const int32_t* head_offsets, int64_t kept,
                          void* k_out, void* v_out, hipStream_t st) {
  const int vecs = d * 2 / 16;
  const int64_t total = kept * vecs;
  const int64_t per_head = head_offsets ? 0 : kept / H;
  hipLaunchKernelGGL(k_compact, dim3((unsigned)((total + 255) / 256), L), dim3(256), 0, st,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), H, n, vecs,
                     idx, head_offsets, kept, per_head, static_cast<u32x4*>(k_out),
                     static_cast<u32x4*>(v_out));
  return hipGetLastError();
}

}  // namespace kvsel
