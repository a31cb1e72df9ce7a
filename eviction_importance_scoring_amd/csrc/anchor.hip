// AnchorKV's anchor stage ([AnchorKV] §3.1-3.2).
//
// Anchor selection is the two-stage selection of select.hip with stage 2
// keyed by uniform draws: (score * 0 + 1) * draw is the draw itself, so
// stage 1 takes floor(rho * (k - W)) positions by pooled score and stage 2
// the largest draws among the rest (uniform sampling without replacement);
// the W recent positions are the window. See kvsel_anchor_select in api.hip.
//
// Assignment: every vector of a head goes to the anchor of largest cosine
// similarity, kept as the anchor's slot and gamma = <x, a> / <a, a>:
//   k_anchor_gather  the head's anchor rows into a contiguous [kpad][128]
//                    block (zero rows past k) and 1/|a| per slot (0 for a
//                    zero or padding anchor, which is never chosen)
//   k_anchor_assign  4-wave workgroups, 256 vectors of one (layer, head),
//                    each wave 64 of them in registers as MFMA operands;
//                    the anchor block streams through the LDS ring of
//                    kvsel_ring.h in 64-row tiles. Per tile the MFMA gives
//                    <x, a> for 64 anchors x 64 vectors; each lane keeps,
//                    per vector, the best <x, a> / |a| (the cosine up to
//                    the vector's own norm) over its anchor rows, visited
//                    in increasing slot order with a strict compare, so the
//                    lower slot wins ties; the two lane halves merge the
//                    same way.
//   k_anchor_self    every anchor position to its own slot, gamma 1.
// Dot products are fp32 sums of exact bf16 products.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"
#include "kvsel_ring.h"

namespace kvsel {

constexpr int kAsWaves = 4;
constexpr int kMaxAnchorPad = 2048;        // anchors per head (LDS for their 1/|a|)
constexpr int kAsBlock = kAsWaves * 64;    // vectors per workgroup
using AsLoader = RingLoader<kAsWaves>;
constexpr int kAsLoads = AsLoader::kLoads;

// max of three floats, a quiet NaN operand ignored (IEEE-mode v_max3_f32);
// as asm so that no canonicalising max is put before each operand.
__device__ __forceinline__ float max3_nan_skip(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// a.lo * a'.lo + a.hi * a'.hi + c over bf16 pairs, in fp32
typedef __bf16 bf16x2_a __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_a, a), __builtin_bit_cast(bf16x2_a, b), c,
                                         false);
}

int anchor_kpad(int k) { return (k + gTile - 1) / gTile * gTile; }

// A slot's score is <x, a> * scale. The scale is 1/|a|, or NaN for a zero
// or padding anchor: its score compares greater than nothing, so it is
// never chosen (and a real anchor's score is the same single rounding of
// <x, a> / |a| as before).
__device__ __forceinline__ float score_scale(float r) {
  return r > 0.f ? r : __builtin_nanf("");
}

// grid (kpad, L*H), block 64: one anchor row per workgroup, its 16-byte
// pieces on 16 lanes (the other 48 idle; the gather is tiny)
__global__ __launch_bounds__(64) void k_anchor_gather(const u32x4* __restrict__ x,
                                                      const int32_t* __restrict__ anchors, int n,
                                                      int k, int kpad, u32x4* __restrict__ arows,
                                                      float* __restrict__ rinv) {
  const int s = blockIdx.x;
  const size_t lh = blockIdx.y;
  const int lane = threadIdx.x;
  constexpr int kPieces = kRowBytes / 16;
  int pos = -1;
  if (s < k) pos = anchors[lh * k + s];
  const bool valid = pos >= 0 && pos < n;
  float ss = 0.f;
  if (lane < kPieces) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (valid) v = x[(lh * n + pos) * kPieces + lane];
    arows[((size_t)lh * kpad + s) * kPieces + lane] = v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xFFFF0000u);
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) rinv[lh * kpad + s] = ss > 0.f ? 1.0f / __builtin_sqrtf(ss) : 0.f;
}

// 1-D grid of key_blocks * H * L workgroups, block 256.
__global__ __launch_bounds__(256, 2) void k_anchor_assign(const __bf16* __restrict__ x,
                                                          const __bf16* __restrict__ arows,
                                                          const float* __restrict__ rinv_g, int H,
                                                          int n, int kpad, int key_blocks,
                                                          int32_t* __restrict__ slot_out,
                                                          float* __restrict__ gamma_out) {
  __shared__ __align__(16) unsigned char ring[gSlots][gRowsBytes];
  __shared__ __align__(16) float rinv[kMaxAnchorPad];   // score_scale per slot
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = id % key_blocks;
  id /= key_blocks;
  const int h = id % H, l = id / H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const int ntiles = kpad / gTile;
  const __bf16* ah = arows + lh * (size_t)kpad * kHeadDim;

  const int key0 = kb * kAsBlock + wave * 64;
  bf16x8 vop[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = key0 + nt * 32 + col;
    if (key < n) load_half_row(x + (lh * n + key) * (size_t)kHeadDim, hf, vop[nt]);
    else zero_ops(vop[nt]);
  }
  for (int s = threadIdx.x; s < kpad; s += 256) rinv[s] = score_scale(rinv_g[lh * kpad + s]);
  AsLoader ld;
  ld.init(kHeadDim);
  auto issue = [&](int t, int slot) { ld.issue(ah, t * gTile, kpad, kHeadDim, ring[slot]); };
  // the rinv stores and the operand loads complete before the ring starts
  __syncthreads();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < gSlots - 1; ++t) issue(min(t, ntiles - 1), t);

  const bool any_key = key0 < n;
  // packed scores as in k_anchor_assign_res: <x, a> / |a| + cx, the low 4
  // bits replaced by 15 - (accumulator row); best packed value per vector
  // and its 32-slot half-tile
  float best[2] = {neg_inf(), neg_inf()};
  int bu[2] = {0, 0};
  float cx[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float ss = 0.f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const u32x4 w = __builtin_bit_cast(u32x4, vop[nt][s8]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = bf16_dot2(w[e], w[e], ss);
    }
    ss += __shfl_xor(ss, 32);   // the other half row
    cx[nt] = __builtin_sqrtf(ss) + 0x1p-100f;
  }

  auto begin_tile = [&](int t) -> const unsigned char* {
    gen_wait_tile<kAsLoads>(t, ntiles);
    gen_barrier();
    if (t + gSlots - 1 < ntiles) issue(t + gSlots - 1, (t + gSlots - 1) % gSlots);
    int soff = (t % gSlots) * gRowsBytes;   // opaque: LDS reads stay inside the tile
    asm volatile("" : "+v"(soff));
    return ring[0] + soff;
  };
  for (int t = 0; t < ntiles; ++t) {
    const unsigned char* slot = begin_tile(t);
    if (!any_key) continue;
    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();
    bf16x8 a[2][2];
    read_step(slot, col, hf, 0, a[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) read_step(slot, col, hf, st + 1, a[(st + 1) & 1]);
      tile_step(a[st & 1], vop, st, acc);
    }
    // half-tile mt of tile t: rows 4j..4j+3 of an accumulator are
    // consecutive slots (one 16-byte read of their scales)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float mx[2] = {neg_inf(), neg_inf()};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 r4 = *reinterpret_cast<const f32x4*>(&rinv[t * gTile + mt * 32 + acc_row(4 * j, lane)]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sc = __builtin_fmaf(acc[mt][nt][4 * j + e], r4[e], cx[nt]);
            p[e] = __uint_as_float((__float_as_uint(sc) & ~15u) | (uint32_t)(15 - (4 * j + e)));
          }
          mx[nt] = max3_nan_skip(mx[nt], p[0], p[1]);
          mx[nt] = max3_nan_skip(mx[nt], p[2], p[3]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (mx[nt] > best[nt]) {
          best[nt] = mx[nt];
          bu[nt] = 2 * t + mt;
        }
    }
  }
  gen_wait<0>();
  if (!any_key) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const bool found = best[nt] > neg_inf();
    const int i = 15 - (int)(__float_as_uint(best[nt]) & 15u);
    int bslot = found ? bu[nt] * 32 + 8 * (i >> 2) + 4 * hf + (i & 3) : 0;
    // the other lane half holds the other 16 anchor rows of every block
    const float ob = __shfl_xor(best[nt], 32);
    const int os = __shfl_xor(bslot, 32);
    if (ob > best[nt] || (ob == best[nt] && os < bslot)) {
      best[nt] = ob;
      bslot = os;
    }
    const int key = key0 + nt * 32 + col;
    if (hf == 0 && key < n) {
      // <x, a> / <a, a> = (<x, a> / |a|) / |a|; no valid anchor: 0
      const float sc = __uint_as_float(__float_as_uint(best[nt]) & ~15u) - cx[nt];
      slot_out[lh * n + key] = bslot;
      gamma_out[lh * n + key] = best[nt] > neg_inf() ? sc * rinv[bslot] : 0.f;
    }
  }
}

// Up to kResAnchors anchors per head: the whole anchor block stays in LDS
// (filled once by direct-to-LDS loads, swizzled like a ring slot) and a
// workgroup streams kResBlocks blocks of 256 vectors of its head through
// it, the next block's vectors loading into registers while the current
// block is compared against every anchor.
constexpr int kResAnchors = 256;            // 64 KB of anchor rows
constexpr int kResBlocks = 16;              // vector blocks per workgroup

// 1-D grid of groups * H * L workgroups (groups = ceil(key_blocks /
// kResBlocks)), block 256.
__global__ __launch_bounds__(256, 2) void k_anchor_assign_res(const __bf16* __restrict__ x,
                                                              const __bf16* __restrict__ arows,
                                                              const float* __restrict__ rinv_g,
                                                              int H, int n, int kpad,
                                                              int key_blocks, int groups,
                                                              int32_t* __restrict__ slot_out,
                                                              float* __restrict__ gamma_out) {
  __shared__ __align__(16) unsigned char abuf[kResAnchors / gTile][gRowsBytes];
  __shared__ __align__(16) float rinv[kResAnchors];   // score_scale per slot
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = id % groups;
  id /= groups;
  const int h = id % H, l = id / H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const int ntiles = kpad / gTile;
  const int b0 = grp * kResBlocks, b1 = min(key_blocks, b0 + kResBlocks);

  // every anchor tile into LDS once
  {
    AsLoader ld;
    ld.init(kHeadDim);
    const __bf16* ah = arows + lh * (size_t)kpad * kHeadDim;
    for (int t = 0; t < ntiles; ++t) ld.issue(ah, t * gTile, kpad, kHeadDim, abuf[t]);
  }
  for (int s = threadIdx.x; s < kpad; s += 256) rinv[s] = score_scale(rinv_g[lh * kpad + s]);
  auto load_vecs = [&](int b, bf16x8 (&v)[2][8]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int key = b * kAsBlock + wave * 64 + nt * 32 + col;
      if (key < n) load_half_row(x + (lh * n + key) * (size_t)kHeadDim, hf, v[nt]);
      else zero_ops(v[nt]);
    }
  };
  bf16x8 vcur[2][8], vnext[2][8];
  load_vecs(b0, vcur);
  __syncthreads();   // the anchors, their table and the first vectors are in place

  // Half-tile u covers anchor slots [32u, 32u + 32): its 16 MFMAs (8 head-
  // dim steps x 2 vector sets) run while the argmax of half-tile u-1 is
  // done in eight parts between them, two accumulator pairs in turn.
  const int nh = 2 * ntiles;
  auto half_op = [&](int u, int st) -> bf16x8 {
    return gen_op(abuf[u >> 1], (u & 1) * 32 + col, hf, st);
  };
  // Scores are compared as packed values: the score plus an offset c >= |x|
  // (so the value is not negative), with its low 4 mantissa bits replaced by
  // 15 - i for the lane's accumulator row i of the half-tile. Among equal
  // scores the lower slot (lower i) then holds the larger value, a half-tile
  // needs one max per two pairs instead of a compare and two selects per
  // pair, and half-tiles are visited in increasing order with a strict
  // compare. The truncated bits move a score by less than 2^-19 of 2|x|.
  float best[2];   // best packed value so far
  int bu[2];       // its half-tile
  float mx[2];     // packed maximum of the current half-tile
  float cx[2];     // offset: |x| (plus 2^-100, so a zero vector's values stay normal)
  // the four scales of rows 4j..4j+3 of half-tile u (consecutive slots)
  auto scales = [&](int u, int j) -> f32x4 {
    return *reinterpret_cast<const f32x4*>(&rinv[u * 32 + acc_row(4 * j, lane)]);
  };
  // part c of the argmax of half-tile u: rows i = 4j + e (e < 4) of vector
  // set c % 2, j = c / 2; row i is slot 32u + 8j + 4hf + e
  auto arg_part = [&](int u, const f32x16 (&acc)[2], int c, const f32x4& r4) {
    const int j = c >> 1, nt = c & 1;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sc = __builtin_fmaf(acc[nt][4 * j + e], r4[e], cx[nt]);
      p[e] = __uint_as_float((__float_as_uint(sc) & ~15u) | (uint32_t)(15 - (4 * j + e)));
    }
    if (j == 0) mx[nt] = neg_inf();
    mx[nt] = max3_nan_skip(mx[nt], p[0], p[1]);
    mx[nt] = max3_nan_skip(mx[nt], p[2], p[3]);
    if (j == 3 && mx[nt] > best[nt]) {
      best[nt] = mx[nt];
      bu[nt] = u;
    }
  };
  // MFMAs of half-tile u into cur, argmax of half-tile u-1 from prev
  // The scales of the argmax are read one part ahead: r4n holds those of
  // the next part, across half-tiles too (part 0 of half-tile u is read
  // during the last part of half-tile u-1's argmax).
  f32x4 r4n;
  auto half = [&](int u, f32x16 (&cur)[2], const f32x16 (&prev)[2]) {
    bf16x8 op[2];
    f32x4 r4;
    op[0] = half_op(u, 0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) op[(st + 1) & 1] = half_op(u, st + 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        cur[nt] = mfma32(op[st & 1], vcur[nt][st], st == 0 ? zero16() : cur[nt]);
      if ((st & 1) == 0) {   // shared by both vector sets
        r4 = r4n;
        r4n = st < 6 ? scales(u - 1, (st >> 1) + 1) : scales(u, 0);
      }
      arg_part(u - 1, prev, st, r4);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int b = b0; b < b1; ++b) {
    if (b + 1 < b1) load_vecs(b + 1, vnext);   // in flight during this block
    const int key0 = b * kAsBlock + wave * 64;
    best[0] = best[1] = neg_inf();
    bu[0] = bu[1] = 0;
    if (key0 < n) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float ss = 0.f;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const u32x4 w = __builtin_bit_cast(u32x4, vcur[nt][s8]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = bf16_dot2(w[e], w[e], ss);
        }
        ss += __shfl_xor(ss, 32);   // the other half row
        cx[nt] = __builtin_sqrtf(ss) + 0x1p-100f;
      }
      f32x16 A[2], B[2];
      {
        bf16x8 op[2];
        op[0] = half_op(0, 0);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          if (st + 1 < 8) op[(st + 1) & 1] = half_op(0, st + 1);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            A[nt] = mfma32(op[st & 1], vcur[nt][st], st == 0 ? zero16() : A[nt]);
        }
        r4n = scales(0, 0);
      }
      int u = 1;
      for (; u + 1 < nh; u += 2) {
        half(u, B, A);
        half(u + 1, A, B);
      }
      half(u, B, A);   // nh is even: the last half-tile is odd
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 r4 = scales(u, j);
        arg_part(u, B, 2 * j, r4);
        arg_part(u, B, 2 * j + 1, r4);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bool found = best[nt] > neg_inf();
        const int i = 15 - (int)(__float_as_uint(best[nt]) & 15u);
        int bslot = found ? bu[nt] * 32 + 8 * (i >> 2) + 4 * hf + (i & 3) : 0;
        // the other lane half holds the other 16 rows of every half-tile
        const float ob = __shfl_xor(best[nt], 32);
        const int os = __shfl_xor(bslot, 32);
        if (ob > best[nt] || (ob == best[nt] && os < bslot)) {
          best[nt] = ob;
          bslot = os;
        }
        const int key = key0 + nt * 32 + col;
        if (hf == 0 && key < n) {
          // <x, a> / <a, a> = (<x, a> / |a|) / |a|; no valid anchor: 0
          const float sc = __uint_as_float(__float_as_uint(best[nt]) & ~15u) - cx[nt];
          slot_out[lh * n + key] = bslot;
          gamma_out[lh * n + key] = best[nt] > neg_inf() ? sc * rinv[bslot] : 0.f;
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) vcur[nt][s8] = vnext[nt][s8];
  }
}

// grid (ceil(k/256), L*H): anchor positions to their own slot
__global__ __launch_bounds__(256) void k_anchor_self(const int32_t* __restrict__ anchors, int n,
                                                     int k, int32_t* __restrict__ slot_out,
                                                     float* __restrict__ gamma_out) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  const size_t lh = blockIdx.y;
  if (s >= k) return;
  const int pos = anchors[lh * k + s];
  if (pos < 0 || pos >= n) return;
  slot_out[lh * n + pos] = s;
  gamma_out[lh * n + pos] = 1.0f;
}

size_t anchor_ws_bytes(int L, int H, int k) {
  const size_t kpad = anchor_kpad(k);
  const size_t rows = ((size_t)L * H * kpad * kRowBytes + 255) & ~size_t(255);
  return rows + (size_t)L * H * kpad * sizeof(float);
}

hipError_t anchor_assign_launch(const void* x, const int32_t* anchors, int L, int H, int n, int k,
                                int32_t* slot, float* gamma, void* ws, hipStream_t st) {
  const int kpad = anchor_kpad(k);
  const size_t LH = (size_t)L * H;
  char* w = static_cast<char*>(ws);
  u32x4* arows = reinterpret_cast<u32x4*>(w);
  float* rinv = reinterpret_cast<float*>(w + ((LH * kpad * kRowBytes + 255) & ~size_t(255)));
  const int key_blocks = (n + kAsBlock - 1) / kAsBlock;
  const long long blocks = (long long)key_blocks * H * L;
  if (blocks > 0x7fffffffLL || LH > 65535u) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_anchor_gather, dim3(kpad, (unsigned)LH), dim3(64), 0, st,
                     static_cast<const u32x4*>(x), anchors, n, k, kpad, arows, rinv);
  if (kpad <= kResAnchors) {
    const int groups = (key_blocks + kResBlocks - 1) / kResBlocks;
    hipLaunchKernelGGL(k_anchor_assign_res, dim3((unsigned)((long long)groups * H * L)), dim3(256),
                       0, st, static_cast<const __bf16*>(x), reinterpret_cast<const __bf16*>(arows),
                       rinv, H, n, kpad, key_blocks, groups, slot, gamma);
  } else {
    hipLaunchKernelGGL(k_anchor_assign, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const __bf16*>(x), reinterpret_cast<const __bf16*>(arows), rinv,
                       H, n, kpad, key_blocks, slot, gamma);
  }
  hipLaunchKernelGGL(k_anchor_self, dim3((k + 255) / 256, (unsigned)LH), dim3(256), 0, st, anchors,
                     n, k, slot, gamma);
  return hipGetLastError();
}

}  // namespace kvsel
