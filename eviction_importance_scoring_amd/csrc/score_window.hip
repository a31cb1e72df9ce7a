// Window-mode scoring, two streaming passes over K ([CriticalKV] §3.3
// Algorithm 2 steps 2-3; the row softmax runs along keys and the aggregate
// along queries, [KVzip] §3.4, so the normaliser of every row is needed
// before any key's weight).
//
// Both kernels serve R = G*W <= 128 query rows per KV head. A workgroup
// owns a range of keys of one (layer, KV head); its 4 waves split the rows
// (wave w: rows 32w..32w+31, held as MFMA operands in registers for the
// whole kernel) and all consume the same K tiles. K streams from HBM once
// per pass through a ring of kSlots LDS slots of kTile keys each, filled by
// direct global->LDS loads (global_load_lds_dwordx4): each instruction reads
// 4 whole 256-byte rows, and the 16-byte pieces of row r are stored XOR-
// swizzled by (r & 15), so the MFMA operand reads (one half row per lane)
// are free of bank conflicts. kSlots-1 tiles are in flight at any time.
// MFMA is 32x32x16 bf16 with fp32 accumulation.
//
//   pass 1 (k_win_stats): keys on the MFMA M side, rows on lanes; every lane
//     keeps an online (max, sum of 2^(x - max)) for its row over the keys.
//   pass 2 (k_win_colsum): rows on the M side, keys on lanes; every lane sums
//     2^(x - c_r) (or takes the max of x - c_r) over its 16 rows of each key,
//     then lane halves and waves are added in a fixed order through LDS.
// Tiles whose keys every window query sees (all but the last tile or two of
// a head) skip the causal mask.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kTile = 64;                     // keys per ring slot (16 KB)
constexpr int kSlots = 3;                     // ring depth (3 keeps 3 workgroups per CU)
constexpr int kSub = kTile / 32;              // 32-key MFMA sub-tiles per slot
constexpr int kLoadsPerTile = kTile * kRowBytes / (4 * 1024);   // per wave
constexpr float kNegBig = -1.0e30f;           // "no key seen yet"
[[maybe_unused]] constexpr int kNonTemporal = 2;              // cache-policy bit: K is read once per pass

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) const void* glb_ptr;

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Workgroup barrier without a memory fence: the ring's LDS-DMA writes are
// waited for explicitly (s_waitcnt vmcnt) before it, so the tiles still in
// flight are not drained.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same barrier for a wave that has written LDS with ds_write since the
// last one (pass 2's column partials and row normalisers): s_barrier by
// itself does not order LDS writes before other waves' reads after it, so
// the wave first waits for its own LDS operations (lgkmcnt(0); vmcnt and
// expcnt left at their maxima).
__device__ __forceinline__ void ring_barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for this wave's loads of tile t. Tiles are issued in order, kSlots-1
// ahead, and none past the last, so all but the last tile may leave the
// next one in flight; the last drains everything (nothing is left in flight
// when the workgroup ends).
static_assert(kSlots == 3 && kSub == 2, "wait_ring and the pass-1 folds assume 3 slots of 64 keys");
__device__ __forceinline__ void wait_ring(bool last) {
  constexpr int n = kLoadsPerTile;
  static_assert(n < 16, "vmcnt field");
  if (last) __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  else __builtin_amdgcn_s_waitcnt(n | (7 << 4) | (15 << 8));
}

// Wait until only the prologue's ring loads may still be outstanding: the
// per-lane operands loaded before them are then in registers, so the loop
// needs no wait for them (otherwise the compiler waits for every load in
// flight inside the loop).
__device__ __forceinline__ void wait_operands() {
  constexpr int n = (kSlots - 1) * kLoadsPerTile;
  static_assert(n < 16, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(n | (7 << 4) | (15 << 8));
}

// A wave's share of the ring loads: chunks [c0, c0 + cnt) of a tile's 16
// chunks of 1 KB (chunk c = key rows 4c..4c+3), cnt <= MAXC. LDS layout: row
// r at r*256, piece p at ((p ^ (r & 15)) * 16). Loads go through a buffer
// resource whose base is the tile's first key and whose size ends at key
// n-1: the lane offsets (row r = 4c + lane/16, swizzled piece) are fixed
// for the whole kernel, so issuing a tile costs no vector instructions, and
// rows past the last key are cut off by the hardware range check (those
// keys are never used) instead of being clamped.
constexpr int kChunks = kTile * kRowBytes / 1024;
static_assert(kChunks == 16, "chunk split of the ring loaders");
[[maybe_unused]] constexpr int kRawBufferWord3 = 0x00020000;  // untyped 32-bit data format
template <int MAXC>
struct RingLoader {
  uint32_t off[MAXC];
  int c0, cnt;
  __device__ __forceinline__ void init(int first, int count) {
    const int lane = threadIdx.x & 63;
    c0 = first;
    cnt = count;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int r = (first + i) * 4 + (lane >> 4);
      off[i] = (uint32_t)(r * kRowBytes + (((lane & 15) ^ (r & 15)) << 4));
    }
  }
  // key0 < n; n * kRowBytes < 2^31 (window_applicable)
  __device__ __forceinline__ void issue(const __bf16* kh, int key0, int n, unsigned char* slot) const {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer resources exist only in the device pass
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(kh + (size_t)key0 * kHeadDim), 0, (n - key0) * kRowBytes, kRawBufferWord3);
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
      if (i < cnt)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(slot + (c0 + i) * 1024), 16, off[i], 0, 0,
                                                 kNonTemporal);
#endif
  }
};

// Pass 2 loads the ring like pass 1 (every wave a quarter of each tile).
// Wave 0 also stores the finished sums, which share vmcnt with its loads;
// wait_ring stays correct (loads return in order, so at most kLoadsPerTile
// outstanding operations leave no load of an older tile in flight) and may
// also wait for a store issued after the newest tile's loads.
// Before the pass-2 loop every load of the prologue is waited for: with
// stores in the loop the compiler otherwise re-waits for all loads in
// flight (vmcnt(0)) at the operands' first use inside the loop.
__device__ __forceinline__ void wait_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// MFMA operand (step s) of key row r (0..kTile-1) for lane half hf.
__device__ __forceinline__ bf16x8 tile_op(const unsigned char* slot, int r, int hf, int s) {
  return ld16(slot + r * kRowBytes + (((hf * 8 + s) ^ (r & 15)) << 4));
}

struct RingShared {
  unsigned char ring[kSlots][kTile * kRowBytes];
};

// Pass 2 keeps its column partials in the same LDS object as the ring: with
// two objects the compiler waits for every direct-to-LDS load in flight
// before each LDS read, which would drain the ring every tile.
struct ColsumShared {
  unsigned char ring[kSlots][kTile * kRowBytes];
  float colbuf[2][4][kTile];
};

// ---------------------------------------------------------------- pass 1 ----
// grid (blocks, H, L); keys [b*kpb, min(n, (b+1)*kpb)); part[lh][b][row].
//
// Software pipelined: the MFMAs of tile t are interleaved (one step at a
// time) with folding tile t-1 into the running (max, sum), two accumulator
// sets in turn, so the vector work hides behind the matrix work and the
// tile loads. A tile's exponentials use the running offset m from before
// the tile; only when the tile's partial sum passes 2^64 (first tile of a
// row, or a large jump of its max) is the tile's max found and the sum
// redone at a new offset, which keeps the max off the per-logit path.
constexpr float kPartialLimit = 1.8446744e19f;   // 2^64

// Three workgroups per CU (LDS) need at most 168 registers a lane.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_win_stats(const __bf16* __restrict__ q,
                                                   const __bf16* __restrict__ k, int H, int R,
                                                   int W, int n, float alpha, int blocks,
                                                   int kpb, float2* __restrict__ part) {
  __shared__ __align__(16) RingShared sm;
  const int b = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const __bf16* kh = k + lh * (size_t)n * kHeadDim;
  const int j0 = b * kpb, j1 = min(n, j0 + kpb);
  const int ntiles = (j1 - j0 + kTile - 1) / kTile;

  const int row = wave * 32 + col;
  const bool active = wave * 32 < R;       // wave has rows (uniform)
  bf16x8 qb[8];
  if (row < R) load_half_row(q + (lh * R + row) * (size_t)kHeadDim, hf, qb);
  else zero_ops(qb);
  asm volatile("" ::: "memory");
  RingLoader<kLoadsPerTile> ld;
  ld.init(wave * kLoadsPerTile, kLoadsPerTile);
#pragma unroll
  for (int t = 0; t < kSlots - 1; ++t) ld.issue(kh, j0 + min(t, ntiles - 1) * kTile, n, sm.ring[t]);
  wait_operands();
  const int last = row < R ? n - W + row % W : -1;   // last key this row sees
  const int open_end = n - W;                        // every row sees keys <= this
  float m = kNegBig, s = 0.f;

  auto begin_tile = [&](int t) -> const unsigned char* {
    wait_ring(t + 1 == ntiles);
    ring_barrier();
    if (t + kSlots - 1 < ntiles)
      ld.issue(kh, j0 + (t + kSlots - 1) * kTile, n, sm.ring[(t + kSlots - 1) % kSlots]);
    // the slot's offset in an opaque vector register: keeps LDS reads from
    // moving across tiles, and each operand address is one add
    int soff = (t % kSlots) * (kTile * kRowBytes);
    asm volatile("" : "+v"(soff));
    return sm.ring[0] + soff;
  };
  auto mask = [&](f32x16 (&acc)[kSub], int t) {
    const int kt = j0 + t * kTile;
    if (kt + kTile - 1 <= open_end && kt + kTile <= j1) return;
#pragma unroll
    for (int u = 0; u < kSub; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kt + u * 32 + acc_row(i, lane);
        if (!(kk <= last && kk < j1)) acc[u][i] = -__builtin_inff();
      }
  };
  // part c (of 8) of a tile: 4 logits into the partial sum at offset m
  auto fold_part = [&](const f32x16 (&acc)[kSub], int c, float& ps) {
    const int u = c >> 2, i0 = (c & 3) * 4;
#pragma unroll
    for (int i = i0; i < i0 + 4; ++i) ps += fast_exp2(__builtin_fmaf(acc[u][i], alpha, -m));
  };
  auto fold_end = [&](const f32x16 (&acc)[kSub], float ps) {
    const float s_old = s;
    s = s_old + ps;            // unconditional: keeps the folds beside the MFMAs
    if (!(ps <= kPartialLimit)) {
      float tm = -__builtin_inff();
#pragma unroll
      for (int u = 0; u < kSub; ++u)
#pragma unroll
        for (int i = 0; i < 16; i += 2) tm = max3f(tm, acc[u][i], acc[u][i + 1]);
      const float mn = __builtin_fmaxf(m, tm * alpha);   // alpha > 0
      float sum = s_old * fast_exp2(m - mn);
#pragma unroll
      for (int u = 0; u < kSub; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(acc[u][i], alpha, -mn));
      s = sum;
      m = mn;
    }
  };
  // operand reads run one step ahead of the MFMAs that use them
  auto read_ops = [&](const unsigned char* slot, int st, bf16x8 (&o)[kSub]) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) o[u] = tile_op(slot, u * 32 + col, hf, st);
  };
  auto mfma_step = [&](const bf16x8 (&o)[kSub], int st, f32x16 (&acc)[kSub]) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) acc[u] = mfma32(o[u], qb[st], acc[u]);
  };
  auto step = [&](int t, f32x16 (&cur)[kSub], f32x16 (&prev)[kSub]) {
    const unsigned char* slot = begin_tile(t);
    if (!active) return;
    mask(prev, t - 1);
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < kSub; ++u) cur[u] = zero16();
    bf16x8 o[2][kSub];
    read_ops(slot, 0, o[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) read_ops(slot, st + 1, o[(st + 1) & 1]);
      mfma_step(o[st & 1], st, cur);
      fold_part(prev, st, ps);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" : "+v"(ps));
    fold_end(prev, ps);
  };
  auto fold_all = [&](f32x16 (&acc)[kSub], int t) {
    mask(acc, t);
    float ps = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) fold_part(acc, c, ps);
    fold_end(acc, ps);
  };

  f32x16 A[kSub], B[kSub];
  {
    const unsigned char* slot = begin_tile(0);
    if (active) {
#pragma unroll
      for (int u = 0; u < kSub; ++u) A[u] = zero16();
      bf16x8 o[2][kSub];
      read_ops(slot, 0, o[0]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st + 1 < 8) read_ops(slot, st + 1, o[(st + 1) & 1]);
        mfma_step(o[st & 1], st, A);
      }
    }
  }
  int t = 1;
  for (; t + 1 < ntiles; t += 2) {
    step(t, B, A);
    step(t + 1, A, B);
  }
  if (t < ntiles) {
    step(t, B, A);
    if (active) fold_all(B, t);
  } else if (active) {
    fold_all(A, t - 1);
  }
  // the other lane half saw the other 16 keys of every 32-key sub-tile
  const float m2 = lane_xor32(m), s2 = lane_xor32(s);
  lse_merge(m, s, m2, s2);
  if (hf == 0 && row < R) part[(lh * blocks + b) * (size_t)R + row] = make_float2(m, s);
}

// ---------------------------------------------------------------- pass 2 ----
// grid (blocks, H, L); raw[lh][key] = sum_r 2^(x - c_r), or 2^(max_r (x - c_r)).
//
// Pipelined like pass 1: while the MFMAs of tile t run, tile t-1 is folded
// into per-key partials over this wave's 32 rows and written to LDS; after
// the next barrier one wave adds the 4 waves' partials of tile t-1 in
// fixed order and stores them. Three workgroups per CU (LDS) need at most
// 168 registers a lane.
template <bool MAXAGG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_win_colsum(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, int H, int R, int W, int n,
    float alpha, const float* __restrict__ stat, int kpb, float* __restrict__ raw) {
  __shared__ __align__(16) ColsumShared sm;
  const int b = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const __bf16* kh = k + lh * (size_t)n * kHeadDim;
  const int j0 = b * kpb, j1 = min(n, j0 + kpb);
  const int ntiles = (j1 - j0 + kTile - 1) / kTile;

  const bool active = wave * 32 < R;
  bf16x8 qa[8];
  {
    const int row = wave * 32 + col;
    if (row < R) load_half_row(q + (lh * R + row) * (size_t)kHeadDim, hf, qa);
    else zero_ops(qa);
  }
  // row normaliser of each accumulator register's row (padding rows weigh 0)
  float crow[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = wave * 32 + acc_row(i, lane);
    crow[i] = r < R ? stat[lh * R + r] : __builtin_inff();
  }
  asm volatile("" ::: "memory");
  RingLoader<kLoadsPerTile> ld;
  ld.init(wave * kLoadsPerTile, kLoadsPerTile);
#pragma unroll
  for (int t = 0; t < kSlots - 1; ++t) ld.issue(kh, j0 + min(t, ntiles - 1) * kTile, n, sm.ring[t]);
  wait_all();
  const int open_end = n - W;
  const float ident = MAXAGG ? -__builtin_inff() : 0.f;

  // one wave adds the 4 waves' partials of tile tt (written before the
  // last barrier) in a fixed order. In the tile loop the LDS reads are
  // issued right after the barrier and the sum is stored after the tile's
  // MFMAs, so the read latency stays off the wave's path to the next
  // barrier; the buffer is written again only after that barrier.
  float rp[4];
  auto reduce_read = [&](int tt) {
    if (tid >= kTile) return;
    const float* cb = &sm.colbuf[tt & 1][0][0];
#pragma unroll
    for (int w = 0; w < 4; ++w) rp[w] = cb[w * kTile + tid];
  };
  auto reduce_store = [&](int tt) {
    if (tid >= kTile) return;
    const int key = j0 + tt * kTile + tid;
    float v;
    if (MAXAGG) v = fast_exp2(__builtin_fmaxf(__builtin_fmaxf(rp[0], rp[1]), __builtin_fmaxf(rp[2], rp[3])));
    else v = (rp[0] + rp[1]) + (rp[2] + rp[3]);
    if (key < j1) raw[lh * n + key] = v;
  };
  auto reduce = [&](int tt) {
    reduce_read(tt);
    reduce_store(tt);
  };
  // tile t-2's sums are read after the barrier and stored by wave 0 after the MFMAs
  auto begin_tile = [&](int t) -> const unsigned char* {
    wait_ring(t + 1 == ntiles);
    ring_barrier_lds();
    if (t >= 2) reduce_read(t - 2);
    if (t + kSlots - 1 < ntiles)
      ld.issue(kh, j0 + (t + kSlots - 1) * kTile, n, sm.ring[(t + kSlots - 1) % kSlots]);
    // the slot's offset in an opaque vector register: keeps LDS reads from
    // moving across tiles, and each operand address is one add
    int soff = (t % kSlots) * (kTile * kRowBytes);
    asm volatile("" : "+v"(soff));
    return sm.ring[0] + soff;
  };
  // window rows hide keys past n - W + (row % W)
  auto mask = [&](f32x16 (&acc)[kSub], int t) {
    const int kt = j0 + t * kTile;
    if (kt + kTile - 1 <= open_end) return;
    // opaque row base: keeps the 16 row % W values from being hoisted out
    // of the tile loop into registers (this branch runs on edge tiles only)
    int rbase = wave * 32 + 4 * hf;
    asm volatile("" : "+v"(rbase));
#pragma unroll
    for (int nt = 0; nt < kSub; ++nt) {
      const int key = kt + nt * 32 + col;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key > n - W + (rbase + 8 * (i >> 2) + (i & 3)) % W) acc[nt][i] = -__builtin_inff();
    }
  };
  // part c (of 8): 4 rows of key set nt = c / 4 into the per-key partial
  auto fold_part = [&](const f32x16 (&acc)[kSub], int c, float (&pa)[kSub]) {
    const int nt = c >> 2, i0 = (c & 3) * 4;
#pragma unroll
    for (int i = i0; i < i0 + 4; ++i) {
      const float x = __builtin_fmaf(acc[nt][i], alpha, -crow[i]);
      if (MAXAGG) pa[nt] = __builtin_fmaxf(pa[nt], x);
      else pa[nt] += fast_exp2(x);
    }
  };
  // this wave's per-key partials of tile tt (other lane half: other 16 rows)
  auto fold_end = [&](const float (&pa)[kSub], int tt) {
#pragma unroll
    for (int nt = 0; nt < kSub; ++nt) {
      const float o = lane_xor32(pa[nt]);
      if (hf == 0)
        sm.colbuf[tt & 1][wave][nt * 32 + col] = MAXAGG ? __builtin_fmaxf(pa[nt], o) : pa[nt] + o;
    }
  };
  // operand reads run one step ahead of the MFMAs that use them
  auto read_ops = [&](const unsigned char* slot, int st, bf16x8 (&o)[kSub]) {
#pragma unroll
    for (int nt = 0; nt < kSub; ++nt) o[nt] = tile_op(slot, nt * 32 + col, hf, st);
  };
  auto mfma_step = [&](const bf16x8 (&o)[kSub], int st, f32x16 (&acc)[kSub]) {
#pragma unroll
    for (int nt = 0; nt < kSub; ++nt) acc[nt] = mfma32(qa[st], o[nt], acc[nt]);
  };
  // tile t into cur while tile t-1 (prev) is folded; tile t-2 is reduced
  auto step = [&](int t, f32x16 (&cur)[kSub], f32x16 (&prev)[kSub]) {
    const unsigned char* slot = begin_tile(t);
    float pa[kSub] = {ident, ident};
    if (active) {
      mask(prev, t - 1);
#pragma unroll
      for (int nt = 0; nt < kSub; ++nt) cur[nt] = zero16();
      bf16x8 o[2][kSub];
      read_ops(slot, 0, o[0]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st + 1 < 8) read_ops(slot, st + 1, o[(st + 1) & 1]);
        mfma_step(o[st & 1], st, cur);
        fold_part(prev, st, pa);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t >= 2) reduce_store(t - 2);
    fold_end(pa, t - 1);
  };

  f32x16 A[kSub], B[kSub];
  {
    const unsigned char* slot = begin_tile(0);
    if (active) {
#pragma unroll
      for (int nt = 0; nt < kSub; ++nt) A[nt] = zero16();
      bf16x8 o[2][kSub];
      read_ops(slot, 0, o[0]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st + 1 < 8) read_ops(slot, st + 1, o[(st + 1) & 1]);
        mfma_step(o[st & 1], st, A);
      }
    }
  }
  int t = 1;
  for (; t + 1 < ntiles; t += 2) {
    step(t, B, A);
    step(t + 1, A, B);
  }
  // the last tile's accumulators: B if one more step runs, else A
  auto finish = [&](f32x16 (&acc)[kSub], int tl) {
    ring_barrier_lds();            // partials of tile tl-1 are in LDS
    if (tl >= 1) reduce(tl - 1);
    float pa[kSub] = {ident, ident};
    if (active) {
      mask(acc, tl);
#pragma unroll
      for (int c = 0; c < 8; ++c) fold_part(acc, c, pa);
    }
    fold_end(pa, tl);
    ring_barrier_lds();
    reduce(tl);
  };
  if (t < ntiles) {
    step(t, B, A);
    finish(B, t);
  } else {
    finish(A, t - 1);
  }
}

// ------------------------------------------------------------------ host ----

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// The ring's buffer resources address a head's K with 31-bit byte offsets.
bool window_applicable(const ScorePlan& p) {
  return p.causal && p.R <= 128 && (long long)p.n * kRowBytes <= 0x7fffffffLL;
}

static int win_keys_per_block(const ScorePlan& p) {
  // >= ~2048 workgroups per pass when the cache is large; kTile granularity
  const long long heads = (long long)p.L * p.H;
  long long kpb = ((long long)p.n * heads + 2047) / 2048;
  kpb = (kpb + kTile - 1) / kTile * kTile;
  if (kpb < 2 * kTile) kpb = 2 * kTile;
  if (kpb > 4096) kpb = 4096;
  return (int)kpb;
}

void window_plan(const ScorePlan& p, WindowLayout* o) {
  const int kpb = win_keys_per_block(p);
  o->kpb = kpb;
  o->blocks = (p.n + kpb - 1) / kpb;
  const size_t LH = (size_t)p.L * p.H;
  o->part_off = 0;
  o->stat_off = al256(LH * o->blocks * p.R * sizeof(float2));
  o->raw_off = o->stat_off + al256(LH * p.R * sizeof(float));
  o->bytes = o->raw_off + (p.need_raw_tmp ? al256(LH * p.n * sizeof(float)) : 0);
}

hipError_t combine_launch(const float2* part, int L, int H, int R, int splits, float* stat,
                          hipStream_t st);

hipError_t window_launch(const ScorePlan& p, const WindowLayout& o, const void* q, const void* k,
                         float* scores, float* raw, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  float2* part = reinterpret_cast<float2*>(w + o.part_off);
  float* stat = reinterpret_cast<float*>(w + o.stat_off);
  float* rawbuf = raw ? raw : reinterpret_cast<float*>(w + o.raw_off);
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const float alpha = p.scale * kLog2e;
  dim3 grid(o.blocks, p.H, p.L);
  // each launch's status is checked before the next one depends on it
  hipLaunchKernelGGL(k_win_stats, grid, dim3(256), 0, st, qb, kb, p.H, p.R, p.W, p.n, alpha,
                     o.blocks, o.kpb, part);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = combine_launch(part, p.L, p.H, p.R, o.blocks, stat, st);
  if (e != hipSuccess) return e;
  if (p.max_agg)
    hipLaunchKernelGGL(k_win_colsum<true>, grid, dim3(256), 0, st, qb, kb, p.H, p.R, p.W, p.n,
                       alpha, stat, o.kpb, rawbuf);
  else
    hipLaunchKernelGGL(k_win_colsum<false>, grid, dim3(256), 0, st, qb, kb, p.H, p.R, p.W, p.n,
                       alpha, stat, o.kpb, rawbuf);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return pool_launch(rawbuf, p.L, p.H, p.n, p.n_cand, p.pool / 2, scores, st);
}

}  // namespace kvsel
