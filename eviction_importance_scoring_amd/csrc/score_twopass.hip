// General two-pass attention scoring for any number R of query rows per KV
// head: KVzip's many external queries ([KVzip] §3.2, max over the group
// queries of the softmax weight), and window scoring with R = G*W > 128
// ([CriticalKV] §3.3 Algorithm 2 steps 2-4). The row softmax runs along the
// keys while the aggregate runs along the queries ([KVzip] §3.4 names this
// cross-dimension dependence), so every row's normaliser is needed before
// any key's aggregate:
//   pass 1  k_gen_stats   per row r: m_r = max_j x_rj, l_r = sum_j 2^(x_rj - m_r),
//                         x = log2(e) * scale * <q_r, k_j>; c_r = m_r + log2 l_r.
//   pass 2  k_gen_colagg  per key j: sum_r 2^(x_rj - c_r), or 2^(max_r (x_rj - c_r)).
//   pool    max over +-pool/2 neighbours inside the candidate range.
// KVzip-logit ([KVzip] §6.5, no softmax): pass 2 alone, every c_r = 0 and
// no exponential: per key j, scale * max_r <q_r, k_j>.
// Chunked scoring ([KVzip] §3.4): a "layer" of the grid is a (layer,
// chunk) pair whose keys are the chunk's m cached keys (a KeyMap says where
// they sit in the cache). Pass 1 folds, per row, the chunk's cached keys
// and then, in the same workgroup, the input's own keys causally (row r
// sees own keys 0 .. r % n_in); the combine gives the rows past a short
// last chunk's input -inf; pass 2 maxes over the chunk's cached keys.
// Both passes are dense Q K^T contractions on MFMA (32x32x16 bf16, fp32
// accumulation) built for operand reuse:
//   pass 1: a workgroup of 4 waves owns 256 rows (a wave: 64 rows, two MFMA
//     N tiles, Q operands in registers) and streams K in 64-key tiles
//     through an LDS ring shared by the 4 waves; two workgroups share a CU,
//     so one computes while the other waits at its tile barrier. Rows sit
//     on lanes, so the online max / sum stays in-lane.
//   pass 2: a workgroup owns 256 keys (a wave: 64 keys in registers; two
//     workgroups share a CU like pass 1's) and
//     streams Q in 64-row tiles through the ring, each with its 64 c_r.
//     The accumulators start at -c_r / (log2(e) * scale), so the MFMA
//     itself subtracts the normaliser and max aggregation costs one max
//     per element.
// Ring slots are filled by direct global->LDS loads, the 16-byte pieces of
// row r XOR-swizzled by (r & 15); fence-free barriers keep the loads of the
// next gSlots-1 tiles in flight. Workgroups are ordered so that those that
// re-read one head's operand run on one XCD (one L2). Every row's and key's
// result comes from one lane and a fixed-order merge: deterministic.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"
#include "kvsel_ring.h"

namespace kvsel {

constexpr int gSlotBytes = gRowsBytes + gTile * 4;             // pass 2: rows + normalisers
constexpr float gNegBig = -1.0e30f;

// The keys of grid layer lv (layer lv / T, chunk lv % T) and head h: rows
// [row0, row0 + nk) of a [L][H][n_total][d] array, chunk t holding keys
// [t*m, t*m + m) of its (layer, head) (the last chunk may be shorter).
// Unchunked: T = 1, m = n_total.
struct KeyMap {
  int T, m, n_total;
};

__device__ __forceinline__ void key_span(const KeyMap& km, int lv, int H, int h, size_t& row0,
                                         int& nk) {
  const int l = lv / km.T, t = lv - l * km.T;
  row0 = ((size_t)l * H + h) * km.n_total + (size_t)t * km.m;
  nk = min(km.m, km.n_total - t * km.m);
}

// ---------------------------------------------------------------- pass 1 ----
// 1-D grid of row_blocks * splits * H * L workgroups, block 512.
// part[lh][sp][row] = (m, l) of the row over split sp's keys.
//
// Software pipelined: the 8 MFMA steps of tile t are interleaved with the
// vector work of tile t-1 (two accumulator sets in turn), an eighth of it
// after each step, so the matrix and vector units run side by side.
// The vector work is the bound here (an exponential costs a quarter-rate
// issue slot), so it is kept to one FMA, one exp2 and one add per logit:
// a tile's exponentials use the running offset m from before the tile, and
// the tile's max is only found (and the sum redone with a new offset) when
// the tile's partial sum passes 2^64: on the first tile of a row, or when
// its max jumps. A partial sum of at most 2^64 bounds every term, so the
// kept sums stay far below fp32's limit (at most n * 2^64).
constexpr float kHeadroomPow2 = 1.8446744e19f;   // 2^64

// part[lh][sp_off + sp] (of sp_stride slots per row block) for split sp.
// SELF (KVzip's chunked scoring): after the grid layer's keys the same
// workgroup runs on the input's own keys, ks[lv][h][n_self][d], causally
// (row r sees own keys 0 .. r % n_self), so both key sources fold into one
// (max, sum) per row and each query block is loaded once.
// Two 4-wave workgroups per CU (256 VGPRs a wave) rather than one of 8
// waves: the same operand reuse per wave, but each workgroup's tile
// barriers no longer stall the other's waves.
constexpr int gStatsWaves = 4;                       // pass-1 waves per workgroup
constexpr int gStatsBlock = gStatsWaves * 64;         // pass-1 rows per workgroup
using StatsLoader = RingLoader<gStatsWaves>;
template <bool CAUSAL, bool SELF = false>
__global__ __launch_bounds__(gStatsBlock, 3) void k_gen_stats(const __bf16* __restrict__ q,
                                                   const __bf16* __restrict__ k, int H, int R,
                                                   int W, KeyMap km, float alpha, int row_blocks,
                                                   int splits, int kps, int sp_off, int sp_stride,
                                                   float2* __restrict__ part,
                                                   const __bf16* __restrict__ ks, int n_self) {
  __shared__ __align__(16) unsigned char ring[gSlots][gTile * kRowBytes];
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int rb = id % row_blocks;
  id /= row_blocks;
  const int sp = id % splits;
  id /= splits;
  const int h = id % H, l = id / H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  size_t krow0;
  int n;
  key_span(km, l, H, h, krow0, n);
  const __bf16* kh = k + krow0 * kHeadDim;
  // causal: no row of this workgroup sees past its largest r % W, so the
  // keys after it are skipped (the window rule's rows are [G][W]; a chunk's
  // own keys have n = W, where this halves the work)
  int vis_end = n;
  if (CAUSAL) {
    const int r0 = rb * gStatsBlock, r1 = min(R, r0 + gStatsBlock);
    const int top = (r1 - 1) / W != r0 / W ? W - 1 : (r1 - 1) % W;
    vis_end = n - W + top + 1;
  }
  const int j0 = sp * kps, j1 = min(min(n, vis_end), j0 + kps);
  // SELF: own-key tiles up to the block's last visible own key; self_open:
  // the own keys every row of the block sees
  int ntiles2 = 0, self_open = -1;
  const __bf16* ksh = ks;
  if constexpr (SELF) {
    const int r0 = rb * gStatsBlock, r1 = min(R, r0 + gStatsBlock);
    const bool spans = (r1 - 1) / n_self != r0 / n_self;
    const int top = spans ? n_self - 1 : (r1 - 1) % n_self;
    self_open = spans ? 0 : r0 % n_self;
    ntiles2 = (top + gTile) / gTile;
    ksh = ks + lh * (size_t)n_self * kHeadDim;
  }
  if (j1 <= j0 && (!SELF || ntiles2 == 0)) {   // a split past every visible key: neutral statistics
    const int row = rb * gStatsBlock + threadIdx.x;
    if (row < R) part[(lh * sp_stride + sp_off + sp) * (size_t)R + row] = make_float2(gNegBig, 0.f);
    return;         // every wave returns here: no barrier is left waiting
  }
  const int ntiles1 = SELF ? (j1 > j0 ? (j1 - j0 + gTile - 1) / gTile : 0) : (j1 - j0 + gTile - 1) / gTile;
  const int ntiles = SELF ? ntiles1 + ntiles2 : ntiles1;

  const int row0 = rb * gStatsBlock + wave * 64;
  const bool active = row0 < R;
  bf16x8 qb[2][8];
  int last[2], last_self[2] = {-1, -1};
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = row0 + nt * 32 + col;
    if (row < R) load_half_row(q + (lh * R + row) * (size_t)kHeadDim, hf, qb[nt]);
    else zero_ops(qb[nt]);
    last[nt] = row < R ? (CAUSAL ? n - W + row % W : n - 1) : -1;   // last visible key
    if constexpr (SELF) last_self[nt] = row < R ? row % n_self : -1;   // last visible own key
  }
  StatsLoader ld;
  ld.init(kHeadDim);
  // tile t of the workgroup: the layer's keys, then (SELF) the own keys
  auto issue_tile = [&](int t, unsigned char* slot) {
    if constexpr (SELF) {
      if (t >= ntiles1) {
        ld.issue(ksh, (t - ntiles1) * gTile, n_self, kHeadDim, slot);
        return;
      }
    }
    ld.issue(kh, j0 + t * gTile, n, kHeadDim, slot);
  };
  asm volatile("" ::: "memory");
  // the first gSlots-1 tiles (repeating the last one if there are fewer)
#pragma unroll
  for (int t = 0; t < gSlots - 1; ++t) issue_tile(min(t, ntiles - 1), ring[t]);
  // Q is in registers once at most the prologue's loads are in flight; an
  // explicit wait here keeps the compiler from waiting inside the loop
  gen_wait<(gSlots - 1) * StatsLoader::kLoads>();
  // keys every row sees
  const int open_end = CAUSAL ? n - W : n - 1;
  float m[2] = {gNegBig, gNegBig}, s[2] = {0.f, 0.f};

  // hide the keys a row does not see (tiles at the causal edge or the split end)
  auto mask = [&](f32x16 (&acc)[2][2], int t) {
    if constexpr (SELF) {   // the layer's keys, then the own keys (causal)
      const bool own = t >= ntiles1;
      const int kt = own ? (t - ntiles1) * gTile : j0 + t * gTile;
      const int end = own ? n_self : j1;
      if (kt + gTile - 1 <= (own ? self_open : open_end) && kt + gTile <= end) return;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int lim = own ? last_self[nt] : last[nt];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt + mt * 32 + acc_row(i, lane);
            if (!(key <= lim && key < end)) acc[mt][nt][i] = neg_inf();
          }
      }
      return;
    }
    const int kt = j0 + t * gTile;
    if (kt + gTile - 1 <= open_end && kt + gTile <= j1) return;
    // opaque key base: keeps the 16 row offsets from being hoisted out of
    // the tile loop into registers (this branch runs on edge tiles only)
    int kbase = kt + acc_row(0, lane);
    asm volatile("" : "+v"(kbase));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + mt * 32 + (acc_row(i, 0) - acc_row(0, 0));
          if (!(key <= last[nt] && key < j1)) acc[mt][nt][i] = neg_inf();
        }
  };
  // part c (of 8) of a tile: 8 logits of row set nt = c / 4 into the
  // tile's partial sum at offset m
  auto fold_part = [&](const f32x16 (&acc)[2][2], int c, float (&ps)[2]) {
    const int nt = c >> 2, mt = (c >> 1) & 1, i0 = (c & 1) * 8;
    float sum = ps[nt];
    const float off = -m[nt];
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) sum += fast_exp2(__builtin_fmaf(acc[mt][nt][i], alpha, off));
    ps[nt] = sum;
  };
  // close a tile: accept its partial sums, or redo a row with a new offset
  auto fold_end = [&](const f32x16 (&acc)[2][2], const float (&ps)[2]) {
    // both rows' sums are taken unconditionally (before any branch), so the
    // partial sums are computed where they were written, beside the MFMAs,
    // rather than sunk towards a branch
    const float s_old[2] = {s[0], s[1]};
    s[0] = s_old[0] + ps[0];
    s[1] = s_old[1] + ps[1];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (!(ps[nt] <= kHeadroomPow2)) {   // also catches an overflow to inf
        float tm = neg_inf();
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; i += 2) tm = gmax3(tm, acc[mt][nt][i], acc[mt][nt][i + 1]);
        const float mn = __builtin_fmaxf(m[nt], tm * alpha);   // alpha > 0
        float sum = s_old[nt] * fast_exp2(m[nt] - mn);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(acc[mt][nt][i], alpha, -mn));
        s[nt] = sum;
        m[nt] = mn;
      }
    }
  };
  auto begin_tile = [&](int t) -> const unsigned char* {
    gen_wait_tile<StatsLoader::kLoads>(t, ntiles);
    gen_barrier();
    if (t + gSlots - 1 < ntiles) issue_tile(t + gSlots - 1, ring[(t + gSlots - 1) % gSlots]);
    // the slot's offset in an opaque vector register: keeps LDS reads from
    // moving across tiles, and each operand address is one add
    int soff = (t % gSlots) * gRowsBytes;
    asm volatile("" : "+v"(soff));
    return ring[0] + soff;
  };
  auto zero_acc = [&](f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();
  };
  // tile t into cur, interleaved with folding tile t-1 (prev)
  auto step = [&](int t, f32x16 (&cur)[2][2], f32x16 (&prev)[2][2]) {
    const unsigned char* slot = begin_tile(t);
    if (!active) return;
    mask(prev, t - 1);
    float ps[2] = {0.f, 0.f};
    zero_acc(cur);
    bf16x8 a[2][2];
    read_step(slot, col, hf, 0, a[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) read_step(slot, col, hf, st + 1, a[(st + 1) & 1]);
      // each of the step's four MFMAs is followed by two logits of part st
      // of the previous tile's fold (the sums of fold_part, in its order)
      const int fnt = st >> 2, fmt = (st >> 1) & 1, fi = (st & 1) * 8;
      const float off = -m[fnt];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int mt = u & 1, nt = u >> 1;
        cur[mt][nt] = mfma32(a[st & 1][mt], qb[nt][st], cur[mt][nt]);
#pragma unroll
        for (int i = fi + 2 * u; i < fi + 2 * u + 2; ++i)
          ps[fnt] += fast_exp2(__builtin_fmaf(prev[fmt][fnt][i], alpha, off));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // pin the partial sums here: otherwise the compiler sinks the second
    // row set's folds past the first row set's branch, behind the MFMAs
    asm volatile("" : "+v"(ps[0]), "+v"(ps[1]));
    fold_end(prev, ps);
  };
  // fold a tile with no MFMA work beside it (one part at a time: fewer
  // exponentials in flight, fewer registers)
  auto fold_all = [&](f32x16 (&acc)[2][2], int t) {
    mask(acc, t);
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      fold_part(acc, c, ps);
      __builtin_amdgcn_sched_barrier(0);
    }
    fold_end(acc, ps);
  };

  // tile t: its MFMAs, then its fold. One accumulator set: three 4-wave
  // workgroups per CU fit, and the other waves' MFMAs cover a wave's
  // exponentials (the fold order, and so the sums, are those of the
  // pipelined step above, which is kept for reference)
  (void)step;
  f32x16 acc[2][2];
  for (int t = 0; t < ntiles; ++t) {
    const unsigned char* slot = begin_tile(t);
    if (!active) continue;
    zero_acc(acc);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      bf16x8 a[2];
      read_step(slot, col, hf, st, a);
      tile_step(a, qb, st, acc);
    }
    fold_all(acc, t);
  }
  // with fewer tiles than the prologue's loads, repeats of the last tile may
  // still be landing in LDS: let them finish before the workgroup ends
  gen_wait<0>();
  // the other lane half holds the other 16 keys of every 32-key block
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float m2 = lane_xor32(m[nt]), s2 = lane_xor32(s[nt]);
    lse_merge(m[nt], s[nt], m2, s2);
    const int row = row0 + nt * 32 + col;
    if (hf == 0 && row < R)
      part[(lh * sp_stride + sp_off + sp) * (size_t)R + row] = make_float2(m[nt], s[nt]);
  }
}

// c_r = m_r + log2(l_r) over the splits, in split order (the window
// kernels' normaliser).
__global__ __launch_bounds__(256) void k_combine(const float2* __restrict__ part,
                                                 int H, int R, int splits,
                                                 float* __restrict__ stat) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, l = blockIdx.z;
  if (r >= R) return;
  const size_t lh = (size_t)l * H + h;
  float m = gNegBig, s = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const float2 p = part[(lh * splits + sp) * (size_t)R + r];
    lse_merge(m, s, p.x, p.y);
  }
  stat[lh * R + r] = m + __log2f(s);
}

// Pass 2's form of the normaliser: -c_r / alpha in rows of Rpad (a multiple
// of the tile), padding rows -inf so they drop out of every aggregate.
// Chunked (T > 0): rows are [G][n_in] per head, and row i of a g block is
// padding past the chunk's input of n_prompt + m_t tokens.
__global__ __launch_bounds__(256) void k_combine_neg(const float2* __restrict__ part,
                                                     int H, int R, int Rpad, int splits,
                                                     float inv_alpha, int T, int n_in,
                                                     int n_prompt, KeyMap km,
                                                     float* __restrict__ stat) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, l = blockIdx.z;
  if (r >= Rpad) return;
  const size_t lh = (size_t)l * H + h;
  bool pad = r >= R;
  if (T > 0 && !pad) {
    const int t = l % T;
    pad = r % n_in >= n_prompt + min(km.m, km.n_total - t * km.m);
  }
  if (pad) {
    stat[lh * Rpad + r] = neg_inf();
    return;
  }
  float m = gNegBig, s = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const float2 p = part[(lh * splits + sp) * (size_t)R + r];
    lse_merge(m, s, p.x, p.y);
  }
  stat[lh * Rpad + r] = -(m + __log2f(s)) * inv_alpha;
}

// KVzip-logit: no normaliser, so pass 2 starts every real row at 0 (and
// padding rows at -inf).
__global__ __launch_bounds__(256) void k_logit_stat(int R, int Rpad, float* __restrict__ stat) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= Rpad) return;
  const size_t lh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  stat[lh * Rpad + r] = r < R ? 0.f : neg_inf();
}

// ---------------------------------------------------------------- pass 2 ----
// 1-D grid of key_blocks * H * L workgroups, block 512. raw[lh][key].
// Pipelined like pass 1: the MFMAs of row tile t run beside the aggregation
// of tile t-1, so the matrix pipe does not wait for the per-tile max / sum.
// Like pass 1: two 4-wave workgroups per CU.
constexpr int gColWaves = 4;                          // pass-2 waves per workgroup
constexpr int gColBlock = gColWaves * 64;             // pass-2 keys per workgroup
using ColLoader = RingLoader<gColWaves>;
template <bool CAUSAL, bool MAXAGG, bool LOGIT = false>
__global__ __launch_bounds__(gColBlock, 3) void k_gen_colagg(const __bf16* __restrict__ q,
                                                    const __bf16* __restrict__ k, int H, int R,
                                                    int W, KeyMap km, float alpha, int key_blocks,
                                                    const float* __restrict__ stat,
                                                    float* __restrict__ raw) {
  // one LDS object: slot = 64 Q rows, then their 64 normalisers (with two
  // objects the compiler waits for every direct-to-LDS load before any read)
  __shared__ __align__(16) unsigned char ring[gSlots][gSlotBytes];
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = id % key_blocks;
  id /= key_blocks;
  const int h = id % H, l = id / H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const __bf16* qh = q + lh * (size_t)R * kHeadDim;
  const int ntiles = (R + gTile - 1) / gTile;
  const float* sh = stat + lh * (size_t)ntiles * gTile;
  size_t krow0;
  int n;
  key_span(km, l, H, h, krow0, n);

  // this wave's 64 keys: MFMA B operands for the whole kernel
  const int key0 = kb * gColBlock + wave * 64;
  bf16x8 kop[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = key0 + nt * 32 + col;
    if (key < n) load_half_row(k + (krow0 + key) * (size_t)kHeadDim, hf, kop[nt]);
    else zero_ops(kop[nt]);
  }
  // a row tile: the Q rows (all waves) and their -c_r / alpha (wave 0)
  ColLoader ld;
  ld.init(kHeadDim);
  auto issue = [&](int t, int slot) {
    ld.issue(qh, t * gTile, R, kHeadDim, ring[slot]);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(sh + t * gTile + lane),
                                       (lds_ptr_t)(ring[slot] + gRowsBytes), 4, 0, 0);
  };
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < gSlots - 1; ++t) issue(min(t, ntiles - 1), t);
  // K operands are in registers once at most the prologue's loads remain
  if (wave == 0) gen_wait<(gSlots - 1) * (ColLoader::kLoads + 1)>();
  else gen_wait<(gSlots - 1) * ColLoader::kLoads>();

  float agg[2];
  agg[0] = agg[1] = MAXAGG ? neg_inf() : 0.f;
  const bool any_key = key0 < n;

  auto begin_tile = [&](int t) -> const unsigned char* {
    if (wave == 0) gen_wait_tile<ColLoader::kLoads + 1>(t, ntiles);
    else gen_wait_tile<ColLoader::kLoads>(t, ntiles);
    gen_barrier();
    if (t + gSlots - 1 < ntiles) issue(t + gSlots - 1, (t + gSlots - 1) % gSlots);
    int soff = (t % gSlots) * gSlotBytes;   // opaque: LDS reads stay inside the tile
    asm volatile("" : "+v"(soff));
    return ring[0] + soff;
  };
  // acc = <q_r, k> - c_r / alpha: start from the tile's normalisers
  // (padding rows: -inf)
  auto init_acc = [&](const unsigned char* slot, f32x16 (&acc)[2][2]) {
    const float* cs = reinterpret_cast<const float*>(slot + gRowsBytes);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 init;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(cs + mt * 32 + 8 * j + 4 * hf);
#pragma unroll
        for (int u = 0; u < 4; ++u) init[4 * j + u] = c4[u];
      }
      acc[mt][0] = init;
      acc[mt][1] = init;
    }
  };
  // window rows: row r sees keys up to n - W + r % W (only keys past n - W
  // can be hidden)
  auto mask = [&](f32x16 (&acc)[2][2], int t) {
    if (!CAUSAL) return;
    const int rt = t * gTile;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int key = key0 + nt * 32 + col;
      if (key > n - W) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rt + mt * 32 + acc_row(i, lane);
            if (key > n - W + row % W) acc[mt][nt][i] = neg_inf();
          }
      }
    }
  };
  // part c (of 8) of a tile: 8 values of key set nt = c / 4
  auto fold_part = [&](const f32x16 (&acc)[2][2], int c, float (&pa)[2]) {
    const int nt = c >> 2, mt = (c >> 1) & 1, i0 = (c & 1) * 8;
    float a = pa[nt];
#pragma unroll
    for (int i = i0; i < i0 + 8; i += 2) {
      if (MAXAGG) a = gmax3(a, acc[mt][nt][i], acc[mt][nt][i + 1]);
      else a += fast_exp2(acc[mt][nt][i] * alpha) + fast_exp2(acc[mt][nt][i + 1] * alpha);
    }
    pa[nt] = a;
  };
  auto step = [&](int t, f32x16 (&cur)[2][2], f32x16 (&prev)[2][2]) {
    const unsigned char* slot = begin_tile(t);
    if (!any_key) return;
    mask(prev, t - 1);
    init_acc(slot, cur);
    bf16x8 a[2][2];
    read_step(slot, col, hf, 0, a[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) read_step(slot, col, hf, st + 1, a[(st + 1) & 1]);
      tile_step(a[st & 1], kop, st, cur);
      fold_part(prev, st, agg);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto fold_all = [&](f32x16 (&acc)[2][2], int t) {
    mask(acc, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) fold_part(acc, c, agg);
  };

  // tile t: its MFMAs, then its fold (in the order of the pipelined step
  // above, kept for reference). One accumulator set: three 4-wave
  // workgroups per CU fit, and the other waves' MFMAs cover a wave's fold.
  (void)step;
  f32x16 acc[2][2];
  for (int t = 0; t < ntiles; ++t) {
    const unsigned char* slot = begin_tile(t);
    if (!any_key) continue;
    init_acc(slot, acc);
    bf16x8 a[2][2];
    read_step(slot, col, hf, 0, a[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) read_step(slot, col, hf, st + 1, a[(st + 1) & 1]);
      tile_step(a[st & 1], kop, st, acc);
    }
    fold_all(acc, t);
  }
  gen_wait<0>();   // repeats of the last tile (fewer tiles than the prologue's)
  // the other lane half holds the other 16 rows of every 32-row block
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float o = lane_xor32(agg[nt]);
    // LOGIT: alpha is the plain scale and the max is the logit itself
    const float tot = LOGIT ? __builtin_fmaxf(agg[nt], o) * alpha
                    : MAXAGG ? fast_exp2(__builtin_fmaxf(agg[nt], o) * alpha) : agg[nt] + o;
    const int key = key0 + nt * 32 + col;
    if (hf == 0 && key < n) raw[krow0 + key] = tot;
  }
}

// ------------------------------------------------------------------ pool ----
// scores[j] = max raw[t], |t - j| <= r, 0 <= t < n_cand.
// grid (ceil(n_cand / kPoolSpan), L*H), block 256. A block stages its
// kPoolSpan + 2r raw values in LDS with all of a thread's loads in flight,
// then each thread writes kPoolOut outputs 256 apart (conflict-free LDS
// reads, coalesced stores).
constexpr int kPoolOut = 4;
constexpr int kPoolSpan = 256 * kPoolOut;

__global__ __launch_bounds__(256) void k_pool(const float* __restrict__ raw, int n,
                                              int n_cand, int r,
                                              float* __restrict__ scores) {
  __shared__ float tile[kPoolSpan + 2 * 32];
  const size_t lh = blockIdx.y;
  const int j0 = blockIdx.x * kPoolSpan;
  const float* src = raw + lh * n;
  const int tid = threadIdx.x;
  const int span = kPoolSpan + 2 * r;
  float v[kPoolOut + 1];
#pragma unroll
  for (int u = 0; u <= kPoolOut; ++u) {
    const int t = tid + u * 256;
    const int j = j0 - r + t;
    // outside the candidates: no part
    v[u] = (t < span && j >= 0 && j < n_cand) ? src[j] : neg_inf();
  }
#pragma unroll
  for (int u = 0; u <= kPoolOut; ++u)
    if (tid + u * 256 < span) tile[tid + u * 256] = v[u];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPoolOut; ++u) {
    const int c = tid + u * 256;
    if (j0 + c < n_cand) {
      float m = tile[c + r];
      for (int o = 1; o <= r; ++o) m = fmaxf(m, fmaxf(tile[c + r - o], tile[c + r + o]));
      scores[lh * n_cand + j0 + c] = m;
    }
  }
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
  if (!scores) return hipSuccess;   // raw scores only
  hipLaunchKernelGGL(k_pool, dim3((n_cand + kPoolSpan - 1) / kPoolSpan, L * H), dim3(256), 0,
                     st, raw, n, n_cand, r, scores);
  return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void twopass_plan(const ScorePlan& p, TwoPassLayout* o) {
  const int Lv = p.chunk_m > 0 ? p.L * ((p.n + p.chunk_m - 1) / p.chunk_m) : p.L;
  const int row_blocks = (p.R + gStatsBlock - 1) / gStatsBlock;
  int splits, kps, stride;
  if (p.chunk_m > 0) {
    // chunked: (layer, chunk) pairs fill the GPU; one workgroup per row
    // block folds the chunk's cached keys and then the input's own keys
    splits = 1;
    kps = (p.chunk_m + gTile - 1) / gTile * gTile;
    stride = 1;
  } else {
    const long long base = (long long)row_blocks * p.H * p.L;
    // split the keys only when the row blocks alone cannot fill the GPU
    splits = (int)((1024 + base - 1) / base);
    const int max_splits = (p.n + 4 * gTile - 1) / (4 * gTile);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    kps = (p.n + splits - 1) / splits;
    kps = (kps + gTile - 1) / gTile * gTile;
    splits = (p.n + kps - 1) / kps;
    stride = splits;
  }
  o->row_blocks = row_blocks;
  o->splits = splits;
  o->sp_stride = stride;
  o->keys_per_split = kps;
  o->Lv = Lv;
  const size_t LHv = (size_t)Lv * p.H;
  o->part_off = 0;
  const size_t Rpad = (size_t)(p.R + gTile - 1) / gTile * gTile;
  o->stat_off = p.logit ? 0 : align256(LHv * stride * p.R * sizeof(float2));   // no pass 1
  o->raw_off = o->stat_off + align256(LHv * Rpad * sizeof(float));
  o->bytes = o->raw_off +
             (p.need_raw_tmp ? align256((size_t)p.L * p.H * p.n * sizeof(float)) : 0);
}

hipError_t twopass_launch(const ScorePlan& p, const TwoPassLayout& o, const void* q,
                          const void* k, const void* k_self, float* scores, float* raw,
                          void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  float2* part = reinterpret_cast<float2*>(w + o.part_off);
  float* stat = reinterpret_cast<float*>(w + o.stat_off);
  float* rawbuf = raw ? raw : reinterpret_cast<float*>(w + o.raw_off);
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const float alpha = p.scale * kLog2e;
  const bool chunked = p.chunk_m > 0;
  const int T = chunked ? (p.n + p.chunk_m - 1) / p.chunk_m : 1;
  const KeyMap km{T, chunked ? p.chunk_m : p.n, p.n};
  const int kmax = km.m;                      // keys a grid layer holds at most
  const long long g1 = (long long)o.row_blocks * o.splits * p.H * o.Lv;
  const int key_blocks = (kmax + gColBlock - 1) / gColBlock;
  const long long g2 = (long long)key_blocks * p.H * o.Lv;
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int Rpad = (p.R + gTile - 1) / gTile * gTile;
  if (p.logit) {
    hipLaunchKernelGGL(k_logit_stat, dim3((Rpad + 255) / 256, p.H, o.Lv), dim3(256), 0, st, p.R,
                       Rpad, stat);
    hipLaunchKernelGGL((k_gen_colagg<false, true, true>), dim3((unsigned)g2), dim3(gColBlock), 0, st, qb,
                       kb, p.H, p.R, p.W, km, p.scale, key_blocks, stat, rawbuf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return pool_launch(rawbuf, p.L, p.H, p.n, p.n_cand, p.pool / 2, scores, st);
  }
  // chunked: the input's own keys (rows are [G][n_in], row r sees own keys
  // 0 .. r % n_in) follow the chunk's cached keys in the same workgroups
  const int n_in = chunked ? p.n_prompt + p.chunk_m : 0;
  const __bf16* ksb = static_cast<const __bf16*>(k_self);
  if (chunked)
    hipLaunchKernelGGL((k_gen_stats<false, true>), dim3((unsigned)g1), dim3(gStatsBlock), 0, st, qb, kb,
                       p.H, p.R, p.W, km, alpha, o.row_blocks, o.splits, o.keys_per_split, 0,
                       o.sp_stride, part, ksb, n_in);
  else if (p.causal)
    hipLaunchKernelGGL(k_gen_stats<true>, dim3((unsigned)g1), dim3(gStatsBlock), 0, st, qb, kb, p.H,
                       p.R, p.W, km, alpha, o.row_blocks, o.splits, o.keys_per_split, 0,
                       o.sp_stride, part, ksb, 1);
  else
    hipLaunchKernelGGL(k_gen_stats<false>, dim3((unsigned)g1), dim3(gStatsBlock), 0, st, qb, kb, p.H,
                       p.R, p.W, km, alpha, o.row_blocks, o.splits, o.keys_per_split, 0,
                       o.sp_stride, part, ksb, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_combine_neg, dim3((Rpad + 255) / 256, p.H, o.Lv), dim3(256), 0, st, part,
                     p.H, p.R, Rpad, o.sp_stride, 1.0f / alpha, chunked ? T : 0, n_in, p.n_prompt,
                     km, stat);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((unsigned)g2);
  if (p.causal) {
    if (p.max_agg)
      hipLaunchKernelGGL((k_gen_colagg<true, true>), grid2, dim3(gColBlock), 0, st, qb, kb, p.H, p.R,
                         p.W, km, alpha, key_blocks, stat, rawbuf);
    else
      hipLaunchKernelGGL((k_gen_colagg<true, false>), grid2, dim3(gColBlock), 0, st, qb, kb, p.H,
                         p.R, p.W, km, alpha, key_blocks, stat, rawbuf);
  } else {
    if (p.max_agg)
      hipLaunchKernelGGL((k_gen_colagg<false, true>), grid2, dim3(gColBlock), 0, st, qb, kb, p.H,
                         p.R, p.W, km, alpha, key_blocks, stat, rawbuf);
    else
      hipLaunchKernelGGL((k_gen_colagg<false, false>), grid2, dim3(gColBlock), 0, st, qb, kb, p.H,
                         p.R, p.W, km, alpha, key_blocks, stat, rawbuf);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return pool_launch(rawbuf, p.L, p.H, p.n, p.n_cand, p.pool / 2, scores, st);
}

}  // namespace kvsel
