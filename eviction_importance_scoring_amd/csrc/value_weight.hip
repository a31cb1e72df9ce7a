// CriticalKV's projected-value norm ([CriticalKV] §3.3 Algorithm 1 steps
// 2-3; Theorem 3.3): weight[l][h][j] = (1/G) sum_g || W_O^(h,g) v_j ||_1
// where W_O^(h,g) is the D x d column slice of the output projection that
// query head h*G+g uses (group mode 0), or || (sum_g W_O^(h,g)) v_j ||_1
// (group mode 1: the slices are summed into a bf16 copy first, then the
// same kernel runs with one slice per KV head). The projection V W^O is a
// bf16 MFMA product accumulated in fp32; each output tile is folded into
// per-key |.| sums in registers and never written ([CriticalKV] §D.4 notes
// the full V W^O would be ~7.8 GB per layer at 7B / 128K).
//
// Tiling (the LDS ring of kvsel_ring.h, 4 waves, three workgroups per CU):
// a workgroup owns 256 keys of one (layer, KV head); each wave holds the
// values of 64 keys (two MFMA N tiles) in registers for the whole kernel. The A operand, W_O^(h,g), is
// streamed in 64-row tiles (64 of the D output features, 128 columns each,
// rows H_q*d elements apart in the [D][H_q*d] matrix) through the ring, for
// every g: G * ceil(D/64) tiles. Workgroups of one (layer, head) run on one XCD, so
// the 4 MB slice they all stream stays in that XCD's L2. Each tile's MFMAs
// run first and its |.| fold after them; a wave's vector work does not run
// beside its own MFMAs, so the other workgroups' waves keep the matrix unit
// busy meanwhile. Every key's sum is accumulated in one lane in a fixed order:
// deterministic, no atomics.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"
#include "kvsel_ring.h"

namespace kvsel {

// Three 4-wave workgroups per CU: each workgroup's tile barriers do not
// stall the others' waves.
constexpr int vWaves = 4;
constexpr int vBlock = vWaves * 64;                    // keys per workgroup
using VLoader = RingLoader<vWaves>;

// 1-D grid of key_blocks * H * L workgroups, block vBlock.
__global__ __launch_bounds__(vBlock, 3) void k_value_weight(const __bf16* __restrict__ v,
                                                      const __bf16* __restrict__ w_o,
                                                      int H, int G, int n, int D, int n_cand,
                                                      int key_blocks,
                                                      float* __restrict__ weight) {
  __shared__ __align__(16) unsigned char ring[gSlots][gRowsBytes];
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = id % key_blocks;
  id /= key_blocks;
  const int h = id % H, l = id / H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const int Hq = H * G;
  const int stride = Hq * kHeadDim;                        // elements between W_O rows
  const __bf16* wl = w_o + (size_t)l * D * (size_t)stride;
  const int dtiles = (D + gTile - 1) / gTile;
  const int ntiles = G * dtiles;

  // this wave's 64 keys: MFMA B operands for the whole kernel
  const int key0 = kb * vBlock + wave * 64;
  bf16x8 vop[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = key0 + nt * 32 + col;
    if (key < n_cand) load_half_row(v + (lh * n + key) * (size_t)kHeadDim, hf, vop[nt]);
    else zero_ops(vop[nt]);
  }
  // tile t: output features [64*dt, 64*dt + 64) of query head h*G + g
  VLoader ld;
  ld.init(stride);
  auto issue = [&](int t, int slot) {
    const int g = t / dtiles, dt = t - g * dtiles;
    ld.issue(wl + (size_t)(h * G + g) * kHeadDim, dt * gTile, D, stride, ring[slot]);
  };
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < gSlots - 1; ++t) issue(min(t, ntiles - 1), t);
  // values are in registers once at most the prologue's loads remain
  gen_wait<(gSlots - 1) * VLoader::kLoads>();

  const bool any_key = key0 < n_cand;
  float part[2] = {0.f, 0.f};

  auto begin_tile = [&](int t) -> const unsigned char* {
    gen_wait_tile<VLoader::kLoads>(t, ntiles);
    gen_barrier();
    if (t + gSlots - 1 < ntiles) issue(t + gSlots - 1, (t + gSlots - 1) % gSlots);
    int soff = (t % gSlots) * gRowsBytes;   // opaque: LDS reads stay inside the tile
    asm volatile("" : "+v"(soff));
    return ring[0] + soff;
  };
  // D % 64 == 32: the last tile of each g has 32 real rows; its other 32
  // MFMA rows get zero operands (|0| adds nothing)
  auto half_tile = [&](int t) { return (t % dtiles) * gTile + 32 >= D; };
  auto read = [&](const unsigned char* slot, int st, bool half, bf16x8 (&a)[2]) {
    read_step(slot, col, hf, st, a);
    if (half) a[1] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  };
  // part c (of 8) of a tile: 8 outputs of key set nt = c / 4
  auto fold_part = [&](const f32x16 (&acc)[2][2], int c, float (&ps)[2]) {
    const int nt = c >> 2, mt = (c >> 1) & 1, i0 = (c & 1) * 8;
    float sum = ps[nt];
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) sum += __builtin_fabsf(acc[mt][nt][i]);
    ps[nt] = sum;
  };
  auto zero_acc = [&](f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();
  };
  // tile t: its MFMAs, then its |.| fold (per-tile partial sums keep the
  // fp32 additions short). One accumulator set: three workgroups per CU
  // fit (<= 168 registers), and the other waves' MFMAs cover a wave's fold.
  f32x16 acc[2][2];
  for (int t = 0; t < ntiles; ++t) {
    const unsigned char* slot = begin_tile(t);
    if (!any_key) continue;
    const bool half = half_tile(t);
    zero_acc(acc);
    bf16x8 a[2][2];
    read(slot, 0, half, a[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) read(slot, st + 1, half, a[(st + 1) & 1]);
      tile_step(a[st & 1], vop, st, acc);
    }
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) fold_part(acc, c, ps);
    part[0] += ps[0];
    part[1] += ps[1];
  }
  gen_wait<0>();   // repeats of the last tile (fewer tiles than the prologue's)
  const float inv_g = 1.0f / (float)G;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float tot = part[nt] + __shfl_xor(part[nt], 32);   // the other 16 output rows
    const int key = key0 + nt * 32 + col;
    if (hf == 0 && key < n_cand) weight[lh * n_cand + key] = tot * inv_g;
  }
}

// Group-summed projection (group mode 1): wsum[l][c][h*d + e] =
// bf16(sum_g w_o[l][c][(h*G + g)*d + e]), the G column slices of KV head
// h added in fp32 in order g = 0..G-1 and rounded once to nearest-even.
// 1-D grid over the L*D*H*d/8 16-byte pieces of wsum, block 256.
__global__ __launch_bounds__(256) void k_wo_group_sum(const __bf16* __restrict__ w_o, int H,
                                                       int G, long long pieces,
                                                       __bf16* __restrict__ wsum) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  constexpr int kPer = kHeadDim / 8;                  // pieces per head row slice
  const long long row = i / ((long long)H * kPer);    // (l, c)
  const int rem = (int)(i - row * H * kPer);
  const int h = rem / kPer, p = rem - h * kPer;
  const u32x4* src = reinterpret_cast<const u32x4*>(w_o + row * (long long)H * G * kHeadDim +
                                                     (long long)h * G * kHeadDim + p * 8);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int g = 0; g < G; ++g) {
    const u32x4 x = src[g * kPer];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(x[e] << 16);
      acc[2 * e + 1] += __uint_as_float(x[e] & 0xFFFF0000u);
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t lo = __float_as_uint(acc[2 * e]), hi = __float_as_uint(acc[2 * e + 1]);
    lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;    // round to nearest-even (finite)
    hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
    out[e] = lo | (hi << 16);
  }
  reinterpret_cast<u32x4*>(wsum)[i] = out;
}

size_t value_weight_ws_bytes(int L, int H, int D, int group_mode) {
  if (group_mode == 0) return 0;
  return (size_t)L * D * H * kHeadDim * sizeof(__bf16);
}

hipError_t value_weight_launch(const void* v, const void* w_o, int L, int H, int G, int n,
                               int D, int n_cand, int group_mode, float* weight, void* ws,
                               hipStream_t st) {
  const int key_blocks = (n_cand + vBlock - 1) / vBlock;
  const long long blocks = (long long)key_blocks * H * L;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const __bf16* proj = static_cast<const __bf16*>(w_o);
  int g_eff = G;
  if (group_mode == 1) {
    // mode 1 is mode 0 with one query head per KV head on the summed slices
    __bf16* wsum = static_cast<__bf16*>(ws);
    const long long pieces = (long long)L * D * H * (kHeadDim / 8);
    const long long pb = (pieces + 255) / 256;
    if (pb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_wo_group_sum, dim3((unsigned)pb), dim3(256), 0, st,
                       static_cast<const __bf16*>(w_o), H, G, pieces, wsum);
    proj = wsum;
    g_eff = 1;
  }
  hipLaunchKernelGGL(k_value_weight, dim3((unsigned)blocks), dim3(vBlock), 0, st,
                     static_cast<const __bf16*>(v), proj, H, g_eff, n, D, n_cand, key_blocks,
                     weight);
  return hipGetLastError();
}

}  // namespace kvsel
