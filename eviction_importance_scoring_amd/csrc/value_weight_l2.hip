// The L2 variant of CriticalKV's projected-value norm ([CriticalKV] §C.3
// and footnote 1: the L1 and L2 distances give similar gains):
//   weight[l][h][j] = (1/G) sum_g || W_O^(h,g) v_j ||_2
// with W_O^(h,g) the D x d column slice of the output projection that query
// head h*G+g uses (the slices and GQA reading of the L1 weight).
//
// ||W v||_2^2 = v^T (W^T W) v = ||R v||_2^2 for any R with R^T R = W^T W.
// So each query head's D x d slice is replaced by the d x d upper-triangular
// factor R = L^T of the Cholesky factorisation W^T W = L L^T, and the weight
// becomes a triangular d-row projection instead of a D-row one. R depends
// on the model weights only, so it is computed once (kvsel_value_l2_factor)
// and reused by every call of the projection (kvsel_value_weight_l2):
//   k_l2_factor  per (layer, query head): W^T W by bf16 MFMA (fp32
//                accumulation, exact products) over W staged transposed in
//                LDS, then an in-LDS Cholesky in fp32; R is written as two
//                bf16 matrices R_hi + R_lo (R_lo = R - R_hi rounded), which
//                together carry R to about 2^-17 relative.
//   k_value_weight_l2  4-wave workgroups (three per CU, so one block's value
//                loads overlap the others' MFMAs) own 256 keys of one
//                (layer, KV head), each wave the values of 64 keys in
//                registers. An LDS ring (kvsel_ring.h) streams, for every g
//                and each 64-row half of R, the R_hi tile then the R_lo tile
//                into the same accumulators, so the MFMA forms
//                (R_hi + R_lo) v. Each MFMA step covers 16 consecutive
//                columns of R, so the 32 x 16 blocks below the diagonal
//                (all zero) are skipped: 20 of 32 block-steps remain. Each
//                pair of tiles is folded into per-key sums of squares; after
//                both halves of g, sqrt.
// The factorisation assumes W^T W has full rank (D >= d and independent
// columns, as for a model's projection): a pivot below 1e-6 of the largest
// diagonal entry is taken as 0 (its direction dropped).
#include "kvsel_internal.h"
#include "kvsel_kernels.h"
#include "kvsel_ring.h"

#include <type_traits>

namespace kvsel {

constexpr int kGcChunk = 64;                     // rows of W per Gram step
constexpr int kWtStride = kGcChunk + 8;          // bf16 per transposed row (144 B: 16-aligned, bank spread)
constexpr int kChStride = kHeadDim + 1;          // fp32 per Cholesky row
constexpr float kPivotFloor = 1.0e-6f;           // relative to the largest diagonal entry

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // finite inputs
}

// grid L * Hq, block 256 (4 waves). factor[l][hq][2][d][d] bf16: R_hi, R_lo.
__global__ __launch_bounds__(256) void k_l2_factor(const __bf16* __restrict__ w_o, int D, int Hq,
                                                   uint16_t* __restrict__ factor) {
  __shared__ __align__(16) uint16_t wt[kHeadDim][kWtStride];   // W chunk, transposed: wt[e][c]
  __shared__ float a[kHeadDim][kChStride];                     // W^T W, then L (lower)
  __shared__ float s_piv;
  const int l = blockIdx.x / Hq, hq = blockIdx.x - l * Hq;
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)Hq * kHeadDim;                     // elements between rows of W_O
  const __bf16* wl = w_o + (size_t)l * D * rs + (size_t)hq * kHeadDim;

  // ---- W^T W: wave w owns output rows [32w, 32w + 32), all 4 column blocks
  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = zero16();
  for (int c0 = 0; c0 < D; c0 += kGcChunk) {
    // 64 rows x 16 pieces of 8 elements; each thread 4 pieces, written transposed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, r = p >> 4, cp = p & 15;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (c0 + r < D) x = *reinterpret_cast<const u32x4*>(wl + (size_t)(c0 + r) * rs + cp * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wt[cp * 8 + 2 * e][r] = (uint16_t)(x[e] & 0xFFFFu);
        wt[cp * 8 + 2 * e + 1][r] = (uint16_t)(x[e] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kGcChunk / 16; ++ks) {
      // A[m = e][k = c] = W[c][e] and B[k = c][n = e'] = W[c][e']: both 8
      // consecutive c of one column, a 16-byte run of the transposed chunk
      const bf16x8 av = ld16(&wt[wave * 32 + col][ks * 16 + hf * 8]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = mfma32(av, ld16(&wt[nb * 32 + col][ks * 16 + hf * 8]), acc[nb]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) a[wave * 32 + acc_row(i, lane)][nb * 32 + col] = acc[nb][i];
  __syncthreads();

  // ---- Cholesky in place (lower triangle): a = L L^T
  float dmax = 0.f;
  for (int i = 0; i < kHeadDim; ++i) dmax = fmaxf(dmax, a[i][i]);
  const float floor_ = kPivotFloor * dmax;
  for (int k = 0; k < kHeadDim; ++k) {
    if (tid == 0) {
      const float dk = a[k][k];
      s_piv = dk > floor_ ? sqrtf(dk) : 0.f;
      a[k][k] = s_piv;
    }
    __syncthreads();
    const float piv = s_piv;
    const float inv = piv > 0.f ? 1.f / piv : 0.f;
    if (tid > k && tid < kHeadDim) a[tid][k] *= inv;
    __syncthreads();
    // trailing lower triangle: a[i][j] -= L[i][k] L[j][k], k < j <= i
    for (int e = (k + 1) * kHeadDim + tid; e < kHeadDim * kHeadDim; e += 256) {
      const int i = e >> 7, j = e & (kHeadDim - 1);
      if (j > k && j <= i) a[i][j] = __builtin_fmaf(-a[i][k], a[j][k], a[i][j]);
    }
    __syncthreads();
  }
  // ---- R = L^T as bf16 hi + lo: R[i][j] = L[j][i] for j >= i
  uint16_t* rh = factor + (((size_t)l * Hq + hq) * 2) * kHeadDim * kHeadDim;
  uint16_t* rl = rh + kHeadDim * kHeadDim;
  for (int e = tid; e < kHeadDim * kHeadDim; e += 256) {
    const int i = e >> 7, j = e & (kHeadDim - 1);
    const float r = j >= i ? a[j][i] : 0.f;
    const uint16_t hi = bf16_rne(r);
    rh[e] = hi;
    rl[e] = bf16_rne(r - __uint_as_float((uint32_t)hi << 16));
  }
}

constexpr int kL2Waves = 4;
constexpr int kL2Block = kL2Waves * 64;   // keys per workgroup
using L2Loader = RingLoader<kL2Waves>;
constexpr int kL2Loads = L2Loader::kLoads;

// MFMA operand of step s for lane half hf: the 16-byte piece 2s + hf of row
// r (columns 16s + 8hf .. +8) of a ring slot, whose pieces are stored
// XOR-swizzled by r & 15.
__device__ __forceinline__ bf16x8 tri_op(const unsigned char* slot, int r, int hf, int s) {
  return ld16(slot + r * kRowBytes + (((2 * s + hf) ^ (r & 15)) << 4));
}

// 1-D grid of key_blocks * H * L workgroups, block 256.
__global__ __launch_bounds__(256, 3) void k_value_weight_l2(const __bf16* __restrict__ v,
                                                            const __bf16* __restrict__ factor,
                                                            int H, int G, int n, int n_cand,
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
  // 4G ring tiles: for each g, rows [0, 64) then [64, 128) of R, each as the
  // R_hi tile then the R_lo tile
  const int ntiles = 4 * G;

  // this wave's 64 keys as MFMA B operands: step s, lane half hf holds
  // columns 16s + 8hf .. +8 of the key's value row
  const int key0 = kb * kL2Block + wave * 64;
  bf16x8 vop[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = key0 + nt * 32 + col;
    if (key < n_cand) {
      const unsigned char* row =
          reinterpret_cast<const unsigned char*>(v + (lh * n + key) * (size_t)kHeadDim);
#pragma unroll
      for (int s = 0; s < 8; ++s) vop[nt][s] = ld16(row + (2 * s + hf) * 16);
    } else {
      zero_ops(vop[nt]);
    }
  }
  L2Loader ld;
  ld.init(kHeadDim);
  auto issue = [&](int t, int slot) {
    const int g = t >> 2, dt = (t >> 1) & 1, lo = t & 1;
    const __bf16* base = factor + ((((size_t)l * Hq + h * G + g) * 2 + lo) * kHeadDim) * kHeadDim;
    ld.issue(base, dt * gTile, kHeadDim, kHeadDim, ring[slot]);
  };
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < gSlots - 1; ++t) issue(min(t, ntiles - 1), t);
  // values are in registers once at most the prologue's loads remain
  gen_wait<(gSlots - 1) * kL2Loads>();

  const bool any_key = key0 < n_cand;
  float ss[2] = {0.f, 0.f}, wsum[2] = {0.f, 0.f};

  auto begin_tile = [&](int t) -> const unsigned char* {
    gen_wait_tile<kL2Loads>(t, ntiles);
    gen_barrier();
    if (t + gSlots - 1 < ntiles) issue(t + gSlots - 1, (t + gSlots - 1) % gSlots);
    int soff = (t % gSlots) * gRowsBytes;   // opaque: LDS reads stay inside the tile
    asm volatile("" : "+v"(soff));
    return ring[0] + soff;
  };
  // One ring tile of rows [64 DT, 64 DT + 64) of R. Row block mt (32 rows
  // starting at 64 DT + 32 mt) is zero left of column 64 DT + 32 mt, so its
  // steps start at 4 DT + 2 mt.
  auto mfma_tile = [&](auto dtc, const unsigned char* slot, f32x16 (&cur)[2][2]) {
    constexpr int DT = decltype(dtc)::value;
    constexpr int s0 = 4 * DT, s1 = 4 * DT + 2;
    bf16x8 av[2][2];
    av[s0 & 1][0] = tri_op(slot, col, hf, s0);
#pragma unroll
    for (int st = s0; st < 8; ++st) {
      if (st + 1 < 8) {
        av[(st + 1) & 1][0] = tri_op(slot, col, hf, st + 1);
        if (st + 1 >= s1) av[(st + 1) & 1][1] = tri_op(slot, 32 + col, hf, st + 1);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        cur[0][nt] = mfma32(av[st & 1][0], vop[nt][st], cur[0][nt]);
        if (st >= s1) cur[1][nt] = mfma32(av[st & 1][1], vop[nt][st], cur[1][nt]);
      }
    }
  };
  using D0 = std::integral_constant<int, 0>;
  using D1 = std::integral_constant<int, 1>;
  // pair p (tiles 2p, 2p+1: R_hi then R_lo of rows [64 DT, 64 DT + 64),
  // DT = p & 1) into fresh accumulators, folded into the sums of squares;
  // after rows [64, 128) of a g, its norm joins the sum over g
  auto pair = [&](auto dtc, int p) {
    constexpr int DT = decltype(dtc)::value;
    f32x16 acc[2][2];
    const unsigned char* slot = begin_tile(2 * p);
    if (any_key) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();
      mfma_tile(dtc, slot, acc);
    }
    slot = begin_tile(2 * p + 1);
    if (any_key) {
      mfma_tile(dtc, slot, acc);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float sum = ss[nt];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sum = __builtin_fmaf(acc[mt][nt][i], acc[mt][nt][i], sum);
        ss[nt] = sum;
      }
    }
    if (DT == 1) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float tot = ss[nt] + __shfl_xor(ss[nt], 32);   // the other 16 output rows
        wsum[nt] += __builtin_sqrtf(tot);
        ss[nt] = 0.f;
      }
    }
  };
  for (int g = 0; g < G; ++g) {
    pair(D0{}, 2 * g);
    pair(D1{}, 2 * g + 1);
  }
  gen_wait<0>();
  const float inv_g = 1.0f / (float)G;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = key0 + nt * 32 + col;
    if (hf == 0 && key < n_cand) weight[lh * n_cand + key] = wsum[nt] * inv_g;
  }
}

hipError_t value_l2_factor_launch(const void* w_o, int L, int H, int G, int D, void* factor,
                                  hipStream_t st) {
  const long long gc = (long long)L * H * G;
  if (gc > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_l2_factor, dim3((unsigned)gc), dim3(256), 0, st,
                     static_cast<const __bf16*>(w_o), D, H * G, static_cast<uint16_t*>(factor));
  return hipGetLastError();
}

hipError_t value_weight_l2_launch(const void* v, const void* factor, int L, int H, int G, int n,
                                  int n_cand, float* weight, hipStream_t st) {
  const int key_blocks = (n_cand + kL2Block - 1) / kL2Block;
  const long long blocks = (long long)key_blocks * H * L;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_value_weight_l2, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const __bf16*>(v), static_cast<const __bf16*>(factor), H, G, n,
                     n_cand, key_blocks, weight);
  return hipGetLastError();
}

}  // namespace kvsel
