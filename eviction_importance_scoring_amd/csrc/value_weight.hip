// CriticalKV's projected-value norm ([CriticalKV] §3.3 Algorithm 1 steps
// 2-3; Theorem 3.3): weight[l][h][j] = (1/G) sum_g || W_O^(h,g) v_j ||_1
// where W_O^(h,g) is the D x d column slice of the output projection that
// query head h*G+g uses. The projection V_proj = V W^O is a bf16 MFMA
// product accumulated in fp32; each 32 x 32 output tile is folded into
// per-key |.| sums in registers and never written ([CriticalKV] §D.4 notes
// the full V_proj would be ~7.8 GB per layer at 7B / 128K).
//
// Tiling: a workgroup owns 256 keys of one (layer, KV head); each of its 4
// waves holds the bf16 values of 64 keys (2 MFMA N-tiles) in registers for
// the whole kernel and streams 32-row tiles of W_O^(h,g) (the MFMA A
// operand) for every g and every 32 of the D output features. Every key's
// sum is accumulated in one lane in a fixed order: deterministic, no
// atomics.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

__global__ __launch_bounds__(256) void k_value_weight(const __bf16* __restrict__ v,
                                                      const __bf16* __restrict__ w_o,
                                                      int H, int G, int n, int D, int n_cand,
                                                      float* __restrict__ weight) {
  const int kb = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const size_t lh = (size_t)l * H + h;
  const int Hq = H * G;
  const __bf16* vh = v + lh * (size_t)n * kHeadDim;
  const __bf16* wl = w_o + (size_t)l * D * (size_t)Hq * kHeadDim;

  bf16x8 b[2][8];
  int key[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    key[nt] = kb * 256 + wave * 64 + nt * 32 + col;
    if (key[nt] < n_cand) load_half_row(vh + (size_t)key[nt] * kHeadDim, hf, b[nt]);
    else zero_ops(b[nt]);
  }
  float part[2] = {0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    const __bf16* wg = wl + (size_t)(h * G + g) * kHeadDim;   // column slice of this query head
    for (int mt = 0; mt < D; mt += 32) {
      bf16x8 a[8];
      load_half_row(wg + (size_t)(mt + col) * Hq * kHeadDim, hf, a);
      f32x16 acc0 = zero16(), acc1 = zero16();
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        acc0 = mfma32(a[st], b[0][st], acc0);
        acc1 = mfma32(a[st], b[1][st], acc1);
      }
      float t0 = 0.f, t1 = 0.f;   // per-tile partials keep the fp32 sums short
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        t0 += fabsf(acc0[i]);
        t1 += fabsf(acc1[i]);
      }
      part[0] += t0;
      part[1] += t1;
    }
  }
  const float inv_g = 1.0f / (float)G;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float tot = part[nt] + __shfl_xor(part[nt], 32);   // the other 16 output rows
    if (hf == 0 && key[nt] < n_cand) weight[lh * n_cand + key[nt]] = tot * inv_g;
  }
}

hipError_t value_weight_launch(const void* v, const void* w_o, int L, int H, int G, int n,
                               int D, int n_cand, float* weight, hipStream_t st) {
  dim3 grid((n_cand + 255) / 256, H, L);
  hipLaunchKernelGGL(k_value_weight, grid, dim3(256), 0, st, static_cast<const __bf16*>(v),
                     static_cast<const __bf16*>(w_o), H, G, n, D, n_cand, weight);
  return hipGetLastError();
}

}  // namespace kvsel
