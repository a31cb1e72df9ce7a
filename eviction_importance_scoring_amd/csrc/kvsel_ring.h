// LDS-ring MFMA building blocks of the 8-wave kernels (general scoring,
// value weight), gfx950 only.
//
// A workgroup of gWaves waves streams a shared [rows][128] bf16 operand in
// 64-row tiles through a ring of gSlots LDS slots. Slots are filled with
// direct-to-LDS loads (buffer_load_dwordx4 ... lds): each instruction
// moves 4 whole 256-byte rows, the 16-byte pieces of row r stored XOR-
// swizzled by (r & 15) so that the MFMA operand reads (one half row per
// lane) are free of bank conflicts. Each wave multiplies every tile by its
// own register-resident operand (two 32-column MFMA tiles), 32x32x16 bf16
// MFMAs with fp32 accumulation.
//
// Ordering: a wave waits for its own loads of a tile (vmcnt), then all
// waves meet at a fence-free barrier, after which the tile is complete in
// LDS and the slot read two tiles ago may be refilled.
#pragma once

#include "kvsel_internal.h"

namespace kvsel {

constexpr int gTile = 64;                                     // rows per ring slot (16 KB)
constexpr int gSlots = 3;
constexpr int gWaves = 8;
constexpr int gBlock = gWaves * 64;                           // rows / keys per workgroup
constexpr int gLoads = gTile * kRowBytes / (gWaves * 1024);   // 16-byte loads per lane per tile
constexpr int gRowsBytes = gTile * kRowBytes;
static_assert(gSlots >= 2, "ring depth");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* glb_ptr_t;

// Workgroup barrier without the vmcnt(0) that __syncthreads implies (the
// ring's loads stay in flight across it); LDS visibility comes from the
// explicit waits below. It does not wait for the wave's own ds_write
// operations either, so the kernels built on it write LDS only through the
// direct-to-LDS loads.
__device__ __forceinline__ void gen_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (vmcnt is 6 bits: low 4 in [3:0], high 2 in [15:14]).
template <int N>
__device__ __forceinline__ void gen_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int PER, int A>
__device__ __forceinline__ void gen_wait_ahead(int ahead) {
  if constexpr (A == 0) {
    gen_wait<0>();
  } else {
    if (ahead >= A) gen_wait<A * PER>();
    else gen_wait_ahead<PER, A - 1>(ahead);
  }
}

// Wait for this wave's loads of tile t (PER loads per tile). The prologue
// issues gSlots-1 tile loads (repeating the last tile when there are fewer
// tiles) and iteration t' issues tile t'+gSlots-1 when it exists, all in
// order; the loads issued after tile t's may stay in flight.
template <int PER>
__device__ __forceinline__ void gen_wait_tile(int t, int ntiles) {
  const int issued = gSlots - 1 + max(0, min(t, ntiles - gSlots + 1));
  gen_wait_ahead<PER, gSlots - 2>(issued - (t + 1));
}

// This wave's share (kLoads chunks of 1 KB, chunk c = tile rows 4c..4c+3)
// of rows [row0, row0 + 64) of a bf16 matrix with `rows` rows of 128
// elements, `stride` elements apart, into `slot`, for a workgroup of NW
// waves. Loads go through a raw buffer resource based at the tile's first
// row and ending after row rows-1: the lane offsets (row r = 4c + lane/16,
// swizzled piece) are fixed per kernel, so a tile costs no vector
// instructions, and rows past the end are cut off by the hardware range
// check (their results are never used). The whole matrix must span less
// than 2^31 bytes (checked by the API).
[[maybe_unused]] constexpr int kRawBufferWord3 = 0x00020000;   // untyped 32-bit data format
template <int NW>
struct RingLoader {
  static constexpr int kLoads = gTile * kRowBytes / (NW * 1024);
  uint32_t off[kLoads];
  __device__ __forceinline__ void init(int stride) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = (wave * kLoads + i) * 4 + (lane >> 4);
      off[i] = (uint32_t)r * (uint32_t)stride * 2u + (uint32_t)(((lane & 15) ^ (r & 15)) << 4);
    }
  }
  // row0 < rows
  __device__ __forceinline__ void issue(const __bf16* base, int row0, int rows, int stride,
                                        unsigned char* slot) const {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer resources exist only in the device pass
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bytes = ((rows - 1 - row0) * stride + kHeadDim) * 2;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(base + (size_t)row0 * stride), 0, bytes, kRawBufferWord3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(slot + (wave * kLoads + i) * 1024), 16,
                                               off[i], 0, 0, 0);
#endif
  }
};
using GenLoader = RingLoader<gWaves>;
static_assert(GenLoader::kLoads == gLoads, "loads per lane per tile");

// MFMA operand of step s, lane half hf, for row r of a ring slot.
__device__ __forceinline__ bf16x8 gen_op(const unsigned char* slot, int r, int hf, int s) {
  return ld16(slot + r * kRowBytes + (((hf * 8 + s) ^ (r & 15)) << 4));
}

__device__ __forceinline__ float gmax3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// MFMA step st of one 64-row ring tile against this wave's two 32-column
// operand sets: acc[mt][nt] += (slot rows [32mt, 32mt + 32)) x b[nt], over
// head-dim slice st. a[] holds the step's two row operands.
__device__ __forceinline__ void tile_step(const bf16x8 (&a)[2], const bf16x8 (&b)[2][8], int st,
                                          f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    acc[0][nt] = mfma32(a[0], b[nt][st], acc[0][nt]);
    acc[1][nt] = mfma32(a[1], b[nt][st], acc[1][nt]);
  }
}

__device__ __forceinline__ void read_step(const unsigned char* slot, int col, int hf, int st,
                                          bf16x8 (&a)[2]) {
  a[0] = gen_op(slot, col, hf, st);
  a[1] = gen_op(slot, 32 + col, hf, st);
}

}  // namespace kvsel
