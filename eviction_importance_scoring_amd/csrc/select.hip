// Top-k selection of cache entries, per head or per layer.
//
// [CriticalKV] §3.3: Algorithm 2 step 6 (Top_k of the pooled window score,
// the window kept) and Algorithm 1 steps 3-9 (stage 1: floor(alpha*k) by
// attention score; stage 2: the rest by (A + eps) * ||V W^O||_1 among the
// remaining entries). [KVzip] §4.2: one budget per layer across its heads.
//
// Each segment (a head, or a whole layer when adaptive) is one workgroup of
// 1024 threads. The order is the 62-bit key (score bits << 31) | (2^31-1-f)
// over the flat candidate index f: a larger score wins, equal scores go to
// the lower index (lower head first when adaptive), and no two keys tie.
// Scores are >= 0, so their IEEE bits order like the values; negative or
// NaN inputs count as 0. The k-th key is found by MSD radix select with
// 11/11/9-bit digits over the score bits, then over the index bits, each
// digit a 2048-bin LDS histogram; it stops as soon as the bucket that holds
// the k-th key is taken whole. Members are then (key >> shift) >= prefix.
// Two-stage selection runs the select twice: first on the score (k1
// entries), then on a key where stage-1 members are +inf and the others
// carry the integrated score, which keeps exactly the k1 stage-1 members
// plus the k - k1 best of the rest.
//
// Segments of up to kResidentMax candidates are read from HBM once into
// LDS; longer ones are streamed from memory on every pass.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kSelThreads = 1024;
constexpr int kBins = 2048;
constexpr int kResidentMax = 34816;          // 136 KiB of u32 keys in LDS
constexpr int kMaxGroups = 1024;             // heads per segment
constexpr uint32_t kInfBits = 0x7F800000u;

struct SelArgs {
  const float* scores;
  const float* weight;
  int32_t* idx;
  int32_t* head_offsets;
  uint8_t* stage;
  uint32_t seg_len, n_cand, groups, W, n;
  uint32_t k, k1;
  int64_t budget;
  int two_stage;
  float score_norm, eps;
};

struct SelShared {
  uint32_t hist[kBins];
  uint32_t sbuf[32];
  uint32_t group_start[kMaxGroups];
  uint64_t prefix;
  int shift;
  uint32_t need;
  uint32_t digit, above, dcount;
};

__device__ __forceinline__ uint32_t score_bits(float x) {
  return x > 0.f ? __float_as_uint(x) : 0u;
}

__device__ __forceinline__ uint64_t make_key(uint32_t bits, uint32_t f) {
  return ((uint64_t)bits << 31) | (uint64_t)(0x7FFFFFFFu - f);
}

// Integrated score of [CriticalKV] Algorithm 1 step 3 in fp32: mul, add,
// mul, each rounded once (no contraction).
__device__ __forceinline__ uint32_t stage2_bits(float s, float w, float norm, float eps) {
  return score_bits(__fmul_rn(__fadd_rn(__fmul_rn(s, norm), eps), w));
}

__device__ __forceinline__ int digit_width(int shift) {
  return (shift == 40 || shift == 9) ? 9 : 11;   // 62->51->40->31->20->9->0
}

// Exclusive scan of v over the 1024 threads; returns the block total too.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* sbuf, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const uint32_t t = sbuf[w];
    off += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

// One stage of radix select over the segment: finds (prefix, shift) such
// that exactly k keys satisfy (key >> shift) >= prefix.
template <typename KeyFn>
__device__ void radix_select(SelShared& sm, uint32_t len, uint32_t k, KeyFn key_of,
                             uint64_t& prefix_out, int& shift_out) {
  const int tid = threadIdx.x;
  if (k == 0 || k == len) {  // nothing, or everything
    prefix_out = (k == 0) ? 1 : 0;
    shift_out = 62;
    return;
  }
  if (tid == 0) {
    sm.prefix = 0;
    sm.shift = 62;
    sm.need = k;
  }
  __syncthreads();
  for (;;) {
    const uint64_t prefix = sm.prefix;
    const int shift = sm.shift;
    const uint32_t need = sm.need;
    const int wdt = digit_width(shift);
    const int nb = 1 << wdt;
    for (int b = tid; b < kBins; b += kSelThreads) sm.hist[b] = 0;
    __syncthreads();
    for (uint32_t f = tid; f < len; f += kSelThreads) {
      const uint64_t key = key_of(f);
      if ((key >> shift) == prefix)
        atomicAdd(&sm.hist[(uint32_t)(key >> (shift - wdt)) & (nb - 1)], 1u);
    }
    __syncthreads();
    // bins in descending order: thread t holds bins nb-1-2t and nb-2-2t
    const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
    const uint32_t h0 = b0 >= 0 ? sm.hist[b0] : 0u;
    const uint32_t h1 = b1 >= 0 ? sm.hist[b1] : 0u;
    uint32_t tot;
    const uint32_t above = block_excl_scan(h0 + h1, sm.sbuf, tot);
    if (above < need && need <= above + h0) {
      sm.digit = b0;
      sm.above = above;
      sm.dcount = h0;
    } else if (above + h0 < need && need <= above + h0 + h1) {
      sm.digit = b1;
      sm.above = above + h0;
      sm.dcount = h1;
    }
    __syncthreads();
    if (tid == 0) {
      sm.prefix = (prefix << wdt) | sm.digit;
      sm.shift = shift - wdt;
      sm.need = need - sm.above;
    }
    __syncthreads();
    if (sm.need == sm.dcount || sm.shift == 0) break;
  }
  prefix_out = sm.prefix;
  shift_out = sm.shift;
  __syncthreads();
}

template <bool RESIDENT>
__global__ __launch_bounds__(kSelThreads) void k_select(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelShared& sm = *reinterpret_cast<SelShared*>(smem_raw);
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem_raw + sizeof(SelShared));
  const int tid = threadIdx.x;
  const size_t seg = blockIdx.x;
  const float* sc = a.scores + seg * a.seg_len;
  const float* wt = a.weight ? a.weight + seg * a.seg_len : nullptr;
  const uint32_t len = a.seg_len;

  if (RESIDENT) {
    for (uint32_t f = tid; f < len; f += kSelThreads) keys[f] = score_bits(sc[f]);
    __syncthreads();
  }
  auto bits1 = [&](uint32_t f) -> uint32_t {
    return RESIDENT ? keys[f] : score_bits(sc[f]);
  };

  // stage 1 (only when two-stage)
  uint64_t p1 = 1;
  int s1 = 62;
  if (a.two_stage) {
    radix_select(sm, len, a.k1, [&](uint32_t f) { return make_key(bits1(f), f); }, p1, s1);
  }
  auto member1 = [&](uint32_t f, uint32_t b1) -> bool {
    return (make_key(b1, f) >> s1) >= p1;
  };
  if (RESIDENT && a.two_stage) {
    for (uint32_t f = tid; f < len; f += kSelThreads) {
      const uint32_t b1 = keys[f];
      keys[f] = member1(f, b1) ? kInfBits : stage2_bits(sc[f], wt[f], a.score_norm, a.eps);
    }
    __syncthreads();
  }
  auto bits_final = [&](uint32_t f) -> uint32_t {
    if (RESIDENT || !a.two_stage) return bits1(f);
    const uint32_t b1 = score_bits(sc[f]);
    return member1(f, b1) ? kInfBits : stage2_bits(sc[f], wt[f], a.score_norm, a.eps);
  };

  uint64_t pf;
  int sf;
  radix_select(sm, len, a.k, [&](uint32_t f) { return make_key(bits_final(f), f); }, pf, sf);

  // ---- emission, in index order, 1024 candidates per round
  int32_t* out = a.idx + seg * (size_t)a.budget;
  uint8_t* st_out = a.stage ? a.stage + seg * (size_t)a.budget : nullptr;
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t running = 0;
  for (uint32_t base = 0; base < len; base += kSelThreads) {
    const uint32_t f = base + tid;
    bool mem = false;
    uint32_t bf = 0;
    if (f < len) {
      bf = bits_final(f);
      mem = (make_key(bf, f) >> sf) >= pf;
    }
    const uint64_t ballot = __ballot(mem);
    const uint32_t lane_rank = __builtin_amdgcn_mbcnt_hi(
        (uint32_t)(ballot >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
    if (lane == 0) sm.sbuf[wave] = __popcll(ballot);
    __syncthreads();
    uint32_t woff = 0, rtot = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      const uint32_t t = sm.sbuf[w];
      woff += (w < wave) ? t : 0u;
      rtot += t;
    }
    const uint32_t before = running + woff + lane_rank;  // members with index < f
    if (f < len) {
      const uint32_t g = f / a.n_cand, pos = f - g * a.n_cand;
      if (pos == 0) sm.group_start[g] = before;
      if (mem) {
        const uint32_t o = before + g * a.W;
        out[o] = (int32_t)pos;
        if (st_out) st_out[o] = (!a.two_stage || bf == kInfBits) ? 1 : 2;
      }
    }
    running += rtot;
    __syncthreads();
  }
  // window entries after each group's members, and the group offsets
  for (uint32_t g = 0; g < a.groups; ++g) {
    const uint32_t end_rank = (g + 1 < a.groups) ? sm.group_start[g + 1] : a.k;
    const uint32_t end = end_rank + (g + 1) * a.W;
    for (uint32_t t = tid; t < a.W; t += kSelThreads) {
      out[end - a.W + t] = (int32_t)(a.n - a.W + t);
      if (st_out) st_out[end - a.W + t] = 0;
    }
    if (a.head_offsets && tid == 0) a.head_offsets[seg * (a.groups + 1) + g] = sm.group_start[g] + g * a.W;
  }
  if (a.head_offsets && tid == 0) a.head_offsets[seg * (a.groups + 1) + a.groups] = (int32_t)a.budget;
}

static size_t lds_bytes(bool resident, uint32_t len) {
  return sizeof(SelShared) + (resident ? (size_t)len * sizeof(uint32_t) : 0);
}

size_t select_ws_bytes(const SelectPlan&) { return 0; }

hipError_t select_launch(const SelectPlan& p, const float* scores, const float* weight,
                         int32_t* idx, int32_t* head_offsets, uint8_t* stage, void*,
                         hipStream_t st) {
  SelArgs a;
  a.scores = scores;
  a.weight = p.two_stage ? weight : nullptr;
  a.idx = idx;
  a.head_offsets = p.adaptive ? head_offsets : nullptr;
  a.stage = stage;
  a.seg_len = (uint32_t)p.seg_len;
  a.n_cand = (uint32_t)p.n_cand;
  a.groups = p.adaptive ? (uint32_t)p.H : 1u;
  a.W = (uint32_t)p.W;
  a.n = (uint32_t)p.n;
  a.k = (uint32_t)p.k;
  a.k1 = (uint32_t)p.k1;
  a.budget = p.budget;
  a.two_stage = p.two_stage ? 1 : 0;
  a.score_norm = p.score_norm;
  a.eps = p.eps;
  const bool resident = p.seg_len <= kResidentMax;
  const size_t lds = lds_bytes(resident, a.seg_len);
  hipError_t e;
  if (resident) {
    e = hipFuncSetAttribute((const void*)k_select<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_select<true>, dim3(p.segments), dim3(kSelThreads), lds, st, a);
  } else {
    e = hipFuncSetAttribute((const void*)k_select<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_select<false>, dim3(p.segments), dim3(kSelThreads), lds, st, a);
  }
  return hipGetLastError();
}

bool select_groups_ok(int groups) { return groups <= kMaxGroups; }

}  // namespace kvsel
