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
        if (o < a.budget) {   // exactly k members: always true; never write past the segment
          out[o] = (int32_t)pos;
          if (st_out) st_out[o] = (!a.two_stage || bf == kInfBits) ? 1 : 2;
        }
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
      if (end - a.W + t < a.budget) {
        out[end - a.W + t] = (int32_t)(a.n - a.W + t);
        if (st_out) st_out[end - a.W + t] = 0;
      }
    }
    if (a.head_offsets && tid == 0) a.head_offsets[seg * (a.groups + 1) + g] = sm.group_start[g] + g * a.W;
  }
  if (a.head_offsets && tid == 0) a.head_offsets[seg * (a.groups + 1) + a.groups] = (int32_t)a.budget;
}

// ------------------------------------------------- many workgroups per segment
//
// Segments longer than kResidentMax (a whole layer when adaptive, or very
// long heads) would leave most CUs idle with one workgroup each, so they
// run the same MSD radix select spread over chunks of kChunk candidates:
//   k_msel_init    per segment: state (prefix, shift, need) for a stage
//   k_msel_hist    per chunk: LDS histogram of the current digit among the
//                  candidates that match the prefix, added to the
//                  segment's global histogram
//   k_msel_pick    per segment: the bin holding the need-th largest key
//                  (bins read in descending order), the next state, and a
//                  cleared histogram for the next digit
// A segment whose bucket is taken whole is done and later rounds return at
// once. The final stage runs only the three rounds of the 31 score bits:
// if the last bucket (keys with equal score bits b) is not taken whole,
// its first `need` entries in index order are members (the index part of
// the key orders equal scores exactly that way), which the emission
// resolves with a second scan instead of three more rounds over the index
// bits. Stage 1 of the two-stage selection runs all six rounds, so that
// its members stay a plain prefix test on the key. Emission:
//   k_msel_count   per chunk: entries above the bucket, and in it
//   k_msel_offsets per segment: exclusive scans over its chunks (members
//                  and bucket entries), head offsets, window entries
//   k_msel_emit    per chunk: members in index order at their ranks
// Chunks never straddle a head (group), so a group's first chunk offset is
// the number of members before the group. Everything is deterministic.
constexpr int kMThreads = 256;
constexpr int kChunk = 8192;                       // candidates per chunk
constexpr int kPerThread = kChunk / kMThreads;     // 32

struct alignas(16) SegState {
  uint64_t prefix;      // current stage: key prefix above `shift`
  uint64_t p1;          // stage-1 result (two-stage)
  int32_t shift, s1;
  uint32_t need, done;
};

struct MselArgs {
  const float* scores;
  const float* weight;
  SegState* states;
  uint32_t* ghist;      // [segments][kBins]
  uint32_t* ccount;     // [segments][chunks][2]: above / in the bucket
  int32_t* idx;
  int32_t* head_offsets;
  uint8_t* stage;
  uint32_t seg_len, n_cand, groups, W, n, cpg, chunks;
  uint32_t k, k1;
  int64_t budget;
  float score_norm, eps;
};

// Key bits of candidate f for the stage being selected (stage 2 of the
// two-stage selection: stage-1 members are +inf, the rest the integrated
// score).
__device__ __forceinline__ uint32_t msel_bits(const MselArgs& a, const SegState& st,
                                              const float* sc, const float* wt, bool stage2,
                                              uint32_t f) {
  const uint32_t b = score_bits(sc[f]);
  if (!stage2) return b;
  return (make_key(b, f) >> st.s1) >= st.p1 ? kInfBits : stage2_bits(sc[f], wt[f], a.score_norm, a.eps);
}

// chunk c of a segment: [begin, end) in flat candidate indices
__device__ __forceinline__ void msel_chunk(const MselArgs& a, uint32_t c, uint32_t& g,
                                           uint32_t& begin, uint32_t& end) {
  g = c / a.cpg;
  const uint32_t cc = c - g * a.cpg;
  begin = g * a.n_cand + cc * kChunk;
  end = min(begin + (uint32_t)kChunk, (g + 1) * a.n_cand);
}

// stage 1 (or the single stage): prefix 0 / need k. stage 2: keep the
// stage-1 result in (p1, s1) first. grid ceil(segments/256).
__global__ __launch_bounds__(kMThreads) void k_msel_init(MselArgs a, int segments, int stage2) {
  const int seg = blockIdx.x * kMThreads + threadIdx.x;
  if (seg >= segments) return;
  SegState& st = a.states[seg];
  if (stage2) {
    st.p1 = st.prefix;
    st.s1 = st.shift;
  } else {
    st.p1 = 1;          // no stage-1 members when single-stage
    st.s1 = 62;
  }
  const uint32_t k = (stage2 || a.k1 == 0xFFFFFFFFu) ? a.k : a.k1;
  st.shift = 62;
  if (k == 0) {          // nothing: (key >> 62) >= 1 holds for no key
    st.prefix = 1;
    st.need = 0;
    st.done = 1;
  } else if (k >= a.seg_len) {   // everything
    st.prefix = 0;
    st.need = 0;
    st.done = 1;
  } else {
    st.prefix = 0;
    st.need = k;
    st.done = 0;
  }
}

// grid segments, block 256: a segment's global histogram to zero
__global__ __launch_bounds__(kMThreads) void k_msel_clear(MselArgs a) {
  uint32_t* gh = a.ghist + (size_t)blockIdx.x * kBins;
  for (int b = threadIdx.x; b < kBins; b += kMThreads) gh[b] = 0u;
}

// grid chunks*segments (1-D), block 256
__global__ __launch_bounds__(kMThreads) void k_msel_hist(MselArgs a, int stage2) {
  __shared__ uint32_t hist[kBins];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = a.states[seg];
  if (st.done) return;
  const int tid = threadIdx.x;
  const int shift = st.shift, wdt = digit_width(shift), nb = 1 << wdt;
  for (int b = tid; b < nb; b += kMThreads) hist[b] = 0;
  __syncthreads();
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  const float* sc = a.scores + (size_t)seg * a.seg_len;
  const float* wt = a.weight ? a.weight + (size_t)seg * a.seg_len : nullptr;
#pragma unroll 8
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t f = begin + i * kMThreads + tid;
    if (f < end) {
      const uint64_t key = make_key(msel_bits(a, st, sc, wt, stage2 != 0, f), f);
      if ((key >> shift) == st.prefix)
        atomicAdd(&hist[(uint32_t)(key >> (shift - wdt)) & (nb - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.ghist + (size_t)seg * kBins;
  for (int b = tid; b < nb; b += kMThreads)
    if (hist[b]) atomicAdd(&gh[b], hist[b]);
}

// grid segments, block 256: thread t owns bins nb-1-8t .. nb-8-8t (descending)
__global__ __launch_bounds__(kMThreads) void k_msel_pick(MselArgs a) {
  __shared__ uint32_t sbuf[kMThreads / 64];
  __shared__ uint32_t s_digit, s_above, s_count;
  const uint32_t seg = blockIdx.x;
  SegState& st = a.states[seg];
  if (st.done) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int shift = st.shift, wdt = digit_width(shift), nb = 1 << wdt;
  const uint32_t need = st.need;
  uint32_t* gh = a.ghist + (size_t)seg * kBins;
  uint32_t h[8], sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int b = nb - 1 - 8 * tid - j;
    h[j] = b >= 0 ? gh[b] : 0u;
    sum += h[j];
  }
  // exclusive scan of the per-thread sums (descending bin order)
  uint32_t x = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  uint32_t above = x - sum;
  for (int w = 0; w < wave; ++w) above += sbuf[w];
  if (above < need && need <= above + sum) {   // exactly one thread
    uint32_t acc = above;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (acc < need && need <= acc + h[j]) {
        s_digit = (uint32_t)(nb - 1 - 8 * tid - j);
        s_above = acc;
        s_count = h[j];
      }
      acc += h[j];
    }
  }
  __syncthreads();
  // clear this digit's bins for the next round
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int b = nb - 1 - 8 * tid - j;
    if (b >= 0) gh[b] = 0u;
  }
  if (tid == 0) {
    st.prefix = (st.prefix << wdt) | s_digit;
    st.shift = shift - wdt;
    st.need = need - s_above;
    st.done = (st.need == s_count || st.shift == 0) ? 1u : 0u;
  }
}

// Membership classes of a key after the rounds: when the segment is done,
// every key with (key >> shift) >= prefix is a member ("above"); otherwise
// shift == 31, prefix holds the bucket's score bits, keys with larger score
// bits are members and keys with equal ones are in the bucket, of which
// the first `need` (index order) are members.
__device__ __forceinline__ void msel_class(const SegState& st, uint32_t bits, uint32_t f,
                                           bool& above, bool& eq) {
  const uint64_t top = make_key(bits, f) >> st.shift;
  if (st.done) {
    above = top >= st.prefix;
    eq = false;
  } else {
    above = top > st.prefix;
    eq = top == st.prefix;
  }
}

__device__ __forceinline__ uint32_t block_sum256(uint32_t v, uint32_t* sbuf) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) sbuf[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kMThreads / 64; ++w) t += sbuf[w];
  __syncthreads();
  return t;
}

// exclusive scan over the 256 threads (in thread order); total returned too
__device__ __forceinline__ uint32_t block_scan256(uint32_t v, uint32_t* sbuf, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  uint32_t off = x - v, tot = 0;
#pragma unroll
  for (int w = 0; w < kMThreads / 64; ++w) {
    off += (w < wave) ? sbuf[w] : 0u;
    tot += sbuf[w];
  }
  __syncthreads();
  total = tot;
  return off;
}

// grid chunks*segments, block 256: per chunk, entries above the bucket and in it
__global__ __launch_bounds__(kMThreads) void k_msel_count(MselArgs a, int stage2) {
  __shared__ uint32_t sbuf[kMThreads / 64];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = a.states[seg];
  const int tid = threadIdx.x;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  const float* sc = a.scores + (size_t)seg * a.seg_len;
  const float* wt = a.weight ? a.weight + (size_t)seg * a.seg_len : nullptr;
  uint32_t na = 0, ne = 0;
#pragma unroll 8
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t f = begin + i * kMThreads + tid;
    if (f < end) {
      bool above, eq;
      msel_class(st, msel_bits(a, st, sc, wt, stage2 != 0, f), f, above, eq);
      na += above;
      ne += eq;
    }
  }
  na = block_sum256(na, sbuf);
  ne = block_sum256(ne, sbuf);
  if (tid == 0) {
    a.ccount[((size_t)seg * a.chunks + c) * 2] = na;
    a.ccount[((size_t)seg * a.chunks + c) * 2 + 1] = ne;
  }
}

// grid segments, block 256: per chunk, the bucket entries before it (eqoff)
// and the members before it (memoff), both in place of the counts; head
// offsets and window entries
__global__ __launch_bounds__(kMThreads) void k_msel_offsets(MselArgs a) {
  __shared__ uint32_t sbuf[kMThreads / 64];
  __shared__ uint32_t gstart[kMaxGroups];   // members before each group
  const uint32_t seg = blockIdx.x;
  const SegState st = a.states[seg];
  const uint32_t need = st.done ? 0u : st.need;
  const int tid = threadIdx.x;
  uint32_t* cc = a.ccount + (size_t)seg * a.chunks * 2;
  uint32_t run_eq = 0, run_mem = 0;
  for (uint32_t base = 0; base < a.chunks; base += kMThreads) {
    const uint32_t c = base + tid;
    const uint32_t na = c < a.chunks ? cc[2 * c] : 0u;
    const uint32_t ne = c < a.chunks ? cc[2 * c + 1] : 0u;
    uint32_t tot_eq, tot_mem;
    const uint32_t eqoff = run_eq + block_scan256(ne, sbuf, tot_eq);
    // bucket members in this chunk: the part of [eqoff, eqoff + ne) below need
    const uint32_t tie = eqoff >= need ? 0u : min(ne, need - eqoff);
    const uint32_t memoff = run_mem + block_scan256(na + tie, sbuf, tot_mem);
    if (c < a.chunks) {
      cc[2 * c] = memoff;
      cc[2 * c + 1] = eqoff;
      if (c % a.cpg == 0) gstart[c / a.cpg] = memoff;
    }
    run_eq += tot_eq;
    run_mem += tot_mem;
  }
  __syncthreads();
  int32_t* out = a.idx + (size_t)seg * (size_t)a.budget;
  uint8_t* st_out = a.stage ? a.stage + (size_t)seg * (size_t)a.budget : nullptr;
  for (uint32_t g = 0; g < a.groups; ++g) {
    const uint32_t end_rank = (g + 1 < a.groups) ? gstart[g + 1] : a.k;
    const int64_t end = (int64_t)end_rank + (int64_t)(g + 1) * a.W;
    for (uint32_t t = tid; t < a.W; t += kMThreads) {
      const int64_t o = end - a.W + t;
      if (o >= 0 && o < a.budget) {
        out[o] = (int32_t)(a.n - a.W + t);
        if (st_out) st_out[o] = 0;
      }
    }
    if (a.head_offsets && tid == 0)
      a.head_offsets[(size_t)seg * (a.groups + 1) + g] = (int32_t)(gstart[g] + g * a.W);
  }
  if (a.head_offsets && tid == 0)
    a.head_offsets[(size_t)seg * (a.groups + 1) + a.groups] = (int32_t)a.budget;
}

// LDS slot of chunk element e: one pad word per 32, so that a thread
// reading its own 32 consecutive elements and a wave writing 64
// consecutive ones both hit distinct banks
__device__ __forceinline__ uint32_t emit_slot(uint32_t e) { return e + (e >> 5); }

// grid chunks*segments, block 256: thread t takes kPerThread consecutive
// candidates of the chunk (their key bits staged through LDS from
// coalesced loads); block scans of the per-thread bucket and member counts
// give each bucket entry its tie rank and each member its rank, in index
// order
__global__ __launch_bounds__(kMThreads) void k_msel_emit(MselArgs a, int stage2) {
  __shared__ uint32_t bits[kChunk + kChunk / 32];
  __shared__ uint32_t sbuf[kMThreads / 64];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = a.states[seg];
  const uint32_t need = st.done ? 0u : st.need;
  const int tid = threadIdx.x;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  const float* sc = a.scores + (size_t)seg * a.seg_len;
  const float* wt = a.weight ? a.weight + (size_t)seg * a.seg_len : nullptr;
#pragma unroll 8
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t e = i * kMThreads + tid;
    const uint32_t f = begin + e;
    bits[emit_slot(e)] = f < end ? msel_bits(a, st, sc, wt, stage2 != 0, f) : 0u;
  }
  __syncthreads();
  uint32_t amask = 0, emask = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const uint32_t e = tid * kPerThread + j;
    const uint32_t f = begin + e;
    if (f < end) {
      bool above, eq;
      msel_class(st, bits[emit_slot(e)], f, above, eq);
      amask |= (uint32_t)above << j;
      emask |= (uint32_t)eq << j;
      ne += eq;
    }
  }
  const uint32_t* cc = a.ccount + ((size_t)seg * a.chunks + c) * 2;
  uint32_t tot;
  uint32_t tierank = cc[1] + block_scan256(ne, sbuf, tot);   // bucket entries before this thread's
  uint32_t mmask = amask;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (emask & (1u << j)) {
      if (tierank < need) mmask |= 1u << j;
      ++tierank;
    }
  }
  uint32_t rank = cc[0] + block_scan256((uint32_t)__popc(mmask), sbuf, tot);
  int32_t* out = a.idx + (size_t)seg * (size_t)a.budget;
  uint8_t* st_out = a.stage ? a.stage + (size_t)seg * (size_t)a.budget : nullptr;
  const uint32_t pos0 = begin - g * a.n_cand;
  for (int j = 0; j < kPerThread; ++j) {
    if (mmask & (1u << j)) {
      const int64_t o = (int64_t)rank + (int64_t)g * a.W;
      if (o < a.budget) {   // exactly k members: always true; never write past the segment
        out[o] = (int32_t)(pos0 + tid * kPerThread + j);
        if (st_out) st_out[o] = (!stage2 || bits[emit_slot(tid * kPerThread + j)] == kInfBits) ? 1 : 2;
      }
      ++rank;
    }
  }
}

static size_t al256s(size_t x) { return (x + 255) & ~size_t(255); }

struct MselLayout {
  uint32_t cpg, chunks;
  size_t states_off, ghist_off, ccount_off, bytes;
};

static MselLayout msel_layout(const SelectPlan& p) {
  MselLayout m;
  const uint32_t groups = p.adaptive ? (uint32_t)p.H : 1u;
  m.cpg = (uint32_t)((p.n_cand + kChunk - 1) / kChunk);
  m.chunks = groups * m.cpg;
  m.states_off = 0;
  m.ghist_off = al256s((size_t)p.segments * sizeof(SegState));
  m.ccount_off = m.ghist_off + al256s((size_t)p.segments * kBins * sizeof(uint32_t));
  m.bytes = m.ccount_off + al256s((size_t)p.segments * m.chunks * 2 * sizeof(uint32_t));
  return m;
}

static bool use_multi(const SelectPlan& p) { return p.seg_len > kResidentMax; }

static hipError_t msel_launch(const SelectPlan& p, const float* scores, const float* weight,
                              int32_t* idx, int32_t* head_offsets, uint8_t* stage, void* ws,
                              hipStream_t st) {
  const MselLayout m = msel_layout(p);
  char* w = static_cast<char*>(ws);
  MselArgs a;
  a.scores = scores;
  a.weight = p.two_stage ? weight : nullptr;
  a.states = reinterpret_cast<SegState*>(w + m.states_off);
  a.ghist = reinterpret_cast<uint32_t*>(w + m.ghist_off);
  a.ccount = reinterpret_cast<uint32_t*>(w + m.ccount_off);
  a.idx = idx;
  a.head_offsets = p.adaptive ? head_offsets : nullptr;
  a.stage = stage;
  a.seg_len = (uint32_t)p.seg_len;
  a.n_cand = (uint32_t)p.n_cand;
  a.groups = p.adaptive ? (uint32_t)p.H : 1u;
  a.W = (uint32_t)p.W;
  a.n = (uint32_t)p.n;
  a.cpg = m.cpg;
  a.chunks = m.chunks;
  a.k = (uint32_t)p.k;
  a.k1 = p.two_stage ? (uint32_t)p.k1 : 0xFFFFFFFFu;   // 0xFFFFFFFF: single stage, select k
  a.budget = p.budget;
  a.score_norm = p.score_norm;
  a.eps = p.eps;
  const long long blocks = (long long)m.chunks * p.segments;
  if (blocks > 0x7fffffffLL || p.segments > 0x7fffffff) return hipErrorInvalidConfiguration;
  // the global histograms start cleared (a kernel, not a memset, so the
  // call can be captured in a graph); each pick clears what it read
  const dim3 gs((p.segments + kMThreads - 1) / kMThreads), gc((unsigned)blocks), gp(p.segments);
  hipLaunchKernelGGL(k_msel_clear, gp, dim3(kMThreads), 0, st, a);
  const int stages = p.two_stage ? 2 : 1;
  for (int stg = 0; stg < stages; ++stg) {
    const int stage2 = stg == 1 ? 1 : 0;
    // the final stage stops after the score bits (ties split in emission)
    const int rounds = stg + 1 < stages ? 6 : 3;
    hipLaunchKernelGGL(k_msel_init, gs, dim3(kMThreads), 0, st, a, p.segments, stage2);
    for (int r = 0; r < rounds; ++r) {
      hipLaunchKernelGGL(k_msel_hist, gc, dim3(kMThreads), 0, st, a, stage2);
      hipLaunchKernelGGL(k_msel_pick, gp, dim3(kMThreads), 0, st, a);
    }
  }
  const int final2 = p.two_stage ? 1 : 0;
  hipLaunchKernelGGL(k_msel_count, gc, dim3(kMThreads), 0, st, a, final2);
  hipLaunchKernelGGL(k_msel_offsets, gp, dim3(kMThreads), 0, st, a);
  hipLaunchKernelGGL(k_msel_emit, gc, dim3(kMThreads), 0, st, a, final2);
  return hipGetLastError();
}

static size_t lds_bytes(bool resident, uint32_t len) {
  return sizeof(SelShared) + (resident ? (size_t)len * sizeof(uint32_t) : 0);
}

size_t select_ws_bytes(const SelectPlan& p) { return use_multi(p) ? msel_layout(p).bytes : 0; }

hipError_t select_launch(const SelectPlan& p, const float* scores, const float* weight,
                         int32_t* idx, int32_t* head_offsets, uint8_t* stage, void* ws,
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
  if (use_multi(p)) return msel_launch(p, scores, weight, idx, head_offsets, stage, ws, st);
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
