// Top-k selection of cache entries, per head or per layer.
//
// [CriticalKV] §3.3: Algorithm 2 step 6 (Top_k of the pooled window score,
// the window kept) and Algorithm 1 steps 3-9 (stage 1: floor(alpha*k) by
// attention score; stage 2: the rest by (A + eps) * ||V W^O||_1 among the
// remaining entries). [KVzip] §4.2: one budget per layer across its heads.
//
// Each segment (a head, or a whole layer when adaptive) is one workgroup of
// 1024 threads. The order is the 63-bit key (score bits << 31) | (2^31-1-f)
// over the flat candidate index f: a larger score wins, equal scores go to
// the lower index (lower head first when adaptive), and no two keys tie.
// The score bits are an order-preserving 32-bit image of the float (sign
// bit flipped for positives, all bits flipped for negatives, -0 as +0), so
// any finite score orders as its value, negative ones included (the
// softmax-free logit scores of [KVzip] §6.5); NaN counts as below every
// number. The k-th key is found by MSD radix select with 11/11/10-bit
// digits over the score bits, then 11/11/9 over the index bits, each digit
// a 2048-bin LDS histogram; it stops as soon as the bucket that holds the
// k-th key is taken whole. Members are then (key >> shift) >= prefix.
// The final select stops after the score bits: if the last bucket (keys of
// one score) is not taken whole, its first `need` entries in index order
// are members, which the index-order emission counts with one more scan
// instead of three more rounds over the index bits (max-pooling makes such
// ties common).
// Two-stage selection runs the select twice: first on the score (k1
// entries, down to a single key), then on a key where stage-1 members are
// +inf and the others carry the integrated score, which keeps exactly the
// k1 stage-1 members plus the k - k1 best of the rest.
//
// Segments of up to kResidentMax candidates are read from HBM once into
// the LDS of one workgroup; longer ones are spread over many workgroups
// (below).
//
// Per-head budget vector ([CriticalKV] §4.1: HeadKV's offline per-head
// budgets): segments are heads, each with its own budget b (window
// included, clamped into [W, n]) and so its own k = b - W (and k1); a
// layer's heads are packed in order into a row of `stride` entries, and
// entries that would land at or past the row's end are not written.
#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kSelThreads = 1024;
constexpr int kBins = 2048;
constexpr int kResidentMax = 34816;          // 136 KiB of u32 keys in LDS (< 2^16)
constexpr int kMaxGroups = 1024;             // heads per segment
constexpr uint32_t kInfBits = 0xFF800000u;     // score bits of +inf
constexpr int kLoadUnroll = 8;              // loads in flight per thread
constexpr int kMaxPer = 35;                  // candidates a thread emits (odd)

struct SelArgs {
  const float* scores;
  const float* weight;
  int32_t* idx;
  int32_t* head_offsets;
  uint8_t* stage;
  const int32_t* budgets;   // [L][H] or null
  uint32_t seg_len, n_cand, groups, W, n, H;
  uint32_t k, k1;
  int64_t budget, stride;
  int two_stage;
  float score_norm, eps, alpha;
};

// What segment `seg` selects and where it writes. Without a budget vector:
// the call's k, k1 and budget, at seg * budget. With one (a segment is a
// head): the head's clamped budget b, k = b - W, k1 = floor(alpha k) in
// double (as the host computes it), packed after the layer's earlier heads.
struct SegSpan {
  uint32_t k, k1;     // k1 = 0xFFFFFFFF: single stage
  int64_t base;       // first output entry of the segment
  int64_t room;       // entries it may write (its budget, cut at the row's end)
  int64_t off, end;   // budget vector: [off, end) in the layer row, clipped to it
};

__device__ __forceinline__ int64_t clamp_budget(int32_t b, uint32_t W, uint32_t n) {
  return b < (int32_t)W ? (int64_t)W : (b > (int32_t)n ? (int64_t)n : (int64_t)b);
}

template <class A>
__device__ __forceinline__ SegSpan seg_span(const A& a, size_t seg) {
  SegSpan s;
  if (!a.budgets) {
    s.k = a.k;
    s.k1 = a.k1;
    s.base = (int64_t)seg * a.budget;
    s.room = a.budget;
    s.off = 0;
    s.end = a.budget;
    return s;
  }
  const size_t l = seg / a.H;
  const uint32_t h = (uint32_t)(seg - l * a.H);
  const int32_t* bl = a.budgets + l * a.H;
  int64_t off = 0;
  for (uint32_t j = 0; j < h; ++j) off += clamp_budget(bl[j], a.W, a.n);
  const int64_t b = clamp_budget(bl[h], a.W, a.n);
  s.k = (uint32_t)(b - a.W);
  s.k1 = a.weight ? (uint32_t)floor((double)a.alpha * (double)s.k) : 0xFFFFFFFFu;
  s.off = min(off, a.stride);
  s.end = min(off + b, a.stride);
  s.base = (int64_t)l * a.stride + s.off;
  s.room = s.end - s.off;
  return s;
}

// Budget vector: the layer row past the last head is filled with -1 (a
// stage byte of 0) by the last head's segment.
__device__ __forceinline__ void fill_row_tail(int32_t* idx, uint8_t* stage, int64_t row0,
                                              int64_t from, int64_t stride, int tid, int nthreads) {
  for (int64_t o = from + tid; o < stride; o += nthreads) {
    idx[row0 + o] = -1;
    if (stage) stage[row0 + o] = 0;
  }
}

// The resident select's digit histogram: kHistCopies copies of 16-bit
// counters, two bins a word (bin 2w in the low half of word w, 2w+1 in the
// high half). Lane l adds to copy l % kHistCopies, so the lanes of one
// atomic instruction that hit the same bin (common on the first digit,
// where keys crowd a few exponent bins) are spread over that many words;
// copies lie kCopyWords apart, an odd count, so those words sit in
// different banks. A copy sees at most ceil(len / kHistCopies) keys, which
// keeps every counter below 2^16.
constexpr int kHistCopies = 4;
constexpr int kCopyWords = kBins / 2 + 1;
static_assert((kResidentMax + kHistCopies * kSelThreads) / kHistCopies < 65536, "16-bit counters");

struct alignas(16) SelShared {   // a multiple of 16 bytes: the keys follow it
  uint32_t hist[kHistCopies * kCopyWords];
  uint32_t sbuf[32];
  uint32_t group_start[kMaxGroups];
  uint64_t prefix;
  int shift;
  uint32_t need;
  uint32_t digit, above, dcount;
};

// Order-preserving 32-bit image of a score: larger value, larger bits.
__device__ __forceinline__ uint32_t score_bits(float x) {
  if (x != x) return 0u;                      // NaN: below everything
  if (x == 0.f) return 0x80000000u;           // -0 and +0 alike
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(uint32_t bits, uint32_t f) {
  return ((uint64_t)bits << 31) | (uint64_t)(0x7FFFFFFFu - f);
}

// Integrated score of [CriticalKV] Algorithm 1 step 3 in fp32: mul, add,
// mul, each rounded once to nearest-even. HIP's __fmul_rn / __fadd_rn are
// plain operators, which the compiler's default contraction would fuse
// into one fma (a single rounding of s*norm + eps); the pragma keeps the
// three operations separate.
__device__ __forceinline__ uint32_t stage2_bits(float s, float w, float norm, float eps) {
#pragma clang fp contract(off)
  const float t = s * norm;
  const float u = t + eps;
  return score_bits(u * w);
}

__device__ __forceinline__ int digit_width(int shift) {
  return shift == 41 ? 10 : (shift == 9 ? 9 : 11);   // 63->52->41->31->20->9->0
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global stores (a plain __syncthreads would drain
// the output stores of every emission round).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Result of one radix-select stage. done: exactly k keys satisfy
// (key >> shift) >= prefix. Otherwise the rounds stopped at shift 31 (the
// score bits): the keys with (key >> 31) > prefix are members, and so are
// the first `need` keys, in index order, of those with (key >> 31) ==
// prefix (the index part of the key orders equal scores that way).
struct SelCut {
  uint64_t prefix;
  int shift;
  uint32_t need;
  bool done;
};

// One stage of radix select over the segment's resident key bits, down to
// stop_shift at most (0: to a single key).
__device__ SelCut radix_select(SelShared& sm, const uint32_t* bits, uint32_t len, uint32_t k,
                               int stop_shift) {
  const int tid = threadIdx.x;
  if (k == 0 || k == len)   // nothing ((key >> 63) >= 1 never holds), or everything
    return SelCut{(k == 0) ? uint64_t(1) : uint64_t(0), 63, 0u, true};
  if (tid == 0) {
    sm.prefix = 0;
    sm.shift = 63;
    sm.need = k;
  }
  __syncthreads();
  for (;;) {
    const uint64_t prefix = sm.prefix;
    const int shift = sm.shift;
    const uint32_t need = sm.need;
    const int wdt = digit_width(shift);
    const int nb = 1 << wdt;
    for (int w = tid; w < kHistCopies * kCopyWords; w += kSelThreads) sm.hist[w] = 0;
    __syncthreads();
    const uint32_t cbase = (uint32_t)(tid & (kHistCopies - 1)) * kCopyWords;
    if (shift - wdt >= 31 && (len & 3u) == 0) {
      // the digit lies in the score bits: 32-bit compares on 4 keys a read
      const uint32_t sh = shift - 31, dsh = shift - wdt - 31, p32 = (uint32_t)prefix;
      const u32x4* b4 = reinterpret_cast<const u32x4*>(bits);
      for (uint32_t i = tid; i < (len >> 2); i += kSelThreads) {
        const u32x4 v = b4[i];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((uint32_t)((uint64_t)v[c] >> sh) == p32) {   // sh may be 31
            const uint32_t bin = (v[c] >> dsh) & (nb - 1);
            atomicAdd(&sm.hist[cbase + (bin >> 1)], 1u << ((bin & 1u) << 4));
          }
      }
    } else {
      for (uint32_t f = tid; f < len; f += kSelThreads) {
        const uint64_t key = make_key(bits[f], f);
        if ((key >> shift) == prefix) {
          const uint32_t bin = (uint32_t)(key >> (shift - wdt)) & (nb - 1);
          atomicAdd(&sm.hist[cbase + (bin >> 1)], 1u << ((bin & 1u) << 4));
        }
      }
    }
    __syncthreads();
    // bins in descending order: thread t holds bins nb-1-2t and nb-2-2t,
    // the high and low halves of word nb/2-1-t in every copy
    const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
    uint32_t h0 = 0u, h1 = 0u;
    if (b0 >= 0) {
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) {
        const uint32_t x = sm.hist[c * kCopyWords + (b0 >> 1)];
        h0 += x >> 16;
        h1 += x & 0xFFFFu;
      }
    }
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
    if (sm.need == sm.dcount || sm.shift <= stop_shift) break;
  }
  const SelCut cut{sm.prefix, sm.shift, sm.need, sm.need == sm.dcount || sm.shift == 0};
  __syncthreads();
  return cut;
}

// One workgroup per segment of at most kResidentMax candidates: the key
// bits are read from HBM once into LDS and every pass runs there.
__global__ __launch_bounds__(kSelThreads) void k_select(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelShared& sm = *reinterpret_cast<SelShared*>(smem_raw);
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem_raw + sizeof(SelShared));
  const int tid = threadIdx.x;
  const size_t seg = blockIdx.x;
  const float* sc = a.scores + seg * a.seg_len;
  const float* wt = a.weight ? a.weight + seg * a.seg_len : nullptr;
  const uint32_t len = a.seg_len;
  const SegSpan sp = seg_span(a, seg);

  // every load of a sweep in flight at once (one wait per sweep)
  if ((len & 3u) == 0) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(sc);
    u32x4* k4 = reinterpret_cast<u32x4*>(keys);
    const uint32_t n4 = len >> 2;
    for (uint32_t base = 0; base < n4; base += kLoadUnroll * kSelThreads) {
      u32x4 v[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const uint32_t i = base + u * kSelThreads + tid;
        v[u] = i < n4 ? __builtin_nontemporal_load(s4 + i) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const uint32_t i = base + u * kSelThreads + tid;
        if (i < n4)
          k4[i] = u32x4{score_bits(__uint_as_float(v[u].x)), score_bits(__uint_as_float(v[u].y)),
                        score_bits(__uint_as_float(v[u].z)), score_bits(__uint_as_float(v[u].w))};
      }
    }
  } else {
    for (uint32_t base = 0; base < len; base += kLoadUnroll * kSelThreads) {
      float v[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const uint32_t f = base + u * kSelThreads + tid;
        v[u] = f < len ? sc[f] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const uint32_t f = base + u * kSelThreads + tid;
        if (f < len) keys[f] = score_bits(v[u]);
      }
    }
  }
  __syncthreads();

  // stage 1 (two-stage only), all the way down: stage-1 membership stays a
  // test on the key, which stage 2 turns into +inf
  if (a.two_stage) {
    const SelCut c1 = radix_select(sm, keys, len, sp.k1, 0);
    for (uint32_t base = 0; base < len; base += kLoadUnroll * kSelThreads) {
      float sv[kLoadUnroll], wv[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const uint32_t f = base + u * kSelThreads + tid;
        sv[u] = f < len ? sc[f] : 0.f;
        wv[u] = f < len ? wt[f] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kLoadUnroll; ++u) {
        const uint32_t f = base + u * kSelThreads + tid;
        if (f < len)
          keys[f] = (make_key(keys[f], f) >> c1.shift) >= c1.prefix
                        ? kInfBits : stage2_bits(sv[u], wv[u], a.score_norm, a.eps);
      }
    }
    __syncthreads();
  }

  const SelCut cf = radix_select(sm, keys, len, sp.k, 31);

  // ---- emission, in index order. Thread t owns the `per` consecutive
  // candidates from t*per (per odd, so the LDS reads of a wave fall in
  // distinct banks); block scans give each thread the members (and tied
  // bucket entries) before its range. Members are staged by rank in LDS
  // (over the keys, which are no longer needed) and then written out with
  // coalesced stores.
  static_assert(((kResidentMax + kSelThreads - 1) / kSelThreads | 1) <= kMaxPer, "one 64-bit mask a thread");
  const uint32_t per = ((len + kSelThreads - 1) / kSelThreads) | 1u;
  const uint32_t f0 = min(len, tid * per), f1 = min(len, f0 + per);
  // (key >> shift) vs prefix on the score bits alone; prefix 1 at shift 63
  // (select nothing) stays out of reach of every score
  const uint32_t csh = (uint32_t)cf.shift - 31u;
  const uint32_t cp = cf.prefix > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)cf.prefix;
  // every read first (clamped in range), then branch-free tests
  uint32_t bv[kMaxPer];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) bv[j] = keys[min(f0 + j, len - 1)];
  const bool done = cf.done;
  uint64_t mmask = 0, emask = 0, imask = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const bool valid = f0 + j < f1;
    const uint32_t top = (uint32_t)((uint64_t)bv[j] >> csh);   // the select stopped at shift >= 31
    const bool eq = top == cp;
    const bool mem = valid && (top > cp || (done && eq));
    const bool tie = valid && !done && eq;
    mmask |= (uint64_t)mem << j;
    emask |= (uint64_t)tie << j;
    imask |= (uint64_t)(bv[j] == kInfBits) << j;
  }
  // one scan of (tied entries, members) before each thread's range: the
  // tied members are the first cf.need tied entries in index order, so the
  // members before the range are mem_before + min(need, tied_before)
  uint32_t tot;
  const uint32_t packed = ((uint32_t)__popcll(emask) << 16) | (uint32_t)__popcll(mmask);
  const uint32_t before = block_excl_scan(packed, sm.sbuf, tot);   // both sums < 2^16
  const uint32_t tied_before = before >> 16;
  const uint32_t need = done ? 0u : cf.need;
  uint32_t rank = (before & 0xFFFFu) + min(need, tied_before);
  for (uint64_t e = emask, t = tied_before; e != 0 && t < need; e &= e - 1, ++t)
    mmask |= e & (~e + 1);
  // staged[r] = position in its head of the member of rank r, bit 31 set
  // for a stage-2 member of the two-stage selection
  uint32_t* staged = keys;
  if (f0 < f1) {
    const uint32_t g0 = f0 / a.n_cand, gstart = g0 * a.n_cand;
    if (gstart == f0) sm.group_start[g0] = rank;   // members before each group
    for (uint32_t gs = gstart + a.n_cand; gs < f1; gs += a.n_cand)
      sm.group_start[gs / a.n_cand] = rank + (uint32_t)__popcll(mmask & ((uint64_t(1) << (gs - f0)) - 1));
    if (a.n_cand >= (uint32_t)kMaxPer) {   // at most one group boundary in the range
      const uint32_t next = gstart + a.n_cand;
      uint32_t r = rank;
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        if ((mmask >> j) & 1u) {
          const uint32_t f = f0 + j;
          const uint32_t pos = f - (f >= next ? next : gstart);
          const bool second = a.two_stage && !((imask >> j) & 1u);
          if (r < sp.k) staged[r] = pos | (second ? 0x80000000u : 0u);   // r < k always
          ++r;
        }
      }
    } else {
      uint32_t gs = gstart;
      for (uint64_t m = mmask; m != 0; m &= m - 1, ++rank) {
        const uint32_t j = (uint32_t)__builtin_ctzll(m);
        const uint32_t f = f0 + j;
        while (f >= gs + a.n_cand) gs += a.n_cand;
        const bool second = a.two_stage && !((imask >> j) & 1u);
        if (rank < sp.k) staged[rank] = (f - gs) | (second ? 0x80000000u : 0u);   // rank < k always
      }
    }
  }
  lds_barrier();
  // output slot o: group g's members then its W window entries, groups in
  // order (slot of group g's first member: group_start[g] + g*W)
  int32_t* out = a.idx + sp.base;
  uint8_t* st_out = a.stage ? a.stage + sp.base : nullptr;
  for (uint32_t o = tid; o < sp.room; o += kSelThreads) {
    uint32_t g = 0;
    if (a.groups > 1) {   // last group whose first slot is <= o
      uint32_t lo = 0, hi = a.groups - 1;
      while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (sm.group_start[mid] + mid * a.W <= o) lo = mid; else hi = mid - 1;
      }
      g = lo;
    }
    const uint32_t first = sm.group_start[g];
    const uint32_t count = (g + 1 < a.groups ? sm.group_start[g + 1] : sp.k) - first;
    const uint32_t local = o - (first + g * a.W);
    int32_t v;
    uint8_t sv;
    if (local < count) {
      const uint32_t e = staged[first + local];
      v = (int32_t)(e & 0x7FFFFFFFu);
      sv = (e >> 31) ? 2 : 1;
    } else {
      v = (int32_t)(a.n - a.W + (local - count));
      sv = 0;
    }
    out[o] = v;
    if (st_out) st_out[o] = sv;
  }
  if (a.budgets) {
    const size_t l = seg / a.H;
    const uint32_t h = (uint32_t)(seg - l * a.H);
    if (tid == 0) a.head_offsets[l * (a.H + 1) + h] = (int32_t)sp.off;
    if (h + 1 == a.H) {
      if (tid == 0) a.head_offsets[l * (a.H + 1) + a.H] = (int32_t)sp.end;
      fill_row_tail(a.idx, a.stage, (int64_t)l * a.stride, sp.end, a.stride, tid, kSelThreads);
    }
    return;
  }
  if (a.head_offsets && tid < (int)a.groups)
    a.head_offsets[seg * (a.groups + 1) + tid] = (int32_t)(sm.group_start[tid] + tid * a.W);
  if (a.head_offsets && tid == 0) a.head_offsets[seg * (a.groups + 1) + a.groups] = (int32_t)a.budget;
}

// ------------------------------------------------- many workgroups per segment
//
// Segments longer than kResidentMax (a whole layer when adaptive, or very
// long heads) would leave most CUs idle with one workgroup each, so they
// run the same MSD radix select spread over chunks of kChunk candidates:
//   k_msel_init    per segment: state (prefix, shift, need) for a stage
//                  (and, for the first, a cleared global histogram)
//   k_msel_hist    per chunk: histogram of the current digit among the
//                  candidates that match the prefix (in LDS: four copies on
//                  a stage's first digit, where keys crowd a few bins; one
//                  copy after it, where few keys match the prefix),
//                  added to the segment's global histogram
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
//   k_msel_emit    per chunk: members in index order at their ranks,
//                  staged in LDS and written with coalesced stores
// Chunks never straddle a head (group), so a group's first chunk offset is
// the number of members before the group. Every sum runs in a fixed order
// or over integers: the result is deterministic.
//
// Every thread issues all of its kPerThread loads before it uses one: a
// chunk's workgroup then waits for memory once.
constexpr int kMThreads = 256;
constexpr int kChunk = 8192;                       // candidates per chunk
constexpr int kPerThread = kChunk / kMThreads;     // 32
constexpr int kMCopies = 4;                        // LDS histogram copies, first digit

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
  const int32_t* budgets;   // [L][H] or null
  uint32_t seg_len, n_cand, groups, W, n, cpg, chunks, H;
  uint32_t k, k1;
  int64_t budget, stride;
  float score_norm, eps, alpha;
};

// Key bits of candidate f for the stage being selected, from its score s
// and weight w (stage 2 of the two-stage selection: stage-1 members are
// +inf, the rest the integrated score).
__device__ __forceinline__ uint32_t msel_bits(const MselArgs& a, const SegState& st, float s,
                                              float w, bool stage2, uint32_t f) {
  const uint32_t b = score_bits(s);
  if (!stage2) return b;
  return (make_key(b, f) >> st.s1) >= st.p1 ? kInfBits : stage2_bits(s, w, a.score_norm, a.eps);
}

// chunk c of a segment: [begin, end) in flat candidate indices
__device__ __forceinline__ void msel_chunk(const MselArgs& a, uint32_t c, uint32_t& g,
                                           uint32_t& begin, uint32_t& end) {
  g = c / a.cpg;
  const uint32_t cc = c - g * a.cpg;
  begin = g * a.n_cand + cc * kChunk;
  end = min(begin + (uint32_t)kChunk, (g + 1) * a.n_cand);
}

// The thread's kPerThread candidates f = begin + i * kMThreads + tid (in
// range: f < end; coalesced), all loads issued before the first is used;
// out-of-range slots read 0.
__device__ __forceinline__ void msel_load(const MselArgs& a, uint32_t seg, uint32_t begin,
                                          uint32_t end, bool stage2, float (&s)[kPerThread],
                                          float (&w)[kPerThread]) {
  const float* sc = a.scores + (size_t)seg * a.seg_len;
  const float* wt = a.weight ? a.weight + (size_t)seg * a.seg_len : nullptr;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t f = begin + i * kMThreads + threadIdx.x;
    s[i] = f < end ? sc[f] : 0.f;
    w[i] = (stage2 && f < end) ? wt[f] : 0.f;
  }
}

// stage 1 (or the single stage): prefix 0 / need k. stage 2: keep the
// stage-1 result in (p1, s1) first. grid segments, block 256; stage 1 also
// clears the segment's global histogram (the workspace may hold anything;
// each pick clears the bins it read).
__global__ __launch_bounds__(kMThreads) void k_msel_init(MselArgs a, int stage2) {
  const uint32_t seg = blockIdx.x;
  if (!stage2) {
    uint32_t* gh = a.ghist + (size_t)seg * kBins;
    for (int b = threadIdx.x; b < kBins; b += kMThreads) gh[b] = 0u;
  }
  if (threadIdx.x != 0) return;
  SegState& st = a.states[seg];
  if (stage2) {
    st.p1 = st.prefix;
    st.s1 = st.shift;
  } else {
    st.p1 = 1;          // no stage-1 members when single-stage
    st.s1 = 63;
  }
  const SegSpan sp = seg_span(a, (size_t)seg);
  const uint32_t k = (stage2 || sp.k1 == 0xFFFFFFFFu) ? sp.k : sp.k1;
  st.shift = 63;
  if (k == 0) {          // nothing: (key >> 63) >= 1 holds for no key
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

// grid chunks*segments (1-D), block 256
template <int COPIES>
__global__ __launch_bounds__(kMThreads) void k_msel_hist(MselArgs a, int stage2) {
  __shared__ uint32_t hist[COPIES][kBins];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = a.states[seg];
  if (st.done) return;
  const int tid = threadIdx.x;
  const int shift = st.shift, wdt = digit_width(shift), nb = 1 << wdt;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  float s[kPerThread], w[kPerThread];
  msel_load(a, seg, begin, end, stage2 != 0, s, w);
#pragma unroll
  for (int cp = 0; cp < COPIES; ++cp)
    for (int b = tid; b < nb; b += kMThreads) hist[cp][b] = 0;
  __syncthreads();
  uint32_t* hc = hist[tid & (COPIES - 1)];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t f = begin + i * kMThreads + tid;
    if (f < end) {
      const uint64_t key = make_key(msel_bits(a, st, s[i], w[i], stage2 != 0, f), f);
      if ((key >> shift) == st.prefix)
        atomicAdd(&hc[(uint32_t)(key >> (shift - wdt)) & (nb - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.ghist + (size_t)seg * kBins;
  for (int b = tid; b < nb; b += kMThreads) {
    uint32_t v = 0;
#pragma unroll
    for (int cp = 0; cp < COPIES; ++cp) v += hist[cp][b];
    if (v) atomicAdd(gh + b, v);
  }
}

// grid segments, block 256: thread t owns bins nb-1-8t .. nb-8-8t
// (descending); exactly one thread holds the bin where the count of larger
// keys first reaches need
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
  const SegSpan sp = seg_span(a, (size_t)seg);
  int32_t* out = a.idx + sp.base;
  uint8_t* st_out = a.stage ? a.stage + sp.base : nullptr;
  for (uint32_t g = 0; g < a.groups; ++g) {
    const uint32_t end_rank = (g + 1 < a.groups) ? gstart[g + 1] : sp.k;
    const int64_t end = (int64_t)end_rank + (int64_t)(g + 1) * a.W;
    for (uint32_t t = tid; t < a.W; t += kMThreads) {
      const int64_t o = end - a.W + t;
      if (o >= 0 && o < sp.room) {
        out[o] = (int32_t)(a.n - a.W + t);
        if (st_out) st_out[o] = 0;
      }
    }
    if (a.head_offsets && !a.budgets && tid == 0)
      a.head_offsets[(size_t)seg * (a.groups + 1) + g] = (int32_t)(gstart[g] + g * a.W);
  }
  if (a.budgets) {
    const size_t l = seg / a.H;
    const uint32_t h = (uint32_t)(seg - l * a.H);
    if (tid == 0) a.head_offsets[l * (a.H + 1) + h] = (int32_t)sp.off;
    if (h + 1 == a.H) {
      if (tid == 0) a.head_offsets[l * (a.H + 1) + a.H] = (int32_t)sp.end;
      fill_row_tail(a.idx, a.stage, (int64_t)l * a.stride, sp.end, a.stride, tid, kMThreads);
    }
    return;
  }
  if (a.head_offsets && tid == 0)
    a.head_offsets[(size_t)seg * (a.groups + 1) + a.groups] = (int32_t)a.budget;
}

// grid chunks*segments, block 256: per chunk, entries above the bucket and in it
__global__ __launch_bounds__(kMThreads) void k_msel_count(MselArgs a, int stage2) {
  __shared__ uint32_t sbuf[kMThreads / 64];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = a.states[seg];
  const int tid = threadIdx.x;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  float s[kPerThread], w[kPerThread];
  msel_load(a, seg, begin, end, stage2 != 0, s, w);
  uint32_t na = 0, ne = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t f = begin + i * kMThreads + tid;
    if (f < end) {
      bool above, eq;
      msel_class(st, msel_bits(a, st, s[i], w[i], stage2 != 0, f), f, above, eq);
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

// LDS slot of chunk element e: one pad word per 32, so that a thread
// reading its own 32 consecutive elements and a wave writing 64
// consecutive ones both hit distinct banks
__device__ __forceinline__ uint32_t emit_slot(uint32_t e) { return e + (e >> 5); }

// grid chunks*segments, block 256: thread t takes kPerThread consecutive
// candidates of the chunk (their key bits staged through LDS from
// coalesced loads); block scans of the per-thread bucket and member counts
// give each bucket entry its tie rank and each member its rank, in index
// order. The chunk's members take consecutive output slots: they are
// staged by rank in LDS and stored with coalesced writes.
__global__ __launch_bounds__(kMThreads) void k_msel_emit(MselArgs a, int stage2) {
  __shared__ uint32_t bits[kChunk + kChunk / 32];
  __shared__ uint32_t sbuf[kMThreads / 64];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = a.states[seg];
  const uint32_t need = st.done ? 0u : st.need;
  const int tid = threadIdx.x;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  {
    float s[kPerThread], w[kPerThread];
    msel_load(a, seg, begin, end, stage2 != 0, s, w);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const uint32_t e = i * kMThreads + tid;
      const uint32_t f = begin + e;
      bits[emit_slot(e)] = f < end ? msel_bits(a, st, s[i], w[i], stage2 != 0, f) : 0u;
    }
  }
  __syncthreads();
  uint32_t amask = 0, emask = 0, ne = 0, imask = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const uint32_t e = tid * kPerThread + j;
    const uint32_t f = begin + e;
    if (f < end) {
      const uint32_t b = bits[emit_slot(e)];
      bool above, eq;
      msel_class(st, b, f, above, eq);
      amask |= (uint32_t)above << j;
      emask |= (uint32_t)eq << j;
      imask |= (uint32_t)(b == kInfBits) << j;
      ne += eq;
    }
  }
  const uint32_t* cc = a.ccount + ((size_t)seg * a.chunks + c) * 2;
  const uint32_t rank0 = cc[0], eq0 = cc[1];
  uint32_t tot;
  uint32_t tierank = eq0 + block_scan256(ne, sbuf, tot);   // bucket entries before this thread's
  uint32_t mmask = amask;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (emask & (1u << j)) {
      if (tierank < need) mmask |= 1u << j;
      ++tierank;
    }
  }
  uint32_t count;
  uint32_t r = block_scan256((uint32_t)__popc(mmask), sbuf, count);   // members before this thread's
  // staged[r] = position in its head of the chunk's member of rank r, bit
  // 31 set for a stage-2 member of the two-stage selection (the key bits
  // are no longer needed: every thread has classified its entries before
  // the scans' barriers)
  uint32_t* staged = bits;
  const uint32_t pos0 = begin - g * a.n_cand + tid * kPerThread;
  for (uint32_t m = mmask; m != 0; m &= m - 1, ++r) {
    const uint32_t j = (uint32_t)__builtin_ctz(m);
    const bool second = stage2 && !((imask >> j) & 1u);
    staged[r] = (pos0 + j) | (second ? 0x80000000u : 0u);
  }
  __syncthreads();
  const SegSpan sp = seg_span(a, (size_t)seg);
  int32_t* out = a.idx + sp.base;
  uint8_t* st_out = a.stage ? a.stage + sp.base : nullptr;
  const int64_t o0 = (int64_t)rank0 + (int64_t)g * a.W;
  for (uint32_t i = tid; i < count; i += kMThreads) {
    const int64_t o = o0 + i;
    if (o < sp.room) {   // k members fit the budget; the room may be cut at the row's end
      const uint32_t e = staged[i];
      out[o] = (int32_t)(e & 0x7FFFFFFFu);
      if (st_out) st_out[o] = (e >> 31) ? 2 : 1;
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
  a.budgets = p.budgets;
  a.H = (uint32_t)p.H;
  a.stride = p.stride;
  a.alpha = p.alpha;
  if (p.budgets) a.head_offsets = head_offsets;
  const long long blocks = (long long)m.chunks * p.segments;
  if (blocks > 0x7fffffffLL || p.segments > 0x7fffffff) return hipErrorInvalidConfiguration;
  // the global histograms start cleared (by a kernel, not a memset, so
  // the call can be captured in a graph); each pick clears what it read
  const dim3 gc((unsigned)blocks), gp(p.segments);
  const int stages = p.two_stage ? 2 : 1;
  for (int stg = 0; stg < stages; ++stg) {
    const int stage2 = stg == 1 ? 1 : 0;
    // the final stage stops after the score bits (ties split in emission)
    const int rounds = stg + 1 < stages ? 6 : 3;
    hipLaunchKernelGGL(k_msel_init, gp, dim3(kMThreads), 0, st, a, stage2);
    for (int r = 0; r < rounds; ++r) {
      if (r == 0)
        hipLaunchKernelGGL(k_msel_hist<kMCopies>, gc, dim3(kMThreads), 0, st, a, stage2);
      else
        hipLaunchKernelGGL(k_msel_hist<1>, gc, dim3(kMThreads), 0, st, a, stage2);
      hipLaunchKernelGGL(k_msel_pick, gp, dim3(kMThreads), 0, st, a);
    }
  }
  const int final2 = p.two_stage ? 1 : 0;
  hipLaunchKernelGGL(k_msel_count, gc, dim3(kMThreads), 0, st, a, final2);
  hipLaunchKernelGGL(k_msel_offsets, gp, dim3(kMThreads), 0, st, a);
  hipLaunchKernelGGL(k_msel_emit, gc, dim3(kMThreads), 0, st, a, final2);
  return hipGetLastError();
}

static size_t lds_bytes(uint32_t len) { return sizeof(SelShared) + (size_t)len * sizeof(uint32_t); }
static_assert(sizeof(SelShared) + (size_t)kResidentMax * sizeof(uint32_t) <= 160 * 1024,
              "a resident segment and the shared state fit the CU's LDS");

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
  a.budgets = p.budgets;
  a.H = (uint32_t)p.H;
  a.stride = p.stride;
  a.alpha = p.alpha;
  if (p.budgets) a.head_offsets = head_offsets;
  if (use_multi(p)) return msel_launch(p, scores, weight, idx, head_offsets, stage, ws, st);
  const size_t lds = lds_bytes(a.seg_len);
  const hipError_t e =
      hipFuncSetAttribute((const void*)k_select, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select, dim3(p.segments), dim3(kSelThreads), lds, st, a);
  return hipGetLastError();
}

bool select_groups_ok(int groups) { return groups <= kMaxGroups; }

}  // namespace kvsel
