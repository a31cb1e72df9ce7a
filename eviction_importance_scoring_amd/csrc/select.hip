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
// the registers of one workgroup; longer ones are spread over many
// workgroups (below).
//
// Per-head budget vector ([CriticalKV] §4.1: HeadKV's offline per-head
// budgets): segments are heads, each with its own budget b (window
// included, clamped into [W, n]) and so its own k = b - W (and k1); a
// layer's heads are packed in order into a row of `stride` entries, and
// entries that would land at or past the row's end are not written.
#include <type_traits>

#include "kvsel_internal.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;
constexpr int kKPT = 34;                              // keys a thread holds
constexpr int kResidentMax = kKPT * kSelThreads;      // 34,816 candidates
constexpr int kMaxGroups = 1024;             // heads per segment
constexpr uint32_t kInfBits = 0xFF800000u;     // score bits of +inf
constexpr int kMaxPoolR = 3;                 // on-chip max-pooling radius (width 7)
constexpr int kStagePad = 4;                 // floats before a staged segment

struct SelArgs {
  const float* scores;      // segment s at scores + s * in_stride
  const float* weight;      // segment s at weight + s * seg_len
  int32_t* idx;
  int32_t* head_offsets;
  uint8_t* stage;
  const int32_t* budgets;   // [L][H] or null
  float* pooled;            // resident path with pool_r > 0: pooled scores out, or null
  uint32_t seg_len, n_cand, groups, W, n, H;
  uint32_t k, k1;
  int64_t budget, stride;
  int64_t in_stride;
  int two_stage;
  int staged;               // resident path: segments staged by 16-byte loads
  int pool_r;               // resident path: max-pool radius applied on chip (0..kMaxPoolR)
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

// The resident select's digit histogram: kHistCopies copies of 32-bit
// counters, one bin a word. Lane l adds to copy l % kHistCopies, so the
// lanes of one atomic instruction that hit the same bin (common on the
// first digit, where keys crowd a few exponent bins, and wherever
// max-pooling repeats a score over neighbouring keys, which sit in
// neighbouring lanes) meet in one word at most four at a time. Copies lie
// kCopyWords apart (2 mod 32 banks), so one bin's words in different
// copies sit in different banks, and each thread's pair of bins in a copy
// is one aligned 8-byte read.
constexpr int kHistCopies = 16;
constexpr int kCopyWords = kBins + 2;
static_assert((kHistCopies * kCopyWords) % 4 == 0, "cleared in 16-byte pieces");

struct alignas(16) SelShared {
  uint32_t hist[kHistCopies * kCopyWords];
  uint32_t sbuf[32];
  uint32_t wcount[2][kSelWaves];        // per wave: members, tied entries
  uint32_t group_start[kMaxGroups];
  uint32_t digit, above, dcount;
};

// Order-preserving 32-bit image of a score: larger value, larger bits.
__device__ __forceinline__ uint32_t score_bits(float x) {
  const float y = x + 0.f;                    // -0 becomes +0 (denormals are kept)
  const uint32_t u = __float_as_uint(y);
  const uint32_t b = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // ~u, or u | 2^31
  return y == y ? b : 0u;                     // NaN: below everything
}

// The score a key's bits stand for (the image of -0 gives +0, of NaN a
// NaN): the inverse of score_bits wherever the keys' order can tell.
__device__ __forceinline__ float bits_score(uint32_t b) {
  const uint32_t u = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return b == 0u ? __uint_as_float(0x7FC00000u) : __uint_as_float(u);
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

// Candidate i of this thread: f = fbase + 64 i (wave w, lane l: fbase =
// 64 w kKPT + l), so each key register of a wave covers 64 consecutive
// candidates.
__device__ __forceinline__ uint32_t cand(uint32_t fbase, int i) { return fbase + 64u * (uint32_t)i; }

// (key >> shift) >= prefix for key = (bits << 31) | (2^31 - 1 - f), in
// 32-bit arithmetic
__device__ __forceinline__ bool key_ge(uint32_t bits, uint32_t f, int shift, uint64_t prefix) {
  if (shift >= 31) {
    const uint32_t s = (uint32_t)shift - 31u;   // 0..32
    const uint32_t top = s >= 32 ? 0u : bits >> s;
    return (uint64_t)top >= prefix;
  }
  const uint32_t pb = (uint32_t)(prefix >> (31 - shift));
  const uint32_t pi = (uint32_t)prefix & ((1u << (31 - shift)) - 1u);
  return bits > pb || (bits == pb && ((0x7FFFFFFFu - f) >> shift) >= pi);
}

// One stage of radix select over the segment's key bits, held in the
// threads' registers (kb), down to stop_shift at most (0: to a single key).
// Every thread keeps the same (prefix, shift, need). nvw: registers that
// hold at least one real candidate in this wave (the rest are skipped).
// Real candidates past the segment's end in a register that has some hold
// score bits 0 and indices f >= len: keys below every real key (a NaN
// score's included), so for 0 < k < len they change neither the k-th key
// nor which real keys are members; they only add to the lowest buckets'
// counts, which can make the final stage stop at the score bits with the
// bucket split by index where it would have been taken whole (the
// emission counts real keys only, so the members are the same).
__device__ __forceinline__ SelCut radix_select(SelShared& sm, const uint32_t (&kb)[kKPT],
                                               uint32_t fbase, uint32_t nvw, uint32_t len,
                                               uint32_t k, int stop_shift) {
  const int tid = threadIdx.x;
  if (k == 0 || k == len)   // nothing ((key >> 63) >= 1 never holds), or everything
    return SelCut{(k == 0) ? uint64_t(1) : uint64_t(0), 63, 0u, true};
  uint64_t prefix = 0;
  int shift = 63;
  uint32_t need = k, dcount = 0;
  // this lane's copy: the atomic's address is one shift-add from the bin
  uint32_t* hc = sm.hist + (tid & (kHistCopies - 1)) * kCopyWords;
  __syncthreads();   // the histogram is clear on entry and stays so between rounds
  for (;;) {
    const int wdt = digit_width(shift);
    const uint32_t nb = 1u << wdt;
    // opaque per round: keeps the per-key indices from being hoisted out
    // of the round loop into 34 more registers
    uint32_t fb = fbase;
    asm volatile("" : "+v"(fb));
    // full: every register of the wave holds real candidates (no tests)
    auto hist = [&](auto full) {
      constexpr bool kFull = decltype(full)::value;
      if (shift == 63) {
        // first digit: every key matches
#pragma unroll
        for (int i = 0; i < kKPT; ++i)
          if (kFull || (uint32_t)i < nvw) atomicAdd(hc + (kb[i] >> 21), 1u);
      } else if (shift - wdt >= 31) {
        // the digit lies in the score bits: keys with (bits >> sh) == prefix
        // are those in [lo, lo + 2^sh)
        const uint32_t sh = shift - 31, dsh = shift - wdt - 31;
        const uint32_t lo = (uint32_t)prefix << sh, span = 1u << sh;
#pragma unroll
        for (int i = 0; i < kKPT; ++i)
          if ((kFull || (uint32_t)i < nvw) && kb[i] - lo < span)
            atomicAdd(hc + __builtin_amdgcn_ubfe(kb[i], dsh, (uint32_t)wdt), 1u);
      } else {
        // the digit lies in the index bits: the score bits are all fixed
        const uint32_t pb = (uint32_t)(prefix >> (31 - shift));
        const uint32_t pi = (uint32_t)prefix & ((1u << (31 - shift)) - 1u);
        const uint32_t ish = (uint32_t)shift, dsh = (uint32_t)(shift - wdt);
#pragma unroll
        for (int i = 0; i < kKPT; ++i) {
          const uint32_t ix = 0x7FFFFFFFu - cand(fb, i);
          if ((kFull || (uint32_t)i < nvw) && kb[i] == pb && (ix >> ish) == pi)
            atomicAdd(hc + __builtin_amdgcn_ubfe(ix, dsh, (uint32_t)wdt), 1u);
        }
      }
    };
    if (nvw == (uint32_t)kKPT) hist(std::true_type{});
    else hist(std::false_type{});
    __syncthreads();
    // bins in descending order: thread t holds bins nb-1-2t and nb-2-2t,
    // one aligned pair in every copy, which it clears for the next round
    // (a round adds to bins below its nb only)
    const int b0 = (int)nb - 1 - 2 * tid, b1 = b0 - 1;
    uint32_t h0 = 0u, h1 = 0u;
    if (b0 >= 0) {
#pragma unroll
      for (int c0 = 0; c0 < kHistCopies; c0 += 4) {
        uint2 x[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = *reinterpret_cast<const uint2*>(&sm.hist[(c0 + c) * kCopyWords + b1]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          h1 += x[c].x;
          h0 += x[c].y;
          *reinterpret_cast<uint2*>(&sm.hist[(c0 + c) * kCopyWords + b1]) = uint2{0u, 0u};
        }
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
    prefix = (prefix << wdt) | sm.digit;
    shift -= wdt;
    need -= sm.above;
    dcount = sm.dcount;
    // sm.digit/above/dcount are written again only after the next round's
    // histogram barrier, which every thread reaches after these reads
    if (need == dcount || shift <= stop_shift) break;
  }
  return SelCut{prefix, shift, need, need == dcount || shift == 0};
}

// lanes below this one whose bit is set in m, plus base
__device__ __forceinline__ uint32_t lanes_below(uint64_t m, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, base));
}

// One workgroup per segment of at most kResidentMax candidates: every key
// is read from HBM once into a register of one thread, and each radix
// round histograms the registers into LDS.
__global__ __launch_bounds__(kSelThreads) void k_select(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelShared& sm = *reinterpret_cast<SelShared*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t seg = blockIdx.x;
  const float* sc = a.scores + seg * a.in_stride;
  const float* wt = a.weight ? a.weight + seg * a.seg_len : nullptr;
  const uint32_t len = a.seg_len;   // >= 1 (the API keeps W < n)
  const SegSpan sp = seg_span(a, seg);
  const uint32_t fbase = (uint32_t)(wave * kKPT) * 64u + (uint32_t)lane;
  // the thread's real candidates: i < nv; the wave's: registers i < nvw
  // hold some (lane 0 has the most), registers i < nvall hold only real ones
  const uint32_t nv = fbase < len ? min((uint32_t)kKPT, (len - fbase + 63u) / 64u) : 0u;
  const uint32_t nvw = __builtin_amdgcn_readfirstlane(nv);
  const uint32_t nvall = __builtin_amdgcn_readlane(nv, 63);

  uint32_t kb[kKPT];
  if (a.staged) {
    // The segment goes to LDS (over the histogram, which is not in use yet)
    // with 16-byte direct-to-LDS loads, 1 KB a wave instruction: the host
    // checks that the row is 16-byte aligned and that len rounded up to 4
    // stays inside it. Stage index 4 + f holds candidate f.
    float* stg = reinterpret_cast<float*>(smem_raw);
#if defined(__HIP_DEVICE_COMPILE__)
    {
      const uint32_t len4 = (len + 3u) & ~3u;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(sc), 0, (int)(len4 * 4u), 0x00020000);
      const uint32_t chunks = (len4 + 255u) / 256u;   // 1 KB each, <= kResidentMax / 256
      for (uint32_t c = wave; c < chunks; c += kSelWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(stg + kStagePad + c * 256u), 16,
            c * 1024u + (uint32_t)lane * 16u, 0, 0, 0);
    }
#endif
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);   // vmcnt(0)
    __syncthreads();
    if (a.pool_r > 0) {
      // max-pool over |t - f| <= r, 0 <= t < len: thread t pools the
      // kKPT consecutive candidates from kKPT * t, reading r more on each
      // side, then writes them back in place once every thread has read
      auto pool = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        constexpr int NX = kKPT + 2 * R;
        const int f0 = tid * kKPT;
        float x[NX];
#pragma unroll
        for (int j = 0; j < NX; ++j) {
          const int t = f0 - R + j;
          x[j] = (uint32_t)t < len ? stg[kStagePad + t] : -__builtin_inff();
        }
        // in place, ascending (each step reads only entries it has not
        // rewritten yet): pairs x[j..j+1], then for R > 1 quads x[j..j+3];
        // the window x[j..j+2R] is the union of two of them
#pragma unroll
        for (int j = 0; j + 1 < NX; ++j) x[j] = __builtin_fmaxf(x[j], x[j + 1]);
        if constexpr (R > 1) {
#pragma unroll
          for (int j = 0; j + 3 < NX; ++j) x[j] = __builtin_fmaxf(x[j], x[j + 2]);
        }
        constexpr int kSecond = R == 3 ? 3 : 1;   // R = 1: pairs j, j+1; 2: quads j, j+1; 3: quads j, j+3
#pragma unroll
        for (int j = 0; j < kKPT; ++j) x[j] = __builtin_fmaxf(x[j], x[j + kSecond]);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kKPT; ++j)
          if ((uint32_t)(f0 + j) < len) stg[kStagePad + f0 + j] = x[j];
        __syncthreads();
      };
      if (a.pool_r == 1) pool(std::integral_constant<int, 1>{});
      else if (a.pool_r == 2) pool(std::integral_constant<int, 2>{});
      else pool(std::integral_constant<int, 3>{});
    }
    const uint32_t flast = len - 1u;
#pragma unroll
    for (int i = 0; i < kKPT; ++i)
      kb[i] = (uint32_t)i < nvw ? __float_as_uint(stg[kStagePad + min(cand(fbase, i), flast)]) : 0u;
    if (a.pooled) {
      float* po = a.pooled + seg * a.seg_len;
#pragma unroll
      for (int i = 0; i < kKPT; ++i)
        if ((uint32_t)i < nv) po[cand(fbase, i)] = __uint_as_float(kb[i]);
    }
    __syncthreads();   // the stage is read: the histogram may take its place
  } else {
    // every load in flight at once (one wait); each load instruction of a
    // wave reads 256 contiguous bytes
    const uint32_t* sc32 = reinterpret_cast<const uint32_t*>(sc);
    const uint32_t flast = len - 1u;   // loads past the end repeat the last candidate
#pragma unroll
    for (int i = 0; i < kKPT; ++i)
      kb[i] = (uint32_t)i < nvw ? __builtin_nontemporal_load(sc32 + min(cand(fbase, i), flast)) : 0u;
  }
  // the histogram starts clear
  {
    u32x4* h4 = reinterpret_cast<u32x4*>(sm.hist);
    for (int q = tid; q < kHistCopies * kCopyWords / 4; q += kSelThreads) h4[q] = u32x4{0u, 0u, 0u, 0u};
  }
  {
    // an opaque copy of nv keeps the compiler from computing the range
    // tests once and keeping them (in spilled scalar registers) for later
    uint32_t nvl = nv;
    asm volatile("" : "+v"(nvl));
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      const uint32_t b = score_bits(__uint_as_float(kb[i]));
      kb[i] = (uint32_t)i < nvl ? b : 0u;
    }
  }

  // stage 1 (two-stage only), all the way down: stage-1 membership stays a
  // test on the key, which stage 2 turns into +inf
  if (a.two_stage) {
    const SelCut c1 = radix_select(sm, kb, fbase, nvw, len, sp.k1, 0);
    uint32_t nvs = nv;
    asm volatile("" : "+v"(nvs));
    constexpr int kParts = 4, kHalf = (kKPT + kParts - 1) / kParts;
#pragma unroll
    for (int h = 0; h < kParts; ++h) {
      // the score is read back from its key bits (the pooled scores of the
      // on-chip pooling exist nowhere else); every score the order can
      // tell apart comes back exactly, and stage2_bits maps the rest (-0
      // and +0, the NaNs) to the same key
      float wv[kHalf];
#pragma unroll
      for (int u = 0; u < kHalf; ++u) {
        const int i = h * kHalf + u;
        const uint32_t f = cand(fbase, i);
        const bool ok = i < kKPT && (uint32_t)i < nvs;
        wv[u] = ok ? wt[f] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kHalf; ++u) {
        const int i = h * kHalf + u;
        if (i < kKPT)
          kb[i] = (uint32_t)i >= nvs ? 0u
                  : key_ge(kb[i], cand(fbase, i), c1.shift, c1.prefix)
                      ? kInfBits : stage2_bits(bits_score(kb[i]), wv[u], a.score_norm, a.eps);
      }
    }
  }

  const SelCut cf = radix_select(sm, kb, fbase, nvw, len, sp.k, 31);

  // ---- emission, in index order. A key register of a wave holds 64
  // consecutive candidates, so a ballot over it orders them; a first sweep
  // counts each wave's members and tied bucket entries, a scan over the 16
  // waves gives every wave the counts before it, and a second sweep writes
  // each member to its output slot (a wave's members of one register go to
  // consecutive slots).
  // The select stopped at shift >= 31, so (key >> shift) vs prefix is a
  // test on the score bits: keys in the bucket are those >= lo, keys above
  // it those > hi. At shift 63 (k = 0 or k = len) the bucket is nothing
  // (no key is 0xFFFFFFFF, a NaN image) or everything.
  const bool done = cf.done;
  uint32_t lo, hi;
  if (cf.shift == 63) {
    lo = cf.prefix == 0 ? 0u : 0xFFFFFFFFu;
    hi = 0xFFFFFFFFu;
  } else {
    const uint32_t csh = (uint32_t)cf.shift - 31u;            // 0..21
    const uint64_t top = (cf.prefix + 1) << csh;               // <= 2^32
    lo = (uint32_t)(cf.prefix << csh);
    hi = (uint32_t)min(top - 1, (uint64_t)0xFFFFFFFFu);
  }
  // per register i, as ballots: its members above the bucket (m) and its
  // entries in the bucket (t), real lanes only; every operation on them
  // is scalar. kDone: the bucket is taken whole (no tied entries); kFull:
  // every lane of every register of the wave is real.
  auto masks = [&](auto dn, auto fl, int i, uint32_t nvx, uint64_t& m, uint64_t& t) {
    constexpr bool kDone = decltype(dn)::value, kFull = decltype(fl)::value;
    const uint64_t ge = __ballot(kb[i] >= lo);
    const uint64_t gt = kDone ? ge : __ballot(kb[i] > hi);
    const uint64_t rl = kFull || (uint32_t)i < nvall ? ~uint64_t(0) : __ballot((uint32_t)i < nvx);
    m = gt & rl;
    t = kDone ? 0 : ge & ~gt & rl;
  };
  auto count = [&](auto dn, auto fl, uint32_t nvx, uint32_t& cm, uint32_t& ct) {
#pragma unroll
    for (int i = 0; i < kKPT; ++i)
      if (decltype(fl)::value || (uint32_t)i < nvw) {
        uint64_t m, t;
        masks(dn, fl, i, nvx, m, t);
        cm += (uint32_t)__popcll(m);
        ct += (uint32_t)__popcll(t);
      }
  };
  uint32_t cm = 0u, ct = 0u;
  {
    uint32_t nva = nv;   // opaque per sweep: the sweeps share no per-key values
    asm volatile("" : "+v"(nva));
    const bool full = nvall == (uint32_t)kKPT;
    if (done) {
      if (full) count(std::true_type{}, std::true_type{}, nva, cm, ct);
      else count(std::true_type{}, std::false_type{}, nva, cm, ct);
    } else {
      if (full) count(std::false_type{}, std::true_type{}, nva, cm, ct);
      else count(std::false_type{}, std::false_type{}, nva, cm, ct);
    }
  }
  if (lane == 0) {
    sm.wcount[0][wave] = cm;
    sm.wcount[1][wave] = ct;
  }
  lds_barrier();
  uint32_t mb = 0u, tb = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    mb += w < wave ? sm.wcount[0][w] : 0u;
    tb += w < wave ? sm.wcount[1][w] : 0u;
  }
  // the tied members are the first `need` tied entries in index order
  const uint32_t need = done ? 0u : cf.need;
  // members before the register's first candidate, tied entries before it
  uint32_t run = __builtin_amdgcn_readfirstlane(mb + min(need, tb));
  uint32_t trun = __builtin_amdgcn_readfirstlane(tb);
  int32_t* out = a.idx + sp.base;
  uint8_t* st_out = a.stage ? a.stage + sp.base : nullptr;
  // slots past lim are never written: r < k always, and a budget row may
  // cut the segment's room below its budget
  const uint32_t lim = (uint32_t)min((int64_t)sp.k, sp.room);
  uint32_t fc = fbase, nvc = nv;
  asm volatile("" : "+v"(fc), "+v"(nvc));
  // register i's member ballot, tied members included
  auto members = [&](auto dn, auto fl, int i) -> uint64_t {
    uint64_t m, t;
    masks(dn, fl, i, nvc, m, t);
    if (!decltype(dn)::value && t) {   // tied entries: the first `need` in index order are members
      m |= __ballot(__builtin_amdgcn_inverse_ballot_w64(t) && lanes_below(t, trun) < need);
      trun += (uint32_t)__popcll(t);
    }
    return m;
  };
  // one head: a member's slot is its rank
  auto write = [&](auto dn, auto fl) {
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      if (!decltype(fl)::value && (uint32_t)i >= nvw) continue;
      const uint64_t m = members(dn, fl, i);
      if (__builtin_amdgcn_inverse_ballot_w64(m)) {
        const uint32_t r = lanes_below(m, run);   // members before f, and f's slot
        if (r < lim) {
          out[r] = (int32_t)cand(fc, i);
          if (st_out) st_out[r] = (a.two_stage && kb[i] != kInfBits) ? 2 : 1;
        }
      }
      run += (uint32_t)__popcll(m);
    }
  };
  // several heads (adaptive): group g's members start at slot
  // group_start[g] + g*W
  auto write_grouped = [&](auto dn, auto fl) {
    // group (head) of the lane's candidate: g, and its first candidate gstart
    uint32_t g = 0u, gstart = 0u;
    if (fbase < len) {
      g = fbase / a.n_cand;
      gstart = g * a.n_cand;
    }
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      if (!decltype(fl)::value && (uint32_t)i >= nvw) continue;
      const uint64_t m = members(dn, fl, i);
      const uint32_t f = cand(fc, i);
      if ((uint32_t)i < nvc) {
        while (f >= gstart + a.n_cand) {
          ++g;
          gstart += a.n_cand;
        }
        if (f == gstart) sm.group_start[g] = lanes_below(m, run);
      }
      if (__builtin_amdgcn_inverse_ballot_w64(m)) {
        const uint32_t r = lanes_below(m, run);
        const uint32_t slot = r + g * a.W;   // < 2^31: r < k, g*W <= budget
        if (r < lim && slot < sp.room) {
          out[slot] = (int32_t)(f - gstart);
          if (st_out) st_out[slot] = (a.two_stage && kb[i] != kInfBits) ? 2 : 1;
        }
      }
      run += (uint32_t)__popcll(m);
    }
  };
  {
    const bool full = nvall == (uint32_t)kKPT;
    if (a.groups == 1) {
      if (tid == 0) sm.group_start[0] = 0u;
      if (done) {
        if (full) write(std::true_type{}, std::true_type{});
        else write(std::true_type{}, std::false_type{});
      } else {
        if (full) write(std::false_type{}, std::true_type{});
        else write(std::false_type{}, std::false_type{});
      }
    } else {
      if (done) write_grouped(std::true_type{}, std::false_type{});
      else write_grouped(std::false_type{}, std::false_type{});
    }
  }
  lds_barrier();
  // each group's W window entries follow its members (slot of group g's
  // first member: group_start[g] + g*W)
  for (uint32_t e = tid; e < a.groups * a.W; e += kSelThreads) {
    const uint32_t gw = a.groups > 1 ? e / a.W : 0u, j = e - gw * a.W;
    const uint32_t end_g = gw + 1 < a.groups ? sm.group_start[gw + 1] : sp.k;
    const uint64_t slot = (uint64_t)end_g + (uint64_t)gw * a.W + j;
    if (slot < (uint64_t)sp.room) {
      out[slot] = (int32_t)(a.n - a.W + j);
      if (st_out) st_out[slot] = 0;
    }
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
// are spread over chunks of kChunk candidates. A stage of the selection is
// four passes over the chunks and one per segment:
//   round 0        per chunk: histogram of the first 11-bit digit of the
//                  score bits (k_msel_hist; k_msel_pool when it also
//                  max-pools the raw scores), added to the segment's global
//                  histogram of the round
//   round 1        per chunk: the bin holding the need-th largest key of
//                  round 0 (every workgroup reads the 2048 bins and finds
//                  the same one; the chunk-0 workgroup keeps the state),
//                  then the histogram of the next 11 bits among the keys in
//                  that bin
//   k_msel_filter  per chunk: round 1's bin the same way; keys above the
//                  bucket are members (final stage: bits of the chunk's
//                  member mask, and its member count); keys in it go to the
//                  segment's short list (score bits and index)
//   k_msel_finish  per segment: the remaining rounds (the last 10 score
//                  bits, then the index bits) over the list in LDS, until
//                  the bucket is taken whole or holds one key. The stage
//                  ends with an exact threshold key K: its members are the
//                  keys >= K. In the final stage the listed members are
//                  added to the mask and the chunk counts; after stage 1 it
//                  sets up stage 2.
// Two digits (22 of the 32 score bits) leave a few dozen keys in the
// bucket on attention scores: each full pass over the scores is a
// histogram or the filter, and the rounds below them run on the list. A
// bucket too long for the list (heavy ties) is narrowed by k_msel_finish
// itself, one workgroup streaming the segment per round. A segment whose
// bucket is taken whole after a round is done there: its members are the
// keys >= prefix << shift. Each round's state sits in a slot of its own
// (0: the stage's start, 1: after round 0, 2: after round 1), written by
// one workgroup of the kernel that computes it and read by later kernels
// only, and each round has its own global histogram. Stage 2 of the
// two-stage selection keys the stage-1 members (keys >= K1) as +inf.
// Emission (k_msel_emit, per chunk): the members of its mask in index
// order at their ranks (members before the chunk: a sum over the
// segment's earlier chunks), staged in LDS and written with coalesced
// stores; a group's last chunk also writes the group's window entries and
// the first chunk its head offsets. Chunks never straddle a head (group).
// Every sum runs in a fixed order or over integers and K is unique (no two
// keys tie; the list's order does not matter): the result is deterministic.
//
// Every thread issues all of its kPerThread loads before it uses one: a
// chunk's workgroup then waits for memory once.
constexpr int kMThreads = 512;
constexpr int kChunk = 16384;                      // candidates per chunk
constexpr int kPerThread = kChunk / kMThreads;     // 32
constexpr int kMCopies = 4;                        // LDS histogram copies, first digit
constexpr int kMaskWords = kChunk / 32;            // a chunk's member mask
constexpr int kListCap = 1024;                     // bucket entries a segment's list holds
constexpr int kSlots = 3;                          // states per segment (above)
constexpr int kHistBufs = 3;                       // global histograms per segment (above)
static_assert(kMaskWords == kMThreads, "k_msel_emit: one mask word a thread");
static_assert(kBins == 4 * kMThreads, "picks: four bins a thread");

struct alignas(16) SegState {
  uint64_t prefix;      // key prefix above `shift`
  uint64_t thr1;        // two-stage, stage 2: stage-1 members are the keys >= thr1
  int32_t shift;
  uint32_t need, done;
  uint32_t count;       // keys in the bucket the last round chose
  uint32_t listed;      // slot 1: entries appended to the segment's list
  uint32_t pad[3];
};

struct MselArgs {
  const float* scores;
  const float* weight;
  SegState* states;     // [kSlots][segments]
  uint32_t* ghist;      // [3][segments][kBins]: round 0 of stage 1, round 1, round 0 of stage 2
  uint32_t* ccount;     // [segments][chunks]: members
  uint2* list;          // [segments][kListCap]: (score bits, index) of bucket keys
  uint32_t* mask;       // [segments][chunks][kMaskWords]: final members
  uint32_t* mask1;      // the same for stage-1 members (two-stage)
  int32_t* idx;
  int32_t* head_offsets;
  uint8_t* stage;
  const int32_t* budgets;   // [L][H] or null
  uint32_t segs, seg_len, n_cand, groups, W, n, cpg, chunks, H;
  uint32_t k, k1;
  int64_t budget, stride;
  float score_norm, eps, alpha;
};

__device__ __forceinline__ SegState* msel_state(const MselArgs& a, int slot, uint32_t seg) {
  return a.states + (size_t)slot * a.segs + seg;
}
__device__ __forceinline__ uint32_t* msel_ghist(const MselArgs& a, int buf, uint32_t seg) {
  return a.ghist + ((size_t)buf * a.segs + seg) * kBins;
}

// Key bits of candidate f for the stage being selected, from its score s
// and weight w (stage 2 of the two-stage selection: stage-1 members are
// +inf, the rest the integrated score).
__device__ __forceinline__ uint32_t msel_bits(const MselArgs& a, const SegState& st, float s,
                                              float w, bool stage2, uint32_t f) {
  const uint32_t b = score_bits(s);
  if (!stage2) return b;
  return make_key(b, f) >= st.thr1 ? kInfBits : stage2_bits(s, w, a.score_norm, a.eps);
}

// chunk c of a segment: [begin, end) in flat candidate indices
__device__ __forceinline__ void msel_chunk(const MselArgs& a, uint32_t c, uint32_t& g,
                                           uint32_t& begin, uint32_t& end) {
  g = c / a.cpg;
  const uint32_t cc = c - g * a.cpg;
  begin = g * a.n_cand + cc * kChunk;
  end = min(begin + (uint32_t)kChunk, (g + 1) * a.n_cand);
}

// Candidate i of the thread in a chunk starting at `begin`: f = begin +
// msel_e<VEC>(i). VEC (every chunk 16-byte aligned and a multiple of 4
// long: n_cand % 4 == 0): four consecutive candidates a 16-byte load,
// 1 KB a wave; else one a 4-byte load. Either way a wave's loads are
// contiguous.
template <bool VEC>
__device__ __forceinline__ uint32_t msel_e(int i) {
  if constexpr (VEC)
    return (uint32_t)(i >> 2) * (4u * kMThreads) + 4u * threadIdx.x + (uint32_t)(i & 3);
  else
    return (uint32_t)i * kMThreads + threadIdx.x;
}

// The thread's kPerThread candidates (in range: f < end), all loads
// issued before the first is used; out-of-range slots read 0.
template <bool VEC>
__device__ __forceinline__ void msel_load(const MselArgs& a, uint32_t seg, uint32_t begin,
                                          uint32_t end, bool stage2, float (&s)[kPerThread],
                                          float (&w)[kPerThread]) {
  const float* sc = a.scores + (size_t)seg * a.seg_len;
  const float* wt = a.weight ? a.weight + (size_t)seg * a.seg_len : nullptr;
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < kPerThread / 4; ++u) {
      const uint32_t f = begin + msel_e<true>(4 * u);
      const bool in = f < end;   // the chunk's length is a multiple of 4
      const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
      const u32x4 x = in ? *reinterpret_cast<const u32x4*>(sc + f) : zero;
      const u32x4 y = (stage2 && in) ? *reinterpret_cast<const u32x4*>(wt + f) : zero;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s[4 * u + c] = __uint_as_float(x[c]);
        w[4 * u + c] = __uint_as_float(y[c]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const uint32_t f = begin + msel_e<false>(i);
      s[i] = f < end ? sc[f] : 0.f;
      w[i] = (stage2 && f < end) ? wt[f] : 0.f;
    }
  }
}

// A stage's start: prefix 0, need k (k1 for stage 1 of the two-stage
// selection); nothing or everything is done at once.
__device__ __forceinline__ SegState msel_start(const MselArgs& a, uint32_t seg, bool stage2,
                                               uint64_t thr1) {
  const SegSpan sp = seg_span(a, (size_t)seg);
  const uint32_t k = (stage2 || sp.k1 == 0xFFFFFFFFu) ? sp.k : sp.k1;
  SegState st;
  st.thr1 = thr1;
  st.shift = 63;
  st.count = 0;
  st.listed = 0;
  st.pad[0] = st.pad[1] = st.pad[2] = 0;
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
  return st;
}

// grid segments: stage 1's (or the single stage's) start, and cleared
// global histograms (the workspace may hold anything)
__global__ __launch_bounds__(kMThreads) void k_msel_init(MselArgs a) {
  const uint32_t seg = blockIdx.x;
  for (int buf = 0; buf < kHistBufs; ++buf) {
    uint32_t* gh = msel_ghist(a, buf, seg);
    for (int b = threadIdx.x; b < kBins; b += kMThreads) gh[b] = 0u;
  }
  if (threadIdx.x == 0) *msel_state(a, 0, seg) = msel_start(a, seg, false, 0u);
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

// exclusive scan over the workgroup's threads (in thread order); total returned too
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

// Thread t's four bins of a round's global histogram, in descending bin
// order (bins 2047-4t .. 2044-4t): loaded before the chunk's scores, so
// that the pick waits for them only.
__device__ __forceinline__ void pick_load(const uint32_t* gh, uint32_t (&h)[4]) {
  const uint32_t* p = gh + (kBins - 4 - 4 * threadIdx.x);
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  h[0] = v[3];
  h[1] = v[2];
  h[2] = v[1];
  h[3] = v[0];
}

// The state after one more 11-bit digit (shift 63 or 52), from the
// round's histogram: the bin where the count of larger keys first reaches
// need (exactly one thread holds it). Every thread returns the same state.
__device__ __forceinline__ SegState msel_pick(SegState st, const uint32_t (&h)[4], uint32_t* sbuf,
                                              uint32_t* pk) {
  if (st.done) return st;
  const int tid = threadIdx.x;
  const uint32_t need = st.need;
  const uint32_t sum = h[0] + h[1] + h[2] + h[3];
  uint32_t tot;
  const uint32_t above = block_scan256(sum, sbuf, tot);
  if (above < need && need <= above + sum) {
    uint32_t acc = above;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (acc < need && need <= acc + h[j]) {
        pk[0] = (uint32_t)(kBins - 1 - 4 * tid - j);
        pk[1] = acc;
        pk[2] = h[j];
      }
      acc += h[j];
    }
  }
  __syncthreads();
  const uint32_t digit = pk[0], ab = pk[1], cnt = pk[2];
  __syncthreads();   // read by every thread before pk is written again
  st.prefix = (st.prefix << 11) | digit;
  st.shift -= 11;
  st.need = need - ab;
  st.count = cnt;
  st.listed = 0;
  st.done = (st.need == cnt) ? 1u : 0u;
  return st;
}

// Histogram of the digit below st.shift (63 or 52: both rounds lie in the
// score bits) among the keys in the bucket, added to the round's global
// histogram. Four candidates at a time (consecutive ones when VEC): when
// all four fall in one bin, as neighbouring max-pooled scores mostly do on
// the first digit, they add 4 with one atomic.
template <int COPIES, bool VEC>
__device__ __forceinline__ void msel_hist_chunk(const MselArgs& a, const SegState& st, bool stage2,
                                                uint32_t begin, uint32_t end,
                                                const float (&s)[kPerThread],
                                                const float (&w)[kPerThread],
                                                uint32_t (*hist)[kBins], uint32_t* gh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int cp = 0; cp < COPIES; ++cp)
    for (int b = tid; b < kBins; b += kMThreads) hist[cp][b] = 0;
  __syncthreads();
  uint32_t* hc = hist[tid & (COPIES - 1)];
  // keys (bits << 31) | (2^31 - 1 - f) with (key >> shift) == prefix are
  // those with bits in [lo, lo + 2^sh)
  const uint32_t sh = st.shift - 31, dsh = sh - 11;
  const uint32_t lo = sh >= 32 ? 0u : (uint32_t)st.prefix << sh;
  const uint32_t span_m1 = sh >= 32 ? 0xFFFFFFFFu : (1u << sh) - 1u;
#pragma unroll
  for (int u = 0; u < kPerThread / 4; ++u) {
    uint32_t bn[4];
    bool ok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * u + q;
      const uint32_t f = begin + msel_e<VEC>(i);
      const uint32_t b = msel_bits(a, st, s[i], w[i], stage2, f);
      ok[q] = f < end && b - lo <= span_m1;
      bn[q] = (b >> dsh) & (kBins - 1u);
    }
    if (ok[0] && ok[1] && ok[2] && ok[3] && bn[0] == bn[1] && bn[1] == bn[2] && bn[2] == bn[3]) {
      atomicAdd(&hc[bn[0]], 4u);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ok[q]) atomicAdd(&hc[bn[q]], 1u);
    }
  }
  __syncthreads();
  for (int b = tid; b < kBins; b += kMThreads) {
    uint32_t v = 0;
#pragma unroll
    for (int cp = 0; cp < COPIES; ++cp) v += hist[cp][b];
    if (v) atomicAdd(gh + b, v);
  }
}

// grid chunks*segments: round 0 of a stage (its start in slot 0). The
// stage is a template argument so that stage 1 holds no weights (fewer
// registers, more workgroups per CU).
template <bool VEC, bool S2>
__global__ __launch_bounds__(kMThreads) void k_msel_hist0(MselArgs a) {
  constexpr int stage2 = S2 ? 1 : 0;
  __shared__ uint32_t hist[kMCopies][kBins];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st = *msel_state(a, 0, seg);
  if (st.done) return;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  float s[kPerThread], w[kPerThread];
  msel_load<VEC>(a, seg, begin, end, stage2 != 0, s, w);
  msel_hist_chunk<kMCopies, VEC>(a, st, stage2 != 0, begin, end, s, w, hist,
                                 msel_ghist(a, S2 ? 2 : 0, seg));
}

// grid chunks*segments: round 1 (round 0's bin picked from its histogram;
// the chunk-0 workgroup keeps the state in slot 1)
template <bool VEC, bool S2>
__global__ __launch_bounds__(kMThreads) void k_msel_hist1(MselArgs a) {
  constexpr int stage2 = S2 ? 1 : 0;
  __shared__ uint32_t hist[1][kBins];
  __shared__ uint32_t sbuf[kMThreads / 64], pk[3];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const SegState st0 = *msel_state(a, 0, seg);
  uint32_t h[4];
  pick_load(msel_ghist(a, S2 ? 2 : 0, seg), h);
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  float s[kPerThread], w[kPerThread];
  msel_load<VEC>(a, seg, begin, end, stage2 != 0, s, w);
  const SegState st = msel_pick(st0, h, sbuf, pk);
  if (c == 0 && threadIdx.x == 0) *msel_state(a, 1, seg) = st;
  if (st.done) return;
  msel_hist_chunk<1, VEC>(a, st, stage2 != 0, begin, end, s, w, hist, msel_ghist(a, 1, seg));
}

// Pooling in the first pass (kvsel_select_pool on raw rows, radius R <=
// kMaxPoolR): the chunk's raw scores and a halo of kPoolHalo on each side
// go to LDS (one pad word per 32, so that 64 lanes reading at a stride of
// 32 or 4 words, and 64 consecutive ones, all hit distinct banks); thread
// t pools the chunk's candidates 32t .. 32t+31 in the order of the pool
// kernel (so the pooled bits are the same), histograms their first digit
// by runs of equal bins along them, and the pooled scores go out to the
// array the later passes read, through LDS again for coalesced stores.
constexpr int kPoolHalo = 4;                       // >= kMaxPoolR; keeps 16-byte units
constexpr int kPoolWin = 32 + 2 * kPoolHalo;       // a thread's window
__device__ __forceinline__ uint32_t pool_slot(uint32_t x) { return x + (x >> 5); }
// the last thread's window ends at 32 * 511 + kPoolWin - 1
constexpr size_t kPoolTileFloats = (size_t)(kChunk - 32 + kPoolWin - 1) + (kChunk - 32 + kPoolWin - 1) / 32 + 1;
constexpr size_t kPoolTileBytes = (kPoolTileFloats * sizeof(float) + 15) & ~size_t(15);
constexpr size_t kPoolLdsBytes = kPoolTileBytes + kBins * sizeof(uint32_t);
constexpr int kPoolLoadsV = ((kChunk + 2 * kPoolHalo) / 4 + kMThreads - 1) / kMThreads;   // 16-byte units
constexpr int kPoolLoads = (kChunk + 2 * kPoolHalo + kMThreads - 1) / kMThreads;          // 4-byte loads

// grid chunks*segments: round 0 of stage 1. raw: row (seg * groups + g) holds group g's
// candidates, in_stride floats apart. VEC: n_cand and in_stride multiples
// of 4 (every chunk and its halo in whole 16-byte units).
template <int R, bool VEC>
__global__ __launch_bounds__(kMThreads) void k_msel_pool(MselArgs a, const float* raw,
                                                         int64_t in_stride, float* pooled) {
  extern __shared__ __align__(16) unsigned char pool_smem[];
  float* tile = reinterpret_cast<float*>(pool_smem);
  uint32_t* hist = reinterpret_cast<uint32_t*>(pool_smem + kPoolTileBytes);
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const int tid = threadIdx.x;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  const uint32_t len = end - begin, pos0 = begin - g * a.n_cand;
  const float* row = raw + ((size_t)seg * a.groups + g) * (size_t)in_stride;
  const bool do_hist = !msel_state(a, 0, seg)->done;
  // tile x holds candidate pos0 - kPoolHalo + x; -inf outside the candidates
  const uint32_t nx = len + 2 * kPoolHalo;
  const float ninf = -__builtin_inff();
  if constexpr (VEC) {
    const uint32_t units = nx / 4;
    u32x4 v[kPoolLoadsV];
#pragma unroll
    for (int j = 0; j < kPoolLoadsV; ++j) {
      const uint32_t q = tid + j * kMThreads;
      const int64_t p = (int64_t)pos0 - kPoolHalo + 4 * (int64_t)q;
      const bool in = q < units && p >= 0 && p + 4 <= (int64_t)a.n_cand;
      const uint32_t ni = __float_as_uint(ninf);
      v[j] = in ? *reinterpret_cast<const u32x4*>(row + p) : u32x4{ni, ni, ni, ni};
    }
#pragma unroll
    for (int j = 0; j < kPoolLoadsV; ++j) {
      const uint32_t q = tid + j * kMThreads;
      if (q < units) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[pool_slot(4 * q + i)] = __uint_as_float(v[j][i]);
      }
    }
  } else {
    float v[kPoolLoads];
#pragma unroll
    for (int j = 0; j < kPoolLoads; ++j) {
      const uint32_t x = tid + j * kMThreads;
      const int64_t p = (int64_t)pos0 - kPoolHalo + x;
      v[j] = (x < nx && p >= 0 && p < (int64_t)a.n_cand) ? row[p] : ninf;
    }
#pragma unroll
    for (int j = 0; j < kPoolLoads; ++j) {
      const uint32_t x = tid + j * kMThreads;
      if (x < nx) tile[pool_slot(x)] = v[j];
    }
  }
  if (do_hist)
    for (int b = tid; b < kBins; b += kMThreads) hist[b] = 0u;
  __syncthreads();
  // thread t: candidates e = 32t + j, window x = 32t .. 32t + kPoolWin - 1
  // (reads past nx feed only candidates e >= len)
  float win[kPoolWin], out[32];
#pragma unroll
  for (int j = 0; j < kPoolWin; ++j) win[j] = tile[pool_slot(32u * tid + j)];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float m = win[j + kPoolHalo];
#pragma unroll
    for (int o = 1; o <= R; ++o) m = fmaxf(m, fmaxf(win[j + kPoolHalo - o], win[j + kPoolHalo + o]));
    out[j] = m;
  }
  if (do_hist) {
    // first digit (score bits >> 21) by runs along the thread's candidates
    uint32_t cur = 0xFFFFFFFFu, cnt = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (32u * tid + j < len) {
        const uint32_t bin = score_bits(out[j]) >> 21;
        if (bin != cur) {
          if (cnt) atomicAdd(&hist[cur], cnt);
          cur = bin;
          cnt = 0;
        }
        ++cnt;
      }
    }
    if (cnt) atomicAdd(&hist[cur], cnt);
  }
  __syncthreads();   // every window read before the tile takes the pooled scores
#pragma unroll
  for (int j = 0; j < 32; ++j) tile[pool_slot(32u * tid + j)] = out[j];
  __syncthreads();
  float* dst = pooled + (size_t)seg * a.seg_len + begin;
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < kPerThread / 4; ++u) {
      const uint32_t e = u * (4u * kMThreads) + 4u * tid;
      if (e < len) {
        float4 x;
        x.x = tile[pool_slot(e)];
        x.y = tile[pool_slot(e + 1)];
        x.z = tile[pool_slot(e + 2)];
        x.w = tile[pool_slot(e + 3)];
        *reinterpret_cast<float4*>(dst + e) = x;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const uint32_t e = tid + i * kMThreads;
      if (e < len) dst[e] = tile[pool_slot(e)];
    }
  }
  if (do_hist) {
    uint32_t* gh = msel_ghist(a, 0, seg);
    for (int b = tid; b < kBins; b += kMThreads)
      if (hist[b]) atomicAdd(gh + b, hist[b]);
  }
}

// grid chunks*segments: round 1's bin picked from its histogram (the
// chunk-0 workgroup keeps the state in slot 2). Then the final stage's
// members above the bucket (all of it when done) go to the chunk's mask
// and count; the bucket's keys, when they fit the list, to the segment's
// list. Both rounds stopped at shift 63, 52 or 41, all in the score bits,
// so (key >> shift) is bits >> (shift - 31).
//
// H2 (stage 1 of the two-stage selection): each key's stage-1 membership is
// known here except in the bucket, so this pass also loads the weights and
// adds stage 2's first-digit histogram (buffer 2) for the other keys;
// k_msel_finish adds the bucket's once it has K1.
template <bool VEC, bool S2, bool H2>
__global__ __launch_bounds__(kMThreads) void k_msel_filter(MselArgs a, int final) {
  constexpr int stage2 = S2 ? 1 : 0;
  __shared__ uint32_t mw[kMaskWords], m1w[kMaskWords];
  __shared__ uint32_t h2[H2 ? kMCopies : 1][kBins];
  __shared__ uint2 lst[kListCap];
  __shared__ uint32_t sbuf[kMThreads / 64], pk[3];
  __shared__ uint32_t s_n, s_base;
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const int tid = threadIdx.x;
  const SegState st1 = *msel_state(a, 1, seg);
  uint32_t h[4];
  pick_load(msel_ghist(a, 1, seg), h);
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  float s[kPerThread], w[kPerThread];
  msel_load<VEC>(a, seg, begin, end, S2 || H2, s, w);
  const SegState st = msel_pick(st1, h, sbuf, pk);
  if (c == 0 && tid == 0) *msel_state(a, 2, seg) = st;
  const bool listing = !st.done && st.count <= (uint32_t)kListCap;
  if (!final && !listing && !H2) return;
  mw[tid] = 0u;
  m1w[tid] = 0u;
  if (tid == 0) s_n = 0u;
  if constexpr (H2) {
#pragma unroll
    for (int cp = 0; cp < kMCopies; ++cp)
      for (int b = tid; b < kBins; b += kMThreads) h2[cp][b] = 0u;
  }
  __syncthreads();
  uint32_t* h2c = h2[H2 ? (tid & (kMCopies - 1)) : 0];
  const uint32_t sh = (uint32_t)st.shift - 31u, pref = (uint32_t)st.prefix;
  uint32_t nmem = 0;
#pragma unroll
  for (int u = 0; u < kPerThread / 4; ++u) {
    // VEC: the four candidates share a mask word (one LDS atomic); else a
    // wave's 64 candidates are two whole words of its own (a ballot)
    uint32_t word = 0u, word1 = 0u, bin2[4];
    bool ok2[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * u + q;
      const uint32_t e = msel_e<VEC>(i), f = begin + e;
      const bool valid = f < end;
      const uint32_t b1 = score_bits(s[i]);
      const bool in1 = valid && stage2 && make_key(b1, f) >= st.thr1;
      const uint32_t b = !stage2 ? b1 : (in1 ? kInfBits : stage2_bits(s[i], w[i], a.score_norm, a.eps));
      const uint32_t top = sh >= 32 ? 0u : b >> sh;
      const bool mem = valid && (top > pref || (st.done && top == pref));
      nmem += mem;
      if constexpr (VEC) {
        word |= (uint32_t)mem << (e & 31);
        word1 |= (uint32_t)in1 << (e & 31);
      } else if (final) {
        const uint64_t bm = __ballot(mem), bm1 = __ballot(in1);
        if ((tid & 63) == 0) {
          mw[e >> 5] = (uint32_t)bm;
          mw[(e >> 5) + 1] = (uint32_t)(bm >> 32);
          if (stage2) {
            m1w[e >> 5] = (uint32_t)bm1;
            m1w[(e >> 5) + 1] = (uint32_t)(bm1 >> 32);
          }
        }
      }
      if (listing && valid && top == pref) {
        const uint32_t p = atomicAdd(&s_n, 1u);   // < count <= kListCap
        if (p < (uint32_t)kListCap) lst[p] = uint2{b, f};
      }
      if constexpr (H2) {   // stage 2's key: stage-1 members +inf
        ok2[q] = valid && (st.done || top != pref);
        bin2[q] = (mem ? kInfBits : stage2_bits(s[i], w[i], a.score_norm, a.eps)) >> 21;
      }
    }
    if constexpr (H2) {
      if (ok2[0] && ok2[1] && ok2[2] && ok2[3] && bin2[0] == bin2[1] && bin2[1] == bin2[2] &&
          bin2[2] == bin2[3]) {
        atomicAdd(&h2c[bin2[0]], 4u);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (ok2[q]) atomicAdd(&h2c[bin2[q]], 1u);
      }
    }
    if constexpr (VEC) {
      const uint32_t wi = msel_e<true>(4 * u) >> 5;
      if (final && word) atomicOr(&mw[wi], word);
      if (final && word1) atomicOr(&m1w[wi], word1);
    }
  }
  __syncthreads();
  if constexpr (H2) {
    uint32_t* gh = msel_ghist(a, 2, seg);
    for (int b = tid; b < kBins; b += kMThreads) {
      uint32_t v = 0;
#pragma unroll
      for (int cp = 0; cp < kMCopies; ++cp) v += h2[cp][b];
      if (v) atomicAdd(gh + b, v);
    }
  }
  if (final) {
    const size_t wb = ((size_t)seg * a.chunks + c) * kMaskWords;
    a.mask[wb + tid] = mw[tid];
    if (stage2) a.mask1[wb + tid] = m1w[tid];
    nmem = block_sum256(nmem, sbuf);
    if (tid == 0) a.ccount[(size_t)seg * a.chunks + c] = nmem;
  }
  if (listing) {
    // slot 1 is read-only in this kernel: its count takes the appends
    const uint32_t nl = min(s_n, (uint32_t)kListCap);
    if (tid == 0 && nl) s_base = atomicAdd(&msel_state(a, 1, seg)->listed, nl);
    __syncthreads();
    uint2* out = a.list + (size_t)seg * kListCap;
    for (uint32_t j = tid; j < nl; j += kMThreads)
      if (s_base + j < (uint32_t)kListCap) out[s_base + j] = lst[j];
  }
}

// Final stage: candidate f of the segment is a member (mask bit, chunk count)
__device__ __forceinline__ void msel_mark(const MselArgs& a, uint32_t seg, uint32_t f) {
  if (f >= a.seg_len) return;
  const uint32_t g = f / a.n_cand, pos = f - g * a.n_cand;
  const uint32_t c = g * a.cpg + pos / kChunk, e = pos % kChunk;
  const size_t ch = (size_t)seg * a.chunks + c;
  atomicOr(&a.mask[ch * kMaskWords + (e >> 5)], 1u << (e & 31));
  atomicAdd(&a.ccount[ch], 1u);
}

// grid segments: the rounds below the filter's bucket (state in slot 2),
// down to an exact threshold key K: the stage's members are the keys >= K.
// Final stage: the bucket's members go to the masks. Stage 1 of the
// two-stage selection: the rest of stage 2's first histogram, its start
// (slot 0) and a cleared round-1 histogram.
__global__ __launch_bounds__(kMThreads) void k_msel_finish(MselArgs a, int stage2, int final) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t lb[kListCap], lf[kListCap];
  __shared__ uint32_t sbuf[kMThreads / 64];
  __shared__ uint32_t s_digit, s_above, s_count;
  const uint32_t seg = blockIdx.x;
  const SegState st = *msel_state(a, 2, seg);
  const int tid = threadIdx.x;
  uint64_t K = st.prefix << st.shift;   // taken whole: the keys >= prefix << shift
  if (!st.done) {
    const bool listed = st.count <= (uint32_t)kListCap;
    const uint32_t m = listed ? st.count : 0u;
    const float* sc = a.scores + (size_t)seg * a.seg_len;
    const float* wt = stage2 ? a.weight + (size_t)seg * a.seg_len : nullptr;
    for (uint32_t j = tid; j < m; j += kMThreads) {
      const uint2 v = a.list[(size_t)seg * kListCap + j];
      lb[j] = v.x;
      lf[j] = v.y;
    }
    for (int b = tid; b < kBins; b += kMThreads) hist[b] = 0u;
    __syncthreads();
    uint64_t prefix = st.prefix;
    int shift = st.shift;
    uint32_t need = st.need;
    for (;;) {
      const int wdt = digit_width(shift);
      const int nb = 1 << wdt;
      const uint32_t dmask = (uint32_t)nb - 1u;
      if (listed) {
        for (uint32_t j = tid; j < m; j += kMThreads) {
          const uint64_t key = make_key(lb[j], lf[j]);
          if ((key >> shift) == prefix) atomicAdd(&hist[(uint32_t)(key >> (shift - wdt)) & dmask], 1u);
        }
      } else {   // the bucket outgrew the list: one workgroup streams the segment
        for (uint32_t f = tid; f < a.seg_len; f += kMThreads) {
          const uint64_t key = make_key(msel_bits(a, st, sc[f], wt ? wt[f] : 0.f, stage2 != 0, f), f);
          if ((key >> shift) == prefix) atomicAdd(&hist[(uint32_t)(key >> (shift - wdt)) & dmask], 1u);
        }
      }
      __syncthreads();
      // bins in descending order, four a thread
      uint32_t h[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = nb - 1 - 4 * tid - j;
        h[j] = b >= 0 ? hist[b] : 0u;
        sum += h[j];
      }
      uint32_t tot;
      const uint32_t above = block_scan256(sum, sbuf, tot);
      if (above < need && need <= above + sum) {   // exactly one thread
        uint32_t acc = above;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (acc < need && need <= acc + h[j]) {
            s_digit = (uint32_t)(nb - 1 - 4 * tid - j);
            s_above = acc;
            s_count = h[j];
          }
          acc += h[j];
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = nb - 1 - 4 * tid - j;
        if (b >= 0) hist[b] = 0u;
      }
      prefix = (prefix << wdt) | s_digit;
      shift -= wdt;
      need -= s_above;
      const uint32_t dcount = s_count;
      __syncthreads();   // s_digit/above/count read and the bins cleared before the next round
      if (need == dcount || shift == 0) break;
    }
    K = prefix << shift;
    if (final) {
      if (listed) {
        for (uint32_t j = tid; j < m; j += kMThreads)
          if (make_key(lb[j], lf[j]) >= K) msel_mark(a, seg, lf[j]);
      } else {
        // the bucket's members: keys in it (the filter marked those above)
        // and >= K, a mask word a thread
        for (uint32_t c = 0; c < a.chunks; ++c) {
          uint32_t g, begin, end;
          msel_chunk(a, c, g, begin, end);
          uint32_t bits = 0u;
          for (int j = 0; j < 32; ++j) {
            const uint32_t f = begin + 32u * tid + j;
            if (f < end) {
              const uint64_t key = make_key(msel_bits(a, st, sc[f], wt ? wt[f] : 0.f, stage2 != 0, f), f);
              if ((key >> st.shift) == st.prefix && key >= K) bits |= 1u << j;
            }
          }
          const size_t ch = (size_t)seg * a.chunks + c;
          if (bits) atomicOr(&a.mask[ch * kMaskWords + tid], bits);
          const uint32_t cnt = block_sum256((uint32_t)__popc(bits), sbuf);
          if (tid == 0 && cnt) atomicAdd(&a.ccount[ch], cnt);
        }
      }
    }
  }
  if (!final) {
    // stage 2's first-digit histogram (buffer 2): the filter added every
    // key outside the bucket; the bucket's keys are added here, +inf for
    // the stage-1 members (keys >= K)
    uint32_t* g2 = msel_ghist(a, 2, seg);
    const float* sc = a.scores + (size_t)seg * a.seg_len;
    const float* wt = a.weight + (size_t)seg * a.seg_len;
    if (!st.done && st.count <= (uint32_t)kListCap) {
      for (uint32_t j = tid; j < st.count; j += kMThreads) {
        const uint32_t f = lf[j];
        if (f < a.seg_len) {
          const uint32_t b2 = make_key(lb[j], f) >= K
                                  ? kInfBits
                                  : stage2_bits(bits_score(lb[j]), wt[f], a.score_norm, a.eps);
          atomicAdd(&g2[b2 >> 21], 1u);
        }
      }
    } else if (!st.done) {
      for (uint32_t f = tid; f < a.seg_len; f += kMThreads) {
        const float x = sc[f];
        const uint64_t key = make_key(score_bits(x), f);
        if ((key >> st.shift) == st.prefix) {
          const uint32_t b2 = key >= K ? kInfBits : stage2_bits(x, wt[f], a.score_norm, a.eps);
          atomicAdd(&g2[b2 >> 21], 1u);
        }
      }
    }
    // round 1's histogram: every stage-1 reader has finished
    uint32_t* g1 = msel_ghist(a, 1, seg);
    for (int b = tid; b < kBins; b += kMThreads) g1[b] = 0u;
    if (tid == 0) *msel_state(a, 0, seg) = msel_start(a, seg, true, K);
  }
}

// grid chunks*segments: thread t takes mask word t (the chunk's candidates
// 32t .. 32t+31); a block scan of the words' member counts gives each
// member its rank in index order after the members of the segment's
// earlier chunks. The chunk's members take consecutive output slots: they
// are staged by rank in LDS and stored with coalesced writes. Two-stage:
// stage-1 members are marked 1, the others 2. A group's first chunk writes
// its head offset (budget vector: the segment's first chunk writes the
// head's and, for a layer's last head, the row tail), its last chunk the
// group's window entries after its members.
__global__ __launch_bounds__(kMThreads) void k_msel_emit(MselArgs a, int two_stage) {
  __shared__ uint16_t staged[kChunk];
  __shared__ uint32_t sbuf[kMThreads / 64];
  const uint32_t seg = blockIdx.x / a.chunks, c = blockIdx.x - seg * a.chunks;
  const int tid = threadIdx.x;
  uint32_t g, begin, end;
  msel_chunk(a, c, g, begin, end);
  const size_t ch = (size_t)seg * a.chunks + c;
  const uint32_t mm = a.mask[ch * kMaskWords + tid];
  const uint32_t m1 = two_stage ? a.mask1[ch * kMaskWords + tid] : 0xFFFFFFFFu;
  uint32_t part = 0;
  for (uint32_t j = tid; j < c; j += kMThreads) part += a.ccount[(size_t)seg * a.chunks + j];
  const uint32_t rank0 = block_sum256(part, sbuf);   // members before the chunk
  uint32_t count;
  uint32_t r = block_scan256((uint32_t)__popc(mm), sbuf, count);   // members before this thread's
  // staged[r] = position in the chunk of its member of rank r (< 2^14),
  // bit 15 set for a stage-2 member of the two-stage selection
  static_assert(kChunk <= (1 << 15), "chunk positions and the stage bit fit 16 bits");
  for (uint32_t m = mm; m != 0; m &= m - 1, ++r) {
    const uint32_t j = (uint32_t)__builtin_ctz(m);
    staged[r] = (uint16_t)((tid * 32u + j) | (((m1 >> j) & 1u) ? 0u : 0x8000u));
  }
  __syncthreads();
  const SegSpan sp = seg_span(a, (size_t)seg);
  int32_t* out = a.idx + sp.base;
  uint8_t* st_out = a.stage ? a.stage + sp.base : nullptr;
  const int64_t o0 = (int64_t)rank0 + (int64_t)g * a.W;
  const uint32_t pos0 = begin - g * a.n_cand;   // the chunk's first position in its head
  for (uint32_t i = tid; i < count; i += kMThreads) {
    const int64_t o = o0 + i;
    if (o < sp.room) {   // k members fit the budget; the room may be cut at the row's end
      const uint32_t e = staged[i];
      out[o] = (int32_t)(pos0 + (e & 0x7FFFu));
      if (st_out) st_out[o] = (e >> 15) ? 2 : 1;
    }
  }
  const uint32_t cc = c - g * a.cpg;
  if (cc + 1 == a.cpg) {
    // the group's window entries, after its members
    const int64_t wb = (int64_t)rank0 + count + (int64_t)g * a.W;
    for (uint32_t t = tid; t < a.W; t += kMThreads) {
      const int64_t o = wb + t;
      if (o >= 0 && o < sp.room) {
        out[o] = (int32_t)(a.n - a.W + t);
        if (st_out) st_out[o] = 0;
      }
    }
  }
  if (a.budgets) {
    if (c == 0) {
      const size_t l = seg / a.H;
      const uint32_t h = (uint32_t)(seg - l * a.H);
      if (tid == 0) a.head_offsets[l * (a.H + 1) + h] = (int32_t)sp.off;
      if (h + 1 == a.H) {
        if (tid == 0) a.head_offsets[l * (a.H + 1) + a.H] = (int32_t)sp.end;
        fill_row_tail(a.idx, a.stage, (int64_t)l * a.stride, sp.end, a.stride, tid, kMThreads);
      }
    }
  } else if (a.head_offsets && tid == 0) {
    if (cc == 0) a.head_offsets[(size_t)seg * (a.groups + 1) + g] = (int32_t)(rank0 + g * a.W);
    if (c == 0) a.head_offsets[(size_t)seg * (a.groups + 1) + a.groups] = (int32_t)a.budget;
  }
}

static size_t al256s(size_t x) { return (x + 255) & ~size_t(255); }

struct MselLayout {
  uint32_t cpg, chunks;
  size_t states_off, ghist_off, ccount_off, list_off, mask_off, mask1_off, bytes;
};

static MselLayout msel_layout(const SelectPlan& p) {
  MselLayout m;
  const uint32_t groups = p.adaptive ? (uint32_t)p.H : 1u;
  m.cpg = (uint32_t)((p.n_cand + kChunk - 1) / kChunk);
  m.chunks = groups * m.cpg;
  const size_t chunks = (size_t)p.segments * m.chunks;
  m.states_off = 0;
  m.ghist_off = al256s((size_t)kSlots * p.segments * sizeof(SegState));
  m.ccount_off = m.ghist_off + al256s((size_t)kHistBufs * p.segments * kBins * sizeof(uint32_t));
  m.list_off = m.ccount_off + al256s(chunks * sizeof(uint32_t));
  m.mask_off = m.list_off + al256s((size_t)p.segments * kListCap * sizeof(uint2));
  m.mask1_off = m.mask_off + al256s(chunks * kMaskWords * sizeof(uint32_t));
  m.bytes = m.mask1_off + (p.two_stage ? al256s(chunks * kMaskWords * sizeof(uint32_t)) : 0);
  return m;
}

static bool use_multi(const SelectPlan& p) { return p.seg_len > kResidentMax; }

// pass 0: k_msel_hist0, 1: k_msel_hist1, 2: k_msel_filter, for the load
// width and the stage
template <int PASS>
static void launch_msel_passes(bool vec, bool s2, dim3 grid, hipStream_t st, const MselArgs& a,
                               int final, bool h2 = false) {
  auto go = [&](auto v, auto t) {
    constexpr bool V = decltype(v)::value, T = decltype(t)::value;
    if constexpr (PASS == 0)
      hipLaunchKernelGGL((k_msel_hist0<V, T>), grid, dim3(kMThreads), 0, st, a);
    else if constexpr (PASS == 1)
      hipLaunchKernelGGL((k_msel_hist1<V, T>), grid, dim3(kMThreads), 0, st, a);
    else if constexpr (T)
      hipLaunchKernelGGL((k_msel_filter<V, true, false>), grid, dim3(kMThreads), 0, st, a, final);
    else if (h2)
      hipLaunchKernelGGL((k_msel_filter<V, false, true>), grid, dim3(kMThreads), 0, st, a, final);
    else
      hipLaunchKernelGGL((k_msel_filter<V, false, false>), grid, dim3(kMThreads), 0, st, a, final);
  };
  if (vec && s2) go(std::true_type{}, std::true_type{});
  else if (vec) go(std::true_type{}, std::false_type{});
  else if (s2) go(std::false_type{}, std::true_type{});
  else go(std::false_type{}, std::false_type{});
}

template <int R>
static hipError_t launch_msel_pool(const MselArgs& a, const float* raw, int64_t in_stride,
                                   float* pooled, bool vec, dim3 grid, hipStream_t st) {
  const void* f = vec ? reinterpret_cast<const void*>(&k_msel_pool<R, true>)
                      : reinterpret_cast<const void*>(&k_msel_pool<R, false>);
  const hipError_t e =
      hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPoolLdsBytes);
  if (e != hipSuccess) return e;
  if (vec)
    hipLaunchKernelGGL((k_msel_pool<R, true>), grid, dim3(kMThreads), kPoolLdsBytes, st, a, raw,
                       in_stride, pooled);
  else
    hipLaunchKernelGGL((k_msel_pool<R, false>), grid, dim3(kMThreads), kPoolLdsBytes, st, a, raw,
                       in_stride, pooled);
  return hipSuccess;
}

static hipError_t msel_launch(const SelectPlan& p, const float* scores, const float* weight,
                              int32_t* idx, int32_t* head_offsets, uint8_t* stage, void* ws,
                              hipStream_t st) {
  const MselLayout m = msel_layout(p);
  char* w = static_cast<char*>(ws);
  // raw rows (kvsel_select_pool): the first pass pools them into
  // p.pooled, which every later pass reads
  const bool pool_first = p.pooled != nullptr;
  MselArgs a;
  a.scores = pool_first ? p.pooled : scores;
  a.weight = p.two_stage ? weight : nullptr;
  a.states = reinterpret_cast<SegState*>(w + m.states_off);
  a.ghist = reinterpret_cast<uint32_t*>(w + m.ghist_off);
  a.ccount = reinterpret_cast<uint32_t*>(w + m.ccount_off);
  a.list = reinterpret_cast<uint2*>(w + m.list_off);
  a.mask = reinterpret_cast<uint32_t*>(w + m.mask_off);
  a.mask1 = p.two_stage ? reinterpret_cast<uint32_t*>(w + m.mask1_off) : nullptr;
  a.idx = idx;
  a.head_offsets = p.adaptive ? head_offsets : nullptr;
  a.stage = stage;
  a.segs = (uint32_t)p.segments;
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
  // the call can be captured in a graph); stage 1's finish clears them for
  // stage 2
  const dim3 gc((unsigned)blocks), gp(p.segments);
  const int stages = p.two_stage ? 2 : 1;
  // 16-byte loads when every chunk starts 16-byte aligned and is a
  // multiple of 4 long (scores and weights are 16-byte aligned)
  const bool vec = p.n_cand % 4 == 0;
  hipLaunchKernelGGL(k_msel_init, gp, dim3(kMThreads), 0, st, a);
  for (int stg = 0; stg < stages; ++stg) {
    const int stage2 = stg == 1 ? 1 : 0, final = stg + 1 == stages ? 1 : 0;
    if (stg == 0 && pool_first) {
      const bool pvec = vec && p.in_stride % 4 == 0;
      hipError_t e;
      switch (p.pool_r) {
        case 0: e = launch_msel_pool<0>(a, scores, p.in_stride, p.pooled, pvec, gc, st); break;
        case 1: e = launch_msel_pool<1>(a, scores, p.in_stride, p.pooled, pvec, gc, st); break;
        case 2: e = launch_msel_pool<2>(a, scores, p.in_stride, p.pooled, pvec, gc, st); break;
        default: e = launch_msel_pool<3>(a, scores, p.in_stride, p.pooled, pvec, gc, st); break;
      }
      if (e != hipSuccess) return e;
    } else if (stg == 0) {
      launch_msel_passes<0>(vec, false, gc, st, a, 0);
    }   // stage 2's round 0 comes with stage 1's filter and finish
    launch_msel_passes<1>(vec, stage2 != 0, gc, st, a, 0);
    launch_msel_passes<2>(vec, stage2 != 0, gc, st, a, final, p.two_stage && stg == 0);
    hipLaunchKernelGGL(k_msel_finish, gp, dim3(kMThreads), 0, st, a, stage2, final);
  }
  hipLaunchKernelGGL(k_msel_emit, gc, dim3(kMThreads), 0, st, a, p.two_stage ? 1 : 0);
  return hipGetLastError();
}

constexpr size_t kStageBytes = (kStagePad + (size_t)kResidentMax) * sizeof(float);
static_assert(sizeof(SelShared) <= 160 * 1024 && kStageBytes <= 160 * 1024,
              "the shared state and a staged segment fit the CU's LDS");

// A resident segment is staged with 16-byte loads when its rows are
// 16-byte aligned (the base is: every tensor is) and its length rounded up
// to 4 stays inside its row.
static bool stageable(const SelectPlan& p, int64_t in_stride) {
  return p.seg_len <= kResidentMax && in_stride % 4 == 0 && ((p.seg_len + 3) & ~int64_t(3)) <= in_stride;
}

bool select_pools_on_chip(const SelectPlan& p, int pool_r) {
  return !p.adaptive && !p.budgets && pool_r >= 0 && pool_r <= kMaxPoolR && stageable(p, p.n);
}

bool select_pools_in_passes(const SelectPlan& p, int pool_r) {
  return use_multi(p) && !p.budgets && pool_r >= 0 && pool_r <= kMaxPoolR;
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
  a.budgets = p.budgets;
  a.H = (uint32_t)p.H;
  a.stride = p.stride;
  a.alpha = p.alpha;
  if (p.budgets) a.head_offsets = head_offsets;
  a.in_stride = p.in_stride > 0 ? p.in_stride : p.seg_len;
  a.pool_r = p.pool_r;
  a.pooled = p.pooled;
  // raw rows (a stride other than seg_len) and pooling: on chip on the
  // staged resident path; in the first pass of the many-workgroup path,
  // into `pooled` (required there)
  const bool raw_in = a.in_stride != p.seg_len || p.pool_r > 0 || p.pooled;
  if (use_multi(p)) {
    if (raw_in && !(select_pools_in_passes(p, p.pool_r) && p.pooled && p.in_stride >= p.n_cand))
      return hipErrorInvalidValue;
    return msel_launch(p, scores, weight, idx, head_offsets, stage, ws, st);
  }
  if (raw_in && !select_pools_on_chip(p, p.pool_r)) return hipErrorInvalidValue;
  a.staged = stageable(p, a.in_stride) ? 1 : 0;
  const size_t lds = a.staged ? std::max(sizeof(SelShared), kStageBytes) : sizeof(SelShared);
  const hipError_t e =
      hipFuncSetAttribute((const void*)k_select, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select, dim3(p.segments), dim3(kSelThreads), lds, st, a);
  return hipGetLastError();
}

bool select_groups_ok(int groups) { return groups <= kMaxGroups; }

}  // namespace kvsel
