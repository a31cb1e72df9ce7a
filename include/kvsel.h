/*
 * kvsel.h -- prefill-end KV-cache importance scoring, selection and
 * compaction on AMD Instinct MI355X (gfx950). C ABI.
 *
 * Sources, cited below by page title and section:
 *   [CriticalKV] "CriticalKV: Optimizing KV Cache Eviction from an Output
 *                Perturbation Perspective" (Korean translation, sumin.im)
 *   [KVzip]      review of "KVzip: Query-Agnostic KV Cache Compression with
 *                Context Reconstruction" (manon006.tistory.com)
 *   [AnchorKV]   review of "AnchorKV: Anchor-Residual KV Cache Compression"
 *                (charstring.tistory.com)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    keeps no pointer after a call returns. bf16 tensors are passed as
 *    `const void*` (IEEE bfloat16, 2 bytes); other types are as declared.
 *    Every tensor is dense, row-major, in the layout documented per call,
 *    and must be 16-byte aligned.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream). Outputs are valid once the stream has been
 *    synchronised. No call allocates device memory or synchronises.
 *  - Every argument check runs before anything is launched: a call that
 *    returns non-zero has launched nothing and written nothing.
 *  - Workspace protocol (kvsel_score, kvsel_score_chunked,
 *    kvsel_value_weight, kvsel_select, kvsel_select_pool, kvsel_select_budgets,
 *    kvsel_head_budgets, kvsel_anchor_select, kvsel_anchor_assign,
 *    kvsel_decode_attention): with ws == NULL the
 *    call stores the bytes it needs in *ws_bytes, returns KVSEL_OK and
 *    launches nothing. Otherwise *ws_bytes is the size of `ws` (checked).
 *    Workspace contents need no initialisation and are scratch afterwards.
 *    Two calls in flight at once must use different workspaces.
 *  - Floating-point inputs must be finite; results are unspecified
 *    otherwise. Results are bitwise reproducible for identical inputs
 *    (no floating-point atomics anywhere).
 *  - Calls are thread-safe when they use distinct outputs and workspaces.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVSEL_OK = 0,
  KVSEL_ERR_ARG = 1,          /* null required pointer, bad size, bad range */
  KVSEL_ERR_UNSUPPORTED = 2,  /* valid request this build does not cover    */
  KVSEL_ERR_WORKSPACE = 3,    /* ws given but *ws_bytes is too small        */
  KVSEL_ERR_HIP = 4,          /* a HIP launch failed; outputs undefined     */
  KVSEL_ERR_SCRATCH = 5       /* needs more than the static scratch holds   */
};

/* Which queries score the cache. */
enum {
  /* The W queries are the cache's own last W tokens ([CriticalKV] §3.3,
     Algorithm 2, step 2: Q_hat = Q[-n':]). Query i sits at position n-W+i
     and sees keys 0..n-W+i (causal). Candidates are positions [0, n-W); the
     window itself is always kept by kvsel_select. */
  KVSEL_Q_WINDOW = 0,
  /* The W queries come from outside the cache (KVzip's reconstruction
     queries, [KVzip] §3.2) and see all n keys. Candidates are [0, n). */
  KVSEL_Q_EXTERNAL = 1
};

/* How the per-query softmax weights of one key are aggregated. */
enum {
  /* Sum over the W queries and the G query heads of the KV head
     ([CriticalKV] §3.3, Algorithm 2, step 3, as a sum: the mean only
     rescales by 1/(W*G)). The raw scores of one head sum to W*G. */
  KVSEL_AGG_SUM = 0,
  /* Max over the W queries and the G query heads ([KVzip] §3.2). */
  KVSEL_AGG_MAX = 1,
  /* No softmax: max over the W queries and the G query heads of the logit
     s itself (KVzip-logit, [KVzip] §6.5). KVSEL_Q_EXTERNAL only. Scores
     may be negative; kvsel_select orders them as signed values. */
  KVSEL_AGG_LOGIT_MAX = 2
};

/*
 * kvsel_score -- attention-based importance of every cached key.
 *
 * Per layer l and KV head h, with query head hq = h*G + g (GQA grouping,
 * [KVzip] §2.2): logits s = scale * <q[l][hq][i], k[l][h][j]>, a softmax
 * over the keys each query sees (all n, or causal in window mode; none for
 * KVSEL_AGG_LOGIT_MAX), the aggregate over (g, i) chosen by `agg`, then
 * 1-D max-pooling of width `pool` along the candidate positions
 * ([CriticalKV] §3.3, Algorithm 2, step 4; stride 1, centred, neighbours
 * outside [0, n_cand) ignored).
 *
 *   q      bf16 [L][H_kv*G][W][d]
 *   k      bf16 [L][H_kv][n][d]
 *   scores f32  [L][H_kv][n_cand]  pooled scores, n_cand = n-W (window)
 *                                  or n (external); may be NULL when raw is
 *                                  given: then no pooling is done (the
 *                                  raw-input selection kvsel_select_pool
 *                                  pools itself)
 *   raw    f32  [L][H_kv][n]       optional (NULL): pre-pool aggregate over
 *                                  all n keys, window keys included
 *   scale  softmax temperature (the model's 1/sqrt(d)), > 0
 *   pool   odd, >= 1 (1 = no pooling)
 *
 * Limits: d == 128; one head's K and one head's query rows must each span
 * less than 2^31 bytes (n <= 8388607 and G*W <= 8388607); else
 * KVSEL_ERR_UNSUPPORTED. Window mode needs 1 <= W < n. Needs a workspace
 * (protocol above).
 */
int32_t kvsel_score(const void* q, const void* k,
                    int32_t L, int32_t H_kv, int32_t G, int32_t d, int32_t n,
                    int32_t W, int32_t q_mode, int32_t agg, float scale,
                    int32_t pool, float* scores, float* raw,
                    void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_score_chunked -- KVzip's chunked scoring with the input's own keys.
 *
 * [KVzip] §3.4: the n cached keys of each (layer, head) are split into
 * T = ceil(n/m) chunks of m (the last one m_T = n - (T-1)*m long). Chunk t
 * is reconstructed from an input of n_in_t = n_prompt + m_t tokens whose
 * queries attend over the chunk's cached keys (all visible) and the
 * input's own keys (causal: input position i sees own keys 0..i):
 *   A = softmax_j(scale * <q[l][t][hq][i], [k_chunk ; k_self][j]>)
 * and the chunk's keys score max over g < G and i < n_in_t of the cached
 * part of A, then max-pooling of width `pool` over all n positions as in
 * kvsel_score. Inputs hold every chunk at the full n_in = n_prompt + m:
 *
 *   q      bf16 [L][T][H_kv*G][n_in][d]  chunk t's queries (rows past n_in_t
 *                                        are ignored but must be finite)
 *   k      bf16 [L][H_kv][n][d]          the cache
 *   k_self bf16 [L][T][H_kv][n_in][d]    chunk t's own keys (rows past n_in_t
 *                                        are ignored)
 *   scores f32  [L][H_kv][n]             pooled
 *   raw    f32  [L][H_kv][n]             optional (NULL): before pooling
 *
 * m larger than n is taken as n (one chunk). Limits: d == 128;
 * G*n_in*d*2 and n*d*2 each below 2^31 bytes; pool odd <= 65. Needs a
 * workspace (protocol above).
 */
int32_t kvsel_score_chunked(const void* q, const void* k, const void* k_self,
                            int32_t L, int32_t H_kv, int32_t G, int32_t d,
                            int32_t n, int32_t m, int32_t n_prompt, float scale,
                            int32_t pool, float* scores, float* raw,
                            void* ws, size_t* ws_bytes, void* stream);

/* How the G query heads of a KV head combine in kvsel_value_weight. */
enum {
  /* Mean over g of the L1 norm of each query head's projection (Theorem
     3.3 of [CriticalKV] is per attention head; the group's attention is
     summed before pooling). */
  KVSEL_GROUP_MEAN_OF_NORMS = 0,
  /* L1 norm of the group-summed projection (sum_g W_O^(h,g)) v: one
     D-vector per KV head and position, the size of the V W^O intermediate
     [CriticalKV] §D.4 quotes; G times fewer matrix flops. */
  KVSEL_GROUP_NORM_OF_SUM = 1
};

/*
 * kvsel_value_weight -- CriticalKV's projected-value norm.
 *
 * [CriticalKV] §3.3, Algorithm 1, steps 2-3: V_proj = V W^O and the L1
 * norm of each row of V_proj (Theorem 3.3: the output perturbation is
 * bounded by attention weight times this norm). W_O^(h,g) is the D x d
 * column slice w_o[l][:][(h*G+g)*d .. +d) of query head h*G+g. For j < n_cand:
 *   group_mode 0 (KVSEL_GROUP_MEAN_OF_NORMS):
 *     weight[l][h][j] = (1/G) sum_g sum_{c<D} | (W_O^(h,g) v[l][h][j])_c |
 *   group_mode 1 (KVSEL_GROUP_NORM_OF_SUM):
 *     weight[l][h][j] = sum_{c<D} | ((sum_g W_O^(h,g)) v[l][h][j])_c |
 * The projection is accumulated in fp32 from bf16 and is never written
 * out. In mode 1 the summed slices are formed in fp32 and rounded once to
 * bf16 (round to nearest-even) in the workspace before the product.
 *
 *   v      bf16 [L][H_kv][n][d]
 *   w_o    bf16 [L][D][H_kv*G*d]     output projection, (out, in) layout
 *   weight f32  [L][H_kv][n_cand]    1 <= n_cand <= n
 *
 * Limits: d == 128, D % 32 == 0, and one layer's w_o must span less than
 * 2^31 bytes (D * H_kv*G*d * 2 < 2^31); else KVSEL_ERR_UNSUPPORTED.
 * Needs a workspace (protocol above): none for mode 0 (0 bytes; any
 * 16-byte-aligned non-NULL ws runs the call), L*D*H_kv*d*2 bytes for mode 1.
 */
int32_t kvsel_value_weight(const void* v, const void* w_o,
                           int32_t L, int32_t H_kv, int32_t G, int32_t d,
                           int32_t n, int32_t D, int32_t n_cand, int32_t group_mode,
                           float* weight, void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_value_l2_factor, kvsel_value_weight_l2 -- the L2 form of the
 * projected-value norm.
 *
 * [CriticalKV] §C.3 and footnote 1 (the L1 and L2 distances of the output
 * perturbation give similar gains), with the GQA mean of kvsel_value_weight:
 *   weight[l][h][j] = (1/G) sum_g sqrt( sum_{c<D} ( sum_{e<d}
 *                        w_o[l][c][(h*G+g)*d + e] * v[l][h][j][e] )^2 )
 * for j < n_cand. Since ||W v||_2^2 = v^T (W^T W) v = ||R v||_2^2 for the
 * Cholesky factor R (upper triangular, R^T R = W^T W) of each query head's
 * d x d Gram matrix, the weight is computed in two calls:
 *
 * kvsel_value_l2_factor: R for every (layer, query head), from the model's
 * output projection alone, so it is computed once per model and reused.
 * The Gram matrix is accumulated in fp32 from bf16 and factored in fp32;
 * R is stored as two bf16 matrices whose sum carries it to ~2^-17
 * relative. W^T W is treated as positive definite: a pivot below 1e-6 of
 * the largest diagonal entry is taken as zero (its direction dropped), so
 * a rank-deficient slice (D < d, or dependent columns) is factored up to
 * that threshold.
 *
 *   w_o    bf16 [L][D][H_kv*G*d]          output projection, (out, in) layout
 *   factor bf16 [L][H_kv*G][2][d][d]      out: R_hi, R_lo (zero below the
 *                                         diagonal); L*H_kv*G*4*d*d bytes
 *
 * kvsel_value_weight_l2: the weight from the values and the factor.
 *
 *   v      bf16 [L][H_kv][n][d]
 *   factor bf16 [L][H_kv*G][2][d][d]      as written by kvsel_value_l2_factor
 *   weight f32  [L][H_kv][n_cand]         1 <= n_cand <= n
 *
 * Limits: d == 128, else KVSEL_ERR_UNSUPPORTED.
 */
int32_t kvsel_value_l2_factor(const void* w_o, int32_t L, int32_t H_kv,
                              int32_t G, int32_t d, int32_t D,
                              void* factor, void* stream);

int32_t kvsel_value_weight_l2(const void* v, const void* factor,
                              int32_t L, int32_t H_kv, int32_t G, int32_t d,
                              int32_t n, int32_t n_cand, float* weight,
                              void* stream);

/*
 * kvsel_select -- which cache entries to keep.
 *
 * Candidates are positions [0, n-W) of every head; the W window positions
 * [n-W, n) are always kept and count toward the budget. Among candidates
 * the k = budget - W (per head) or k = budget - H_kv*W (per layer, when
 * adaptive) largest keys are kept; equal keys go to the lower index
 * (adaptive: lower head, then lower position). Keys compare as signed
 * floats (-0 equal to +0); a NaN key counts as below every number.
 *
 *  - weight == NULL: key = scores ([CriticalKV] §3.3, Algorithm 2, step 6).
 *  - weight != NULL: CriticalKV's two-stage selection ([CriticalKV] §3.3,
 *    Algorithm 1, steps 3-9): stage 1 keeps k1 = floor(alpha*k) entries by
 *    score; stage 2 keeps k - k1 of the rest by the integrated score
 *      (score*score_norm + eps) * weight
 *    computed in fp32 as mul, add, mul, each rounded once.
 *  - adaptive == 0: one budget per head. adaptive == 1: one budget per
 *    layer shared by its heads, selected over the flattened candidates of
 *    all heads (the non-uniform head budget of [KVzip] §4.2 / AdaKV).
 *
 *   scores       f32 [L][H_kv][n-W]
 *   weight       f32 [L][H_kv][n-W]    optional
 *   idx          i32 adaptive == 0: [L][H_kv][budget]  (may be NULL if budget == 0)
 *                    adaptive == 1: [L][budget], grouped by head
 *                Per head: kept candidates ascending, then n-W..n-1.
 *   head_offsets i32 [L][H_kv+1]  adaptive == 1 only (required there):
 *                head h of layer l owns idx[l][head_offsets[l][h] ..
 *                head_offsets[l][h+1]).
 *   stage        u8 same shape as idx, optional: 0 window, 1 stage 1 (or
 *                the single stage), 2 stage 2.
 *
 * Ranges: 0 <= W < n; W <= budget <= n (per head) or
 * H_kv*W <= budget <= H_kv*n (per layer); 0 <= alpha <= 1;
 * score_norm > 0, eps >= 0. Needs a workspace (protocol above).
 */
int32_t kvsel_select(const float* scores, const float* weight,
                     int32_t L, int32_t H_kv, int32_t n, int32_t W,
                     int64_t budget, int32_t adaptive,
                     float score_norm, float eps, float alpha,
                     int32_t* idx, int32_t* head_offsets, uint8_t* stage,
                     void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_select_pool -- kvsel_select on scores it max-pools itself.
 *
 * The same selection as kvsel_score(..., pool, scores, raw, ...) followed
 * by kvsel_select(scores, ...), from the raw aggregates alone: the keys
 * are raw max-pooled with width `pool` over each head's candidate
 * positions [0, n-W) (stride 1, centred, neighbours outside [0, n-W)
 * ignored: [CriticalKV] §3.3, Algorithm 2, steps 4 and 6), then selected
 * as kvsel_select selects. With a per-head budget (adaptive == 0),
 * pool <= 7, n a multiple of 4 and n-W <= 34,816, each head's raw row is
 * read once and pooled on chip: the pooled scores need not pass through
 * memory. Otherwise the pooled scores go to `pooled`, or the workspace:
 * written by the selection's first pass over the raw rows when the
 * segments are longer than 34,816 candidates and pool <= 7, else by a
 * pooling pass before the selection.
 *
 *   raw     f32 [L][H_kv][n]      kvsel_score's raw output (window keys
 *                                 included; they are not pooled)
 *   pool    odd, 1 <= pool <= 65 (else KVSEL_ERR_ARG / _UNSUPPORTED)
 *   pooled  f32 [L][H_kv][n-W]    optional (NULL): the pooled scores
 *   weight, idx, head_offsets, stage and every other argument as in
 *   kvsel_select; the results are those of kvsel_select on the pooled
 *   scores, bit for bit. Needs a workspace (protocol above).
 */
int32_t kvsel_select_pool(const float* raw, const float* weight, int32_t pool,
                          int32_t L, int32_t H_kv, int32_t n, int32_t W,
                          int64_t budget, int32_t adaptive,
                          float score_norm, float eps, float alpha,
                          int32_t* idx, int32_t* head_offsets, uint8_t* stage,
                          float* pooled, void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_select_static -- kvsel_select without a workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same
 * arguments, outputs and results as kvsel_select, bit for bit; the scratch
 * memory kvsel_select takes from `ws` comes instead from a static device
 * array of kvsel_static_scratch_bytes() bytes (16 MiB) that each GPU the
 * library runs on holds until the process ends. The call allocates
 * nothing. A request whose workspace (kvsel_select's *ws_bytes) exceeds
 * that size returns KVSEL_ERR_SCRATCH and launches nothing. All calls on
 * one GPU share its array: calls that overlap on a GPU (concurrent streams
 * or threads) race and give undefined results; calls ordered on one
 * stream are safe. The first call on a device looks up that device's copy
 * of the array (the device current at the call).
 */
int32_t kvsel_select_static(const float* scores, const float* weight,
                            int32_t L, int32_t H_kv, int32_t n, int32_t W,
                            int64_t budget, int32_t adaptive,
                            float score_norm, float eps, float alpha,
                            int32_t* idx, int32_t* head_offsets, uint8_t* stage,
                            void* stream);

/* Size in bytes of kvsel_select_static's static scratch (per GPU). */
size_t kvsel_static_scratch_bytes(void);

/*
 * kvsel_select_budgets -- per-head selection under a budget vector.
 *
 * [CriticalKV] §4.1 combines the method with HeadKV, whose offline budget
 * allocation gives every head of every layer its own budget. Head h of
 * layer l keeps b = budgets[l][h] entries, its W window positions included;
 * b is clamped into [W, n]. Among its candidates [0, n-W) it keeps the
 * k = b - W largest keys exactly as kvsel_select does per head (equal keys
 * to the lower index; two-stage when weight != NULL, with
 * k1 = floor(alpha*k) computed in double).
 *
 *   scores       f32 [L][H_kv][n-W]
 *   weight       f32 [L][H_kv][n-W]    optional
 *   budgets      i32 [L][H_kv]         DEVICE memory, read by the kernels
 *   idx          i32 [L][layer_stride] out: the layer's heads packed in
 *                order, each as its kept candidates ascending then
 *                n-W..n-1; entries past the last head hold -1
 *   head_offsets i32 [L][H_kv+1]       out: head h owns idx[l][head_offsets
 *                [l][h] .. head_offsets[l][h+1])
 *   stage        u8 [L][layer_stride]  optional, as for kvsel_select
 *                (0 also past the last head)
 *
 * layer_stride should be at least the largest per-layer sum of the clamped
 * budgets. If a layer's sum is larger, nothing is written past its row:
 * its head offsets are clipped to layer_stride and the heads that cross it
 * lose their trailing entries (a truncated selection for those heads).
 * The idx rows, the head offsets and kvsel_compact / kvsel_decode_attention
 * then use kept_per_layer = layer_stride.
 *
 * Ranges: 0 <= W < n; 1 <= layer_stride <= H_kv*n; alpha, score_norm and
 * eps as for kvsel_select. Needs a workspace (protocol above).
 */
int32_t kvsel_select_budgets(const float* scores, const float* weight,
                             int32_t L, int32_t H_kv, int32_t n, int32_t W,
                             const int32_t* budgets, int64_t layer_stride,
                             float score_norm, float eps, float alpha,
                             int32_t* idx, int32_t* head_offsets, uint8_t* stage,
                             void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_head_score -- head-level importance.
 *
 * [KVzip] §3.4: the score of a head is the maximum of its per-position
 * scores over the sequence, head_score[l][h] = max_i scores[l][h][i].
 *
 *   scores     f32 [L][H_kv][n_pos]   e.g. kvsel_score's scores or raw
 *   head_score f32 [L][H_kv]
 *
 * NaN entries are ignored (a row of NaN gives -inf).
 */
int32_t kvsel_head_score(const float* scores, int32_t L, int32_t H_kv,
                         int32_t n_pos, float* head_score, void* stream);

/*
 * kvsel_head_budgets -- budgets of head-level eviction.
 *
 * [KVzip] §3.6 / §5.4: context-independent eviction keeps or drops whole
 * heads by their head score, in DuoAttention's structure where a dropped
 * head holds only a recent window. The `keep` heads with the largest
 * head_score over all layers and heads (equal scores to the lower flat
 * index l*H_kv + h; scores ordered as by kvsel_select) get budget n, the
 * others budget W: the budget vector kvsel_select_budgets takes.
 *
 *   head_score f32 [L][H_kv]
 *   budgets    i32 [L][H_kv]   out
 *
 * Ranges: 0 <= keep <= L*H_kv; 0 <= W <= n. Needs a workspace (protocol
 * above).
 */
int32_t kvsel_head_budgets(const float* head_score, int32_t L, int32_t H_kv,
                           int32_t keep, int32_t n, int32_t W, int32_t* budgets,
                           void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_anchor_select -- AnchorKV's anchor positions.
 *
 * [AnchorKV] §3.2 (anchor selection): each KV head keeps k anchors. The W
 * most recent positions [n-W, n) are always anchors and count toward k;
 * of the remaining k - W slots, k1 = floor(rho * (k - W)) (computed in
 * double) go to the candidates [0, n-W) with the largest pooled score
 * (equal scores to the lower position), the rest are drawn uniformly
 * without replacement among the other candidates: the ones with the
 * largest draws rand[l][h][j] (equal draws to the lower position). The
 * draws are the caller's (e.g. uniform in [0, 1)). The page's settings
 * are k = n/128, W = 32, rho = 0.7.
 *
 *   scores  f32 [L][H_kv][n-W]   pooled (kvsel_score)
 *   rand    f32 [L][H_kv][n-W]   finite draws
 *   anchors i32 [L][H_kv][k]     out: ascending positions
 *
 * Ranges: 0 <= W < n; W <= k <= n; 0 <= rho <= 1. Needs a workspace
 * (protocol above).
 */
int32_t kvsel_anchor_select(const float* scores, const float* rand,
                            int32_t L, int32_t H_kv, int32_t n, int32_t W,
                            int32_t k, float rho, int32_t* anchors,
                            void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_anchor_assign -- AnchorKV's nearest-anchor representation.
 *
 * [AnchorKV] §3.1: anchors are stored exactly; every other vector of the
 * head is projected onto the span of the single anchor with the largest
 * cosine similarity and kept as that anchor's slot and the coefficient
 *   gamma = <x, a> / <a, a>.
 * Equal cosines go to the lower slot; an anchor of zero norm is never
 * chosen; an anchor position is its own slot with gamma = 1. Call once for
 * the keys (the page projects pre-RoPE keys) and once for the values.
 * Dot products are fp32 sums of exact bf16 products. Scores <x, a>/|a| are
 * compared after adding |x| (so none is negative) with their last 4
 * mantissa bits replaced by a code of the slot's row, which makes equal
 * scores go to the lower slot; two anchors whose cosines agree to within
 * ~4e-6 may therefore be chosen either way, and gamma carries a relative
 * error below 4e-6 of |x|/|a|.
 *
 *   x       bf16 [L][H_kv][n][d]
 *   anchors i32  [L][H_kv][k]    positions (kvsel_anchor_select)
 *   slot    i32  [L][H_kv][n]    out: index into anchors[l][h]
 *   gamma   f32  [L][H_kv][n]    out
 *
 * Limits: d == 128, k <= 2048, L*H_kv <= 65535 (else
 * KVSEL_ERR_UNSUPPORTED). Anchor positions outside [0, n) count as zero
 * vectors. Positions are expected to be distinct (kvsel_anchor_select's
 * are); a position listed twice maps to one of its slots, which one is
 * unspecified. Needs a workspace (protocol above).
 */
int32_t kvsel_anchor_assign(const void* x, const int32_t* anchors,
                            int32_t L, int32_t H_kv, int32_t d, int32_t n,
                            int32_t k, int32_t* slot, float* gamma,
                            void* ws, size_t* ws_bytes, void* stream);

/*
 * kvsel_compact -- gather the kept rows of K and V.
 *
 * Eviction acts on the un-replicated cache ([KVzip] §4.2): kept row t of
 * layer l, head h, is a bit copy of k[l][h][idx[...]][:] (same for v).
 *
 *   k, v         bf16 [L][H_kv][n][d]
 *   idx          i32  as written by kvsel_select: head_offsets == NULL ->
 *                     [L][H_kv][B] with B = kept_per_layer / H_kv;
 *                     otherwise [L][kept_per_layer] grouped by head
 *   head_offsets i32  [L][H_kv+1] or NULL
 *   k_out, v_out bf16 [L][kept_per_layer][d]  (uniform: = [L][H_kv][B][d])
 *
 * Every idx entry must lie in [0, n); out-of-range entries are not read
 * (their rows are written as zeros). With head_offsets, only the rows
 * before head_offsets[l][H_kv] (clamped into [0, kept_per_layer]) are
 * written; a layer's later rows (the unused end of a kvsel_select_budgets
 * row) are left as they were. d % 8 == 0.
 */
int32_t kvsel_compact(const void* k, const void* v,
                      int32_t L, int32_t H_kv, int32_t d, int32_t n,
                      const int32_t* idx, const int32_t* head_offsets,
                      int64_t kept_per_layer, void* k_out, void* v_out,
                      void* stream);

/*
 * kvsel_decode_attention -- one decoding step over the kept rows.
 *
 * [KVzip] §7.1 (decoding efficiency): after eviction every KV head keeps
 * its own number of rows, and a new token's attention runs over each
 * head's kept rows with a variable-length kernel. The query of query head
 * h*G+g attends over the kept rows of KV head h:
 *   out[l][h*G+g] = sum_t softmax_t(scale * <q[l][h*G+g], k_t>) * v_t
 * over the rows t that kvsel_compact wrote for head h. A head with no kept
 * rows gives zeros. The new token's own key and value are not part of the
 * call (append them to the kept rows to include them).
 *
 *   q            bf16 [L][H_kv*G][d]          the new token's queries
 *   k, v         bf16 [L][kept_per_layer][d]  kept rows (kvsel_compact's
 *                                             output layouts)
 *   head_offsets i32  [L][H_kv+1] or NULL: head h of layer l owns rows
 *                [head_offsets[l][h], head_offsets[l][h+1]) (as written by
 *                kvsel_select); NULL: every head owns kept_per_layer/H_kv
 *                consecutive rows. Each offset is clamped into
 *                [0, kept_per_layer] and then raised to the largest offset
 *                before it in the row, so heads are disjoint ranges of the
 *                layer's rows (valid offsets are unchanged; a head whose
 *                end is not past its start is empty).
 *   out          f32  [L][H_kv*G][d]
 *   scale        softmax temperature (the model's 1/sqrt(d)), > 0
 *
 * fp32 from bf16: exact products, fp32 sums, base-2 exponentials with the
 * scale folded in. Limits: d == 128, 1 <= G <= 8, H_kv <= 1024 (else
 * KVSEL_ERR_UNSUPPORTED); kept_per_layer >= 1, divisible by H_kv when
 * head_offsets is NULL. Needs a workspace (protocol above).
 */
int32_t kvsel_decode_attention(const void* q, const void* k, const void* v,
                               int32_t L, int32_t H_kv, int32_t G, int32_t d,
                               int64_t kept_per_layer, const int32_t* head_offsets,
                               float scale, float* out,
                               void* ws, size_t* ws_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* kvsel_status_str(int32_t status);

/* ABI version of this header: 2. */
int32_t kvsel_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
