"""Plain CPU oracle for prefill-end KV-cache importance scoring and selection.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this package. The library's
own path never does, and shares no code with it (inputs come from the
separate `synth` generator).

Everything is float64 numpy, written as the plain definition: no blocking,
fusion or reordering beyond what the definition states. Library primitives
used as steps: matrix product, exp, sort.

Sources (cited by page title and section):
  [CriticalKV]  the sumin.im Korean translation of "CriticalKV: Optimizing
                KV Cache Eviction from an Output Perturbation Perspective"
  [KVzip]       the manon006.tistory.com review of "KVzip: Query-Agnostic KV
                Cache Compression with Context Reconstruction"

Readings taken where the pages are silent (each repeated where it is used):
  scale     logits are scale * <q, k> with scale an argument (the model's
            1/sqrt(d)); the pages print softmax(QK^T) with no scale.
  causal    window query i (of W) sits at cache position n-W+i and sees
            keys 0..n-W+i; external queries see all n keys.
  sum       window scores sum (not average) over the W queries and the G
            query heads of a KV head; the mean only rescales by 1/(W*G).
  window    candidates are positions [0, n-W); the W window positions are
            always kept and count toward the budget.
  pool      max-pooling: kernel `pool`, stride 1, centred, over candidates
            only; out-of-range neighbours are ignored.
  weight    value weight of KV head h at position j:
            mean over g of || W_O[:, slice(h*G+g)] v_j ||_1, in fp64
            (|| . ||_2 for the L2 variant); or, summed over the group,
            || sum_g W_O[:, slice(h*G+g)] v_j ||_1.
  key       two-stage key = (pooled * score_norm + eps) * weight, applied
            after pooling; stage 1 takes floor(alpha*k) by pooled score.
  ties      larger key first; equal keys go to the lower index (adaptive:
            lower head, then lower position). Output positions ascending.
  max mode  KVzip's max over queries, softmax over the n cached keys only.
  decode    attention of one new query per query head over its KV head's
            kept rows only; an empty head gives zeros.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "window_raw_scores", "external_raw_scores", "maxpool", "value_weight",
    "value_weight_group_sum",
    "topk_indices", "select_layer", "compact_layer",
]


# --------------------------------------------------------------- scoring ----

def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Row softmax; -inf entries (masked) get weight 0."""
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def window_raw_scores(q: np.ndarray, k: np.ndarray, G: int, scale: float,
                      agg: str = "sum") -> np.ndarray:
    """Observation-window attention scores of every cached key.

    [CriticalKV, §3.3 Algorithm 2, steps 2-3]: Q_hat = the last n' queries,
    A = softmax(Q_hat K^T), then aggregated over the window queries.
    GQA grouping (query head h*G+g reads KV head h) follows [KVzip, §2.2].
    Readings: causal window, explicit scale, sum over W and G (or max over
    them when agg='max'; masked entries contribute nothing).

    q: [H_kv*G][W][d], k: [H_kv][n][d] (float64). Returns raw [H_kv][n].
    """
    H, n, d = k.shape
    Hq, W, _ = q.shape
    assert Hq == H * G and 0 < W < n
    pos = n - W + np.arange(W)                       # cache position of query i
    visible = np.arange(n)[None, :] <= pos[:, None]  # causal mask [W][n]
    raw = np.zeros((H, n))
    for h in range(H):
        for g in range(G):
            logits = scale * (q[h * G + g] @ k[h].T)  # [W][n]
            logits = np.where(visible, logits, -np.inf)
            p = _softmax_rows(logits)
            if agg == "sum":
                raw[h] += p.sum(axis=0)
            else:
                raw[h] = np.maximum(raw[h], p.max(axis=0))
    return raw


def external_raw_scores(q: np.ndarray, k: np.ndarray, G: int, scale: float,
                        agg: str = "max", q_chunk: int = 512) -> np.ndarray:
    """Scores from queries outside the cache (KVzip's reconstruction queries).

    [KVzip, §3.2]: A = Softmax(Q K^T) for the G x n_in group queries, then
    S = max over g and i of the slice of A on the cached keys. Reading: the
    softmax runs over the n cached keys only (synthetic queries have no
    self-keys). agg='sum' sums over g and i instead. Queries are processed
    q_chunk at a time ([KVzip, §3.4] processes the input in chunks); max and
    sum over queries do not depend on the chunking.

    q: [H_kv*G][Q_s][d], k: [H_kv][n][d]. Returns raw [H_kv][n].
    """
    H, n, d = k.shape
    Hq, Qs, _ = q.shape
    assert Hq == H * G
    raw = np.zeros((H, n))
    for h in range(H):
        for g in range(G):
            for c0 in range(0, Qs, q_chunk):
                p = _softmax_rows(scale * (q[h * G + g, c0:c0 + q_chunk] @ k[h].T))
                if agg == "max":
                    raw[h] = np.maximum(raw[h], p.max(axis=0))
                else:
                    raw[h] += p.sum(axis=0)
    return raw


def chunked_scores(q: np.ndarray, k_cache: np.ndarray, k_self: np.ndarray, G: int,
                   scale: float, m: int, n_prompt: int) -> np.ndarray:
    """KVzip's chunked scoring, with the input's own keys in the softmax.

    [KVzip, §3.4]: the context's n cached keys are split into T = ceil(n/m)
    chunks of m. Chunk t is reconstructed on its own from an input of
    n_in = n_prompt + m_t tokens (the repeat prompt, then the chunk), whose
    queries attend over the chunk's cached keys followed by the input's own
    n_in keys: A = Softmax(Q [K_chunk; K_self]^T), an n_in x (m_t + n_in)
    matrix per query head. The slice of A on the cached keys, maxed over the
    group queries and input positions, scores the chunk's keys.
    Readings: the logits carry the model's scale; the input's own keys are
    causal (input position i sees its keys 0..i), the cached keys all
    visible (the context precedes the input); the last chunk may be shorter
    (m_t = n - t*m), its input then n_prompt + m_t tokens long.

    q: [T][H_kv*G][n_in_max][d], k_cache: [H_kv][n][d],
    k_self: [T][H_kv][n_in_max][d] with n_in_max = n_prompt + m (rows past a
    chunk's own n_in are ignored). Returns [H_kv][n].
    """
    H, n, d = k_cache.shape
    T = (n + m - 1) // m
    assert q.shape[0] == T and q.shape[1] == H * G and k_self.shape[0] == T
    S = np.zeros((H, n))
    for t in range(T):
        c0 = t * m
        mt = min(m, n - c0)
        nin = n_prompt + mt
        for h in range(H):
            keys = np.concatenate([k_cache[h, c0:c0 + mt], k_self[t, h, :nin]])   # [mt + nin][d]
            hidden = np.zeros((nin, mt + nin), bool)
            hidden[:, mt:] = np.triu(np.ones((nin, nin), bool), 1)   # self key j > position i
            for g in range(G):
                logits = scale * (q[t, h * G + g, :nin] @ keys.T)
                a = _softmax_rows(np.where(hidden, -np.inf, logits))
                S[h, c0:c0 + mt] = np.maximum(S[h, c0:c0 + mt], a[:, :mt].max(axis=0))
    return S


def external_logit_scores(q: np.ndarray, k: np.ndarray, G: int, scale: float) -> np.ndarray:
    """The softmax-free scores of KVzip-logit.

    [KVzip, §6.5]: the variant drops the softmax normalisation and scores a
    cached key by the raw attention logits it receives, aggregated like the
    softmax scores of §3.2 (max over the group queries and input positions).
    Reading: the logit is the model's scaled one, scale * <q, k> (the scale
    is common to every head, so it changes no ordering); scores may be
    negative.

    q: [H_kv*G][Q_s][d], k: [H_kv][n][d]. Returns [H_kv][n].
    """
    H, n, d = k.shape
    assert q.shape[0] == H * G
    out = np.full((H, n), -np.inf)
    for h in range(H):
        for g in range(G):
            lg = scale * (q[h * G + g] @ k[h].T)    # [Q_s][n] logits
            out[h] = np.maximum(out[h], lg.max(axis=0))
    return out


def head_scores(scores: np.ndarray) -> np.ndarray:
    """Head-level importance.

    [KVzip, §3.4 and §3.6]: the score of a head is the maximum of its
    per-position scores over the sequence, S_head = max_i S[:, :, i].
    scores: [..., n_pos]. Returns scores.shape[:-1].
    """
    return scores.max(axis=-1)


def head_budgets(head_score: np.ndarray, keep: int, n: int, W: int) -> np.ndarray:
    """Budgets of head-level eviction.

    [KVzip, §3.6 and §5.4]: context-independent eviction keeps or drops
    whole heads by their head score, in DuoAttention's structure, where the
    heads not kept hold only a recent window. Readings: `keep` heads with
    the largest score over all layers and heads keep all n entries (ties to
    the lower flat (layer, head) index); the others keep the last W entries.

    head_score: [L][H]. Returns budgets [L][H] (n or W), the input of the
    per-head budget selection.
    """
    flat = head_score.reshape(-1)
    top = topk_indices(flat, keep)
    b = np.full(flat.shape, W, np.int64)
    b[top] = n
    return b.reshape(head_score.shape)


def maxpool(raw: np.ndarray, n_cand: int, pool: int) -> np.ndarray:
    """[CriticalKV, §3.3 Algorithm 2, step 4] (SnapKV's max-pooling, kernel 7
    in [CriticalKV, §4.1]). Reading: stride 1, centred, over candidate
    positions [0, n_cand) only; neighbours outside that range are ignored.

    raw: [..., n] with n >= n_cand. Returns pooled [..., n_cand].
    """
    assert pool >= 1 and pool % 2 == 1
    r = pool // 2
    src = raw[..., :n_cand]
    out = src.copy()
    for off in range(1, r + 1):
        if off >= n_cand:
            break
        out[..., off:] = np.maximum(out[..., off:], src[..., :n_cand - off])
        out[..., :n_cand - off] = np.maximum(out[..., :n_cand - off], src[..., off:])
    return out


# ---------------------------------------------------------- value weight ----

def value_weight(v: np.ndarray, w_o: np.ndarray, G: int,
                 positions: np.ndarray | None = None) -> np.ndarray:
    """CriticalKV's projected-value norm.

    [CriticalKV, §3.3 Algorithm 1, steps 2-3]: V_proj = V W^O and the L1 norm
    of each row of V_proj (Theorem 3.3 bounds the output perturbation by
    attention weight times this norm; the L1 distance is the paper's choice,
    footnote 1 and §C.3). Reading under GQA: query head hq = h*G+g projects
    KV head h's values through its own d columns of W_O, and the weight of
    KV head h is the mean over its G query heads.

    v: [H_kv][n][d], w_o: [D][H_kv*G*d] (torch Linear layout).
    positions: optional subset of positions. Returns [H_kv][len(positions)].
    """
    H, n, d = v.shape
    if positions is None:
        positions = np.arange(n)
    out = np.zeros((H, len(positions)))
    for h in range(H):
        vh = v[h, positions]                           # [m][d]
        for g in range(G):
            hq = h * G + g
            w_slice = w_o[:, hq * d:(hq + 1) * d]      # [D][d]
            proj = vh @ w_slice.T                      # [m][D] rows of V W^O
            out[h] += np.abs(proj).sum(axis=1)
        out[h] /= G
    return out


def value_weight_group_sum(v: np.ndarray, w_o: np.ndarray, G: int,
                           positions: np.ndarray | None = None) -> np.ndarray:
    """CriticalKV's projected-value norm with the GQA group summed first.

    [CriticalKV, §3.3 Algorithm 1, steps 2-3]: V_proj = V W^O, then the L1
    norm of each row. The alternative GQA reading: the G query heads that
    share KV head h see the same value row, and their attention outputs
    enter the output projection side by side, so one projected row per KV
    head is (sum_g W_O^(h,g)) v_j, with W_O^(h,g) the D x d column slice of
    query head h*G+g. This is the size of the V W^O intermediate that
    [CriticalKV, §D.4] quotes (one D-vector per KV head and position).
    Weight = || (sum_g W_O^(h,g)) v_j ||_1, the slices summed exactly.

    v: [H_kv][n][d], w_o: [D][H_kv*G*d]. Returns [H_kv][len(positions)].
    """
    H, n, d = v.shape
    if positions is None:
        positions = np.arange(n)
    out = np.zeros((H, len(positions)))
    for h in range(H):
        w_sum = np.zeros((w_o.shape[0], d))
        for g in range(G):
            hq = h * G + g
            w_sum += w_o[:, hq * d:(hq + 1) * d]      # [D][d]
        proj = v[h, positions] @ w_sum.T              # [m][D]
        out[h] = np.abs(proj).sum(axis=1)
    return out


def value_weight_l2(v: np.ndarray, w_o: np.ndarray, G: int,
                    positions: np.ndarray | None = None) -> np.ndarray:
    """The L2 variant of CriticalKV's projected-value norm.

    [CriticalKV, §C.3 and footnote 1]: the L1 and L2 distances are compared
    and the L2 one gives similar gains. Weight of KV head h at position j:
    mean over its G query heads of || W_O^(h,g) v_j ||_2, with the same
    column slices and GQA reading as value_weight.

    v: [H_kv][n][d], w_o: [D][H_kv*G*d]. Returns [H_kv][len(positions)].
    """
    H, n, d = v.shape
    if positions is None:
        positions = np.arange(n)
    out = np.zeros((H, len(positions)))
    for h in range(H):
        vh = v[h, positions]
        for g in range(G):
            hq = h * G + g
            proj = vh @ w_o[:, hq * d:(hq + 1) * d].T      # [m][D]
            out[h] += np.sqrt((proj * proj).sum(axis=1))
        out[h] /= G
    return out


# -------------------------------------------------------------- selection ----

def topk_indices(key: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries, equal keys to the lower index,
    returned ascending. ([CriticalKV, §3.3] Top_k; tie rule is a reading.)"""
    order = np.lexsort((np.arange(key.shape[0]), -key))
    return np.sort(order[:k])


def _stage_key(score, weight, score_norm, eps, dtype):
    """Integrated score (A*score_norm + eps) * weight, in `dtype`.

    [CriticalKV, §3.3 Algorithm 1, step 3 and footnote 3 (eps = 1E-4)].
    With dtype float32 each operation rounds once, in this order:
    mul, add, mul (the precision a float32 kernel decides in)."""
    if dtype == np.float32:
        s = np.asarray(score, np.float32)
        t = s * np.float32(score_norm)
        t = t + np.float32(eps)
        return t * np.asarray(weight, np.float32)
    return (np.asarray(score, np.float64) * score_norm + eps) * np.asarray(weight, np.float64)


def _two_stage(score, weight, k, alpha, score_norm, eps, dtype):
    """[CriticalKV, §3.3 Algorithm 1, steps 4-9]: b' = floor(alpha*b) picked by
    attention score (stage 1); the remaining b - b' picked among the rest by
    the integrated score (stage 2). Returns (ascending indices, stage 1|2)."""
    k1 = int(np.floor(alpha * k))
    s1 = topk_indices(score, k1)
    rest = np.ones(score.shape[0], dtype=bool)
    rest[s1] = False
    cand = np.nonzero(rest)[0]
    key = _stage_key(score, weight, score_norm, eps, dtype)
    s2 = cand[topk_indices(key[cand], k - k1)]
    idx = np.concatenate([s1, s2])
    stage = np.concatenate([np.ones(len(s1), np.uint8), np.full(len(s2), 2, np.uint8)])
    o = np.argsort(idx, kind="stable")
    return idx[o], stage[o]


def select_layer(scores: np.ndarray, budget: int, W: int, n: int,
                 adaptive: bool = False, weight: np.ndarray | None = None,
                 alpha: float = 0.5, score_norm: float = 1.0, eps: float = 1e-4,
                 dtype=np.float64):
    """Kept positions of one layer.

    scores: pooled [H][n_cand] (n_cand = n - W). weight: optional [H][n_cand].
    budget: kept entries incl. the W window positions, per head, or per layer
    when adaptive (reading: the window counts toward the budget, so
    k = budget - W per head, or budget - H*W per layer).
    adaptive: one top-k over all heads' candidates of the layer — the
    non-uniform head budget of [KVzip, §4.2] / AdaKV in [CriticalKV, §3.3
    Algorithm 2, step 1], ties by (head, position).
    weight given: CriticalKV two-stage selection [CriticalKV, Algorithm 1].

    Returns (idx, head_offsets, stage): uniform -> idx [H][budget],
    head_offsets None; adaptive -> idx [budget] packed by head and
    head_offsets [H+1]. Per head: candidates ascending, then the window
    n-W..n-1. stage: 0 window, 1 stage 1 / single stage, 2 stage 2.
    """
    H, n_cand = scores.shape
    assert n_cand == n - W
    window = np.arange(n - W, n)
    if not adaptive:
        k = budget - W
        assert 0 <= k <= n_cand
        idx = np.empty((H, budget), np.int64)
        stage = np.empty((H, budget), np.uint8)
        for h in range(H):
            if weight is None:
                pick, st = topk_indices(scores[h], k), None
                st = np.ones(k, np.uint8)
            else:
                pick, st = _two_stage(scores[h], weight[h], k, alpha, score_norm, eps, dtype)
            idx[h] = np.concatenate([pick, window])
            stage[h] = np.concatenate([st, np.zeros(W, np.uint8)])
        return idx, None, stage
    k = budget - H * W
    assert 0 <= k <= H * n_cand
    flat = scores.reshape(-1)
    if weight is None:
        pick = topk_indices(flat, k)
        st = np.ones(k, np.uint8)
    else:
        pick, st = _two_stage(flat, weight.reshape(-1), k, alpha, score_norm, eps, dtype)
    heads, pos = np.divmod(pick, n_cand)
    idx_parts, st_parts, offs = [], [], [0]
    for h in range(H):
        sel = heads == h
        idx_parts += [pos[sel], window]
        st_parts += [st[sel], np.zeros(W, np.uint8)]
        offs.append(offs[-1] + int(sel.sum()) + W)
    return np.concatenate(idx_parts), np.asarray(offs, np.int64), np.concatenate(st_parts)


def select_budgets(scores: np.ndarray, budgets, W: int, n: int,
                   weight: np.ndarray | None = None, alpha: float = 0.5,
                   score_norm: float = 1.0, eps: float = 1e-4, dtype=np.float64):
    """Kept positions of one layer under a per-head budget vector.

    [CriticalKV, §4.1]: the method is combined with HeadKV, whose offline
    budget allocation gives every head of every layer its own budget.
    Reading: budgets[h] counts head h's W window positions, as the uniform
    budget does, and is clamped into [W, n] (a head keeps at least its window
    and at most everything). Each head is then selected on its own, exactly
    as by select_layer with a uniform budget: the top k_h = budgets[h] - W
    candidates (two-stage when weight is given), then the window.

    scores, weight: [H][n_cand], n_cand = n - W. budgets: [H].
    Returns (idx [sum of clamped budgets] packed by head, head_offsets [H+1],
    stage), the packing of the adaptive layout.
    """
    H, n_cand = scores.shape
    assert n_cand == n - W
    b = np.clip(np.asarray(budgets, np.int64), W, n)
    window = np.arange(n - W, n)
    idx_parts, st_parts, offs = [], [], [0]
    for h in range(H):
        k = int(b[h]) - W
        if weight is None:
            pick = topk_indices(scores[h], k)
            st = np.ones(k, np.uint8)
        else:
            pick, st = _two_stage(scores[h], weight[h], k, alpha, score_norm, eps, dtype)
        idx_parts += [pick, window]
        st_parts += [st, np.zeros(W, np.uint8)]
        offs.append(offs[-1] + k + W)
    return np.concatenate(idx_parts), np.asarray(offs, np.int64), np.concatenate(st_parts)


def anchor_select(pooled: np.ndarray, rand: np.ndarray, n: int, W: int, k: int,
                  rho: float) -> np.ndarray:
    """AnchorKV's anchor positions of one layer.

    [AnchorKV, §3.2, anchor selection]: each KV head keeps k anchors. The
    W most recent positions are always anchors and count toward k; of the
    remaining k - W slots a fraction rho goes to the best positions by the
    pooled SnapKV score, the rest to positions drawn uniformly at random
    from the context. Readings: floor(rho * (k - W)) slots by score (ties to
    the lower position); the random ones are drawn without replacement from
    the candidates not already taken, as the largest of per-position uniform
    draws `rand` (the draws are an input: equal draws to the lower position).

    pooled, rand: [H][n - W]. Returns anchors [H][k]: ascending positions.
    """
    H, n_cand = pooled.shape
    assert n_cand == n - W and W <= k <= n
    k1 = int(np.floor(rho * (k - W)))
    out = np.empty((H, k), np.int64)
    for h in range(H):
        by_score = topk_indices(pooled[h], k1)
        rest = np.setdiff1d(np.arange(n_cand), by_score)
        drawn = rest[topk_indices(rand[h][rest], k - W - k1)]
        out[h] = np.sort(np.concatenate([by_score, drawn, np.arange(n - W, n)]))
    return out


def anchor_assign(x: np.ndarray, anchors: np.ndarray):
    """AnchorKV's anchor-residual representation of one layer (no residual).

    [AnchorKV, §3.1]: anchors are stored exactly; every other vector is
    projected orthogonally onto the span of the single anchor with the
    largest cosine similarity, kept as that anchor's index and the scalar
    coefficient gamma = <x, a> / <a, a>. Readings: keys and values are
    assigned separately (call once per tensor); equal cosines go to the
    lower anchor slot; an anchor with zero norm is never chosen; an anchor
    position is its own slot with gamma = 1.

    x: [H][n][d]; anchors: [H][k] positions. Returns (slot [H][n] indices
    into anchors[h], gamma [H][n]).
    """
    H, n, d = x.shape
    k = anchors.shape[1]
    slot = np.empty((H, n), np.int64)
    gamma = np.empty((H, n))
    for h in range(H):
        A = x[h, anchors[h]]                                  # [k][d]
        na = np.sqrt((A * A).sum(axis=1))
        nx = np.sqrt((x[h] * x[h]).sum(axis=1))
        dots = x[h] @ A.T                                     # [n][k]
        with np.errstate(divide="ignore", invalid="ignore"):
            cos = dots / (nx[:, None] * na[None, :])
        cos = np.where(na[None, :] > 0, np.nan_to_num(cos, nan=0.0), -np.inf)
        best = np.argmax(cos, axis=1)                         # first of equal maxima
        slot[h] = best
        gamma[h] = dots[np.arange(n), best] / np.where(na[best] > 0, na[best] ** 2, 1.0)
        slot[h, anchors[h]] = np.arange(k)
        gamma[h, anchors[h]] = 1.0
    return slot, gamma


# -------------------------------------------------------------- compaction ----

def compact_layer(k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                  head_offsets: np.ndarray | None = None):
    """Gather the kept rows from the un-replicated KV cache.

    [KVzip, §4.2]: eviction acts on the original cache before GQA
    replication, so the kept rows of KV head h come from k[h], v[h].
    Bit copies: works on any dtype (bf16 bit patterns included).
    Uniform: idx [H][B] -> [H][B][d]; packed: idx [B_layer] with
    head_offsets [H+1] -> [B_layer][d].
    """
    if head_offsets is None:
        H = k.shape[0]
        return (np.stack([k[h, idx[h]] for h in range(H)]),
                np.stack([v[h, idx[h]] for h in range(H)]))
    ko, vo = [], []
    for h in range(len(head_offsets) - 1):
        sl = idx[head_offsets[h]:head_offsets[h + 1]]
        ko.append(k[h, sl])
        vo.append(v[h, sl])
    return np.concatenate(ko), np.concatenate(vo)


# ------------------------------------------------ decode over the kept rows ----

def decode_attention(q: np.ndarray, k_kept: np.ndarray, v_kept: np.ndarray, G: int,
                     scale: float, head_offsets: np.ndarray | None = None) -> np.ndarray:
    """One decoding step of attention over the compacted cache of one layer.

    [KVzip, §7.1] (decoding efficiency): after eviction every KV head keeps
    its own number of rows (non-uniform head budgets), and a new token's
    attention runs over each head's kept rows with a variable-length kernel.
    The query of query head h*G+g attends over the kept rows of KV head h:
        out[h*G+g] = softmax_t(scale * <q[h*G+g], k_t>) . v_t   (t kept in h)
    Readings: the call covers the kept rows only (the new token's own K/V
    are the caller's to append); a head with no kept rows gives zeros.

    q [H*G][d]; uniform layout: k_kept, v_kept [H][B][d]; packed layout:
    [B_layer][d] with head_offsets [H+1] (the kvsel_compact layouts).
    Returns [H*G][d] float64.
    """
    q = np.asarray(q, np.float64)
    k_kept = np.asarray(k_kept, np.float64)
    v_kept = np.asarray(v_kept, np.float64)
    if head_offsets is None:
        heads = [(k_kept[h], v_kept[h]) for h in range(k_kept.shape[0])]
    else:
        heads = [(k_kept[head_offsets[h]:head_offsets[h + 1]], v_kept[head_offsets[h]:head_offsets[h + 1]])
                 for h in range(len(head_offsets) - 1)]
    out = np.zeros((len(heads) * G, q.shape[-1]))
    for h, (kh, vh) in enumerate(heads):
        if kh.shape[0] == 0:
            continue
        for g in range(G):
            p = _softmax_rows(scale * (q[h * G + g] @ kh.T)[None, :])[0]
            out[h * G + g] = p @ vh
    return out
