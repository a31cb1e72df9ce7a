"""Pins that tie the CPU oracle to something other than itself.

Each check takes an oracle module `o` and raises AssertionError (or any
exception) when the oracle disagrees with:
  - brute force: explicit Python loops over tiny inputs (full causal n x n
    attention, triple-loop projections, pairwise top-k conditions);
  - closed forms and hand-worked examples (tests/golden/*.txt, each with its
    derivation and citation);
  - special cases that reduce to a library routine (scipy softmax,
    torch max_pool1d, torch index_select);
  - invariants (scores of a head sum to W*G, max-mode scores in [1/n, 1]).
The mutation tests run the same checks against copies of the oracle with a
planted mistake and require each copy to fail at least one check.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = [float(x) for x in val.split()]
    return out


def _embed_1d(vals, d=4):
    """d=1 vectors embedded as (x, 0, ..., 0) in d dims."""
    a = np.zeros((len(vals), d))
    a[:, 0] = vals
    return a


# ------------------------------------------------------- window scoring ----

def _bruteforce_window(q, k, G, scale, extra_queries):
    """Full causal attention over all n positions with explicit loops; keeps
    the last W rows and sums them per KV head."""
    H, n, d = k.shape
    Hq, W, _ = q.shape
    raw = [[0.0] * n for _ in range(H)]
    for hq in range(Hq):
        h = hq // G
        # queries for every position: earlier ones arbitrary, last W = window
        qfull = [list(extra_queries[hq][p]) for p in range(n - W)] + \
                [list(q[hq][i]) for i in range(W)]
        for p in range(n):
            logits = []
            for j in range(p + 1):
                s = 0.0
                for e in range(d):
                    s += qfull[p][e] * k[h][j][e]
                logits.append(scale * s)
            mx = max(logits)
            z = sum(math.exp(x - mx) for x in logits)
            if p >= n - W:
                for j in range(p + 1):
                    raw[h][j] += math.exp(logits[j] - mx) / z
    return np.array(raw)


def check_window_bruteforce(o):
    rng = np.random.default_rng(11)
    for (H, G, d, n, W) in [(2, 3, 3, 7, 2), (1, 1, 2, 5, 1), (2, 2, 4, 9, 4), (3, 2, 3, 6, 5)]:
        q = rng.standard_normal((H * G, W, d)) * 1.5
        k = rng.standard_normal((H, n, d)) * 1.5
        extra = rng.standard_normal((H * G, n, d))
        scale = 0.7
        ref = _bruteforce_window(q, k, G, scale, extra)
        got = o.window_raw_scores(q, k, G, scale)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def check_window_sum_invariant(o):
    rng = np.random.default_rng(12)
    H, G, d, n, W = 3, 4, 16, 300, 32
    q = rng.standard_normal((H * G, W, d))
    k = rng.standard_normal((H, n, d)) * rng.uniform(0.5, 4, size=(H, n, 1))
    raw = o.window_raw_scores(q, k, G, 1 / math.sqrt(d))
    np.testing.assert_allclose(raw.sum(axis=1), W * G, rtol=1e-12)
    assert (raw >= 0).all()


def check_window_equal_keys(o):
    g = load_golden("window_equal_keys.txt")
    n, W, G = int(g["n"][0]), int(g["W"][0]), int(g["G"][0])
    rng = np.random.default_rng(13)
    d = 8
    q = rng.standard_normal((G, W, d))
    k = np.tile(rng.standard_normal(d), (1, n, 1))
    raw = o.window_raw_scores(q, k, G, 0.3)[0]
    np.testing.assert_allclose(raw, g["raw"], rtol=1e-12)
    # general (n, W, G) against exact harmonic sums
    for (n, W, G) in [(40, 7, 3), (17, 16, 1), (64, 32, 4)]:
        q = rng.standard_normal((2 * G, W, d))
        k = np.tile(rng.standard_normal(d), (2, n, 1))
        raw = o.window_raw_scores(q, k, G, 0.25)
        pre = G * sum(Fraction(1, n - W + i + 1) for i in range(W))
        win = [G * sum(Fraction(1, n - W + i + 1) for i in range(t, W)) for t in range(W)]
        exp = np.array([float(pre)] * (n - W) + [float(x) for x in win])
        for h in range(2):
            np.testing.assert_allclose(raw[h], exp, rtol=1e-12)


def check_window_hand_example(o):
    g = load_golden("window_hand_example.txt")
    q = _embed_1d(g["q"])[None]              # [1][W=2][d]
    k = _embed_1d(g["k"])[None]              # [1][n=4][d]
    raw = o.window_raw_scores(q, k, 1, 1.0)[0]
    np.testing.assert_allclose(raw, g["raw"], rtol=1e-12)
    # the same closed form written out here
    e = math.e
    z2, z3 = 2 + e, 2 + 2 * e
    np.testing.assert_allclose(raw, [1 / z2 + 1 / z3, e / z2 + e / z3, 1 / z2 + 1 / z3, e / z3],
                               rtol=1e-13)


def check_window_single_query_softmax(o):
    """W = 1, G = 1: the last query sees every key -> one softmax row."""
    from scipy.special import softmax
    rng = np.random.default_rng(14)
    for n, d, scale in [(50, 8, 0.35), (257, 16, 1.0)]:
        q = rng.standard_normal((1, 1, d))
        k = rng.standard_normal((1, n, d))
        raw = o.window_raw_scores(q, k, 1, scale)[0]
        np.testing.assert_allclose(raw, softmax(scale * (k[0] @ q[0, 0])), rtol=1e-12)


def check_window_max_agg(o):
    rng = np.random.default_rng(15)
    H, G, d, n, W = 2, 2, 3, 8, 3
    q = rng.standard_normal((H * G, W, d))
    k = rng.standard_normal((H, n, d))
    scale = 0.8
    got = o.window_raw_scores(q, k, G, scale, agg="max")
    ref = np.zeros((H, n))
    for hq in range(H * G):
        h = hq // G
        for i in range(W):
            p = n - W + i
            lg = [scale * sum(q[hq, i, e] * k[h, j, e] for e in range(d)) for j in range(p + 1)]
            mx = max(lg)
            z = sum(math.exp(x - mx) for x in lg)
            for j in range(p + 1):
                ref[h, j] = max(ref[h, j], math.exp(lg[j] - mx) / z)
    np.testing.assert_allclose(got, ref, rtol=1e-12)


# ----------------------------------------------------- external scoring ----

def check_external(o):
    from scipy.special import softmax
    g = load_golden("external_hand_example.txt")
    q = _embed_1d(g["q"])[None]
    k = _embed_1d(g["k"])[None]
    raw = o.external_raw_scores(q, k, 1, 1.0, agg="max")[0]
    np.testing.assert_allclose(raw, g["raw"], rtol=1e-12)
    rng = np.random.default_rng(16)
    # one query, G = 1 -> one softmax row over all n keys
    n, d = 77, 8
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, n, d))
    np.testing.assert_allclose(o.external_raw_scores(q, k, 1, 0.5)[0],
                               softmax(0.5 * (k[0] @ q[0, 0])), rtol=1e-12)
    # brute force (loops), ranges, and chunk independence
    H, G, Qs, n, d = 2, 3, 5, 9, 3
    q = rng.standard_normal((H * G, Qs, d)) * 2
    k = rng.standard_normal((H, n, d)) * 2
    scale = 0.6
    ref = np.zeros((H, n))
    refsum = np.zeros((H, n))
    for hq in range(H * G):
        h = hq // G
        for i in range(Qs):
            lg = [scale * sum(q[hq, i, e] * k[h, j, e] for e in range(d)) for j in range(n)]
            mx = max(lg)
            z = sum(math.exp(x - mx) for x in lg)
            for j in range(n):
                pj = math.exp(lg[j] - mx) / z
                ref[h, j] = max(ref[h, j], pj)
                refsum[h, j] += pj
    for ch in (1, 2, 512):
        np.testing.assert_allclose(o.external_raw_scores(q, k, G, scale, "max", ch), ref, rtol=1e-12)
    np.testing.assert_allclose(o.external_raw_scores(q, k, G, scale, "sum", 2), refsum, rtol=1e-12)
    np.testing.assert_allclose(refsum.sum(axis=1), G * Qs, rtol=1e-12)
    big = o.external_raw_scores(rng.standard_normal((4, 64, 16)), rng.standard_normal((2, 300, 16)), 2, 0.25)
    assert (big <= 1 + 1e-15).all() and (big.max(axis=1) >= 1 / 300).all()


def check_external_logit(o):
    g = load_golden("logit_head_example.txt")
    qv = g["logit.q"]
    q = _embed_1d(qv).reshape(2, 2, 4)            # query heads of one KV head, 2 queries each
    k = _embed_1d(g["logit.k"])[None]
    sc = g["logit.scale"][0]
    np.testing.assert_allclose(o.external_logit_scores(q, k, 2, sc)[0], g["logit.scores"], rtol=1e-15)
    q1 = _embed_1d([-1.0])[None]
    np.testing.assert_allclose(o.external_logit_scores(q1, k, 1, sc)[0], g["logit.one_query_scores"],
                               rtol=1e-15)
    rng = np.random.default_rng(45)
    # brute force with loops
    H, G, Qs, n, d = 2, 3, 4, 7, 3
    q = rng.standard_normal((H * G, Qs, d))
    k = rng.standard_normal((H, n, d))
    ref = np.full((H, n), -np.inf)
    for hq in range(H * G):
        for i in range(Qs):
            for j in range(n):
                x = 0.7 * sum(q[hq, i, e] * k[hq // G, j, e] for e in range(d))
                ref[hq // G, j] = max(ref[hq // G, j], x)
    got = o.external_logit_scores(q, k, G, 0.7)
    np.testing.assert_allclose(got, ref, rtol=1e-13)
    # a positive factor on the scale scales the max
    np.testing.assert_allclose(o.external_logit_scores(q, k, G, 1.4), 2 * got, rtol=1e-13)
    # one query: the same order as the softmax scores (softmax is monotonic
    # along a row)
    q1 = rng.standard_normal((1, 1, 16))
    kk = rng.standard_normal((1, 200, 16))
    a = o.external_logit_scores(q1, kk, 1, 0.25)[0]
    b = o.external_raw_scores(q1, kk, 1, 0.25)[0]
    np.testing.assert_array_equal(np.argsort(a), np.argsort(b))


def check_head_scores_and_budgets(o):
    g = load_golden("logit_head_example.txt")
    sc = np.asarray(g["heads.scores"]).reshape(2, 3, 4)
    hs = o.head_scores(sc)
    np.testing.assert_array_equal(hs.reshape(-1), g["heads.head_scores"])
    np.testing.assert_array_equal(o.head_budgets(hs, 3, 100, 8).reshape(-1), g["heads.budgets_keep3"])
    np.testing.assert_array_equal(o.head_budgets(hs, 2, 100, 8).reshape(-1), g["heads.budgets_keep2"])
    rng = np.random.default_rng(46)
    for trial in range(10):
        L, H, m = 3, 4, 9
        sc = rng.integers(0, 4, size=(L, H, m)).astype(np.float64)
        hs = o.head_scores(sc)
        for l in range(L):
            for h in range(H):
                assert hs[l, h] == max(sc[l, h, i] for i in range(m))
        keep = int(rng.integers(0, L * H + 1))
        b = o.head_budgets(hs, keep, 50, 5)
        assert set(np.unique(b)) <= {5, 50} and (b == 50).sum() == keep
        _assert_topk_property(hs.reshape(-1), list(np.nonzero(b.reshape(-1) == 50)[0]), keep)


def check_chunked(o):
    g = load_golden("chunked_example.txt")
    m, npr = int(g["m"][0]), int(g["n_prompt"][0])
    k = _embed_1d(g["k_cache"])[None]
    q = np.stack([_embed_1d(g["q_chunk0"]), _embed_1d(g["q_chunk1"])])[:, None]     # [T][1][3][4]
    ks = np.stack([_embed_1d(g["kself_chunk0"]), _embed_1d(g["kself_chunk1"])])[:, None]
    np.testing.assert_allclose(o.chunked_scores(q, k, ks, 1, 1.0, m, npr)[0], g["scores"], rtol=1e-14)
    rng = np.random.default_rng(47)
    # brute force with loops: H = 2, G = 2, n = 7, m = 3 (chunks 3, 3, 1)
    H, G, n, m, npr, d, sc = 2, 2, 7, 3, 2, 3, 0.8
    T, nin_max = 3, npr + m
    q = rng.standard_normal((T, H * G, nin_max, d))
    k = rng.standard_normal((H, n, d))
    ks = rng.standard_normal((T, H, nin_max, d))
    ref = np.zeros((H, n))
    for t in range(T):
        mt = min(m, n - t * m)
        nin = npr + mt
        for hq in range(H * G):
            h = hq // G
            for i in range(nin):
                lg = [sc * sum(q[t, hq, i, e] * k[h, t * m + j, e] for e in range(d)) for j in range(mt)]
                own = [sc * sum(q[t, hq, i, e] * ks[t, h, j, e] for e in range(d)) for j in range(i + 1)]
                mx = max(lg + own)
                z = sum(math.exp(x - mx) for x in lg + own)
                for j in range(mt):
                    ref[h, t * m + j] = max(ref[h, t * m + j], math.exp(lg[j] - mx) / z)
    got = o.chunked_scores(q, k, ks, G, sc, m, npr)
    np.testing.assert_allclose(got, ref, rtol=1e-12)
    # a chunk's scores depend on its own inputs only; rows past a chunk's
    # input (the last chunk's padding) are ignored; every weight is <= 1
    q2, ks2 = q.copy(), ks.copy()
    q2[0] += 1.0
    ks2[0] -= 1.0
    q2[2, :, npr + 1:] = 50.0
    ks2[2, :, npr + 1:] = -3.0
    got2 = o.chunked_scores(q2, k, ks2, G, sc, m, npr)
    np.testing.assert_allclose(got2[:, m:], got[:, m:], rtol=1e-15)
    assert not np.allclose(got2[:, :m], got[:, :m])
    assert (got <= 1).all() and (got > 0).all()


def check_anchor_select(o):
    g = load_golden("anchor_example.txt")
    n, W, k = int(g["select.n"][0]), int(g["select.W"][0]), int(g["select.k"][0])
    got = o.anchor_select(np.array([g["select.pooled"]]), np.array([g["select.rand"]]), n, W, k,
                          g["select.rho"][0])
    np.testing.assert_array_equal(got[0], g["select.anchors"])
    rng = np.random.default_rng(48)
    for trial in range(10):
        H, n, W = 3, 60, 4
        k = int(rng.integers(W, n + 1))
        rho = float(rng.choice([0.0, 0.3, 0.7, 1.0]))
        pooled = rng.integers(0, 5, size=(H, n - W)).astype(np.float64)
        rand = rng.random((H, n - W))
        got = o.anchor_select(pooled, rand, n, W, k, rho)
        k1 = int(math.floor(rho * (k - W)))
        for h in range(H):
            row = list(got[h])
            assert row == sorted(row) and len(set(row)) == k and row[-W:] == list(range(n - W, n))
            cand = [p for p in row if p < n - W]
            # some k1 of them are a top-k1 by score; the others a top by the
            # draws among what the score part left
            by_score = [int(p) for p in o.topk_indices(pooled[h], k1)]
            _assert_topk_property(pooled[h], by_score, k1)
            assert set(by_score) <= set(cand)
            rest = [p for p in range(n - W) if p not in set(by_score)]
            drawn = [rest.index(p) for p in cand if p not in set(by_score)]
            _assert_topk_property(np.array([rand[h][p] for p in rest]), drawn, k - W - k1)
        # the same as the two-stage selection with stage 2 keyed by the draws:
        # (score * 0 + 1) * rand
        idx, _, _ = o.select_layer(pooled, k, W, n, weight=rand, alpha=rho, score_norm=0.0, eps=1.0)
        np.testing.assert_array_equal(np.sort(idx, axis=1), got)


def check_anchor_assign(o):
    g = load_golden("anchor_example.txt")
    x = np.asarray(g["assign.x"]).reshape(1, -1, 2)
    anchors = np.asarray(g["assign.anchors"], np.int64)[None]
    slot, gamma = o.anchor_assign(x, anchors)
    np.testing.assert_array_equal(slot[0], g["assign.slot"])
    np.testing.assert_allclose(gamma[0], g["assign.gamma"], rtol=1e-15, atol=1e-15)
    rng = np.random.default_rng(49)
    H, n, d, k = 2, 40, 5, 6
    x = rng.standard_normal((H, n, d))
    anchors = np.sort(np.stack([rng.choice(n, k, replace=False) for _ in range(H)]), axis=1)
    slot, gamma = o.anchor_assign(x, anchors)
    for h in range(H):
        for j in range(n):
            if j in set(anchors[h]):
                assert anchors[h][slot[h, j]] == j and gamma[h, j] == 1.0
                continue
            best, bs = -2.0, -1
            for s_ in range(k):
                a = x[h, anchors[h][s_]]
                c = sum(a[e] * x[h, j, e] for e in range(d)) / (
                    math.sqrt(sum(v * v for v in a)) * math.sqrt(sum(v * v for v in x[h, j])))
                if c > best:
                    best, bs = c, s_
            assert slot[h, j] == bs
            a = x[h, anchors[h][bs]]
            gm = sum(a[e] * x[h, j, e] for e in range(d)) / sum(v * v for v in a)
            assert abs(gamma[h, j] - gm) <= 1e-12 * max(1.0, abs(gm))
            # gamma * a is the orthogonal projection onto the anchor's span
            r = x[h, j] - gamma[h, j] * a
            assert abs(r @ a) <= 1e-10 * (a @ a)
    # scaling an anchor by c > 0 keeps the slots and divides its gammas by c
    x2 = x.copy()
    x2[0, anchors[0][2]] *= 4.0
    slot2, gamma2 = o.anchor_assign(x2, anchors)
    np.testing.assert_array_equal(slot2, slot)
    m = (slot[0] == 2) & ~np.isin(np.arange(n), anchors[0])
    np.testing.assert_allclose(gamma2[0][m], gamma[0][m] / 4.0, rtol=1e-12)


# ---------------------------------------------------------------- pool ----

def check_maxpool(o):
    import torch
    rng = np.random.default_rng(17)
    raw = rng.random((3, 103))
    for pool in (1, 3, 7, 9):
        for n_cand in (103, 96, 5, 1):
            got = o.maxpool(raw, n_cand, pool)
            t = torch.from_numpy(raw[:, :n_cand].copy())[:, None, :]
            ref = torch.nn.functional.max_pool1d(t, pool, stride=1, padding=pool // 2)[:, 0, :].numpy()
            np.testing.assert_array_equal(got, ref)
            assert (got >= raw[:, :n_cand]).all()
    np.testing.assert_array_equal(o.maxpool(raw, 50, 1), raw[:, :50])
    # hand example: a single spike spreads 3 positions each way, clipped
    x = np.zeros((1, 12))
    x[0, 1] = 5.0
    np.testing.assert_array_equal(o.maxpool(x, 10, 7)[0], [5, 5, 5, 5, 5, 0, 0, 0, 0, 0])


# -------------------------------------------------------- value weight ----

def check_value_weight(o):
    rng = np.random.default_rng(18)
    # brute force with explicit loops
    H, G, d, n, D = 2, 3, 3, 5, 4
    v = rng.standard_normal((H, n, d))
    w_o = rng.standard_normal((D, H * G * d))
    ref = np.zeros((H, n))
    for h in range(H):
        for j in range(n):
            tot = 0.0
            for g in range(G):
                for c in range(D):
                    s = 0.0
                    for e in range(d):
                        s += w_o[c, (h * G + g) * d + e] * v[h, j, e]
                    tot += abs(s)
            ref[h, j] = tot / G
    np.testing.assert_allclose(o.value_weight(v, w_o, G), ref, rtol=1e-12)
    pos = np.array([4, 0, 2])
    np.testing.assert_allclose(o.value_weight(v, w_o, G, pos), ref[:, pos], rtol=1e-12)
    # identity slices -> plain L1 norm of v
    H, G, d, n = 2, 2, 6, 11
    D = 2 * d
    v = rng.standard_normal((H, n, d))
    w_o = np.zeros((D, H * G * d))
    for hq in range(H * G):
        w_o[:d, hq * d:(hq + 1) * d] = np.eye(d)
    np.testing.assert_allclose(o.value_weight(v, w_o, G), np.abs(v).sum(axis=2), rtol=1e-12)
    # homogeneity and linearity in |c|
    w_o = rng.standard_normal((D, H * G * d))
    base = o.value_weight(v, w_o, G)
    np.testing.assert_allclose(o.value_weight(-2.5 * v, w_o, G), 2.5 * base, rtol=1e-12)
    # only the group's own columns matter: zero them for head 1, head 0 unchanged
    w2 = w_o.copy()
    w2[:, G * d:] = 0
    got = o.value_weight(v, w2, G)
    np.testing.assert_allclose(got[0], base[0], rtol=1e-12)
    np.testing.assert_array_equal(got[1], 0)
    # rank-one slice u e_0^T -> ||u||_1 |v_0|, averaged over the group
    w3 = np.zeros((D, H * G * d))
    u = rng.standard_normal((H * G, D))
    for hq in range(H * G):
        w3[:, hq * d] = u[hq]
    exp = np.stack([np.mean([np.abs(u[h * G + g]).sum() for g in range(G)]) * np.abs(v[h, :, 0])
                    for h in range(H)])
    np.testing.assert_allclose(o.value_weight(v, w3, G), exp, rtol=1e-12)


def check_value_weight_group_sum(o):
    g = load_golden("value_weight_group_example.txt")
    w_o = np.array([g["w_o.row0"], g["w_o.row1"]])
    v = np.array([[g["v.pos0"], g["v.pos1"]]])
    np.testing.assert_allclose(o.value_weight(v, w_o, 2)[0], g["mean_of_norms"], rtol=1e-15)
    np.testing.assert_allclose(o.value_weight_group_sum(v, w_o, 2)[0], g["norm_of_sum"], rtol=1e-15)
    rng = np.random.default_rng(28)
    # brute force with explicit loops: the slices summed inside the |.|
    H, G, d, n, D = 2, 3, 3, 5, 4
    v = rng.standard_normal((H, n, d))
    w_o = rng.standard_normal((D, H * G * d))
    ref = np.zeros((H, n))
    for h in range(H):
        for j in range(n):
            tot = 0.0
            for c in range(D):
                s = 0.0
                for gg in range(G):
                    for e in range(d):
                        s += w_o[c, (h * G + gg) * d + e] * v[h, j, e]
                tot += abs(s)
            ref[h, j] = tot
    np.testing.assert_allclose(o.value_weight_group_sum(v, w_o, G), ref, rtol=1e-12)
    pos = np.array([3, 1])
    np.testing.assert_allclose(o.value_weight_group_sum(v, w_o, G, pos), ref[:, pos], rtol=1e-12)
    # one query head per KV head: both group modes are the same norm
    w1 = rng.standard_normal((D, H * d))
    np.testing.assert_allclose(o.value_weight_group_sum(v, w1, 1), o.value_weight(v, w1, 1),
                               rtol=1e-12)
    # triangle inequality: || sum_g W_g v ||_1 <= sum_g || W_g v ||_1 = G * mode 0,
    # with equality when every slice of the group is the same
    assert (o.value_weight_group_sum(v, w_o, G) <= G * o.value_weight(v, w_o, G) + 1e-12).all()
    same = np.concatenate([np.tile(w1[:, h * d:(h + 1) * d], (1, G)) for h in range(H)], axis=1)
    np.testing.assert_allclose(o.value_weight_group_sum(v, same, G),
                               G * o.value_weight(v, same, G), rtol=1e-12)
    # scaled identity slices a_g [I; 0] -> |sum_g a_g| * ||v||_1 (0 when they cancel)
    H, G, d, n = 2, 3, 4, 6
    D = 2 * d
    v = rng.standard_normal((H, n, d))
    a = np.array([[1.5, -0.5, 2.0], [1.0, -1.0, 0.0]])
    w_o = np.zeros((D, H * G * d))
    for h in range(H):
        for gg in range(G):
            w_o[:d, (h * G + gg) * d:(h * G + gg + 1) * d] = a[h, gg] * np.eye(d)
    exp = np.abs(a.sum(axis=1))[:, None] * np.abs(v).sum(axis=2)
    np.testing.assert_allclose(o.value_weight_group_sum(v, w_o, G), exp, rtol=1e-12, atol=1e-15)
    # homogeneity
    w_o = rng.standard_normal((D, H * G * d))
    np.testing.assert_allclose(o.value_weight_group_sum(-3.0 * v, w_o, G),
                               3.0 * o.value_weight_group_sum(v, w_o, G), rtol=1e-12)


# ----------------------------------------------------------- selection ----

def _assert_topk_property(key, picked, k):
    """Every picked entry beats every unpicked one: larger key, or equal key
    and lower index. Checked pairwise with loops."""
    picked = list(picked)
    assert len(picked) == k and len(set(picked)) == k
    ps = set(picked)
    for i in picked:
        for j in range(len(key)):
            if j in ps:
                continue
            assert key[i] > key[j] or (key[i] == key[j] and i < j), (i, j)


def check_select_examples(o):
    g = load_golden("select_examples.txt")
    ties_pooled = np.array([g["ties.pooled"]])
    idx, _, st = o.select_layer(ties_pooled, int(g["ties.budget"][0]), int(g["ties.W"][0]),
                                int(g["ties.n"][0]))
    np.testing.assert_array_equal(idx[0], g["ties.kept"])
    for name in ("two_stage", "odd_k", "eps"):
        idx, _, st = o.select_layer(np.array([g[name + ".pooled"]]), int(g[name + ".budget"][0]),
                                    int(g[name + ".W"][0]), int(g[name + ".n"][0]),
                                    weight=np.array([g[name + ".weight"]]),
                                    alpha=g[name + ".alpha"][0], score_norm=1.0,
                                    eps=g[name + ".eps"][0])
        np.testing.assert_array_equal(idx[0], g[name + ".kept"], err_msg=name)
        np.testing.assert_array_equal(st[0], g[name + ".stage"], err_msg=name)


def check_select_examples_f32(o):
    """The float32 two-stage key, worked by hand (select_examples.txt): the
    rounding of mul, add, mul decides a pick that float64 makes the other
    way, with eps and score_norm both non-trivial."""
    g = load_golden("select_examples.txt")
    for name in ("f32_tie", "f32_even", "f32_fma"):
        args = (np.array([g[name + ".pooled"]]), int(g[name + ".budget"][0]),
                int(g[name + ".W"][0]), int(g[name + ".n"][0]))
        kw = dict(weight=np.array([g[name + ".weight"]]), alpha=g[name + ".alpha"][0],
                  score_norm=g[name + ".score_norm"][0], eps=g[name + ".eps"][0])
        idx, _, st = o.select_layer(*args, dtype=np.float32, **kw)
        np.testing.assert_array_equal(idx[0], g[name + ".kept"], err_msg=name)
        np.testing.assert_array_equal(st[0], g[name + ".stage"], err_msg=name)
        idx64, _, _ = o.select_layer(*args, dtype=np.float64, **kw)
        np.testing.assert_array_equal(idx64[0], g[name + ".kept64"], err_msg=name + " (float64)")


def _f32_key_by_hand(s, w, norm, eps):
    """(s*norm + eps)*w with each operation rounded to float32: the exact
    result of every product and sum is formed as a Fraction and rounded to
    the nearest float32, ties to even."""
    def rnd(x: Fraction) -> Fraction:
        if x == 0:
            return Fraction(0)
        sign = -1 if x < 0 else 1
        a = abs(x)
        e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        e = max(e, -126)                     # subnormal spacing below 2^-126
        ulp = Fraction(2) ** (e - 23)
        q, r = divmod(a, ulp)
        if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
            q += 1
        return sign * q * ulp
    f = lambda v: Fraction(float(np.float32(v)))
    return float(rnd(rnd(rnd(f(s) * f(norm)) + f(eps)) * f(w)))


def check_select_two_stage_f32_bruteforce(o):
    """Two-stage selection in float32 on random tied inputs: stage 1 is a
    top-k1 by score, stage 2 a top-(k-k1) of the rest by the key rounded as
    mul, add, mul to float32 (computed here with exact rationals and
    explicit round-to-nearest-even, not with float32 arithmetic)."""
    rng = np.random.default_rng(23)
    for trial in range(6):
        H, n, W = 2, 24, 3
        n_cand = n - W
        scores = rng.integers(0, 5, size=(H, n_cand)).astype(np.float64) * 0.37
        w = rng.integers(1, 4, size=(H, n_cand)).astype(np.float64) * 1.3
        budget = int(rng.integers(W, n + 1))
        alpha = float(rng.choice([0.0, 0.5, 1.0]))
        norm, eps = 1.0 / 96, 1e-4
        idx, _, st = o.select_layer(scores, budget, W, n, weight=w, alpha=alpha,
                                    score_norm=norm, eps=eps, dtype=np.float32)
        k = budget - W
        k1 = int(math.floor(alpha * k))
        for h in range(H):
            s1 = [int(i) for i, s in zip(idx[h], st[h]) if s == 1]
            s2 = [int(i) for i, s in zip(idx[h], st[h]) if s == 2]
            _assert_topk_property(scores[h], s1, k1)
            rest = [j for j in range(n_cand) if j not in set(s1)]
            sub = np.array([_f32_key_by_hand(scores[h][j], w[h][j], norm, eps) for j in rest])
            _assert_topk_property(sub, [rest.index(j) for j in s2], k - k1)


def check_select_bruteforce(o):
    rng = np.random.default_rng(19)
    for trial in range(20):
        H, n, W = 3, 40, 4
        n_cand = n - W
        # few distinct values -> many ties
        scores = rng.integers(0, 6, size=(H, n_cand)).astype(np.float64)
        budget = int(rng.integers(W, n + 1))
        idx, _, st = o.select_layer(scores, budget, W, n)
        for h in range(H):
            row = list(idx[h])
            assert row == sorted(row)
            assert row[-W:] == list(range(n - W, n))
            _assert_topk_property(scores[h], row[:budget - W], budget - W)
            assert (st[h][-W:] == 0).all() and (st[h][:budget - W] == 1).all()
        # adaptive: one flattened top-k, ties by (head, position)
        budget = int(rng.integers(H * W, H * n + 1))
        idx, offs, st = o.select_layer(scores, budget, W, n, adaptive=True)
        assert offs[0] == 0 and offs[-1] == budget == len(idx)
        flat_pick = []
        for h in range(H):
            seg = list(idx[offs[h]:offs[h + 1]])
            assert seg == sorted(seg) and seg[-W:] == list(range(n - W, n))
            flat_pick += [h * n_cand + p for p in seg[:-W]]
        _assert_topk_property(scores.reshape(-1), flat_pick, budget - H * W)
        # two-stage: stage-1 set is a top-k1 by score; stage-2 set a top-k2
        # of the rest by (score*norm + eps)*w
        w = rng.integers(0, 4, size=(H, n_cand)).astype(np.float64)
        budget = int(rng.integers(W, n + 1))
        alpha = float(rng.choice([0.0, 0.25, 0.5, 1.0]))
        idx, _, st = o.select_layer(scores, budget, W, n, weight=w, alpha=alpha,
                                    score_norm=0.5, eps=0.01)
        k = budget - W
        k1 = int(math.floor(alpha * k))
        for h in range(H):
            s1 = [int(i) for i, s in zip(idx[h], st[h]) if s == 1]
            s2 = [int(i) for i, s in zip(idx[h], st[h]) if s == 2]
            _assert_topk_property(scores[h], s1, k1)
            rest = [j for j in range(n_cand) if j not in set(s1)]
            key = (scores[h] * 0.5 + 0.01) * w[h]
            sub = np.array([key[j] for j in rest])
            _assert_topk_property(sub, [rest.index(j) for j in s2], k - k1)


def check_select_reductions(o):
    rng = np.random.default_rng(20)
    H, n, W = 4, 64, 8
    scores = rng.random((H, n - W))
    w = rng.random((H, n - W)) + 0.1
    budget = 30
    plain, _, _ = o.select_layer(scores, budget, W, n)
    # alpha = 1: two-stage collapses to plain top-k by score
    a1, _, _ = o.select_layer(scores, budget, W, n, weight=w, alpha=1.0)
    np.testing.assert_array_equal(a1, plain)
    # alpha = 0, eps = 0, weight = 1, norm = 1: top-k by score again
    a0, _, _ = o.select_layer(scores, budget, W, n, weight=np.ones_like(w), alpha=0.0,
                              eps=0.0, score_norm=1.0)
    np.testing.assert_array_equal(a0, plain)
    # adaptive with identical heads and k divisible by H -> per-head k/H
    same = np.tile(rng.random(n - W), (H, 1))
    per_head, _, _ = o.select_layer(same, W + 5, W, n)
    ada, offs, _ = o.select_layer(same, H * (W + 5), W, n, adaptive=True)
    np.testing.assert_array_equal(ada, per_head.reshape(-1))
    np.testing.assert_array_equal(offs, np.arange(H + 1) * (W + 5))
    # budget = W keeps only the window; budget = n keeps everything
    only_w, _, _ = o.select_layer(scores, W, W, n)
    np.testing.assert_array_equal(only_w, np.tile(np.arange(n - W, n), (H, 1)))
    full, _, _ = o.select_layer(scores, n, W, n)
    np.testing.assert_array_equal(full, np.tile(np.arange(n), (H, 1)))


# ----------------------------------------------------------- compaction ----

def check_compact(o):
    import torch
    rng = np.random.default_rng(21)
    H, n, d, B = 3, 50, 8, 7
    k = rng.integers(0, 65535, size=(H, n, d)).astype(np.uint16)
    v = rng.integers(0, 65535, size=(H, n, d)).astype(np.uint16)
    idx = np.stack([np.sort(rng.choice(n, B, replace=False)) for _ in range(H)])
    ko, vo = o.compact_layer(k, v, idx)
    for h in range(H):
        ti = torch.from_numpy(idx[h])
        np.testing.assert_array_equal(ko[h], torch.index_select(torch.from_numpy(k[h].astype(np.int32)), 0, ti).numpy())
        np.testing.assert_array_equal(vo[h], torch.index_select(torch.from_numpy(v[h].astype(np.int32)), 0, ti).numpy())
    offs = np.array([0, 2, 2, 9])
    flat = np.concatenate([idx[0][:2], idx[2]])
    ko, vo = o.compact_layer(k, v, flat, offs)
    np.testing.assert_array_equal(ko, np.concatenate([k[0, idx[0][:2]], k[2, idx[2]]]))
    np.testing.assert_array_equal(vo, np.concatenate([v[0, idx[0][:2]], v[2, idx[2]]]))


# ------------------------------------------------------- value weight, L2 ----

def check_value_weight_l2(o):
    rng = np.random.default_rng(41)
    H, G, n, d = 2, 3, 7, 4
    v = rng.normal(size=(H, n, d))
    # identity slices: the L2 norm of v itself
    w_id = np.tile(np.eye(d), (1, H * G))
    np.testing.assert_allclose(o.value_weight_l2(v, w_id, G), np.linalg.norm(v, axis=2), rtol=1e-13)
    # brute force with loops
    D = 5
    w = rng.normal(size=(D, H * G * d))
    got = o.value_weight_l2(v, w, G)
    for h in range(H):
        for j in range(n):
            acc = 0.0
            for g in range(G):
                hq = h * G + g
                ss = 0.0
                for c in range(D):
                    x = sum(w[c, hq * d + e] * v[h, j, e] for e in range(d))
                    ss += x * x
                acc += math.sqrt(ss)
            assert abs(got[h, j] - acc / G) <= 1e-12 * max(1.0, acc)
    # a rotation of the output space changes nothing (true of L2, not of L1)
    qm, _ = np.linalg.qr(rng.normal(size=(D, D)))
    np.testing.assert_allclose(o.value_weight_l2(v, qm @ w, G), got, rtol=1e-12)
    # homogeneity in v, and a rank-one slice: ||a||_2 |b . v|
    np.testing.assert_allclose(o.value_weight_l2(-2.5 * v, w, G), 2.5 * got, rtol=1e-13)
    a_vec, b_vec = rng.normal(size=D), rng.normal(size=d)
    w1 = np.tile(np.outer(a_vec, b_vec), (1, H * G))
    np.testing.assert_allclose(o.value_weight_l2(v, w1, G),
                               np.linalg.norm(a_vec) * np.abs(v @ b_vec), rtol=1e-12)
    # positions select columns of the full result
    pos = np.array([5, 0, 3])
    np.testing.assert_allclose(o.value_weight_l2(v, w, G, pos), got[:, pos], rtol=1e-15)


# ---------------------------------------------------- per-head budgets ----

def check_select_budgets_example(o):
    g = load_golden("select_budgets_example.txt")
    n, W = int(g["n"][0]), int(g["W"][0])
    scores = np.array([g[f"pooled{h}"] for h in range(4)])
    idx, offs, st = o.select_budgets(scores, [int(b) for b in g["budgets"]], W, n)
    np.testing.assert_array_equal(idx, g["kept"])
    np.testing.assert_array_equal(offs, g["head_offsets"])
    np.testing.assert_array_equal(st == 0, np.isin(np.arange(len(idx)), np.concatenate(
        [np.arange(offs[h + 1] - W, offs[h + 1]) for h in range(4)])))


def check_select_budgets_bruteforce(o):
    rng = np.random.default_rng(43)
    for trial in range(15):
        H, n, W = 4, 30, 3
        n_cand = n - W
        scores = rng.integers(0, 5, size=(H, n_cand)).astype(np.float64)
        budgets = rng.integers(W - 2, n + 3, size=H)      # some outside [W, n]
        idx, offs, st = o.select_budgets(scores, budgets, W, n)
        eff = [min(max(int(b), W), n) for b in budgets]
        assert list(offs) == [sum(eff[:h]) for h in range(H + 1)] and len(idx) == offs[-1]
        for h in range(H):
            seg = [int(x) for x in idx[offs[h]:offs[h + 1]]]
            assert seg == sorted(seg) and seg[len(seg) - W:] == list(range(n - W, n))
            _assert_topk_property(scores[h], seg[:len(seg) - W], eff[h] - W)
            assert (st[offs[h]:offs[h + 1] - W] == 1).all() and (st[offs[h + 1] - W:offs[h + 1]] == 0).all()
        # two-stage, per head with its own k: stage-1 a top-floor(alpha k) by
        # score, stage-2 a top of the rest by (score*norm + eps)*w
        w = rng.integers(0, 4, size=(H, n_cand)).astype(np.float64)
        alpha = float(rng.choice([0.0, 0.5, 1.0]))
        idx, offs, st = o.select_budgets(scores, budgets, W, n, weight=w, alpha=alpha,
                                         score_norm=0.5, eps=0.01)
        for h in range(H):
            k = eff[h] - W
            k1 = int(math.floor(alpha * k))
            seg, sst = idx[offs[h]:offs[h + 1]], st[offs[h]:offs[h + 1]]
            s1 = [int(i) for i, s in zip(seg, sst) if s == 1]
            s2 = [int(i) for i, s in zip(seg, sst) if s == 2]
            _assert_topk_property(scores[h], s1, k1)
            rest = [j for j in range(n_cand) if j not in set(s1)]
            key = (scores[h] * 0.5 + 0.01) * w[h]
            _assert_topk_property(np.array([key[j] for j in rest]), [rest.index(j) for j in s2], k - k1)


def check_select_budgets_reductions(o):
    rng = np.random.default_rng(44)
    H, n, W = 4, 50, 5
    scores = rng.random((H, n - W))
    w = rng.random((H, n - W)) + 0.1
    # one budget for every head: the uniform selection, packed
    for weight in (None, w):
        uni, _, ust = o.select_layer(scores, 20, W, n, weight=weight)
        idx, offs, st = o.select_budgets(scores, [20] * H, W, n, weight=weight)
        np.testing.assert_array_equal(idx, uni.reshape(-1))
        np.testing.assert_array_equal(st, ust.reshape(-1))
        np.testing.assert_array_equal(offs, 20 * np.arange(H + 1))
    # each head alone: the one-head uniform selection with its own budget
    budgets = [W, 7, 31, n]
    idx, offs, _ = o.select_budgets(scores, budgets, W, n)
    for h in range(H):
        one, _, _ = o.select_layer(scores[h:h + 1], budgets[h], W, n)
        np.testing.assert_array_equal(idx[offs[h]:offs[h + 1]], one[0])


# ------------------------------------------------- decode over kept rows ----

def check_decode_hand_example(o):
    g = load_golden("decode_hand_example.txt")
    k = np.zeros((1, 3, 4))
    k[0, :, 0] = g["key_x"]
    v = np.asarray(g["values"]).reshape(1, 3, 4)
    q = np.array([[1.0, 0, 0, 0]])
    np.testing.assert_allclose(o.decode_attention(q, k, v, 1, 1.0)[0], g["out"], rtol=1e-12, atol=1e-14)


def check_decode_bruteforce(o):
    """Explicit loops (exp, sums, no matrix products) on ragged heads,
    one of them empty."""
    rng = np.random.default_rng(31)
    H, G, d, scale = 3, 2, 5, 0.7
    offs = np.array([0, 4, 4, 11])
    k = rng.normal(size=(11, d))
    v = rng.normal(size=(11, d))
    q = rng.normal(size=(H * G, d))
    got = o.decode_attention(q, k, v, G, scale, offs)
    for h in range(H):
        rows = range(offs[h], offs[h + 1])
        for g in range(G):
            hq = h * G + g
            if not len(rows):
                np.testing.assert_array_equal(got[hq], np.zeros(d))
                continue
            logits = [scale * sum(q[hq, e] * k[t, e] for e in range(d)) for t in rows]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            z = sum(w)
            ref = [sum(w[i] / z * v[t, e] for i, t in enumerate(rows)) for e in range(d)]
            np.testing.assert_allclose(got[hq], ref, rtol=1e-12, atol=1e-14)


def check_decode_sdpa(o):
    """Uniform heads against torch's scaled_dot_product_attention (fp64),
    the KV heads repeated for their G query heads."""
    import torch
    rng = np.random.default_rng(32)
    H, G, B, d, scale = 2, 3, 9, 8, 0.35
    k = rng.normal(size=(H, B, d))
    v = rng.normal(size=(H, B, d))
    q = rng.normal(size=(H * G, d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], torch.from_numpy(k).repeat_interleave(G, 0),
        torch.from_numpy(v).repeat_interleave(G, 0), scale=scale)[:, 0].numpy()
    np.testing.assert_allclose(o.decode_attention(q, k, v, G, scale), ref, rtol=1e-12, atol=1e-14)


def check_decode_closed_forms(o):
    rng = np.random.default_rng(33)
    d = 6
    q = rng.normal(size=(2, d))
    # equal keys: the mean of the values
    k = np.tile(rng.normal(size=(1, 1, d)), (1, 5, 1))
    v = rng.normal(size=(1, 5, d))
    np.testing.assert_allclose(o.decode_attention(q, k, v, 2, 0.5), np.tile(v[0].mean(0), (2, 1)),
                               rtol=1e-12, atol=1e-14)
    # one row: its value exactly
    np.testing.assert_allclose(o.decode_attention(q[:1], k[:, :1], v[:, :1], 1, 0.5)[0], v[0, 0],
                               rtol=1e-15)
    # a dominant key: its value
    k2 = rng.normal(size=(1, 5, d)) * 0.01
    k2[0, 2] = q[0] * 100
    np.testing.assert_allclose(o.decode_attention(q[:1], k2, v, 1, 1.0)[0], v[0, 2], rtol=1e-9)
    # the order of a head's rows does not matter
    k3 = rng.normal(size=(1, 5, d))
    perm = rng.permutation(5)
    np.testing.assert_allclose(o.decode_attention(q, k3, v, 2, 0.3),
                               o.decode_attention(q, k3[:, perm], v[:, perm], 2, 0.3), rtol=1e-12)


ALL_CHECKS = [
    check_window_bruteforce, check_window_sum_invariant, check_window_equal_keys,
    check_window_hand_example, check_window_single_query_softmax, check_window_max_agg,
    check_external, check_maxpool, check_value_weight, check_select_examples,
    check_select_bruteforce, check_select_reductions, check_compact,
    check_decode_hand_example, check_decode_bruteforce, check_decode_sdpa, check_decode_closed_forms,
    check_value_weight_l2, check_select_budgets_example, check_select_budgets_bruteforce,
    check_select_budgets_reductions, check_external_logit, check_head_scores_and_budgets,
    check_chunked, check_anchor_select, check_anchor_assign,
    check_select_examples_f32, check_select_two_stage_f32_bruteforce, check_value_weight_group_sum,
]
