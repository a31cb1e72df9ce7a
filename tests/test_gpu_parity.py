"""GPU parity against the oracle at small sizes (several tiles, ragged
tails, edge cases). Every call goes through the C ABI via the ctypes
binding; nothing here falls back to a CPU path."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import eviction_importance_scoring_amd as kv
import oracle
import synth
from harness import (assert_logits_close, assert_scores_close, assert_topk_within_band, gen,
                     logit_error_bound,
                     oracle_scores_layer, split_heads, to_dev)

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="t", L=1, H_kv=2, G=4, d=128, n=100, W=8, pool=7, heavy="zipf")
    base.update(kw)
    base["name"] = "t_" + "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return synth.Workload(**base)


def _run_scores(wl, data, return_raw=True):
    q, k = to_dev(data["q"]), to_dev(data["k"])
    mode = kv.Q_WINDOW if wl.q_mode == "window" else kv.Q_EXTERNAL
    agg = kv.AGG_SUM if wl.agg == "sum" else kv.AGG_MAX
    print(f"[gpu] kvsel_score {wl.name} L={wl.L} H={wl.H_kv} G={wl.G} n={wl.n} W={wl.W}",
          flush=True)
    scores, raw = kv.kvsel_score(q, k, G=wl.G, q_mode=mode, agg=agg, scale=wl.scale,
                                 pool=wl.pool, return_raw=return_raw)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), (raw.cpu().numpy() if raw is not None else None)


WINDOW_CASES = [
    dict(n=100, W=8),
    dict(L=2, H_kv=3, n=257, W=32),
    dict(G=1, n=1000, W=1, pool=3),
    dict(H_kv=1, G=7, n=4097, W=32, pool=1),
    dict(n=33, W=32),                      # a single candidate
    dict(n=2, W=1, G=2),                   # smallest cache
    dict(n=300, W=16, pool=5, agg="max"),
    dict(n=1500, W=40, G=4),               # R = 160 rows: more than one row block
    dict(n=4096, W=32, heavy="uniform1pct"),
    # workgroup key ranges (128 keys at these sizes) against pool halos
    dict(n=513, W=1, G=1, pool=17),
    dict(n=768, W=32, pool=7),             # candidates end inside a range
    dict(n=771, W=3, G=4, pool=9),         # 7 ranges, the last one 3 keys
    dict(L=3, H_kv=2, n=2048, W=8, G=8),   # R = 64
    dict(n=1000, W=30, G=3, pool=1),       # R = 90, no pooling
    # general kernels (R > 128): several 512-row blocks, ragged row / key tails
    dict(n=2000, W=160, G=4),              # R = 640
    dict(n=1537, W=130, G=5, agg="max"),   # R = 650
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_window_scores(case):
    wl = _wl(**case)
    data = gen(wl, seed=1, which=("q", "k"))
    scores, raw = _run_scores(wl, data)
    for l in range(wl.L):
        ref_raw, ref_pool = oracle_scores_layer(wl, data["q"][l], data["k"][l])
        assert_scores_close(raw[l], ref_raw, "raw")
        assert_scores_close(scores[l], ref_pool, "pooled")
        if wl.agg == "sum":
            np.testing.assert_allclose(raw[l].astype(np.float64).sum(axis=1), wl.W * wl.G, rtol=1e-5)


POOL_CASES = WINDOW_CASES + [
    dict(n=3000, W=32, pool=65),                   # r = 32: the widest halo
    dict(L=2, H_kv=2, n=5000, W=7, pool=33, agg="max"),
    dict(n=4160, W=100, G=1, pool=63),             # candidates end before the last range
    dict(L=4, H_kv=8, n=20000, W=32, pool=7),      # many pooling blocks per head
]


@pytest.mark.parametrize("case", POOL_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_pool_with_and_without_raw(case):
    """The pooled scores are the same bits whether the raw sums are returned
    or kept in the workspace, on every call, and match the oracle."""
    wl = _wl(**case)
    data = gen(wl, seed=4, which=("q", "k"))
    with_raw, _ = _run_scores(wl, data, return_raw=True)
    alone, raw = _run_scores(wl, data, return_raw=False)
    assert raw is None
    np.testing.assert_array_equal(alone, with_raw)
    again, _ = _run_scores(wl, data, return_raw=False)
    np.testing.assert_array_equal(again, alone)
    _, ref_pool = oracle_scores_layer(wl, data["q"][0], data["k"][0])
    assert_scores_close(alone[0], ref_pool, "pooled")


EXTERNAL_CASES = [
    dict(n=300, W=50, G=3, agg="max"),
    dict(H_kv=1, G=7, n=1000, W=129, agg="max"),
    dict(L=2, n=33, W=1, G=2, agg="max"),
    dict(n=700, W=64, G=2, agg="sum"),
    dict(n=5000, W=300, G=1, agg="max", pool=3),
    dict(H_kv=1, G=7, n=1100, W=600, agg="max"),   # R = 4200: many row blocks
    dict(n=2049, W=520, G=1, agg="sum"),           # R = 520, keys split
]


@pytest.mark.parametrize("case", EXTERNAL_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_external_scores(case):
    wl = _wl(q_mode="external", pool=case.pop("pool", 1), **case)
    data = gen(wl, seed=2, which=("q", "k"))
    scores, raw = _run_scores(wl, data)
    for l in range(wl.L):
        ref_raw, ref_pool = oracle_scores_layer(wl, data["q"][l], data["k"][l])
        assert_scores_close(raw[l], ref_raw, "raw")
        assert_scores_close(scores[l], ref_pool, "pooled")
        if wl.agg == "max":
            assert (raw[l] <= 1.0 + 1e-6).all()


@pytest.mark.parametrize("case", [
    dict(L=2, n=3000, W=32),
    # many tiles per workgroup, all heads busy: cross-wave LDS hand-offs
    dict(L=4, H_kv=8, n=20000, W=32),
    dict(L=2, H_kv=2, G=7, n=4000, W=600, q_mode="external", agg="max", pool=1),
    dict(n=2000, W=160, G=4),
])
def test_scores_deterministic(case):
    """Bit-identical results on repeated calls (no atomics, fixed orders)."""
    wl = _wl(**case)
    data = gen(wl, seed=3, which=("q", "k"))
    a = _run_scores(wl, data)
    for _ in range(2):
        b = _run_scores(wl, data)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_value_weight_deterministic():
    wl = _wl(L=1, H_kv=2, G=4, n=3000, W=1, value_weight=True, D=512)
    data = gen(wl, seed=7, which=("v", "w_o"))
    v, w_o = to_dev(data["v"]), to_dev(data["w_o"])
    a = kv.kvsel_value_weight(v, w_o, G=wl.G, n_cand=wl.n).cpu().numpy()
    for _ in range(2):
        b = kv.kvsel_value_weight(v, w_o, G=wl.G, n_cand=wl.n).cpu().numpy()
        np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------- selection ----

def _quantised_scores(rng, shape, levels):
    """Scores with many exact ties (few distinct levels)."""
    return (rng.integers(0, levels, size=shape) / levels).astype(np.float32)


SELECT_CASES = [
    # (L, H, n, W, budget_frac, adaptive, two_stage, alpha, levels)
    (1, 2, 100, 8, 0.5, False, False, 0.5, 7),
    (2, 3, 1000, 32, 0.2, False, False, 0.5, 1000000),
    (1, 4, 3000, 32, 0.4, True, False, 0.5, 50),
    (2, 2, 2000, 16, 0.3, False, True, 0.5, 30),
    (1, 3, 1500, 8, 0.25, True, True, 0.5, 1000000),
    (1, 2, 500, 4, 0.3, False, True, 0.0, 10),
    (1, 2, 500, 4, 0.3, False, True, 1.0, 10),
    (1, 8, 4000, 8, 0.3, True, False, 0.5, 5),            # one workgroup: 33 candidates a thread, head starts inside ranges
    (1, 8, 40, 8, 0.5, True, False, 0.5, 3),              # heads shorter than a thread's range
    (1, 16, 30, 4, 0.5, True, True, 0.5, 3),              # the same, two-stage
    (1, 1, 50000, 32, 0.1, False, False, 0.5, 1000),      # longer than LDS: many workgroups
    (1, 2, 40000, 32, 0.1, True, True, 0.5, 100000),      # many workgroups, two-stage, adaptive
    # segments over the LDS size run on many workgroups (chunks of 16,384)
    (2, 8, 9032, 32, 0.2, True, False, 0.5, 50),          # adaptive, 8 heads, ties
    (1, 3, 20000, 0, 0.3, True, False, 0.5, 5),           # adaptive, no window, heavy ties
    (1, 1, 36000, 16, 1.0, False, False, 0.5, 3),         # keep everything
    (1, 2, 50000, 32, 0.3, False, True, 0.0, 1000),       # two-stage, alpha 0
    (1, 2, 50000, 32, 0.3, False, True, 1.0, 1000),       # two-stage, alpha 1
    (1, 4, 12000, 8, 0.25, True, True, 0.5, 7),           # adaptive two-stage, ties
    (1, 2, 64, 32, 1.0, False, False, 0.5, 3),            # keep everything
    (1, 2, 64, 32, 0.5, False, False, 0.5, 3),            # keep only the window
    (1, 2, 64, 0, 0.0, False, False, 0.5, 3),             # external: nothing kept
    # many workgroups with n - W not a multiple of 4 (4-byte loads)
    (1, 1, 40001, 0, 0.2, False, False, 0.5, 100),
    (1, 3, 15001, 3, 0.3, True, True, 0.5, 30),
    # many workgroups on near-continuous scores: the bucket after two digits
    # goes to the short list (the tie-heavy cases above outgrow it)
    (1, 8, 9032, 32, 0.2, True, True, 0.5, 1000000),     # adaptive two-stage, 8 heads
    (2, 2, 50000, 32, 0.1, False, True, 0.5, 1000000),   # per head, two-stage
    (1, 1, 40000, 32, 0.00083, False, False, 0.5, 1000000),   # k = 1
    (1, 1, 40000, 32, 0.99998, False, False, 0.5, 1000000),   # k = n - W - 1
]


@pytest.mark.parametrize("case", SELECT_CASES, ids=lambda c: "L{}H{}n{}W{}b{}a{}t{}al{}lv{}".format(*c))
def test_select_exact_on_same_fp32_scores(case):
    L, H, n, W, frac, adaptive, two_stage, alpha, levels = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    n_cand = n - W
    sc = _quantised_scores(rng, (L, H, n_cand), levels)
    wt = (rng.random((L, H, n_cand)).astype(np.float32) * 3 + 0.01) if two_stage else None
    groups = H if adaptive else 1
    budget = max(groups * W, int(np.floor(frac * groups * n)))
    print(f"[gpu] kvsel_select case={case} budget={budget}", flush=True)
    idx, offs, stage = kv.kvsel_select(torch.from_numpy(sc).cuda(), n=n, W=W, budget=budget,
                                       adaptive=adaptive,
                                       weight=None if wt is None else torch.from_numpy(wt).cuda(),
                                       score_norm=1.0 / 128, eps=1e-4, alpha=alpha,
                                       return_stage=True)
    torch.cuda.synchronize()
    idx, stage = idx.cpu().numpy(), stage.cpu().numpy()
    offs = None if offs is None else offs.cpu().numpy()
    for l in range(L):
        ri, ro, rs = oracle.select_layer(sc[l].astype(np.float64), budget, W, n, adaptive=adaptive,
                                         weight=None if wt is None else wt[l].astype(np.float64),
                                         alpha=float(np.float32(alpha)), score_norm=float(np.float32(1 / 128)),
                                         eps=float(np.float32(1e-4)), dtype=np.float32)
        np.testing.assert_array_equal(idx[l], ri)
        np.testing.assert_array_equal(stage[l], rs)
        if adaptive:
            np.testing.assert_array_equal(offs[l], ro)


POOL_SELECT_CASES = [
    # (L, H, n, W, budget_frac, adaptive, two_stage, alpha, levels, pool)
    # pooled on chip: per-head budget, pool <= 7, n % 4 == 0, n - W <= 34,816
    (1, 2, 100, 8, 0.5, False, False, 0.5, 7, 7),
    (2, 3, 1000, 7, 0.2, False, False, 0.5, 1000000, 7),    # n - W not a multiple of 4
    (1, 2, 4096, 32, 0.3, False, False, 0.5, 9, 5),
    (1, 3, 2048, 16, 0.4, False, False, 0.5, 11, 3),
    (1, 2, 3000, 8, 0.3, False, False, 0.5, 5, 1),          # no pooling, raw rows n apart
    (2, 2, 2000, 16, 0.3, False, True, 0.5, 30, 7),         # two-stage
    (1, 2, 500, 4, 0.3, False, True, 0.0, 10, 7),
    (1, 2, 500, 4, 0.3, False, True, 1.0, 10, 5),
    (1, 1, 34848, 32, 0.25, False, False, 0.5, 1000, 7),    # the largest resident head
    (1, 2, 64, 0, 0.5, False, False, 0.5, 3, 7),            # external: no window
    (1, 2, 64, 32, 1.0, False, False, 0.5, 3, 7),           # keep everything
    (1, 2, 64, 32, 0.5, False, False, 0.5, 3, 7),           # keep only the window
    # pooled through memory first
    (1, 2, 1001, 9, 0.3, False, False, 0.5, 50, 7),         # n % 4 != 0
    (1, 2, 1000, 8, 0.3, False, False, 0.5, 50, 9),         # pool > 7
    (1, 4, 3000, 32, 0.4, True, False, 0.5, 50, 7),         # adaptive
    (1, 1, 50000, 32, 0.1, False, True, 0.5, 1000, 7),      # many workgroups
    # many workgroups, pooled in the selection's first pass (radius <= 3)
    (1, 2, 40000, 8, 0.3, True, False, 0.5, 50, 7),         # adaptive
    (1, 2, 40001, 9, 0.3, True, True, 0.5, 300, 5),         # n % 4 != 0: 4-byte loads
    (1, 1, 50003, 32, 0.2, False, False, 0.5, 1000, 3),     # n - W odd
    (1, 1, 40000, 0, 0.2, False, False, 0.5, 1000, 1),      # no window, pool 1 (a copy)
    (1, 3, 36000, 32, 0.5, False, False, 0.5, 1000000, 7),  # three heads
    (2, 2, 35000, 32, 0.05, False, True, 1.0, 1000000, 7),  # two layers, two-stage
    (1, 1, 40000, 16, 0.2, False, True, 0.5, 1000, 9),      # pool 9: the pool kernel first
]


@pytest.mark.parametrize("case", POOL_SELECT_CASES,
                         ids=lambda c: "L{}H{}n{}W{}b{}a{}t{}al{}lv{}p{}".format(*c))
def test_select_pool_exact(case):
    """kvsel_select_pool on raw scores: the oracle's max-pooling then its
    selection, bit for bit; the window's raw values (made the largest) must
    neither pool into a candidate nor be selected."""
    L, H, n, W, frac, adaptive, two_stage, alpha, levels, pool = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    n_cand = n - W
    raw = _quantised_scores(rng, (L, H, n), levels)
    raw[..., n_cand:] = 5.0
    wt = (rng.random((L, H, n_cand)).astype(np.float32) * 3 + 0.01) if two_stage else None
    groups = H if adaptive else 1
    budget = max(groups * W, int(np.floor(frac * groups * n)))
    print(f"[gpu] kvsel_select_pool case={case} budget={budget}", flush=True)
    idx, offs, stage, pooled = kv.kvsel_select_pool(
        torch.from_numpy(raw).cuda(), n=n, W=W, budget=budget, pool=pool, adaptive=adaptive,
        weight=None if wt is None else torch.from_numpy(wt).cuda(), score_norm=1.0 / 128,
        eps=1e-4, alpha=alpha, return_stage=True, return_pooled=True)
    torch.cuda.synchronize()
    idx, stage, pooled = idx.cpu().numpy(), stage.cpu().numpy(), pooled.cpu().numpy()
    offs = None if offs is None else offs.cpu().numpy()
    ref_pooled = oracle.maxpool(raw.astype(np.float64), n_cand, pool)
    np.testing.assert_array_equal(pooled, ref_pooled.astype(np.float32))
    for l in range(L):
        ri, ro, rs = oracle.select_layer(ref_pooled[l], budget, W, n, adaptive=adaptive,
                                         weight=None if wt is None else wt[l].astype(np.float64),
                                         alpha=float(np.float32(alpha)), score_norm=float(np.float32(1 / 128)),
                                         eps=float(np.float32(1e-4)), dtype=np.float32)
        np.testing.assert_array_equal(idx[l], ri)
        np.testing.assert_array_equal(stage[l], rs)
        if adaptive:
            np.testing.assert_array_equal(offs[l], ro)


def test_select_pool_matches_score_then_select():
    """Raw-only scoring followed by kvsel_select_pool gives the same kept
    entries as pooled scoring followed by kvsel_select, on real scores."""
    wl = _wl(L=2, H_kv=2, n=2048, W=32)
    data = gen(wl, seed=3)
    q, k = to_dev(data["q"]), to_dev(data["k"])
    scores, raw = kv.kvsel_score(q, k, G=wl.G, pool=wl.pool, return_raw=True)
    none, raw2 = kv.kvsel_score(q, k, G=wl.G, pool=wl.pool, pooled=False)
    assert none is None
    budget = 700
    idx, _, _ = kv.kvsel_select(scores, n=wl.n, W=wl.W, budget=budget)
    idx2, _, _, pooled = kv.kvsel_select_pool(raw2, n=wl.n, W=wl.W, budget=budget, pool=wl.pool,
                                              return_pooled=True)
    torch.cuda.synchronize()
    assert torch.equal(raw, raw2)
    assert torch.equal(pooled, scores)
    assert torch.equal(idx, idx2)


@pytest.mark.parametrize("name", ["f32_tie", "f32_even", "f32_fma"])
@pytest.mark.parametrize("pad", [0, 40000])
def test_select_two_stage_f32_hand_examples(name, pad):
    """The hand-worked float32 stage-2 keys (tests/golden/select_examples.txt):
    the kernel's mul, add, mul rounding decides the pick exactly as worked
    out by hand. pad > 0 appends zero-weight candidates after the two, so the
    segment runs on the many-workgroup path; they never beat the two."""
    from oracle_pins import load_golden
    g = load_golden("select_examples.txt")
    sc = np.zeros((1, 1, 2 + pad), np.float32)
    wt = np.zeros((1, 1, 2 + pad), np.float32)
    sc[0, 0, :2] = g[name + ".pooled"]
    wt[0, 0, :2] = g[name + ".weight"]
    W = int(g[name + ".W"][0])
    n = 2 + pad + W
    budget = int(g[name + ".budget"][0])
    print(f"[gpu] kvsel_select fp32 hand example {name} pad={pad}", flush=True)
    idx, _, stage = kv.kvsel_select(torch.from_numpy(sc).cuda(), n=n, W=W, budget=budget,
                                    weight=torch.from_numpy(wt).cuda(),
                                    score_norm=g[name + ".score_norm"][0], eps=g[name + ".eps"][0],
                                    alpha=g[name + ".alpha"][0], return_stage=True)
    torch.cuda.synchronize()
    want = [int(x) for x in g[name + ".kept"]]
    want = want[:1] + list(range(n - W, n))
    np.testing.assert_array_equal(idx.cpu().numpy()[0, 0], want)
    np.testing.assert_array_equal(stage.cpu().numpy()[0, 0], [2] + [0] * W)


BUDGET_CASES = [
    # (L, H, n, W, two_stage, alpha, levels, stride_extra)
    (2, 4, 300, 8, False, 0.5, 7, 0),
    (2, 3, 1000, 32, True, 0.5, 30, 0),
    (1, 8, 64, 32, False, 0.5, 3, 17),          # budgets W .. n, a padded row
    (3, 2, 2500, 16, True, 1.0, 1000000, 5),
    (1, 4, 50000, 32, False, 0.5, 1000, 0),     # longer than LDS: many workgroups per head
    (1, 2, 40000, 16, True, 0.5, 100, 3),       # many workgroups, two-stage
    (2, 4, 600, 8, False, 0.5, 5, -40),         # rows shorter than layer 0's budgets: truncated
    (2, 4, 40000, 8, False, 0.5, 1000000, -40), # the same on many workgroups
    (1, 3, 36000, 32, True, 0.5, 1000000, 2),   # many workgroups, two-stage, short lists
]


@pytest.mark.parametrize("case", BUDGET_CASES, ids=lambda c: "L{}H{}n{}W{}t{}al{}lv{}s{}".format(*c))
def test_select_budgets_exact(case):
    L, H, n, W, two_stage, alpha, levels, extra = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    n_cand = n - W
    sc = _quantised_scores(rng, (L, H, n_cand), levels)
    wt = (rng.random((L, H, n_cand)).astype(np.float32) * 3 + 0.01) if two_stage else None
    budgets = rng.integers(W - 3, n + 4, size=(L, H)).astype(np.int32)   # some outside [W, n]
    budgets[0, 0] = W                                                      # window only
    if extra < 0:
        budgets[0] = n                      # layer 0 needs H*n entries
        budgets[1:] = W + 3
    sums = np.clip(budgets, W, n).astype(np.int64).sum(axis=1)
    stride = int(sums.max()) + extra
    print(f"[gpu] kvsel_select_budgets case={case} stride={stride}", flush=True)
    idx, offs, stage = kv.kvsel_select_budgets(
        torch.from_numpy(sc).cuda(), torch.from_numpy(budgets).cuda(), n=n, W=W,
        layer_stride=stride, weight=None if wt is None else torch.from_numpy(wt).cuda(),
        score_norm=1.0 / 128, eps=1e-4, alpha=alpha, return_stage=True)
    torch.cuda.synchronize()
    idx, offs, stage = idx.cpu().numpy(), offs.cpu().numpy(), stage.cpu().numpy()
    assert idx.shape == (L, stride)
    for l in range(L):
        ri, ro, rs = oracle.select_budgets(sc[l].astype(np.float64), budgets[l], W, n,
                                           weight=None if wt is None else wt[l].astype(np.float64),
                                           alpha=float(np.float32(alpha)),
                                           score_norm=float(np.float32(1 / 128)),
                                           eps=float(np.float32(1e-4)), dtype=np.float32)
        m = min(len(ri), stride)
        np.testing.assert_array_equal(offs[l], np.minimum(ro, stride))
        np.testing.assert_array_equal(idx[l, :m], ri[:m])
        np.testing.assert_array_equal(stage[l, :m], rs[:m])
        assert (idx[l, m:] == -1).all() and (stage[l, m:] == 0).all()


def test_select_budgets_feed_compact_and_decode():
    """Budget-vector output in the packed layout drives compaction and decode."""
    rng = np.random.default_rng(12)
    L, H, G, n, W = 2, 4, 2, 700, 16
    sc = rng.random((L, H, n - W)).astype(np.float32)
    budgets = np.array([[16, 100, 700, 40], [300, 16, 17, 5]], np.int32)
    idx, offs, _ = kv.kvsel_select_budgets(torch.from_numpy(sc).cuda(),
                                           torch.from_numpy(budgets).cuda(), n=n, W=W,
                                           layer_stride=900)
    k = synth.bf16_bits(rng.standard_normal((L, H, n, 128)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((L, H, n, 128)).astype(np.float32))
    ko, vo = kv.kvsel_compact(to_dev(k), to_dev(v), idx, offs)
    torch.cuda.synchronize()
    idx_h, offs_h = idx.cpu().numpy(), offs.cpu().numpy()
    ko_h = ko.cpu().view(torch.int16).numpy().view(np.uint16)
    vo_h = vo.cpu().view(torch.int16).numpy().view(np.uint16)
    for l in range(L):
        end = offs_h[l, -1]
        rk, rv = oracle.compact_layer(k[l], v[l], idx_h[l, :end], offs_h[l])
        np.testing.assert_array_equal(ko_h[l, :end], rk)
        np.testing.assert_array_equal(vo_h[l, :end], rv)
    # rows past each layer's last head are left as they were
    fill = torch.full((L, 900, 128), 1.5, dtype=torch.bfloat16, device="cuda")
    ko2, vo2 = kv.kvsel_compact(to_dev(k), to_dev(v), idx, offs, k_out=fill.clone(), v_out=fill.clone())
    torch.cuda.synchronize()
    for l in range(L):
        end = offs_h[l, -1]
        assert torch.equal(ko2[l, :end], ko[l, :end]) and torch.equal(vo2[l, :end], vo[l, :end])
        assert (ko2[l, end:] == 1.5).all() and (vo2[l, end:] == 1.5).all()
    qb = synth.bf16_bits(rng.standard_normal((L, H * G, 128)).astype(np.float32))
    out = kv.kvsel_decode_attention(to_dev(qb), ko, vo, G=G, scale=0.088, head_offsets=offs)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for l in range(L):
        end = offs_h[l, -1]   # rows past it were never written
        vl = synth.bf16_to_f64(vo_h[l, :end])
        ref = oracle.decode_attention(synth.bf16_to_f64(qb[l]), synth.bf16_to_f64(ko_h[l, :end]), vl,
                                      G, 0.088, head_offsets=offs_h[l])
        np.testing.assert_allclose(out[l], ref, rtol=1e-4, atol=1e-4 * np.abs(vl).max())


# KVzip-logit: scale * max <q, k> in fp32 from bf16 (exact products, fp32
# sums of 128 terms), checked with the logit rule of harness.py.
LOGIT_CASES = [
    # (L, H, G, n, Q per query head, pool)
    (1, 2, 3, 1000, 70, 1),
    (2, 1, 7, 4097, 130, 5),      # several key blocks, ragged, pooled negatives
    (1, 2, 1, 300, 600, 1),       # more queries than keys
    (1, 4, 4, 2048, 512, 3),
    (1, 2, 1, 777, 1, 5),         # one query: about half the scores negative, pooled
]


@pytest.mark.parametrize("case", LOGIT_CASES, ids=lambda c: "L{}H{}G{}n{}Q{}p{}".format(*c))
def test_logit_scores(case):
    L, H, G, n, Qn, pool = case
    wl = _wl(L=L, H_kv=H, G=G, n=n, W=Qn, q_mode="external", agg="max", pool=pool)
    data = gen(wl, seed=11, which=("q", "k"))
    print(f"[gpu] kvsel_score logit {case}", flush=True)
    s, r = kv.kvsel_score(to_dev(data["q"]), to_dev(data["k"]), G=G, q_mode=kv.Q_EXTERNAL,
                          agg=kv.AGG_LOGIT_MAX, scale=wl.scale, pool=pool, return_raw=True)
    torch.cuda.synchronize()
    s, r = s.cpu().numpy(), r.cpu().numpy()
    for l in range(L):
        q64, k64 = synth.bf16_to_f64(data["q"][l]), synth.bf16_to_f64(data["k"][l])
        ref = oracle.external_logit_scores(q64, k64, G, wl.scale)
        refp = oracle.maxpool(ref, n, pool)
        bound = logit_error_bound(q64, k64, G, wl.scale)
        assert_logits_close(r[l], ref, bound, f"logit raw l{l}")
        assert_logits_close(s[l], refp, oracle.maxpool(bound, n, pool), f"logit pooled l{l}")


CHUNKED_CASES = [
    # (L, H, G, n, m, n_prompt, pool)
    (1, 2, 2, 1000, 256, 8, 1),       # 4 chunks, the last 232 keys
    (2, 1, 7, 3000, 1024, 40, 3),     # pooled
    (1, 1, 1, 100, 500, 0, 1),        # m past n: one chunk, no prompt
    (1, 2, 4, 2048, 512, 100, 1),     # an exact multiple
    (1, 1, 3, 700, 64, 200, 5),       # chunks shorter than the prompt
    (1, 2, 7, 100, 16, 4, 1),         # inputs of 20 rows: a row block spans all 7 group heads
]


@pytest.mark.parametrize("case", CHUNKED_CASES, ids=lambda c: "L{}H{}G{}n{}m{}p{}pool{}".format(*c))
def test_score_chunked(case):
    L, H, G, n, m, npr, pool = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    me = min(m, n)
    T, n_in = (n + me - 1) // me, npr + me
    q = rng.standard_normal((L, T, H * G, n_in, 128)).astype(np.float32)
    ks = rng.standard_normal((L, T, H, n_in, 128)).astype(np.float32)
    k = rng.standard_normal((L, H, n, 128)).astype(np.float32)
    k[..., :8, :] *= 3.0          # a few heavy keys
    last = npr + (n - (T - 1) * me)
    q[:, T - 1, :, last:] = 30.0  # rows past the last chunk's input: ignored
    ks[:, T - 1, :, last:] = -7.0
    qb, kb, kb_self = synth.bf16_bits(q), synth.bf16_bits(k), synth.bf16_bits(ks)
    scale = 1 / np.sqrt(128)
    print(f"[gpu] kvsel_score_chunked case={case}", flush=True)
    s, r = kv.kvsel_score_chunked(to_dev(qb), to_dev(kb), to_dev(kb_self), G=G, m=m, n_prompt=npr,
                                  scale=scale, pool=pool, return_raw=True)
    torch.cuda.synchronize()
    s, r = s.cpu().numpy(), r.cpu().numpy()
    for l in range(L):
        ref = oracle.chunked_scores(synth.bf16_to_f64(qb[l]), synth.bf16_to_f64(kb[l]),
                                    synth.bf16_to_f64(kb_self[l]), G, scale, me, npr)
        assert_scores_close(r[l], ref, f"chunked raw l{l}")
        assert_scores_close(s[l], oracle.maxpool(ref, n, pool), f"chunked pooled l{l}")


ANCHOR_SELECT_CASES = [
    # (L, H, n, W, k, rho, levels)
    (1, 2, 1000, 8, 32, 0.7, 5),
    (2, 3, 4096, 32, 32, 0.7, 1000),      # window only
    (1, 2, 3000, 16, 3000, 0.5, 3),       # everything
    (1, 4, 50000, 32, 390, 0.7, 100),     # many workgroups per head
    (1, 1, 700, 0, 100, 0.0, 7),          # no window, all random
    (1, 1, 700, 4, 100, 1.0, 7),          # no random
]


@pytest.mark.parametrize("case", ANCHOR_SELECT_CASES, ids=lambda c: "L{}H{}n{}W{}k{}r{}lv{}".format(*c))
def test_anchor_select_exact(case):
    L, H, n, W, k, rho, levels = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    sc = _quantised_scores(rng, (L, H, n - W), levels)
    rd = (rng.integers(0, 1000, size=(L, H, n - W)) / 1000).astype(np.float32)   # ties in the draws too
    print(f"[gpu] kvsel_anchor_select case={case}", flush=True)
    got = kv.kvsel_anchor_select(torch.from_numpy(sc).cuda(), torch.from_numpy(rd).cuda(), n=n, W=W,
                                 k=k, rho=float(np.float32(rho))).cpu().numpy()
    for l in range(L):
        ref = oracle.anchor_select(sc[l].astype(np.float64), rd[l].astype(np.float64), n, W, k,
                                   float(np.float32(rho)))
        np.testing.assert_array_equal(got[l], ref)


ANCHOR_ASSIGN_CASES = [
    # (L, H, n, k)
    (1, 2, 1000, 8),
    (2, 3, 3000, 24),
    (1, 1, 5000, 100),       # two anchor tiles, the second partly padding
    (1, 2, 300, 300),        # every position an anchor
    (1, 1, 777, 1),
    (1, 1, 2100, 130),       # three tiles, ragged vectors
    (1, 2, 3000, 400),       # more than 256 anchors: the anchor rows stream through the ring
]


@pytest.mark.parametrize("case", ANCHOR_ASSIGN_CASES, ids=lambda c: "L{}H{}n{}k{}".format(*c))
def test_anchor_assign(case):
    """Exact slot where the fp64 best cosine leads by more than 1e-5; within
    1e-5 of it otherwise (fp32 dot products decide near-ties). gamma against
    <x, a>/<a, a> for the chosen anchor in fp64."""
    L, H, n, k = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = rng.standard_normal((L, H, n, 128)).astype(np.float32)
    anchors = np.sort(np.stack([[rng.choice(n, k, replace=False) for _ in range(H)] for _ in range(L)]),
                      axis=-1).astype(np.int32)
    if k >= 4:
        x[0, 0, anchors[0, 0, 3]] = x[0, 0, anchors[0, 0, 1]]   # a duplicate anchor: ties to slot 1
        x[0, 0, anchors[0, 0, 2]] = 0.0                         # a zero anchor: never chosen
        x[0, 0, (anchors[0, 0, 0] + 1) % n] = 0.0               # a zero vector (unless an anchor)
    xb = synth.bf16_bits(x)
    print(f"[gpu] kvsel_anchor_assign case={case}", flush=True)
    slot, gamma = kv.kvsel_anchor_assign(to_dev(xb), torch.from_numpy(anchors).cuda())
    torch.cuda.synchronize()
    slot, gamma = slot.cpu().numpy(), gamma.cpu().numpy()
    xf = synth.bf16_to_f64(xb)
    for l in range(L):
        for h in range(H):
            A = xf[l, h, anchors[l, h]]
            na = np.sqrt((A * A).sum(1))
            nx = np.sqrt((xf[l, h] ** 2).sum(1))
            dots = xf[l, h] @ A.T
            with np.errstate(divide="ignore", invalid="ignore"):
                cos = np.where(na > 0, np.nan_to_num(dots / (nx[:, None] * na[None, :])), -np.inf)
            is_anchor = np.zeros(n, bool)
            is_anchor[anchors[l, h]] = True
            np.testing.assert_array_equal(slot[l, h, anchors[l, h]], np.arange(k))
            np.testing.assert_array_equal(gamma[l, h, anchors[l, h]], 1.0)
            j = np.nonzero(~is_anchor)[0]
            s = slot[l, h, j]
            assert ((s >= 0) & (s < k)).all()
            best = cos[j].max(axis=1)
            assert (cos[j, s] >= best - 1e-5).all(), "a chosen anchor is not among the most similar"
            ref_slot, _ = oracle.anchor_assign(xf[l, h][None], anchors[l, h][None].astype(np.int64))
            second = np.sort(cos[j], axis=1)[:, -2] if k > 1 else np.full(len(j), -np.inf)
            clear = best - second > 1e-5
            np.testing.assert_array_equal(s[clear], ref_slot[0, j][clear])
            g_ref = dots[j, s] / np.where(na[s] > 0, na[s] ** 2, 1.0)
            tol = 1e-3 * np.abs(g_ref) + 1e-5 * nx[j] / np.where(na[s] > 0, na[s], 1.0)
            assert (np.abs(gamma[l, h, j] - g_ref) <= tol).all()
            if l == 0 and h == 0 and k >= 4:
                assert not (s == 3).any() and not (s == 2).any()   # duplicate and zero anchors


@pytest.mark.parametrize("k", [8, 300], ids=["resident", "ring"])
def test_anchor_assign_negative_ties(k):
    """Vectors whose every cosine is negative, with the least negative one
    shared by three copies of one anchor (slots 1, 3 and k-2: same lane,
    other lane half or tile): the lower slot wins the exact tie, as the
    oracle reads equal cosines."""
    rng = np.random.default_rng(1000 + k)
    n, d = 900, 128
    e0 = np.zeros(d, np.float32)
    e0[0] = 1.0
    anchors = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
    x = (-5.0 * e0 + 0.02 * rng.standard_normal((n, d))).astype(np.float32)
    a = (rng.uniform(2.0, 3.0, (k, 1)) * e0 + 0.3 * rng.standard_normal((k, d))).astype(np.float32)
    a[1] = 0.2 * e0 + 0.3 * rng.standard_normal(d)
    a[3] = a[1]
    a[k - 2] = a[1]
    x[anchors] = a
    xb = synth.bf16_bits(x[None, None])
    print(f"[gpu] kvsel_anchor_assign negative ties k={k}", flush=True)
    slot, gamma = kv.kvsel_anchor_assign(to_dev(xb), torch.from_numpy(anchors[None, None]).cuda())
    torch.cuda.synchronize()
    slot = slot.cpu().numpy()[0, 0]
    xf = synth.bf16_to_f64(xb)[0, 0]
    A = xf[anchors]
    cos = (xf @ A.T) / (np.linalg.norm(xf, axis=1)[:, None] * np.linalg.norm(A, axis=1)[None, :])
    j = np.setdiff1d(np.arange(n), anchors)
    others = np.delete(cos[j], [1, 3, k - 2], axis=1).max(axis=1)
    tied = (cos[j, 1] < 0) & (cos[j, 1] - others > 1e-5)
    assert tied.sum() > n // 2, "the construction should give most vectors a negative tied best"
    np.testing.assert_array_equal(slot[j][tied], 1)


SIGNED_CASES = [
    # (L, H, n, W, frac, adaptive, two_stage)
    (1, 3, 2000, 0, 0.3, False, False),
    (2, 2, 1000, 8, 0.2, True, False),
    (1, 2, 3000, 16, 0.4, False, True),
    (1, 1, 50000, 0, 0.1, False, False),      # many workgroups
    (1, 2, 40000, 8, 0.3, True, True),        # many workgroups, adaptive two-stage
]


@pytest.mark.parametrize("case", SIGNED_CASES, ids=lambda c: "L{}H{}n{}W{}b{}a{}t{}".format(*c))
def test_select_signed_scores(case):
    """Negative scores (logit scores), -0 beside +0, and infinities."""
    L, H, n, W, frac, adaptive, two_stage = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    n_cand = n - W
    sc = (rng.integers(-40, 40, size=(L, H, n_cand)) * 0.125).astype(np.float32)
    sc[sc == 0] = np.where(rng.random((sc == 0).sum()) < 0.5, -0.0, 0.0)
    flat = sc.reshape(-1)
    flat[rng.choice(flat.size, 5, replace=False)] = np.inf
    flat[rng.choice(flat.size, 5, replace=False)] = -np.inf
    wt = (rng.random((L, H, n_cand)).astype(np.float32) * 3 + 0.01) if two_stage else None
    groups = H if adaptive else 1
    budget = max(groups * W, int(np.floor(frac * groups * n)))
    print(f"[gpu] kvsel_select signed case={case}", flush=True)
    idx, offs, stage = kv.kvsel_select(torch.from_numpy(sc).cuda(), n=n, W=W, budget=budget,
                                       adaptive=adaptive,
                                       weight=None if wt is None else torch.from_numpy(wt).cuda(),
                                       score_norm=1.0 / 128, eps=1e-4, alpha=0.5, return_stage=True)
    torch.cuda.synchronize()
    idx, stage = idx.cpu().numpy(), stage.cpu().numpy()
    for l in range(L):
        ri, ro, rs = oracle.select_layer(sc[l].astype(np.float64), budget, W, n, adaptive=adaptive,
                                         weight=None if wt is None else wt[l].astype(np.float64),
                                         alpha=0.5, score_norm=float(np.float32(1 / 128)),
                                         eps=float(np.float32(1e-4)), dtype=np.float32)
        np.testing.assert_array_equal(idx[l], ri)
        np.testing.assert_array_equal(stage[l], rs)
        if adaptive:
            np.testing.assert_array_equal(offs[l].cpu().numpy(), ro)


@pytest.mark.parametrize("L,H,n_pos", [(2, 3, 1), (1, 4, 3), (3, 8, 4096), (2, 2, 33333)])
def test_head_score_exact(L, H, n_pos):
    """The max is exact: bit-equal to the oracle on signed scores."""
    rng = np.random.default_rng(L * 1000 + n_pos)
    sc = (rng.standard_normal((L, H, n_pos)) * 5 - 2).astype(np.float32)
    print(f"[gpu] kvsel_head_score L={L} H={H} n_pos={n_pos}", flush=True)
    got = kv.kvsel_head_score(torch.from_numpy(sc).cuda()).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.head_scores(sc.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("L,H,keep,levels", [
    (2, 3, 3, 4), (4, 8, 0, 10), (4, 8, 32, 10), (32, 8, 128, 7),
    (100, 400, 20000, 50),    # 40000 heads: the many-workgroup selection
])
def test_head_budgets_exact(L, H, keep, levels):
    rng = np.random.default_rng(keep + L)
    hs = _quantised_scores(rng, (L, H), levels) - 0.5
    n, W = 5000, 16
    print(f"[gpu] kvsel_head_budgets L={L} H={H} keep={keep}", flush=True)
    got = kv.kvsel_head_budgets(torch.from_numpy(hs).cuda(), keep=keep, n=n, W=W).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.head_budgets(hs.astype(np.float64), keep, n, W))


def test_head_level_eviction_pipeline():
    """Head score -> head budgets -> budget-vector select -> compaction: the
    kept heads keep every entry, the others their last W."""
    L, H, n, W, keep = 2, 4, 900, 24, 3
    rng = np.random.default_rng(77)
    sc = rng.random((L, H, n - W)).astype(np.float32)
    hs = kv.kvsel_head_score(torch.from_numpy(sc).cuda())
    b = kv.kvsel_head_budgets(hs, keep=keep, n=n, W=W)
    idx, offs, _ = kv.kvsel_select_budgets(torch.from_numpy(sc).cuda(), b, n=n, W=W)
    torch.cuda.synchronize()
    rb = oracle.head_budgets(oracle.head_scores(sc.astype(np.float64)), keep, n, W)
    np.testing.assert_array_equal(b.cpu().numpy(), rb)
    idx, offs = idx.cpu().numpy(), offs.cpu().numpy()
    for l in range(L):
        ri, ro, _ = oracle.select_budgets(sc[l].astype(np.float64), rb[l], W, n, dtype=np.float32)
        np.testing.assert_array_equal(offs[l], ro)
        np.testing.assert_array_equal(idx[l, :len(ri)], ri)
        for h in range(H):
            want = np.arange(n) if rb[l, h] == n else np.arange(n - W, n)
            np.testing.assert_array_equal(idx[l, offs[l, h]:offs[l, h + 1]], want)


def test_largest_head():
    """The largest head the scoring accepts (n * 256 B just under 2^31), with
    every key equal: each window row's softmax is then uniform over the keys
    it sees, so every score has a closed form; all candidates tie, so the
    selection (many workgroups at this size) keeps the lowest ones; the
    compaction copies the value rows they name."""
    n, W, G, budget = 8_388_607, 32, 4, 1000
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    row = torch.randn(128, device=dev, generator=g).to(torch.bfloat16)
    k = row.expand(1, 1, n, 128).contiguous()
    q = torch.randn((1, G, W, 128), device=dev, generator=g).to(torch.bfloat16)
    print(f"[gpu] kvsel_score largest head n={n}", flush=True)
    scores, raw = kv.kvsel_score(q, k, G=G, pool=7, return_raw=True)
    torch.cuda.synchronize()
    # window row i (query position n - W + i) sees keys 0 .. n - W + i
    inv = 1.0 / (n - W + np.arange(W) + 1.0)
    tail = G * np.cumsum(inv[::-1])[::-1]            # key n - W + t: rows t .. W - 1
    ref_raw = np.full(n, G * inv.sum())
    ref_raw[n - W:] = tail
    assert_scores_close(raw.cpu().numpy()[0], ref_raw[None], "raw")
    assert_scores_close(scores.cpu().numpy()[0], np.full((1, n - W), G * inv.sum()), "pooled")
    del raw
    print("[gpu] kvsel_select largest head", flush=True)
    idx, _, _ = kv.kvsel_select(scores, n=n, W=W, budget=budget)
    torch.cuda.synchronize()
    want = np.concatenate([np.arange(budget - W), np.arange(n - W, n)])
    np.testing.assert_array_equal(idx.cpu().numpy()[0, 0], want)
    del scores, k
    v = torch.randn((1, 1, n, 128), device=dev, generator=g).to(torch.bfloat16)
    print("[gpu] kvsel_compact largest head", flush=True)
    k_out, v_out = kv.kvsel_compact(v, v, idx)
    torch.cuda.synchronize()
    sel = torch.from_numpy(want).to(dev)
    assert torch.equal(v_out.reshape(-1, 128), v[0, 0, sel])
    assert torch.equal(k_out, v_out)


def test_select_end_to_end_band():
    """GPU scores + GPU select against the fp64 oracle's selection."""
    wl = _wl(L=2, H_kv=2, n=3000, W=32)
    data = gen(wl, seed=4, which=("q", "k"))
    q, k = to_dev(data["q"]), to_dev(data["k"])
    scores, _ = kv.kvsel_score(q, k, G=wl.G, pool=7)
    budget = int(0.3 * wl.n)
    idx, _, _ = kv.kvsel_select(scores, n=wl.n, W=wl.W, budget=budget)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for l in range(wl.L):
        _, pooled = oracle_scores_layer(wl, data["q"][l], data["k"][l])
        picks = split_heads(idx[l], None, wl.H_kv, wl.W, wl.n)
        for h in range(wl.H_kv):
            assert_topk_within_band(picks[h], pooled[h], budget - wl.W, f"l{l}h{h}")


# -------------------------------------------------------------- compaction ----

@pytest.mark.parametrize("adaptive,d", [(False, 128), (True, 128), (False, 64), (True, 72)])
def test_compact_bit_exact(adaptive, d):
    rng = np.random.default_rng(5)
    L, H, n = 2, 3, 777
    k = rng.integers(0, 65536, size=(L, H, n, d), dtype=np.uint16)
    v = rng.integers(0, 65536, size=(L, H, n, d), dtype=np.uint16)
    if adaptive:
        counts = [[5, 0, 40], [17, 3, 25]]
        kept = 45
        idx = np.zeros((L, kept), np.int32)
        offs = np.zeros((L, H + 1), np.int32)
        for l in range(L):
            parts = [np.sort(rng.choice(n, c, replace=False)) for c in counts[l]]
            idx[l] = np.concatenate(parts)
            offs[l] = np.concatenate([[0], np.cumsum(counts[l])])
    else:
        B = 31
        idx = np.stack([np.stack([np.sort(rng.choice(n, B, replace=False)) for _ in range(H)])
                        for _ in range(L)]).astype(np.int32)
        offs = None
    ko, vo = kv.kvsel_compact(to_dev(k), to_dev(v), torch.from_numpy(idx).cuda(),
                              None if offs is None else torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    ko = ko.cpu().view(torch.int16).numpy().view(np.uint16)
    vo = vo.cpu().view(torch.int16).numpy().view(np.uint16)
    for l in range(L):
        rk, rv = oracle.compact_layer(k[l], v[l], idx[l], None if offs is None else offs[l])
        np.testing.assert_array_equal(ko[l].reshape(rk.shape), rk)
        np.testing.assert_array_equal(vo[l].reshape(rv.shape), rv)


# ------------------------------------------------------------ value weight ----

@pytest.mark.parametrize("group_mode", [kv.GROUP_MEAN_OF_NORMS, kv.GROUP_NORM_OF_SUM])
@pytest.mark.parametrize("L,H,G,n,D,n_cand", [
    (1, 2, 4, 300, 256, 290),
    (1, 1, 7, 97, 64, 97),
    (1, 3, 1, 1000, 32, 999),     # half a W_O tile
    (2, 2, 3, 1500, 96, 1400),    # several key blocks, ragged, last tile half
    (2, 3, 8, 700, 4096, 650),    # the model's D, G = 8
])
def test_value_weight(L, H, G, n, D, n_cand, group_mode):
    """Mode 0 against the fp64 mean of per-query-head norms; mode 1 against
    the fp64 norm of the exactly summed slices (the kernel rounds the summed
    slices to bf16 once, ~2^-9 relative per element, which averages out in
    the L1 sum far below the 1e-3 bar on these inputs)."""
    wl = _wl(L=L, H_kv=H, G=G, n=n, W=n - n_cand if n_cand < n else 1, value_weight=True, D=D)
    data = gen(wl, seed=6, which=("v", "w_o"))
    print(f"[gpu] kvsel_value_weight L={L} H={H} G={G} n={n} D={D} mode={group_mode}", flush=True)
    w = kv.kvsel_value_weight(to_dev(data["v"]), to_dev(data["w_o"]), G=G, n_cand=n_cand,
                              group_mode=group_mode)
    torch.cuda.synchronize()
    w = w.cpu().numpy()
    norm = oracle.value_weight if group_mode == kv.GROUP_MEAN_OF_NORMS else oracle.value_weight_group_sum
    for l in range(L):
        ref = norm(synth.bf16_to_f64(data["v"][l]), synth.bf16_to_f64(data["w_o"][l]), G,
                   np.arange(n_cand))
        assert_scores_close(w[l], ref, "value weight")


def test_value_weight_group_sum_single_head_is_mode0():
    """With G = 1 the summed slice is the slice itself (no rounding): both
    group modes give the same bits."""
    wl = _wl(L=2, H_kv=3, G=1, n=900, W=1, value_weight=True, D=256)
    data = gen(wl, seed=9, which=("v", "w_o"))
    v, w_o = to_dev(data["v"]), to_dev(data["w_o"])
    print("[gpu] kvsel_value_weight G=1 both modes", flush=True)
    a = kv.kvsel_value_weight(v, w_o, G=1, group_mode=kv.GROUP_MEAN_OF_NORMS)
    b = kv.kvsel_value_weight(v, w_o, G=1, group_mode=kv.GROUP_NORM_OF_SUM)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# L2 form: the kernel factors each query head's W^T W (Cholesky, fp32) and
# projects by the factor held as bf16 hi + lo (~2^-17 relative), so the
# weight meets the same rel 1e-3 bar as the L1 form. D < d (rank-deficient
# W^T W) exercises the dropped pivots.
@pytest.mark.parametrize("L,H,G,n,D,n_cand", [
    (1, 2, 4, 300, 256, 290),
    (1, 1, 7, 97, 4096, 97),
    (1, 3, 1, 1000, 32, 999),     # rank 32 of 128
    (2, 2, 3, 1500, 100, 1400),   # several key blocks, ragged, D not a multiple of 64
    (1, 1, 2, 600, 128, 513),     # square slice
])
def test_value_weight_l2(L, H, G, n, D, n_cand):
    wl = _wl(L=L, H_kv=H, G=G, n=n, W=n - n_cand if n_cand < n else 1, value_weight=True, D=D)
    data = gen(wl, seed=8, which=("v", "w_o"))
    print(f"[gpu] kvsel_value_weight_l2 L={L} H={H} G={G} n={n} D={D}", flush=True)
    fac = kv.kvsel_value_l2_factor(to_dev(data["w_o"]), G=G, H_kv=H)
    w = kv.kvsel_value_weight_l2(to_dev(data["v"]), fac, G=G, n_cand=n_cand)
    torch.cuda.synchronize()
    w = w.cpu().numpy()
    for l in range(L):
        ref = oracle.value_weight_l2(synth.bf16_to_f64(data["v"][l]),
                                     synth.bf16_to_f64(data["w_o"][l]), G, np.arange(n_cand))
        assert_scores_close(w[l], ref, "value weight l2")


def test_value_weight_l2_deterministic():
    wl = _wl(L=1, H_kv=2, G=4, n=3000, W=1, value_weight=True, D=512)
    data = gen(wl, seed=9, which=("v", "w_o"))
    v, w_o = to_dev(data["v"]), to_dev(data["w_o"])
    fac = kv.kvsel_value_l2_factor(w_o, G=wl.G, H_kv=wl.H_kv)
    a = kv.kvsel_value_weight_l2(v, fac, G=wl.G, n_cand=wl.n).cpu().numpy()
    f0 = fac.cpu().view(torch.int16).numpy()
    for _ in range(2):
        fac = kv.kvsel_value_l2_factor(w_o, G=wl.G, H_kv=wl.H_kv)
        np.testing.assert_array_equal(fac.cpu().view(torch.int16).numpy(), f0)
        b = kv.kvsel_value_weight_l2(v, fac, G=wl.G, n_cand=wl.n).cpu().numpy()
        np.testing.assert_array_equal(a, b)


def test_value_l2_factor_properties():
    """The factor is upper triangular with a non-negative diagonal, and
    (R_hi + R_lo)^T (R_hi + R_lo) reproduces the fp64 Gram matrix W^T W of
    each query head's slice."""
    wl = _wl(L=2, H_kv=2, G=3, n=64, W=1, value_weight=True, D=700)
    data = gen(wl, seed=10, which=("w_o",))
    fac = kv.kvsel_value_l2_factor(to_dev(data["w_o"]), G=wl.G, H_kv=wl.H_kv)
    torch.cuda.synchronize()
    r = fac.float().cpu().numpy().astype(np.float64)
    for l in range(wl.L):
        w = synth.bf16_to_f64(data["w_o"][l])
        for hq in range(wl.H_kv * wl.G):
            hi, lo = r[l, hq, 0], r[l, hq, 1]
            assert not np.tril(hi, -1).any() and not np.tril(lo, -1).any()
            assert (np.diag(hi) >= 0).all()
            R = hi + lo
            M = w[:, hq * 128:(hq + 1) * 128].T @ w[:, hq * 128:(hq + 1) * 128]
            err = np.abs(R.T @ R - M).max()
            assert err <= 1e-4 * np.abs(M).max(), (l, hq, err)


# ------------------------------------------------- decode over kept rows ----
#
# Tolerance: outputs are weighted means of v rows, so their error is
# measured against the head's largest |v|: |gpu - ref| <= 1e-4 * max|v| +
# 1e-4 * |ref|. fp32 logits from exact bf16 products (|error| ~ 1e-5 of a
# logit of magnitude ~10), base-2 exponentials and fp32 sums over <= 10^4
# rows keep the weights within ~1e-5 relative.

DECODE_CASES = [
    # (L, H_kv, G, head lengths per layer (None: uniform B), B)
    (1, 2, 4, None, 300),        # two items per head, the second ragged
    (2, 8, 4, None, 13),         # tiny heads
    (1, 1, 8, None, 1000),       # G = 8, four items
    (1, 3, 7, None, 256),        # exactly one item
    (1, 4, 1, None, 512),
    (2, 4, 4, [[0, 1, 600, 257], [300, 0, 0, 5]], None),   # ragged, empty heads
    (1, 3, 2, [[2000, 3, 513]], None),
]


def _decode_inputs(rng, L, H, G, lengths, B):
    if lengths is None:
        lengths = [[B] * H for _ in range(L)]
    kept = max(sum(x) for x in lengths)
    offs = np.zeros((L, H + 1), np.int32)
    for l in range(L):
        offs[l, 1:] = np.cumsum(lengths[l])
    q = synth.bf16_bits(rng.normal(size=(L, H * G, 128)).astype(np.float32))
    k = synth.bf16_bits((rng.normal(size=(L, kept, 128)) * 1.5).astype(np.float32))
    v = synth.bf16_bits(rng.normal(size=(L, kept, 128)).astype(np.float32))
    return q, k, v, offs, kept


def _assert_decode_close(got, ref, vmax, what):
    bad = np.abs(got - ref) > 1e-4 * vmax + 1e-4 * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} entries off; max err {np.abs(got - ref).max():.3g}"


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"L{c[0]}H{c[1]}G{c[2]}{'r' if c[3] else 'u'}")
def test_decode_attention(case):
    L, H, G, lengths, B = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v, offs, kept = _decode_inputs(rng, L, H, G, lengths, B)
    scale = 1.0 / np.sqrt(128.0)
    ragged = lengths is not None
    print(f"[gpu] kvsel_decode_attention L={L} H={H} G={G} kept={kept} ragged={ragged}", flush=True)
    out = kv.kvsel_decode_attention(to_dev(q), to_dev(k), to_dev(v), G=G, scale=scale,
                                    head_offsets=torch.from_numpy(offs).cuda() if ragged else None)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for l in range(L):
        kl, vl = synth.bf16_to_f64(k[l]), synth.bf16_to_f64(v[l])
        if ragged:
            ref = oracle.decode_attention(synth.bf16_to_f64(q[l]), kl, vl, G, scale, offs[l])
        else:
            ref = oracle.decode_attention(synth.bf16_to_f64(q[l]), kl.reshape(H, B, 128),
                                          vl.reshape(H, B, 128), G, scale)
        _assert_decode_close(out[l], ref, np.abs(vl).max(), f"decode layer {l}")


@pytest.mark.parametrize("kept,offsets", [
    (300, [-5, 100, 40, 290, 9999]),
    # overlapping heads: each clamped offset alone would give 8 work items
    # against the 7 the grid and workspace hold (regression test)
    (1024, [0, 1024, 0, 1024]),
])
def test_decode_attention_clamps_offsets(kept, offsets):
    """Offsets are clamped into [0, kept] and raised to the largest earlier
    one, so the heads are disjoint ranges inside the layer: nothing outside
    the layer's rows or the workspace is read."""
    rng = np.random.default_rng(77)
    L, G = 1, 2
    H = len(offsets) - 1
    q = synth.bf16_bits(rng.normal(size=(L, H * G, 128)).astype(np.float32))
    k = synth.bf16_bits(rng.normal(size=(L, kept, 128)).astype(np.float32))
    v = synth.bf16_bits(rng.normal(size=(L, kept, 128)).astype(np.float32))
    offs = np.array([offsets], np.int32)
    print(f"[gpu] kvsel_decode_attention offsets {offsets} kept={kept}", flush=True)
    out = kv.kvsel_decode_attention(to_dev(q), to_dev(k), to_dev(v), G=G, scale=0.09,
                                    head_offsets=torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()[0]
    # [-5, 100, 40, 290, 9999] -> [0, 100, 100, 290, 300]: head 1 empty, head 2 = [100, 290)
    # [0, 1024, 0, 1024] -> [0, 1024, 1024, 1024]: heads 1 and 2 empty
    eff = np.maximum.accumulate(np.clip(offs[0], 0, kept))
    ref = oracle.decode_attention(synth.bf16_to_f64(q[0]), synth.bf16_to_f64(k[0]),
                                  synth.bf16_to_f64(v[0]), G, 0.09, eff)
    _assert_decode_close(out, ref, np.abs(synth.bf16_to_f64(v[0])).max(), "clamped offsets")
