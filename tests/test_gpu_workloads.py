"""The five named workloads at full size, in the launch configuration the
bench times, checked against the oracle on sampled outputs.

Every layer runs on the GPU. Sampled layers carry the host generator's
exact data so the oracle can recompute them; the other layers are seeded
device-side Gaussian draws of the same shape (layers are independent, so
they do not affect the sampled results). Checks:
  - scores (raw and pooled) of sampled layers, all heads, against the fp64
    oracle (relative 1e-3); window scoring with sum aggregation also checks
    every head of every layer for sum_j raw_j = W*G (each of the W*G query
    rows' softmax sums to one);
  - value weights at sampled positions against the fp64 oracle;
  - selection: bit-exact against the oracle run in fp32 on the GPU's own
    scores (same precision decides), and within the tolerance band of the
    fp64 oracle's selection where that is affordable;
  - compaction: bit-exact given the GPU's index set;
  - one decoding step over the compacted cache of a sampled layer against
    the fp64 oracle.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import eviction_importance_scoring_amd as kv
import oracle
import synth
from harness import (RTOL, assert_logits_close, assert_scores_close, assert_topk_within_band,
                     logit_error_bound, oracle_scores_layer, split_heads, to_dev)

pytestmark = pytest.mark.gpu

SEED = 0


def device_inputs(wl: synth.Workload, sampled, which):
    shapes = {name: wl.shape(name) for name in which}
    std = {"q": 1.0, "k": 1.0, "v": 1.0, "w_o": 0.02, "kself": 1.0}
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    dev, host = {}, {}
    for name in which:
        t = torch.empty((wl.L, *shapes[name]), dtype=torch.bfloat16, device="cuda")
        for l in range(wl.L):
            if l in sampled:
                u = getattr(synth, "gen_" + name)(wl, SEED, l)
                host[(name, l)] = u
                t[l] = to_dev(u)
            else:
                t[l] = (torch.randn(shapes[name], generator=g, device="cuda") * std[name]).to(torch.bfloat16)
        dev[name] = t
    torch.cuda.synchronize()
    return dev, host


def _mode(wl):
    return kv.Q_WINDOW if wl.q_mode == "window" else kv.Q_EXTERNAL


def _agg(wl):
    return {"sum": kv.AGG_SUM, "max": kv.AGG_MAX, "logit": kv.AGG_LOGIT_MAX}[wl.agg]


def _score(wl, dev):
    print(f"[gpu] kvsel_score {wl.name}", flush=True)
    s, r = kv.kvsel_score(dev["q"], dev["k"], G=wl.G, q_mode=_mode(wl), agg=_agg(wl),
                          scale=wl.scale, pool=wl.pool, return_raw=True)
    torch.cuda.synchronize()
    return s, r


def _check_scores(wl, s, r, host, layers):
    if wl.q_mode == "window" and wl.agg == "sum":
        # [KVzip, §3.2]: the softmax runs along keys, the sum over the W*G
        # window rows, so a head's raw scores add up to W*G; fp32 sums of
        # n terms stay within 1e-4 of it
        tot = r.sum(dim=-1, dtype=torch.float64).cpu().numpy()
        err = np.abs(tot - wl.W * wl.G).max()
        assert err <= 1e-4 * wl.W * wl.G, f"{wl.name}: sum of raw scores off W*G by {err:.3g}"
    for l in layers:
        ref_raw, ref_pool = oracle_scores_layer(wl, host[("q", l)], host[("k", l)])
        assert_scores_close(r[l].cpu().numpy(), ref_raw, f"{wl.name} raw l{l}")
        assert_scores_close(s[l].cpu().numpy(), ref_pool, f"{wl.name} pooled l{l}")


def _check_select_exact(wl, s, w, idx, offs, stage, layers):
    for l in layers:
        ri, ro, rs = oracle.select_layer(
            s[l].cpu().numpy().astype(np.float64), wl.budget, wl.W_kept, wl.n, adaptive=wl.adaptive,
            weight=None if w is None else w[l].cpu().numpy().astype(np.float64),
            alpha=wl.alpha, score_norm=float(np.float32(1.0 / (wl.W * wl.G))),
            eps=float(np.float32(wl.eps)), dtype=np.float32)
        np.testing.assert_array_equal(idx[l].cpu().numpy(), ri)
        np.testing.assert_array_equal(stage[l].cpu().numpy(), rs)
        if offs is not None:
            np.testing.assert_array_equal(offs[l].cpu().numpy(), ro)


def _check_compact(dev, host, idx, offs, l, wl):
    ko, vo = kv.kvsel_compact(dev["k"], dev["v"], idx, offs)
    torch.cuda.synchronize()
    k_l = dev["k"][l].cpu().view(torch.int16).numpy().view(np.uint16)
    v_l = dev["v"][l].cpu().view(torch.int16).numpy().view(np.uint16)
    rk, rv = oracle.compact_layer(k_l, v_l, idx[l].cpu().numpy(),
                                  None if offs is None else offs[l].cpu().numpy())
    np.testing.assert_array_equal(ko[l].cpu().view(torch.int16).numpy().view(np.uint16).reshape(rk.shape), rk)
    np.testing.assert_array_equal(vo[l].cpu().view(torch.int16).numpy().view(np.uint16).reshape(rv.shape), rv)
    _check_decode(wl, ko, vo, offs, l)


def _check_decode(wl, ko, vo, offs, l):
    """One decoding step over the compacted cache of every layer; layer l
    against the fp64 oracle (|err| <= 1e-4 * max|v| + 1e-4 * |ref|)."""
    rng = np.random.default_rng(99)
    qd = synth.bf16_bits(rng.normal(size=(wl.L, wl.H_q, wl.d)).astype(np.float32))
    print(f"[gpu] kvsel_decode_attention {wl.name}", flush=True)
    out = kv.kvsel_decode_attention(to_dev(qd), ko, vo, G=wl.G, scale=wl.scale, head_offsets=offs)
    torch.cuda.synchronize()
    k_u = ko[l].cpu().view(torch.int16).numpy().view(np.uint16)
    v_u = vo[l].cpu().view(torch.int16).numpy().view(np.uint16)
    if offs is None:
        k_l, v_l = synth.bf16_to_f64(k_u), synth.bf16_to_f64(v_u)
        ref = oracle.decode_attention(synth.bf16_to_f64(qd[l]), k_l.reshape(wl.H_kv, -1, wl.d),
                                      v_l.reshape(wl.H_kv, -1, wl.d), wl.G, wl.scale)
    else:
        o = offs[l].cpu().numpy()
        # rows past the last head are not written: cut before converting
        k_l, v_l = synth.bf16_to_f64(k_u[:o[-1]]), synth.bf16_to_f64(v_u[:o[-1]])
        ref = oracle.decode_attention(synth.bf16_to_f64(qd[l]), k_l, v_l, wl.G, wl.scale, o)
    got = out[l].cpu().numpy()
    bad = np.abs(got - ref) > 1e-4 * np.abs(v_l).max() + 1e-4 * np.abs(ref)
    assert not bad.any(), f"decode layer {l}: {bad.sum()} entries off, max err {np.abs(got - ref).max():.3g}"


def test_snapkv_L1_n4k_full():
    wl = synth.WORKLOADS["snapkv_L1_n4k"]
    dev, host = device_inputs(wl, {0}, ("q", "k", "v"))
    s, r = _score(wl, dev)
    _check_scores(wl, s, r, host, [0])
    idx, offs, stage = kv.kvsel_select(s, n=wl.n, W=wl.W, budget=wl.budget, return_stage=True)
    torch.cuda.synchronize()
    _check_select_exact(wl, s, None, idx, offs, stage, [0])
    _, ref_pool = oracle_scores_layer(wl, host[("q", 0)], host[("k", 0)])
    picks = split_heads(idx[0].cpu().numpy(), None, wl.H_kv, wl.W, wl.n)
    for h in range(wl.H_kv):
        assert_topk_within_band(picks[h], ref_pool[h], wl.budget - wl.W, f"h{h}")
    _check_compact(dev, host, idx, offs, 0, wl)


@pytest.mark.parametrize("name", ["llama8b_n32k", "adakv_llama8b_n64k", "h2o_llama8b_n32k"])
def test_window_workload_full(name):
    wl = synth.WORKLOADS[name]
    sampled = [0, wl.L - 1]
    dev, host = device_inputs(wl, set(sampled), ("q", "k", "v"))
    s, r = _score(wl, dev)
    _check_scores(wl, s, r, host, sampled)
    # without a raw output (the call the bench times) the pooled scores are
    # the same bits
    print(f"[gpu] kvsel_score {wl.name} (no raw output)", flush=True)
    s2, _ = kv.kvsel_score(dev["q"], dev["k"], G=wl.G, q_mode=_mode(wl), agg=_agg(wl),
                           scale=wl.scale, pool=wl.pool)
    torch.cuda.synchronize()
    assert torch.equal(s2, s), "pooled scores depend on whether raw sums are returned"
    del s2
    idx, offs, stage = kv.kvsel_select(s, n=wl.n, W=wl.W, budget=wl.budget, adaptive=wl.adaptive,
                                       return_stage=True)
    torch.cuda.synchronize()
    _check_select_exact(wl, s, None, idx, offs, stage, sampled)
    # end-to-end band check on layer 0 against the fp64 oracle
    _, ref_pool = oracle_scores_layer(wl, host[("q", 0)], host[("k", 0)])
    if wl.adaptive:
        flat = []
        o = offs[0].cpu().numpy()
        picks = split_heads(idx[0].cpu().numpy(), o, wl.H_kv, wl.W, wl.n)
        for h in range(wl.H_kv):
            flat += list(h * wl.n_cand + picks[h])
        assert_topk_within_band(flat, ref_pool.reshape(-1), wl.budget - wl.H_kv * wl.W, "layer0")
    else:
        picks = split_heads(idx[0].cpu().numpy(), None, wl.H_kv, wl.W, wl.n)
        for h in range(wl.H_kv):
            assert_topk_within_band(picks[h], ref_pool[h], wl.budget - wl.W, f"h{h}")
    _check_compact(dev, host, idx, offs, 0, wl)


def test_headkv_budget_vector_full():
    wl = synth.WORKLOADS["headkv_llama8b_n32k"]
    sampled = [0, wl.L - 1]
    dev, host = device_inputs(wl, set(sampled), ("q", "k", "v"))
    s, r = _score(wl, dev)
    _check_scores(wl, s, r, host, [0])
    budgets = synth.gen_budgets(wl, SEED)
    print("[gpu] kvsel_select_budgets full", flush=True)
    idx, offs, stage = kv.kvsel_select_budgets(s, torch.from_numpy(budgets).cuda(), n=wl.n,
                                               W=wl.W, return_stage=True)
    torch.cuda.synchronize()
    eff = np.clip(budgets, wl.W, wl.n).astype(np.int64)
    assert idx.shape[1] == eff.sum(axis=1).max()
    for l in sampled:
        ri, ro, rs = oracle.select_budgets(s[l].cpu().numpy().astype(np.float64), budgets[l], wl.W,
                                           wl.n, dtype=np.float32)
        m = len(ri)
        np.testing.assert_array_equal(offs[l].cpu().numpy(), ro)
        np.testing.assert_array_equal(idx[l, :m].cpu().numpy(), ri)
        np.testing.assert_array_equal(stage[l, :m].cpu().numpy(), rs)
        assert (idx[l, m:].cpu().numpy() == -1).all()
    # end-to-end band check on layer 0 against the fp64 oracle
    _, ref_pool = oracle_scores_layer(wl, host[("q", 0)], host[("k", 0)])
    o = offs[0].cpu().numpy()
    picks = split_heads(idx[0].cpu().numpy(), o, wl.H_kv, wl.W, wl.n)
    for h in range(wl.H_kv):
        assert_topk_within_band(picks[h], ref_pool[h], int(eff[0, h]) - wl.W, f"h{h}")
    # compaction of layer 0 (rows past the last head are not written), then decode
    ko, vo = kv.kvsel_compact(dev["k"], dev["v"], idx, offs)
    torch.cuda.synchronize()
    end = int(o[-1])
    k_l = dev["k"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    v_l = dev["v"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    rk, rv = oracle.compact_layer(k_l, v_l, idx[0, :end].cpu().numpy(), o)
    ko0 = ko[0].cpu().view(torch.int16).numpy().view(np.uint16)
    vo0 = vo[0].cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ko0[:end], rk)
    np.testing.assert_array_equal(vo0[:end], rv)
    _check_decode(wl, ko, vo, offs, 0)


def test_headlevel_eviction_full():
    wl = synth.WORKLOADS["headlevel_llama8b_n32k"]
    sampled = [0, wl.L - 1]
    dev, host = device_inputs(wl, set(sampled), ("q", "k", "v"))
    s, r = _score(wl, dev)
    _check_scores(wl, s, r, host, [0])
    keep = int(round(wl.head_keep * wl.L * wl.H_kv))
    print("[gpu] kvsel_head_score + kvsel_head_budgets full", flush=True)
    hs = kv.kvsel_head_score(s)
    b = kv.kvsel_head_budgets(hs, keep=keep, n=wl.n, W=wl.W)
    torch.cuda.synchronize()
    s_h = s.cpu().numpy()
    # exact on the GPU's own scores; within the score tolerance of the fp64 oracle
    np.testing.assert_array_equal(hs.cpu().numpy(), oracle.head_scores(s_h.astype(np.float64)).astype(np.float32))
    _, ref_pool = oracle_scores_layer(wl, host[("q", 0)], host[("k", 0)])
    assert_scores_close(hs[0].cpu().numpy(), oracle.head_scores(ref_pool), "head score l0")
    bh = b.cpu().numpy()
    np.testing.assert_array_equal(bh, oracle.head_budgets(hs.cpu().numpy().astype(np.float64), keep,
                                                          wl.n, wl.W))
    full = min(wl.H_kv, keep)
    stride = full * wl.n + (wl.H_kv - full) * wl.W
    idx, offs, _ = kv.kvsel_select_budgets(s, b, n=wl.n, W=wl.W, layer_stride=stride)
    torch.cuda.synchronize()
    for l in sampled:
        o = offs[l].cpu().numpy()
        ri, ro, _ = oracle.select_budgets(s_h[l].astype(np.float64), bh[l], wl.W, wl.n, dtype=np.float32)
        np.testing.assert_array_equal(o, ro)
        np.testing.assert_array_equal(idx[l, :len(ri)].cpu().numpy(), ri)
    ko, vo = kv.kvsel_compact(dev["k"], dev["v"], idx, offs)
    torch.cuda.synchronize()
    o = offs[0].cpu().numpy()
    end = int(o[-1])
    k_l = dev["k"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    v_l = dev["v"][0].cpu().view(torch.int16).numpy().view(np.uint16)
    rk, rv = oracle.compact_layer(k_l, v_l, idx[0, :end].cpu().numpy(), o)
    np.testing.assert_array_equal(ko[0, :end].cpu().view(torch.int16).numpy().view(np.uint16), rk)
    np.testing.assert_array_equal(vo[0, :end].cpu().view(torch.int16).numpy().view(np.uint16), rv)
    _check_decode(wl, ko, vo, offs, 0)


def _check_assign(x_u16, anchors, slot, gamma, what):
    """Anchors exact; elsewhere the chosen anchor within 1e-5 of the best
    fp64 cosine (fp32 dot products decide near-ties) and gamma within 1e-3
    of <x, a>/<a, a> for it (plus 1e-5 |x|/|a| for near-zero gamma)."""
    xf = synth.bf16_to_f64(x_u16)
    H, n, _ = xf.shape
    for h in range(H):
        a_pos = anchors[h]
        A = xf[h, a_pos]
        na = np.sqrt((A * A).sum(1))
        nx = np.sqrt((xf[h] ** 2).sum(1))
        dots = xf[h] @ A.T
        cos = dots / (nx[:, None] * na[None, :])
        np.testing.assert_array_equal(slot[h, a_pos], np.arange(len(a_pos)), err_msg=what)
        np.testing.assert_array_equal(gamma[h, a_pos], 1.0, err_msg=what)
        j = np.setdiff1d(np.arange(n), a_pos)
        s = slot[h, j]
        assert (cos[j, s] >= cos[j].max(axis=1) - 1e-5).all(), f"{what} h{h}: slots"
        g_ref = dots[j, s] / na[s] ** 2
        assert (np.abs(gamma[h, j] - g_ref) <= 1e-3 * np.abs(g_ref) + 1e-5 * nx[j] / na[s]).all(), \
            f"{what} h{h}: gamma"


def test_anchorkv_full():
    wl = synth.WORKLOADS["anchorkv_llama8b_n32k"]
    sampled = [0, wl.L - 1]
    dev, host = device_inputs(wl, set(sampled), ("q", "k", "v"))
    s, r = _score(wl, dev)
    _check_scores(wl, s, r, host, [0])
    rand = synth.gen_rand(wl, SEED)
    print("[gpu] kvsel_anchor_select + kvsel_anchor_assign full", flush=True)
    anchors = kv.kvsel_anchor_select(s, torch.from_numpy(rand).cuda(), n=wl.n, W=wl.W,
                                     k=wl.anchor_k, rho=wl.rho)
    ks, kg = kv.kvsel_anchor_assign(dev["k"], anchors)
    vs, vg = kv.kvsel_anchor_assign(dev["v"], anchors)
    torch.cuda.synchronize()
    s_h, a_h = s.cpu().numpy(), anchors.cpu().numpy()
    for l in sampled:
        ref = oracle.anchor_select(s_h[l].astype(np.float64), rand[l].astype(np.float64), wl.n, wl.W,
                                   wl.anchor_k, float(np.float32(wl.rho)))
        np.testing.assert_array_equal(a_h[l], ref)
        _check_assign(host[("k", l)], a_h[l], ks[l].cpu().numpy(), kg[l].cpu().numpy(), f"keys l{l}")
        _check_assign(host[("v", l)], a_h[l], vs[l].cpu().numpy(), vg[l].cpu().numpy(), f"values l{l}")


@pytest.mark.parametrize("name", ["criticalkv_llama8b_n128k", "criticaladakv_llama8b_n32k",
                                  "criticalkv_l2_llama8b_n128k"])
def test_criticalkv_full(name):
    wl = synth.WORKLOADS[name]
    sampled = [0, wl.L - 1]
    dev, host = device_inputs(wl, set(sampled), ("q", "k", "v", "w_o"))
    s, r = _score(wl, dev)
    _check_scores(wl, s, r, host, [0])
    if wl.value_norm == "l2":
        print("[gpu] kvsel_value_l2_factor + kvsel_value_weight_l2 full", flush=True)
        fac = kv.kvsel_value_l2_factor(dev["w_o"], G=wl.G, H_kv=wl.H_kv)
        w = kv.kvsel_value_weight_l2(dev["v"], fac, G=wl.G, n_cand=wl.n_cand)
        del fac
        norm = oracle.value_weight_l2
    else:
        print("[gpu] kvsel_value_weight full", flush=True)
        w = kv.kvsel_value_weight(dev["v"], dev["w_o"], G=wl.G, n_cand=wl.n_cand)
        norm = oracle.value_weight
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    # every head: 96 scattered positions, a contiguous block of 4096 across
    # several 512-key workgroup boundaries, and the ragged last block
    block = np.arange(wl.n_cand // 2 - 2048, wl.n_cand // 2 + 2048)
    tail = np.arange(max(0, (wl.n_cand - 1) // 512 * 512 - 64), wl.n_cand)
    for l in sampled:
        pos = np.unique(np.concatenate([rng.choice(wl.n_cand, 96, replace=False), block, tail]))
        print(f"[host] oracle value weight l{l}: {pos.size} positions x {wl.H_kv} heads", flush=True)
        ref = norm(synth.bf16_to_f64(host[("v", l)]), synth.bf16_to_f64(host[("w_o", l)]), wl.G, pos)
        assert_scores_close(w[l].cpu().numpy()[:, pos], ref, f"value weight l{l}")
    idx, offs, stage = kv.kvsel_select(s, n=wl.n, W=wl.W, budget=wl.budget, weight=w,
                                       adaptive=wl.adaptive, score_norm=1.0 / (wl.W * wl.G),
                                       eps=wl.eps, alpha=wl.alpha, return_stage=True)
    torch.cuda.synchronize()
    _check_select_exact(wl, s, w, idx, offs, stage, sampled)
    st = stage[0].cpu().numpy()
    k = wl.budget - (wl.H_kv * wl.W if wl.adaptive else wl.W)
    assert ((st == 1).sum(axis=-1) == int(np.floor(wl.alpha * k))).all()
    assert ((st == 2).sum(axis=-1) == k - int(np.floor(wl.alpha * k))).all()
    if wl.value_norm == "l1":
        # uniform budgets select per head: two heads; one budget per layer: all
        heads = list(range(wl.H_kv)) if wl.adaptive else [0, wl.H_kv - 1]
        _check_two_stage_band(wl, host, idx[0].cpu().numpy(), None if offs is None else offs[0].cpu().numpy(),
                              stage[0].cpu().numpy(), heads)
    _check_compact(dev, host, idx, offs, 0, wl)


def _ref_weights_head(v64, w64, wl, h, chunk=4096):
    """fp64 value weight of every candidate of KV head h: the oracle on the
    head's own values and its G column slices of W_O, in position chunks."""
    d = wl.d
    v_h = v64[h:h + 1]
    w_h = w64[:, h * wl.G * d:(h + 1) * wl.G * d]
    out = np.empty(wl.n_cand)
    for c in range(0, wl.n_cand, chunk):
        pos = np.arange(c, min(c + chunk, wl.n_cand))
        out[pos] = oracle.value_weight(v_h, w_h, wl.G, pos)[0]
    return out


def _check_two_stage_band(wl, host, idx0, offs0, stage0, heads):
    """Layer 0's two-stage selection against fp64 oracle keys ([CriticalKV,
    §3.3 Algorithm 1, steps 4-9]). Stage 1: the GPU's stage-1 picks are the
    top floor(alpha*k) fp64 pooled scores up to the score band. Stage 2: over
    the candidates the GPU's own stage 1 left, its stage-2 picks are the top
    k - k1 of the fp64 integrated score (pooled * score_norm + eps) * weight,
    up to the band of a product of two quantities within RTOL each.
    Uniform budgets: each listed head on its own; one budget per layer: the
    heads' candidates flattened (all heads listed)."""
    print(f"[host] oracle two-stage keys l0: heads {heads}", flush=True)
    _, ref_pool = oracle_scores_layer(wl, host[("q", 0)], host[("k", 0)])
    v64, w64 = synth.bf16_to_f64(host[("v", 0)]), synth.bf16_to_f64(host[("w_o", 0)])
    ref_w = {h: _ref_weights_head(v64, w64, wl, h) for h in heads}
    norm = 1.0 / (wl.W * wl.G)
    rtol2 = (1.0 + RTOL) ** 2 - 1.0

    def check(pool, weight, s1, s2, k, what):
        k1 = int(np.floor(wl.alpha * k))
        assert s1.size == k1 and s2.size == k - k1, what
        assert_topk_within_band(s1, pool, k1, f"{what} stage 1")
        rest = np.ones(pool.size, bool)
        rest[s1] = False
        cand = np.nonzero(rest)[0]
        assert np.isin(s2, cand).all(), f"{what}: a stage-2 pick was also picked in stage 1"
        key = (pool[cand] * norm + wl.eps) * weight[cand]
        assert_topk_within_band(np.searchsorted(cand, s2), key, k - k1, f"{what} stage 2", rtol=rtol2)

    def segment(h):
        if offs0 is None:
            return idx0[h], stage0[h]
        return idx0[offs0[h]:offs0[h + 1]], stage0[offs0[h]:offs0[h + 1]]

    if not wl.adaptive:
        for h in heads:
            row, st = segment(h)
            check(ref_pool[h], ref_w[h], row[st == 1], row[st == 2], wl.budget - wl.W, f"h{h}")
        return
    assert heads == list(range(wl.H_kv))
    s1, s2 = [], []
    for h in heads:
        row, st = segment(h)
        s1.append(h * wl.n_cand + row[st == 1])
        s2.append(h * wl.n_cand + row[st == 2])
    check(ref_pool.reshape(-1), np.concatenate([ref_w[h] for h in heads]), np.concatenate(s1),
          np.concatenate(s2), wl.budget - wl.H_kv * wl.W, "layer 0")


@functools.lru_cache(maxsize=None)
def _chunked_run():
    """GPU chunked scores and selection of the KVzip chunked workload, kept
    on the host for the per-head checks (layer 0 carries host data)."""
    wl = synth.WORKLOADS["kvzip_chunked_qwen7b_n32k"]
    dev, host = device_inputs(wl, {0}, ("q", "k", "kself"))
    print(f"[gpu] kvsel_score_chunked {wl.name}", flush=True)
    s, r = kv.kvsel_score_chunked(dev["q"], dev["k"], dev["kself"], G=wl.G, m=wl.chunk,
                                  n_prompt=wl.n_prompt, scale=wl.scale, pool=wl.pool,
                                  return_raw=True)
    idx, offs, stage = kv.kvsel_select(s, n=wl.n, W=0, budget=wl.budget, return_stage=True)
    torch.cuda.synchronize()
    _check_select_exact(wl, s, None, idx, offs, stage, [0, wl.L - 1])
    return wl, host, r[0].cpu().numpy(), s[0].cpu().numpy(), idx[0].cpu().numpy()


@pytest.mark.parametrize("h", [0, 1, 2, 3])
def test_kvzip_chunked_full(h):
    wl, host, r0, s0, idx0 = _chunked_run()
    # oracle on KV head h of layer 0: 16 chunks of 2080 x 7 query rows
    print(f"[host] oracle chunked scores l0 h{h}", flush=True)
    q = synth.bf16_to_f64(host[("q", 0)][:, h * wl.G:(h + 1) * wl.G])
    k = synth.bf16_to_f64(host[("k", 0)][h:h + 1])
    ks = synth.bf16_to_f64(host[("kself", 0)][:, h:h + 1])
    ref = oracle.chunked_scores(q, k, ks, wl.G, wl.scale, wl.chunk, wl.n_prompt)[0]
    assert_scores_close(r0[h][None], ref[None], "chunked raw")
    assert_scores_close(s0[h][None], ref[None], "chunked scores")
    assert_topk_within_band(idx0[h], ref, wl.budget, "chunked select")


@functools.lru_cache(maxsize=None)
def _many_query_run(name):
    """GPU scores and selection of a many-query KVzip workload, kept on the
    host for the per-head checks (first and last layer carry host data)."""
    wl = synth.WORKLOADS[name]
    last = wl.L - 1
    dev, host = device_inputs(wl, {0, last}, ("q", "k"))
    s, r = _score(wl, dev)
    idx, offs, stage = kv.kvsel_select(s, n=wl.n, W=0, budget=wl.budget, return_stage=True)
    torch.cuda.synchronize()
    _check_select_exact(wl, s, None, idx, offs, stage, [0, last])
    keep = (0, last)
    return (wl, host, {l: r[l].cpu().numpy() for l in keep}, {l: s[l].cpu().numpy() for l in keep},
            {l: idx[l].cpu().numpy() for l in keep})


@pytest.mark.parametrize("name", ["kvzip_qwen7b_n32k", "kvzip_logit_qwen7b_n32k"])
@pytest.mark.parametrize("layer,h", [(0, 0), (0, 1), (0, 2), (0, 3), (-1, 1)])
def test_kvzip_many_query_full(name, layer, h):
    wl, host, r, s, idx = _many_query_run(name)
    l = layer % wl.L
    logit = wl.agg == "logit"
    # oracle on KV head h of layer l (28672 query rows x 32768 keys)
    print(f"[host] oracle {wl.agg} scores l{l} h{h}", flush=True)
    q = synth.bf16_to_f64(host[("q", l)][h * wl.G:(h + 1) * wl.G])
    k = synth.bf16_to_f64(host[("k", l)][h:h + 1])
    if logit:
        ref = oracle.external_logit_scores(q, k, wl.G, wl.scale)[0]
        bound = logit_error_bound(q, k, wl.G, wl.scale)     # pool = 1: the same for both
        assert_logits_close(r[l][h][None], ref[None], bound, "kvzip raw")
        assert_logits_close(s[l][h][None], ref[None], bound, "kvzip scores")
    else:
        ref = oracle.external_raw_scores(q, k, wl.G, wl.scale, "max", q_chunk=512)[0]
        assert_scores_close(r[l][h][None], ref[None], "kvzip raw")
        assert_scores_close(s[l][h][None], ref[None], "kvzip scores")
    assert_topk_within_band(idx[l][h], ref, wl.budget, "kvzip select", logit)
