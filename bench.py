#!/usr/bin/env python3
"""Throughput of the prefill-end KV-cache scoring -> selection -> compaction
path on one MI355X.

One step = the whole hot path over one synthetic cache, all layers at once:
kvsel_score (window attention scores + max-pool), kvsel_value_weight (only
for the value-weighted workload), kvsel_select and kvsel_compact. Inputs are
seeded synthetic bf16 tensors from `synth`, resident in HBM before timing.

Prints ONE JSON line. `value` = KV entries (KV head x cached token) scored,
selected and compacted per second over the whole step, which equals the
per-layer rate (n*H_kv per layer / time per layer). `roofline` is for the
dominant kernel (the scoring call), timed with HIP events on the stream it
runs on, over the timed steps. `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
METRIC = "KV entries scored+selected/sec per layer at n=32K; % of HBM roofline"
SCORE_SOURCES = ["score_dispatch.hip", "score_window.hip", "score_twopass.hip", "kvsel_internal.h",
                 "kvsel_ring.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "eviction_importance_scoring_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(key, sha):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(key)
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, host, seconds, w_host=None, budgets=None, rand=None):
    """The oracle (fp64 numpy) on the same inputs, timed twice: with one BLAS
    thread, then with the BLAS thread pool as configured for this process
    (OMP_NUM_THREADS, the host's CPU share). Reported in KV entries per
    second, the all-thread rate as the value."""
    from threadpoolctl import threadpool_limits
    usable = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=1):
        one = _cpu_baseline_run(wl, host, seconds / 2, w_host, budgets, rand)
    allt = _cpu_baseline_run(wl, host, seconds, w_host, budgets, rand)
    allt["value_1thread"] = one["value"]
    allt["sample_1thread"] = one["sample"]
    allt["cpu_model"] = cpu_model()
    allt["logical_cpus_usable"] = usable
    allt["logical_cpus_host"] = os.cpu_count()
    return allt


def _cpu_baseline_run(wl, host, seconds, w_host=None, budgets=None, rand=None):
    """The oracle (fp64 numpy) on the same inputs, one (layer, KV head) at a
    time in order, until `seconds` of CPU work: attention scores, max-pool,
    the value weight when the workload uses it, and top-k selection.
    Reported in KV entries per second; `cores` = the BLAS threads in use."""
    import numpy as np

    import oracle
    import synth
    from threadpoolctl import threadpool_info
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    units = 0
    head_rows = []
    pairs = [(l, h) for l in range(min(wl.L, host["q"].shape[0])) for h in range(wl.H_kv)]
    t0 = time.perf_counter()
    # the sample's pairs in order, repeated until `seconds` of CPU work
    while time.perf_counter() - t0 < seconds:
        l, h = pairs[units % len(pairs)]
        q = None if wl.chunk else synth.bf16_to_f64(host["q"][l][h * wl.G:(h + 1) * wl.G])
        k = synth.bf16_to_f64(host["k"][l][h:h + 1])
        if wl.chunk:
            qc = synth.bf16_to_f64(host["q"][l][:, h * wl.G:(h + 1) * wl.G])
            ks = synth.bf16_to_f64(host["kself"][l][:, h:h + 1])
            raw = oracle.chunked_scores(qc, k, ks, wl.G, wl.scale, wl.chunk, wl.n_prompt)
        elif wl.q_mode == "window":
            raw = oracle.window_raw_scores(q, k, wl.G, wl.scale, wl.agg)
        else:
            raw = (oracle.external_logit_scores(q, k, wl.G, wl.scale) if wl.agg == "logit"
                   else oracle.external_raw_scores(q, k, wl.G, wl.scale, wl.agg))
        pooled = oracle.maxpool(raw, wl.n_cand, wl.pool)
        if wl.anchor_k:        # AnchorKV's anchor stage for this head
            anchors = oracle.anchor_select(pooled, rand[l, h:h + 1], wl.n, wl.W_kept, wl.anchor_k,
                                           wl.rho)
            oracle.anchor_assign(k, anchors)
            oracle.anchor_assign(synth.bf16_to_f64(host["v"][l][h:h + 1]), anchors)
            units += 1
            continue
        if wl.head_keep > 0:   # selected below, once the sample's head scores are known
            head_rows.append(pooled)
            units += 1
            continue
        weight = None
        if wl.value_weight and w_host is not None:
            v = synth.bf16_to_f64(host["v"][l][h:h + 1])
            wo = synth.bf16_to_f64(w_host[l][:, h * wl.G * wl.d:(h + 1) * wl.G * wl.d])
            norm = oracle.value_weight_l2 if wl.value_norm == "l2" else oracle.value_weight
            weight = norm(v, wo, wl.G, np.arange(wl.n_cand))
        if budgets is not None:
            oracle.select_budgets(pooled, budgets[l, h:h + 1], wl.W_kept, wl.n, weight=weight,
                                  alpha=wl.alpha, score_norm=1.0 / (wl.W * wl.G), eps=wl.eps)
        else:
            oracle.select_layer(pooled, wl.budget if not wl.adaptive else wl.budget // wl.H_kv,
                                wl.W_kept, wl.n, weight=weight, alpha=wl.alpha,
                                score_norm=1.0 / (wl.W * wl.G), eps=wl.eps)
        units += 1
    if head_rows:
        # head-level eviction over the sample's heads: head score, keep the
        # same fraction whole, select each head under its budget
        hs = oracle.head_scores(np.concatenate(head_rows))[None]
        b = oracle.head_budgets(hs, int(round(wl.head_keep * hs.size)), wl.n, wl.W_kept)
        for i, row in enumerate(head_rows):
            oracle.select_budgets(row, b[0, i:i + 1], wl.W_kept, wl.n)
    dt = time.perf_counter() - t0
    what = ("scores, max-pool" + (", value weight" if wl.value_weight else "")
            + (", head scores and head budgets" if head_rows else "")
            + (", anchor selection and key/value assignment" if wl.anchor_k else " and top-k selection"))
    return {"value": units * wl.n / dt, "unit": "entries/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} (layer, KV head) pairs of {wl.name} in order from layer 0"
                      f"{' (the sample repeated)' if units > len(pairs) else ''}: "
                      f"{what} in fp64 numpy ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_n32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not overwrite a 1 GiB buffer between timed steps")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw the inputs on the GPU (default for caches above 4 GB)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the scoring path shards "
                                   "by layer / KV head with no communication, and this build "
                                   "runs and reports a single GPU",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import eviction_importance_scoring_amd as kv
    import synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # a plain copy of known size: reads and writes exactly 1 GiB each
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 3}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    which = ("q", "k", "v", "w_o") if wl.value_weight else ("q", "k", "v")
    if wl.chunk:
        which = which + ("kself",)
    input_bytes = sum(wl.L * int(np.prod(wl.shape(name))) * 2 for name in which
                      if name != "w_o" or wl.value_weight)
    t0 = time.time()
    if args.device_inputs or input_bytes > (4 << 30):
        log(f"[bench] drawing {wl.name} on the GPU (seed {args.seed})")
        t = synth.gen_all_device(wl, args.seed, which, dev)
        host = None
    else:
        log(f"[bench] generating {wl.name} on the host (seed {args.seed})")
        host = synth.gen_all(wl, args.seed, which)
        t = {name: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
             for name, a in host.items()}
    torch.cuda.synchronize(dev)
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    q, k, v = t["q"], t["k"], t["v"]
    w_o = t.get("w_o")
    mode = kv.Q_WINDOW if wl.q_mode == "window" else kv.Q_EXTERNAL
    agg = {"sum": kv.AGG_SUM, "max": kv.AGG_MAX, "logit": kv.AGG_LOGIT_MAX}[wl.agg]
    W_kept = wl.W_kept
    scores = torch.empty((wl.L, wl.H_kv, wl.n_cand), dtype=torch.float32, device=dev)
    weight = (torch.empty((wl.L, wl.H_kv, wl.n_cand), dtype=torch.float32, device=dev)
              if wl.value_weight else None)
    ws_s = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    l2 = wl.value_weight and wl.value_norm == "l2"
    factor, ms_factor = None, None
    if l2:
        # the L2 norm's per-query-head factor depends on the model weights
        # only: computed once, outside the timed steps (timed on its own)
        factor = kv.kvsel_value_l2_factor(w_o, G=wl.G, H_kv=wl.H_kv)
        torch.cuda.synchronize(dev)
        f0, f1 = ev(), ev()
        f0.record()
        kv.kvsel_value_l2_factor(w_o, G=wl.G, H_kv=wl.H_kv, factor=factor)
        f1.record()
        torch.cuda.synchronize(dev)
        ms_factor = f0.elapsed_time(f1)

    budgets, b_host, stride = None, None, None
    if wl.budget_vector:
        b_host = synth.gen_budgets(wl, args.seed)
        budgets = torch.from_numpy(b_host).to(dev)
        stride = int(np.clip(b_host, W_kept, wl.n).astype(np.int64).sum(axis=1).max())
    keep = 0
    if wl.head_keep > 0:
        # head-level eviction: the budgets come from the head scores inside
        # the step; a layer holds at most min(H, keep) whole heads
        keep = int(round(wl.head_keep * wl.L * wl.H_kv))
        full = min(wl.H_kv, keep)
        stride = full * wl.n + (wl.H_kv - full) * W_kept
        head_sc = torch.empty((wl.L, wl.H_kv), dtype=torch.float32, device=dev)
        budgets = torch.empty((wl.L, wl.H_kv), dtype=torch.int32, device=dev)

    # Where the selection reads every head's raw scores itself (kvsel_select_pool),
    # the scoring call writes raw scores only and the selection max-pools
    # them on chip; the head-level, budget-vector, anchor and chunked steps
    # read pooled scores from the scoring call.
    pool_in_select = not (wl.chunk or wl.budget_vector or wl.head_keep > 0 or wl.anchor_k)
    raw = torch.empty((wl.L, wl.H_kv, wl.n), dtype=torch.float32, device=dev) if pool_in_select else None

    def score():
        if wl.chunk:
            kv.kvsel_score_chunked(q, k, t["kself"], G=wl.G, m=wl.chunk, n_prompt=wl.n_prompt,
                                   scale=wl.scale, pool=wl.pool, scores=scores)
        elif pool_in_select:
            kv.kvsel_score(q, k, G=wl.G, q_mode=mode, agg=agg, scale=wl.scale, pool=wl.pool,
                           raw=raw, pooled=False)
        else:
            kv.kvsel_score(q, k, G=wl.G, q_mode=mode, agg=agg, scale=wl.scale, pool=wl.pool,
                           scores=scores)

    if wl.anchor_k:
        rand = torch.from_numpy(synth.gen_rand(wl, args.seed)).to(dev)
        anchors = torch.empty((wl.L, wl.H_kv, wl.anchor_k), dtype=torch.int32, device=dev)
        a_slot = [torch.empty((wl.L, wl.H_kv, wl.n), dtype=torch.int32, device=dev) for _ in range(2)]
        a_gamma = [torch.empty((wl.L, wl.H_kv, wl.n), dtype=torch.float32, device=dev) for _ in range(2)]

    def anchor_step(marks=None):
        # AnchorKV's anchor stage: score, anchors, keys and values assigned
        if marks is not None:
            marks[0].record()
        score()
        if marks is not None:
            marks[1].record()
        kv.kvsel_anchor_select(scores, rand, n=wl.n, W=W_kept, k=wl.anchor_k, rho=wl.rho,
                               out=anchors)
        if marks is not None:
            marks[2].record()
        kv.kvsel_anchor_assign(k, anchors, slot=a_slot[0], gamma=a_gamma[0])
        if marks is not None:
            marks[3].record()
        kv.kvsel_anchor_assign(v, anchors, slot=a_slot[1], gamma=a_gamma[1])
        if marks is not None:
            marks[4].record()
        return None, None

    def step(marks=None):
        if wl.anchor_k:
            return anchor_step(marks)
        if marks is not None:
            marks[0].record()
        score()
        if marks is not None:
            marks[1].record()
        if keep:
            kv.kvsel_head_score(scores, out=head_sc)
            kv.kvsel_head_budgets(head_sc, keep=keep, n=wl.n, W=W_kept, out=budgets)
        if l2:
            kv.kvsel_value_weight_l2(v, factor, G=wl.G, n_cand=wl.n_cand, weight=weight)
        elif weight is not None:
            kv.kvsel_value_weight(v, w_o, G=wl.G, n_cand=wl.n_cand, weight=weight)
        if marks is not None:
            marks[2].record()
        if budgets is not None:
            idx, offs, _ = kv.kvsel_select_budgets(scores, budgets, n=wl.n, W=W_kept,
                                                   layer_stride=stride, weight=weight,
                                                   score_norm=1.0 / (wl.W * wl.G), eps=wl.eps,
                                                   alpha=wl.alpha)
        elif pool_in_select:
            idx, offs, _, _ = kv.kvsel_select_pool(raw, n=wl.n, W=W_kept, budget=wl.budget,
                                                   pool=wl.pool, adaptive=wl.adaptive,
                                                   weight=weight, score_norm=1.0 / (wl.W * wl.G),
                                                   eps=wl.eps, alpha=wl.alpha)
        else:
            idx, offs, _ = kv.kvsel_select(scores, n=wl.n, W=W_kept, budget=wl.budget,
                                           adaptive=wl.adaptive, weight=weight,
                                           score_norm=1.0 / (wl.W * wl.G), eps=wl.eps,
                                           alpha=wl.alpha)
        if marks is not None:
            marks[3].record()
        kept = kv.kvsel_compact(k, v, idx, offs)
        if marks is not None:
            marks[4].record()
        return kept, offs

    # Between timed steps a 1 GiB buffer is overwritten, so no step finds its
    # inputs in the 256 MB memory-side cache (the small workloads' K would
    # fit there); each step is timed on its own with events, the overwrite
    # outside them.
    flush_buf = None if args.no_flush else torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        if flush_buf is not None:
            flush_buf.fill_(1.0)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize(dev)
    marks = [[ev() for _ in range(5)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    start, end = ev(), ev()
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        flush()
        kept_kv, kept_offs = step(marks[s])
    end.record()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    per_step = [m[0].elapsed_time(m[4]) for m in marks]
    ms_step = float(np.mean(per_step))
    span = lambda a, b: [m[a].elapsed_time(m[b]) for m in marks]
    part = lambda a, b: float(np.mean(span(a, b)))
    ms_score, ms_vw, ms_sel, ms_cmp = part(0, 1), part(1, 2), part(2, 3), part(3, 4)
    stats = lambda xs: {"mean": float(np.mean(xs)), "median": float(np.median(xs)),
                        "min": float(np.min(xs))}

    entries = wl.L * wl.H_kv * wl.n
    # algorithmic bytes of one scoring call: K read once, Q read once,
    # pooled scores (or, when the selection pools, raw scores) written once
    score_bytes = (wl.L * wl.H_kv * wl.n * wl.d * 2 + wl.L * wl.H_q * wl.W * wl.d * 2
                   + wl.L * wl.H_kv * (wl.n if pool_in_select else wl.n_cand) * 4)
    if wl.chunk:   # every chunk's queries and own keys
        score_bytes = (wl.L * wl.H_kv * wl.n * wl.d * 2 + wl.L * wl.T * (wl.H_q + wl.H_kv) * wl.n_in * wl.d * 2
                       + wl.L * wl.H_kv * wl.n_cand * 4)
    achieved = score_bytes / (ms_score * 1e-3) / 1e9
    sha = source_sha(SCORE_SOURCES)
    traffic = traffic_from_profiles(f"kvsel_score:{wl.name}", sha)
    out = {
        "metric": METRIC,
        "value": entries / (ms_step * 1e-3),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "L": wl.L, "H_kv": wl.H_kv, "G": wl.G, "d": wl.d,
                   "n": wl.n, "W": wl.W, "q_mode": wl.q_mode, "agg": wl.agg, "pool": wl.pool,
                   "pooling": "kvsel_select_pool" if pool_in_select else "kvsel_score",
                   "budget": wl.budget, "adaptive": wl.adaptive,
                   **({"chunk": wl.chunk, "n_prompt": wl.n_prompt} if wl.chunk else {}),
                   **({"budget_vector": True, "layer_stride": stride} if wl.budget_vector else {}),
                   **({"head_keep": wl.head_keep, "heads_kept": keep, "layer_stride": stride}
                      if keep else {}),
                   "value_weight": wl.value_weight,
                   **({"value_norm": wl.value_norm} if wl.value_weight else {}),
                   "seed": args.seed,
                   **({"anchor_k": wl.anchor_k, "rho": wl.rho} if wl.anchor_k else {}),
                   "step": ("score+anchor_select+anchor_assign(K)+anchor_assign(V)" if wl.anchor_k
                            else "score+head_score+head_budgets+select_budgets+compact" if keep
                            else "score+select_budgets+compact" if wl.budget_vector
                            else "score+value_weight+select+compact" if wl.value_weight
                            else "score+select+compact")},
        "roofline": None,   # the dominant call's, set below
        "per_call_ms": ({"score": ms_score, "anchor_select": ms_vw, "anchor_assign_k": ms_sel,
                         "anchor_assign_v": ms_cmp} if wl.anchor_k else
                        {"score": ms_score, **({"value_weight": ms_vw} if wl.value_weight else {}),
                         **({"head_score+head_budgets": ms_vw} if keep else {}),
                         "select": ms_sel, "compact": ms_cmp}),
        "per_call_ms_stats": ({
            "step": stats(per_step), "score": stats(span(0, 1)),
            "anchor_select": stats(span(1, 2)), "anchor_assign_k": stats(span(2, 3)),
            "anchor_assign_v": stats(span(3, 4))} if wl.anchor_k else {
            "step": stats(per_step), "score": stats(span(0, 1)),
            **({"value_weight": stats(span(1, 2))} if wl.value_weight else {}),
            **({"head_score+head_budgets": stats(span(1, 2))} if keep else {}),
            "select": stats(span(2, 3)), "compact": stats(span(3, 4))}),
        "scored_selected_entries_per_s": entries / ((ms_score + ms_sel) * 1e-3),
        "score_source_sha": sha,   # the scoring kernels' sources (SCORE_SOURCES) this line ran on
        "wall_s_timed": wall,
        "timing": ("each step between HIP events on the stream it runs on; a 1 GiB buffer "
                   "overwritten before every step, outside its events" if flush_buf is not None
                   else "each step between HIP events on the stream it runs on; no cache flush"),
        "ms_per_step_incl_flush": start.elapsed_time(end) / args.steps,
    }
    # rooflines of the calls: the window score is HBM-bound (algorithmic bytes:
    # K read once, Q read once, pooled scores written once); the many-query
    # score (two passes of Q K^T) and the value weight are MFMA contractions
    score_hbm = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                 "kernel": "kvsel_score", "bytes_per_launch": score_bytes,
                 "ms_per_launch": ms_score, "source_sha": sha}
    calls = []
    # two passes of Q K^T (R = G*W rows per KV head against n keys; one for
    # the softmax-free logit max); the call is MFMA-bound when those flops
    # take longer at peak than its bytes
    passes = 1 if wl.agg == "logit" else 2
    sc_flops = passes * 2.0 * wl.L * wl.H_q * wl.W * wl.n * wl.d
    if wl.chunk:
        # per (layer, chunk, KV head): pass 1 over the chunk's m cached keys
        # and the n_in own keys, pass 2 over the m cached keys (own keys as
        # whole tiles, the MFMA work issued)
        sc_flops = 2.0 * wl.L * wl.T * wl.H_q * wl.n_in * wl.d * (2 * wl.chunk + wl.n_in)
    if sc_flops / (MFMA_BF16_PEAK_TFS * 1e12) > score_bytes / (HBM_PEAK_GBS * 1e9):
        tfs = sc_flops / (ms_score * 1e-3) / 1e12
        calls.append((ms_score, {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS,
                                 "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFS, "traffic": None,
                                 "kernel": "kvsel_score", "flops_per_launch": sc_flops,
                                 "ms_per_launch": ms_score}))
        out["score_hbm"] = score_hbm
    else:
        calls.append((ms_score, score_hbm))
    if wl.value_weight and not l2:
        vw_flops = 2.0 * wl.L * wl.H_kv * wl.n_cand * wl.G * wl.D * wl.d
        tfs = vw_flops / (ms_vw * 1e-3) / 1e12
        calls.append((ms_vw, {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS,
                              "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFS, "traffic": None,
                              "kernel": "kvsel_value_weight", "flops_per_launch": vw_flops,
                              "ms_per_launch": ms_vw}))
    elif l2:
        # R v with R upper triangular (d(d+1)/2 products per key and query
        # head), once for R_hi and once for R_lo
        vw_flops = 2.0 * 2.0 * wl.L * wl.H_kv * wl.n_cand * wl.G * (wl.d * (wl.d + 1) // 2)
        tfs = vw_flops / (ms_vw * 1e-3) / 1e12
        calls.append((ms_vw, {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS,
                              "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFS, "traffic": None,
                              "kernel": "kvsel_value_weight_l2", "flops_per_launch": vw_flops,
                              "ms_per_launch": ms_vw,
                              "factor_ms_once": ms_factor}))
    calls.sort(key=lambda c: -c[0])
    out["roofline"] = calls[0][1]
    if len(calls) > 1:
        out["other_rooflines"] = [c[1] for c in calls[1:]]
    # the next step after eviction: one decoding step over the kept rows of
    # every layer (not part of `value`), on the last step's compacted cache
    if wl.anchor_k:
        # assignment: each vector read once (256 B) and its slot and gamma
        # written (8 B); 2 * kpad * d MFMA flops per vector
        kpad = (wl.anchor_k + 63) // 64 * 64
        a_bytes = wl.L * wl.H_kv * wl.n * (wl.d * 2 + 8)
        a_flops = 2.0 * wl.L * wl.H_kv * wl.n * kpad * wl.d
        a_ms = (ms_sel + ms_cmp) / 2
        out["anchor_assign"] = {
            "bound": "hbm", "ms_per_call": a_ms, "bytes_per_launch": a_bytes,
            "achieved": a_bytes / (a_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a_bytes / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_tflops": a_flops / (a_ms * 1e-3) / 1e12}
    if wl.G <= 8 and kept_kv is not None:
        gq = torch.Generator(device=dev)
        gq.manual_seed(args.seed + 7)
        q_dec = torch.randn((wl.L, wl.H_q, wl.d), generator=gq, device=dev).to(torch.bfloat16)
        ko, vo = kept_kv
        out_dec = torch.empty((wl.L, wl.H_q, wl.d), dtype=torch.float32, device=dev)
        dec = lambda: kv.kvsel_decode_attention(q_dec, ko, vo, G=wl.G, scale=wl.scale,
                                                head_offsets=kept_offs, out=out_dec)
        for _ in range(3):
            dec()
        torch.cuda.synchronize(dev)
        d0, d1 = ev(), ev()
        reps = 10
        d0.record()
        for _ in range(reps):
            dec()
        d1.record()
        torch.cuda.synchronize(dev)
        ms_dec = d0.elapsed_time(d1) / reps
        # kept rows actually read: the packed rows before each layer's last
        # head offset (a budget-vector row may end before its stride)
        rows = (int(kept_offs[:, -1].sum().item()) if kept_offs is not None
                else ko.shape[0] * ko.shape[1])
        dec_bytes = 2 * rows * wl.d * 2 + q_dec.numel() * 2 + out_dec.numel() * 4
        out["next_rows"] = {"decode_attention": {
            "bound": "hbm", "ms_per_call": ms_dec, "bytes_per_launch": dec_bytes,
            "achieved": dec_bytes / (ms_dec * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dec_bytes / (ms_dec * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kept_rows": rows}}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        if host is None:   # bring back the first layers, which the sample uses
            nl = min(wl.L, 2)
            host = {name: t[name][:nl].cpu().view(torch.int16).numpy().view(np.uint16)
                    for name in t if name != "w_o"}
        w_host = None
        if wl.value_weight:
            w_host = t["w_o"][:2].cpu().view(torch.int16).numpy().view(np.uint16)
        out["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_seconds, w_host, b_host,
                                           synth.gen_rand(wl, args.seed) if wl.anchor_k else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
