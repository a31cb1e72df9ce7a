"""kvsel_select_static (scratch in the library's static device array, no
workspace) against kvsel_select on the same inputs: the same bits, on two
calls in a row, the second with a smaller input that reuses the scratch
the first one left behind. Both calls take the many-workgroup path, the
one that needs scratch (histograms, per-segment state, chunk counts)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import eviction_importance_scoring_amd as kv

pytestmark = pytest.mark.gpu


def _scores(rng, L, H, n_cand, levels):
    return (rng.integers(0, levels, size=(L, H, n_cand)) / levels).astype(np.float32)


def _ws_bytes(L, H, n, W, budget, adaptive, two_stage):
    nb = ctypes.c_size_t(0)
    w = ctypes.c_void_p(16) if two_stage else None
    rc = kv.lib().kvsel_select(None, w, L, H, n, W, budget, int(adaptive), 1.0 / 128, 1e-4, 0.5,
                               None, None, None, None, ctypes.byref(nb), None)
    assert rc == 0
    return nb.value


CASES = [
    # (L, H, n, W, frac, adaptive, two_stage, levels)
    (2, 8, 40000, 32, 0.2, True, True, 50),      # large: adaptive two-stage, 8 heads a layer
    (1, 2, 36000, 16, 0.3, False, False, 7),     # smaller: per head, single stage
]


def test_select_static_matches_select_twice():
    rng = np.random.default_rng(2024)
    for case in CASES:
        L, H, n, W, frac, adaptive, two_stage, levels = case
        groups = H if adaptive else 1
        budget = int(np.floor(frac * groups * n))
        need = _ws_bytes(L, H, n, W, budget, adaptive, two_stage)
        assert 0 < need <= kv.kvsel_static_scratch_bytes(), (case, need)
        sc = torch.from_numpy(_scores(rng, L, H, n - W, levels)).cuda()
        wt = torch.from_numpy(rng.random((L, H, n - W)).astype(np.float32) + 0.01).cuda() \
            if two_stage else None
        kw = dict(n=n, W=W, budget=budget, adaptive=adaptive, weight=wt, score_norm=1.0 / 128,
                  eps=1e-4, alpha=0.5)
        print(f"[gpu] kvsel_select vs kvsel_select_static case={case} scratch={need}", flush=True)
        ri, ro, rs = kv.kvsel_select(sc, return_stage=True, **kw)
        gi, go, gs = kv.kvsel_select_static(sc, stage=torch.empty_like(rs), **kw)
        torch.cuda.synchronize()
        assert torch.equal(gi, ri), f"{case}: indices differ"
        assert torch.equal(gs, rs), f"{case}: stages differ"
        if adaptive:
            assert torch.equal(go, ro), f"{case}: head offsets differ"
