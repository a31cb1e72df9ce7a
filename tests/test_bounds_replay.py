"""Every global read and write of the selection, compaction, decoding and
AnchorKV kernels stays inside the buffers the library was given, for arbitrary
contents of the integer buffers those kernels trust (index lists, head
offsets, budget vectors, the many-workgroup select's segment states and
chunk counts). The kernels' index arithmetic is replayed on the host
(bounds_replay.py); no GPU is used."""
from __future__ import annotations

import numpy as np
import pytest

import bounds_replay as br

I32_MIN, I32_MAX = -(1 << 31), (1 << 31) - 1


def _arbitrary_i32(rng, size, n):
    """Random int32 values mixed with the edge values an unwritten or
    corrupted buffer may hold."""
    edge = np.array([I32_MIN, I32_MIN + 1, -n, -1, 0, 1, n - 1, n, n + 1, I32_MAX - 1, I32_MAX],
                    np.int64)
    x = rng.integers(I32_MIN, I32_MAX, size=size, endpoint=True)
    pick = rng.random(size) < 0.5
    x[pick] = rng.choice(edge, size=int(pick.sum()))
    small = rng.random(size) < 0.3
    x[small] = rng.integers(-2, n + 3, size=int(small.sum()))
    return x.astype(np.int64)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("ragged", [False, True])
def test_compact_stays_in_bounds(seed, ragged):
    rng = np.random.default_rng(seed)
    L, H = 2, int(rng.integers(1, 9))
    n = int(rng.integers(1, 3000))
    vecs = int(rng.choice([16, 8, 9]))            # d = 128, 64, 72
    kept = int(rng.integers(1, 4 * H * n // 3 + 2))
    if not ragged:
        kept = max(H, kept // H * H)
    kept = min(kept, H * n)
    idx = _arbitrary_i32(rng, L * kept, n)
    offs = _arbitrary_i32(rng, L * (H + 1), kept) if ragged else None
    acc = br.compact_accesses(L, H, n, vecs, kept, idx, offs)
    acc.check(br.compact_sizes(L, H, n, vecs, kept, offs))


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("ragged", [False, True])
def test_decode_stays_in_bounds(seed, ragged):
    rng = np.random.default_rng(100 + seed)
    L, H, G = 2, int(rng.choice([1, 3, 8, 65])), int(rng.integers(1, 9))
    kept = int(rng.integers(1, 5000))
    if not ragged:
        kept = max(H, kept // H * H)
    offs = None
    if ragged:
        mode = seed % 4
        if mode == 0:      # arbitrary
            offs = _arbitrary_i32(rng, L * (H + 1), kept)
        elif mode == 1:    # decreasing
            offs = np.sort(rng.integers(-10, kept + 10, size=L * (H + 1)))[::-1].copy()
        elif mode == 2:    # valid
            cuts = np.sort(rng.integers(0, kept + 1, size=(L, H - 1)), axis=1)
            offs = np.concatenate([np.zeros((L, 1), np.int64), cuts, np.full((L, 1), kept)], 1).ravel()
        else:              # all heads empty but one huge
            offs = np.zeros(L * (H + 1), np.int64)
            offs[H] = I32_MAX
    acc = br.decode_accesses(L, H, G, kept, offs)
    acc.check(br.decode_sizes(L, H, G, kept, offs))


def _valid_uniform_plan(rng, adaptive, two_stage, long_segments):
    L = 2
    H = int(rng.integers(1, 9))
    n = int(rng.integers(br.K_CHUNK * 2, 40000)) if long_segments else int(rng.integers(2, 3000))
    W = int(rng.integers(0, min(n, 300)))
    groups = H if adaptive else 1
    budget = int(rng.integers(groups * W, groups * n + 1))
    return br.select_plan(L, H, n, W, budget=budget, adaptive=adaptive, two_stage=two_stage)


def _budget_plan(rng, two_stage, long_segments):
    L, H = 2, int(rng.integers(1, 9))
    n = int(rng.integers(br.K_CHUNK * 2, 40000)) if long_segments else int(rng.integers(2, 3000))
    W = int(rng.integers(0, min(n, 300)))
    stride = int(rng.integers(1, H * n + 1))
    budgets = _arbitrary_i32(rng, L * H, n)
    return br.select_plan(L, H, n, W, two_stage=two_stage, budgets=budgets, stride=stride), budgets


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("variant", ["uniform", "adaptive", "two_stage", "budgets"])
def test_select_resident_stays_in_bounds(seed, variant):
    rng = np.random.default_rng(200 + seed)
    if variant == "budgets":
        p, budgets = _budget_plan(rng, two_stage=bool(seed % 2), long_segments=False)
    else:
        p = _valid_uniform_plan(rng, variant == "adaptive", variant == "two_stage", False)
        budgets = None
    acc = br.select_resident_accesses(p, budgets)
    acc.check(br.select_sizes(p))


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("variant", ["uniform", "adaptive", "two_stage", "budgets"])
def test_select_many_workgroups_stays_in_bounds(seed, variant):
    rng = np.random.default_rng(300 + seed)
    if variant == "budgets":
        p, budgets = _budget_plan(rng, two_stage=bool(seed % 2), long_segments=True)
    else:
        p = _valid_uniform_plan(rng, variant == "adaptive", variant == "two_stage", True)
        budgets = None
    S, C = p["segments"], p["chunks"]
    # arbitrary segment states, chunk counts and list entries (uint32 fields)
    states = [dict(shift=int(rng.integers(I32_MIN, I32_MAX)), need=int(rng.integers(0, 1 << 32)),
                   done=int(rng.integers(0, 2)), count=int(rng.integers(0, 1 << 32)))
              for _ in range(S)]
    for st in states[: S // 2]:       # and some near the values a select leaves
        st["shift"] = int(rng.choice([63, 52, 41, 31, 20, 9, 0]))
        st["need"] = int(rng.integers(0, p["seg_len"] + 2))
        st["count"] = int(rng.integers(0, br.K_LIST_CAP + 2))
    ccount = [rng.integers(0, 1 << 32, size=C, dtype=np.int64) for _ in range(S)]
    for cc in ccount[: S // 2]:
        cc[:] = rng.integers(0, br.K_CHUNK + 1, size=C)
    lists = [rng.integers(0, 1 << 32, size=br.K_LIST_CAP, dtype=np.int64) for _ in range(S)]
    for ls in lists[: S // 2]:
        ls[:] = rng.integers(0, p["seg_len"] + 2, size=br.K_LIST_CAP)
    acc = br.msel_accesses(p, states, ccount, rng, budgets, lists)
    acc.check(br.select_sizes(p))


def test_replay_sees_an_unguarded_access():
    """The checker fails a replay whose access leaves its buffer (here: the
    compaction's source row without its pos < n guard)."""
    acc = br.Accesses()
    n, vecs = 10, 16
    pos = np.array([0, 5, n])              # n: one past the head
    acc.add("kv", pos * vecs)
    with pytest.raises(AssertionError):
        acc.check({"kv": n * vecs})


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("adaptive", [False, True])
def test_select_pool_first_pass_stays_in_bounds(seed, adaptive):
    rng = np.random.default_rng(500 + seed + 10 * adaptive)
    p = _valid_uniform_plan(rng, adaptive, bool(seed % 2), True)
    acc = br.msel_pool_accesses(p, p["n"])
    acc.check({"raw": p["L"] * p["H"] * p["n"], "pooled": p["segments"] * p["seg_len"]})


@pytest.mark.parametrize("seed", range(6))
def test_anchor_assign_stays_in_bounds(seed):
    """Arbitrary anchor positions (outside the head, negative, repeated) and
    every slot a packed score can decode to stay inside the buffers and the
    kernels' LDS tables, for anchor counts on both sides of the resident
    kernel's limit."""
    rng = np.random.default_rng(seed)
    L, H = 1, int(rng.integers(1, 4))
    n = int(rng.integers(1, 3000))
    k = int(rng.choice([1, 7, 64, 200, 256, 257, 400, min(2048, n)]))
    k = max(1, min(k, n))
    anchors = _arbitrary_i32(rng, L * H * k, n)
    acc, sizes = br.anchor_accesses(L, H, n, k, anchors)
    acc.check(sizes)
