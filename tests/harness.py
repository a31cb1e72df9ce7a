"""Shared helpers for the parity tests: upload of generator output, and the
comparison rules between the HIP path and the oracle.

Score rule (fp32 accumulation from bf16 inputs against the fp64 oracle):
    |gpu - ref| <= RTOL * |ref| + ATOL_REL * max(ref of that head)
RTOL = 1e-3 is the relative error the scores must meet. The absolute floor
tau = ATOL_REL * max (1e-6 of the head's largest score) only covers entries
whose exact value is below fp32 resolution of that head's softmax terms,
e.g. keys whose every weight underflows.

Logit rule (KVzip-logit scores, any sign): |gpu - ref| <= RTOL * |ref| +
LOGIT_ATOL_REL * max |ref| of that head. A logit is an fp32 sum of 128
exact bf16 products: its absolute error scales with the terms, not with
the (possibly cancelling) sum, so near-zero logits get the floor.

Selection rule: let t be the oracle's k-th largest key of a segment and
A = {j : |key_j - t| <= RTOL * |t|}, the relative band alone. The GPU keeps
exactly as many entries as the oracle and the two sets agree outside A.
Guard: |t| > 100 * tau (tau as above, LOGIT_ATOL_REL * max |key| for
logits), so the absolute floor of the score rule is at most 1 % of the
band at the selection boundary and never decides which side of it an
entry falls on; a segment that fails the guard fails the check.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

RTOL = 1e-3
ATOL_REL = 1e-6
LOGIT_ATOL_REL = 1e-4


def to_dev(u16: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> torch.bfloat16 on the device."""
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, what: str = "scores"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    floor = ATOL_REL * ref.max(axis=-1, keepdims=True)
    err = np.abs(gpu - ref)
    bad = err > RTOL * np.abs(ref) + floor
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} entries outside tolerance; first at {tuple(i)}: "
            f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r} rel={err[tuple(i)] / max(abs(ref[tuple(i)]), 1e-300):.3e}")
    return float((err / np.maximum(np.abs(ref), 1e-30)).max())


def _band(key: np.ndarray, k: int, logit: bool = False, what: str = "", rtol: float = RTOL):
    """Oracle's k-th key t and the relative tolerance band around it (a
    boolean mask). Asserts the guard |t| > 100 * tau."""
    if k == 0 or k == key.size:
        return None, np.zeros(key.shape, bool)
    order = np.lexsort((np.arange(key.size), -key))
    t = key[order[k - 1]]
    tau = LOGIT_ATOL_REL * np.abs(key).max() if logit else ATOL_REL * key.max()
    assert abs(t) > 100 * tau, (f"{what}: k-th key {t!r} is within 100x the absolute score floor "
                                f"{tau!r}; the selection band would depend on it")
    return t, np.abs(key - t) <= rtol * abs(t)


def assert_logits_close(gpu: np.ndarray, ref: np.ndarray, what: str = "logit scores"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    tol = RTOL * np.abs(ref) + LOGIT_ATOL_REL * np.abs(ref).max(axis=-1, keepdims=True)
    bad = np.abs(gpu - ref) > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} entries outside tolerance, "
                           f"max err {np.abs(gpu - ref).max():.3g}")


def assert_topk_within_band(gpu_pick, ref_key: np.ndarray, k: int, what: str, logit: bool = False,
                            rtol: float = RTOL):
    """gpu_pick: candidate indices the GPU kept (any order). rtol: the
    relative error the GPU's keys may carry (RTOL for a score; a product of
    two quantities each within RTOL, such as CriticalKV's integrated score,
    carries (1 + RTOL)^2 - 1)."""
    gpu_pick = np.asarray(gpu_pick)
    assert gpu_pick.size == k, f"{what}: kept {gpu_pick.size}, expected {k}"
    assert np.unique(gpu_pick).size == k, f"{what}: duplicate indices"
    ref_pick = oracle.topk_indices(ref_key, k)
    t, band = _band(ref_key, k, logit, what, rtol)
    g = np.zeros(ref_key.size, bool)
    g[gpu_pick] = True
    r = np.zeros(ref_key.size, bool)
    r[ref_pick] = True
    diff = (g != r) & ~band
    assert not diff.any(), (f"{what}: {diff.sum()} selections differ outside the tolerance band "
                            f"(k-th key {t!r}); first index {np.argmax(diff)}")
    return int(((g != r) & band).sum())


def split_heads(idx, offs, H, W, n):
    """Per-head kept candidate positions and window check from select output."""
    out = []
    for h in range(H):
        if offs is None:
            row = np.asarray(idx[h])
        else:
            row = np.asarray(idx[offs[h]:offs[h + 1]])
        assert (np.diff(row) > 0).all(), "indices must ascend"
        assert list(row[len(row) - W:]) == list(range(n - W, n)), "window must be kept last"
        out.append(row[:len(row) - W])
    return out


def gen(wl: synth.Workload, seed: int = 0, which=("q", "k", "v", "w_o")):
    return synth.gen_all(wl, seed, which)


def oracle_scores_layer(wl: synth.Workload, q_u16, k_u16):
    """Oracle raw [H][n] and pooled [H][n_cand] for one layer."""
    q = synth.bf16_to_f64(q_u16)
    k = synth.bf16_to_f64(k_u16)
    if wl.q_mode == "window":
        raw = oracle.window_raw_scores(q, k, wl.G, wl.scale, wl.agg)
    elif wl.agg == "logit":
        raw = oracle.external_logit_scores(q, k, wl.G, wl.scale)
    else:
        raw = oracle.external_raw_scores(q, k, wl.G, wl.scale, wl.agg)
    return raw, oracle.maxpool(raw, wl.n_cand, wl.pool)
