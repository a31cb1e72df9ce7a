"""Shared helpers for the parity tests: upload of generator output, and the
comparison rules between the HIP path and the oracle.

Score rule (fp32 accumulation from bf16 inputs against the fp64 oracle):
    |gpu - ref| <= RTOL * |ref| + ATOL_REL * max(ref of that head)
RTOL = 1e-3 is the relative error the scores must meet. The absolute floor
tau = ATOL_REL * max (1e-6 of the head's largest score) only covers entries
whose exact value is below fp32 resolution of that head's softmax terms,
e.g. keys whose every weight underflows.

Logit rule (KVzip-logit scores, any sign): |gpu - ref| <= 4 * gamma_{d+1} *
B_j, with B_j = scale * max over the head's query rows r of
sum_e |q_re k_je| and gamma_m = m u / (1 - m u), u = 2^-24. A logit is a sum
of d products of bf16 values (each exact in fp32) accumulated in fp32, then
scaled: in any summation order its error is within gamma_{d+1} times the sum
of the magnitudes of its terms (Higham, Accuracy and Stability of Numerical
Algorithms, 2nd ed., §3.1), and the max over rows of perturbed logits is
within the largest row error of the exact max. The factor 4 covers directed
rounding inside the matrix unit (2u per operation) and the fp32 rounding of
the scale; the oracle's own fp64 error is far below. Near-zero logits need
no floor: the bound scales with the terms, not with their (possibly
cancelling) sum.

Selection rule: let t be the oracle's k-th largest key of a segment and
A = {j : |key_j - t| <= RTOL * |t|}, the relative band alone. The GPU keeps
exactly as many entries as the oracle and the two sets agree outside A.
Guard: |t| > 100 * tau (tau as above; LOGIT_ATOL_REL * max |key| for
logits, a guard constant only), so the absolute floor of the score rule is at most 1 % of the
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


def logit_error_bound(q: np.ndarray, k: np.ndarray, G: int, scale: float, chunk: int = 512):
    """gamma_{d+1} * B_j per key (the logit rule above): q [H*G][T][d], k
    [H][n][d] (fp64 copies of the bf16 inputs). Returns [H][n]."""
    H, n, d = k.shape
    ak = np.abs(k)
    b = np.zeros((H, n))
    for h in range(H):
        for g in range(G):
            aq = np.abs(q[h * G + g])
            for r0 in range(0, aq.shape[0], chunk):
                b[h] = np.maximum(b[h], (aq[r0:r0 + chunk] @ ak[h].T).max(axis=0))
    m = d + 1
    u = 2.0 ** -24
    return m * u / (1 - m * u) * scale * b


def assert_logits_close(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray,
                        what: str = "logit scores"):
    """bound: logit_error_bound of the inputs (max-pooled like the scores
    when the scores are pooled)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape == bound.shape, (gpu.shape, ref.shape, bound.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bad = err > 4.0 * bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} entries outside the error bound, "
                           f"max err / bound {(err / (4.0 * bound)).max():.3g}")
    return float((err / bound).max())


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
