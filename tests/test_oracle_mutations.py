"""Plant plausible mistakes in copies of the oracle and require the pins to
catch every one of them. CPU only; the real oracle is never modified."""
import importlib.util
import os
import sys

import pytest

from oracle_pins import ALL_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "__init__.py")

MUTANTS = {
    "causal_off_by_one": ("pos = n - W + np.arange(W)", "pos = n - W - 1 + np.arange(W)"),
    "causal_off_by_one_late": ("pos = n - W + np.arange(W)", "pos = n - W + 1 + np.minimum(np.arange(W), W - 2)"),
    "non_causal": ("logits = np.where(visible, logits, -np.inf)", "logits = logits"),
    "no_scale": ("logits = scale * (q[h * G + g] @ k[h].T)", "logits = (q[h * G + g] @ k[h].T)"),
    "gqa_interleaved": ("logits = scale * (q[h * G + g] @ k[h].T)", "logits = scale * (q[g * H + h] @ k[h].T)"),
    "softmax_wrong_axis": ("m = logits.max(axis=1, keepdims=True)\n    e = np.exp(logits - m)\n    return e / e.sum(axis=1, keepdims=True)",
                           "m = logits.max(axis=0, keepdims=True)\n    e = np.exp(logits - m)\n    return e / e.sum(axis=0, keepdims=True)"),
    "mean_instead_of_sum": ("raw[h] += p.sum(axis=0)\n            else:", "raw[h] += p.mean(axis=0)\n            else:"),
    "external_sum_for_max": ("                if agg == \"max\":", "                if agg == \"sum\":"),
    "external_causal": ("p = _softmax_rows(scale * (q[h * G + g, c0:c0 + q_chunk] @ k[h].T))",
                        "p = _softmax_rows(np.where(np.tri(min(q_chunk, Qs - c0), n, n - min(q_chunk, Qs - c0), bool), scale * (q[h * G + g, c0:c0 + q_chunk] @ k[h].T), -np.inf))"),
    "pool_radius": ("r = pool // 2\n", "r = max(pool // 2 - 1, 0)\n"),
    "pool_one_sided": ("out[..., :n_cand - off] = np.maximum(out[..., :n_cand - off], src[..., off:])", "pass"),
    "pool_over_all_n": ("src = raw[..., :n_cand]\n    out = src.copy()", "src = raw\n    out = src.copy()[..., :n_cand]"),
    "weight_no_abs": ("out[h] += np.abs(proj).sum(axis=1)", "out[h] += proj.sum(axis=1)"),
    "weight_l2": ("out[h] += np.abs(proj).sum(axis=1)", "out[h] += np.sqrt((proj ** 2).sum(axis=1))"),
    "weight_no_mean": ("            out[h] += np.abs(proj).sum(axis=1)\n        out[h] /= G",
                       "            out[h] += np.abs(proj).sum(axis=1)\n        out[h] /= 1"),
    "weight_wrong_slice": ("w_slice = w_o[:, hq * d:(hq + 1) * d]", "w_slice = w_o[:, h * d:(h + 1) * d]"),
    "ties_to_higher_index": ("order = np.lexsort((np.arange(key.shape[0]), -key))", "order = np.lexsort((-np.arange(key.shape[0]), -key))"),
    "k1_ceil": ("k1 = int(np.floor(alpha * k))", "k1 = int(np.ceil(alpha * k))"),
    "no_eps_f64": ("(np.asarray(score, np.float64) * score_norm + eps)", "(np.asarray(score, np.float64) * score_norm)"),
    "no_eps_f32": ("        t = t + np.float32(eps)\n", "        t = t + np.float32(0.0)\n"),
    "no_norm_f32": ("        t = s * np.float32(score_norm)\n", "        t = s * np.float32(1.0)\n"),
    "f32_reassociated": ("        t = t + np.float32(eps)\n        return t * np.asarray(weight, np.float32)",
                         "        wf = np.asarray(weight, np.float32)\n        return t * wf + np.float32(eps) * wf"),
    "f32_fused_add": ("        t = s * np.float32(score_norm)\n        t = t + np.float32(eps)\n",
                      "        t = np.float32(np.asarray(score, np.float64) * np.float32(score_norm) + np.float64(np.float32(eps)))\n"),
    "grpsum_mean_of_norms": ("        proj = v[h, positions] @ w_sum.T              # [m][D]\n        out[h] = np.abs(proj).sum(axis=1)",
                             "        proj = v[h, positions] @ w_sum.T              # [m][D]\n        out[h] = np.abs(proj).sum(axis=1) / G"),
    "grpsum_abs_inside": ("            w_sum += w_o[:, hq * d:(hq + 1) * d]      # [D][d]",
                          "            w_sum += np.abs(w_o[:, hq * d:(hq + 1) * d])      # [D][d]"),
    "grpsum_first_slice_only": ("            w_sum += w_o[:, hq * d:(hq + 1) * d]      # [D][d]",
                                "            w_sum += w_o[:, h * G * d:(h * G + 1) * d]      # [D][d]"),
    "grpsum_wrong_head": ("        proj = v[h, positions] @ w_sum.T              # [m][D]",
                          "        proj = v[0, positions] @ w_sum.T              # [m][D]"),
    "stage2_from_all": ("cand = np.nonzero(rest)[0]", "cand = np.arange(score.shape[0])"),
    "adaptive_transposed": ("flat = scores.reshape(-1)", "flat = scores.T.reshape(-1)"),
    "window_not_counted": ("        k = budget - W\n        assert 0 <= k <= n_cand", "        k = max(budget - 2 * W, 0)\n        assert 0 <= k <= n_cand"),
    "decode_no_scale": ("p = _softmax_rows(scale * (q[h * G + g] @ kh.T)[None, :])[0]",
                        "p = _softmax_rows((q[h * G + g] @ kh.T)[None, :])[0]"),
    "decode_gqa_interleaved": ("p = _softmax_rows(scale * (q[h * G + g] @ kh.T)[None, :])[0]",
                               "p = _softmax_rows(scale * (q[g * len(heads) + h] @ kh.T)[None, :])[0]"),
    "decode_values_from_keys": ("out[h * G + g] = p @ vh", "out[h * G + g] = p @ kh"),
    "decode_offsets_shifted": ("heads = [(k_kept[head_offsets[h]:head_offsets[h + 1]], v_kept[head_offsets[h]:head_offsets[h + 1]])",
                               "heads = [(k_kept[head_offsets[h]:head_offsets[h + 1]], v_kept[head_offsets[h] + 1:head_offsets[h + 1] + 1])"),
    "decode_uniform_weights": ("out[h * G + g] = p @ vh", "out[h * G + g] = vh.mean(axis=0)"),
    "l2_no_sqrt": ("out[h] += np.sqrt((proj * proj).sum(axis=1))", "out[h] += (proj * proj).sum(axis=1)"),
    "l2_is_l1": ("out[h] += np.sqrt((proj * proj).sum(axis=1))", "out[h] += np.abs(proj).sum(axis=1) * 1.0"),
    "l2_no_mean": ("            out[h] += np.sqrt((proj * proj).sum(axis=1))\n        out[h] /= G",
                   "            out[h] += np.sqrt((proj * proj).sum(axis=1))\n        out[h] /= 1"),
    "l2_wrong_slice": ("proj = vh @ w_o[:, hq * d:(hq + 1) * d].T      # [m][D]", "proj = vh @ w_o[:, h * d:(h + 1) * d].T      # [m][D]"),
    "budgets_no_clamp": ("b = np.clip(np.asarray(budgets, np.int64), W, n)", "b = np.asarray(budgets, np.int64)"),
    "budgets_window_not_counted": ("        k = int(b[h]) - W\n", "        k = max(int(b[h]) - 2 * W, 0)\n"),
    "budgets_head_shifted": ("        k = int(b[h]) - W\n", "        k = int(b[(h + 1) % H]) - W\n"),
    "budgets_offsets_no_window": ("offs.append(offs[-1] + k + W)", "offs.append(offs[-1] + k)"),
    "logit_softmax": ("lg = scale * (q[h * G + g] @ k[h].T)    # [Q_s][n] logits",
                      "lg = _softmax_rows(scale * (q[h * G + g] @ k[h].T))    # [Q_s][n] logits"),
    "logit_no_scale": ("lg = scale * (q[h * G + g] @ k[h].T)    # [Q_s][n] logits", "lg = (q[h * G + g] @ k[h].T)    # [Q_s][n] logits"),
    "logit_floor_zero": ("out = np.full((H, n), -np.inf)", "out = np.zeros((H, n))"),
    "head_scores_mean": ("    return scores.max(axis=-1)", "    return scores.mean(axis=-1)"),
    "head_budgets_ties_high": ("    top = topk_indices(flat, keep)", "    top = len(flat) - 1 - topk_indices(flat[::-1], keep)"),
    "head_budgets_drop_all": ("    b = np.full(flat.shape, W, np.int64)", "    b = np.full(flat.shape, 0, np.int64)"),
    "chunked_self_not_causal": ("hidden[:, mt:] = np.triu(np.ones((nin, nin), bool), 1)", "hidden[:, mt:] = False"),
    "chunked_self_excluded": ("hidden[:, mt:] = np.triu(np.ones((nin, nin), bool), 1)", "hidden[:, mt:] = True"),
    "chunked_padding_rows": ("        nin = n_prompt + mt\n", "        nin = n_prompt + m\n"),
    "chunked_offset": ("        c0 = t * m\n", "        c0 = min(t * m + 1, n - 1)\n"),
    "chunked_no_scale": ("logits = scale * (q[t, h * G + g, :nin] @ keys.T)", "logits = (q[t, h * G + g, :nin] @ keys.T)"),
    "anchor_rho_of_k": ("    k1 = int(np.floor(rho * (k - W)))\n    out = np.empty((H, k), np.int64)",
                        "    k1 = min(int(np.floor(rho * k)), k - W)\n    out = np.empty((H, k), np.int64)"),
    "anchor_no_window": ("out[h] = np.sort(np.concatenate([by_score, drawn, np.arange(n - W, n)]))",
                         "out[h] = np.sort(np.concatenate([by_score, drawn, np.arange(n - W - 1, n - 1)]))"),
    "anchor_random_from_all": ("drawn = rest[topk_indices(rand[h][rest], k - W - k1)]",
                               "drawn = rest[topk_indices(rand[h][:len(rest)], k - W - k1)]"),
    "assign_dot_not_cos": ("cos = dots / (nx[:, None] * na[None, :])", "cos = dots / (nx[:, None] * 1.0)"),
    "assign_gamma_unnormed": ("gamma[h] = dots[np.arange(n), best] / np.where(na[best] > 0, na[best] ** 2, 1.0)",
                              "gamma[h] = dots[np.arange(n), best] / np.where(na[best] > 0, na[best], 1.0)"),
    "assign_ties_high": ("best = np.argmax(cos, axis=1)                         # first of equal maxima",
                         "best = k - 1 - np.argmax(cos[:, ::-1], axis=1)     # first of equal maxima"),
    "compact_wrong_head": ("return (np.stack([k[h, idx[h]] for h in range(H)]),", "return (np.stack([k[0, idx[h]] for h in range(H)]),"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} must occur exactly once"
    mod_name = f"oracle_mutant_{name}"
    spec = importlib.util.spec_from_loader(mod_name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), f"<{mod_name}>", "exec"), mod.__dict__)
    sys.modules.pop(mod_name, None)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _load_mutant(name, *MUTANTS[name])
    failed = []
    for check in ALL_CHECKS:
        try:
            check(mod)
        except Exception:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
