"""Python binding of libkvsel: prefill-end KV-cache importance scoring,
selection and compaction on MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/kvsel.h: each
function below checks tensor dtypes / shapes / devices (caller-supplied
outputs included), allocates missing outputs and the workspace with torch
on the inputs' device, and calls the C entry
point of the same name on the current torch stream. Every step of the
computation runs in the HIP kernels of libkvsel.so. There is no fallback:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "library_path", "KvselError", "kvsel_score", "kvsel_score_chunked", "kvsel_value_weight",
    "kvsel_value_l2_factor", "kvsel_value_weight_l2",
    "kvsel_select", "kvsel_select_pool", "kvsel_select_static", "kvsel_static_scratch_bytes", "kvsel_select_budgets", "kvsel_head_score", "kvsel_head_budgets",
    "kvsel_anchor_select", "kvsel_anchor_assign",
    "kvsel_compact", "kvsel_decode_attention", "kvsel_status_str",
    "kvsel_abi_version",
    "Q_WINDOW", "Q_EXTERNAL", "AGG_SUM", "AGG_MAX", "AGG_LOGIT_MAX",
    "GROUP_MEAN_OF_NORMS", "GROUP_NORM_OF_SUM",
]

Q_WINDOW, Q_EXTERNAL = 0, 1
AGG_SUM, AGG_MAX, AGG_LOGIT_MAX = 0, 1, 2
GROUP_MEAN_OF_NORMS, GROUP_NORM_OF_SUM = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libkvsel.so")

_c_void_p = ctypes.c_void_p
_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_f32 = ctypes.c_float
_c_size_p = ctypes.POINTER(ctypes.c_size_t)

_SIGNATURES = {
    "kvsel_score": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                    _c_i32, _c_i32, _c_f32, _c_i32, _c_void_p, _c_void_p, _c_void_p,
                    _c_size_p, _c_void_p],
    "kvsel_score_chunked": [_c_void_p, _c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32,
                            _c_i32, _c_i32, _c_i32, _c_f32, _c_i32, _c_void_p, _c_void_p,
                            _c_void_p, _c_size_p, _c_void_p],
    "kvsel_value_weight": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                           _c_i32, _c_i32, _c_i32, _c_void_p, _c_void_p, _c_size_p, _c_void_p],
    "kvsel_value_l2_factor": [_c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_void_p,
                              _c_void_p],
    "kvsel_value_weight_l2": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                              _c_i32, _c_void_p, _c_void_p],
    "kvsel_select": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                     _c_f32, _c_f32, _c_f32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                     _c_size_p, _c_void_p],
    "kvsel_select_pool": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                          _c_i32, _c_f32, _c_f32, _c_f32, _c_void_p, _c_void_p, _c_void_p,
                          _c_void_p, _c_void_p, _c_size_p, _c_void_p],
    "kvsel_select_budgets": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_void_p,
                             _c_i64, _c_f32, _c_f32, _c_f32, _c_void_p, _c_void_p, _c_void_p,
                             _c_void_p, _c_size_p, _c_void_p],
    "kvsel_head_score": [_c_void_p, _c_i32, _c_i32, _c_i32, _c_void_p, _c_void_p],
    "kvsel_head_budgets": [_c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_void_p,
                           _c_void_p, _c_size_p, _c_void_p],
    "kvsel_anchor_select": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                            _c_void_p, _c_void_p, _c_size_p, _c_void_p],
    "kvsel_anchor_assign": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                            _c_void_p, _c_void_p, _c_void_p, _c_size_p, _c_void_p],
    "kvsel_compact": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_void_p,
                      _c_void_p, _c_i64, _c_void_p, _c_void_p, _c_void_p],
    "kvsel_decode_attention": [_c_void_p, _c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32,
                               _c_i64, _c_void_p, _c_f32, _c_void_p, _c_void_p, _c_size_p,
                               _c_void_p],
    "kvsel_select_static": [_c_void_p, _c_void_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                            _c_f32, _c_f32, _c_f32, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "kvsel_status_str": [_c_i32],
    "kvsel_abi_version": [],
}

_LIB = None


class KvselError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded libkvsel.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise KvselError(f"{library_path} is missing: build it with __graft_entry__.build()")
        l = ctypes.CDLL(library_path)
        for name, args in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = _c_i32
        l.kvsel_status_str.restype = ctypes.c_char_p
        l.kvsel_static_scratch_bytes.argtypes = []
        l.kvsel_static_scratch_bytes.restype = ctypes.c_size_t
        _LIB = l
    return _LIB


def kvsel_status_str(status: int) -> str:
    return lib().kvsel_status_str(status).decode()


def kvsel_abi_version() -> int:
    return lib().kvsel_abi_version()


def _check(rc: int) -> None:
    if rc != 0:
        raise KvselError(kvsel_status_str(rc))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, dims=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")


def _out(t, dtype, name, shape, device):
    """A caller-supplied output is checked (dtype, device, contiguity and the
    exact shape the kernels write); None allocates one."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, dtype, name, len(shape), device)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
    return t


def _workspace(nbytes: int, device, workspace=None):
    """A caller-supplied workspace (any dtype, contiguous, on the device) or a
    new one. Returns (tensor, size in bytes)."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
            raise ValueError("workspace must be a GPU tensor")
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, expected {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        size = workspace.numel() * workspace.element_size()
        if size < nbytes:
            raise ValueError(f"workspace too small: {size} < {nbytes} bytes")
        return workspace, size
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


def kvsel_score(q, k, *, G: int, q_mode: int = Q_WINDOW, agg: int = AGG_SUM,
                scale: float | None = None, pool: int = 7, return_raw: bool = False,
                scores=None, raw=None, workspace=None, pooled: bool = True):
    """Pooled attention scores [L][H_kv][n_cand] (and raw [L][H_kv][n]).

    q bf16 [L][H_kv*G][W][d], k bf16 [L][H_kv][n][d]. pooled=False: raw
    scores only (returned as (None, raw)), for kvsel_select_pool."""
    _need(q, torch.bfloat16, "q", 4)
    _need(k, torch.bfloat16, "k", 4)
    L, Hq, W, d = q.shape
    L2, H, n, d2 = k.shape
    if L2 != L or d2 != d or Hq != H * G:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, G={G}")
    if scale is None:
        scale = 1.0 / d ** 0.5
    n_cand = n - W if q_mode == Q_WINDOW else n
    dev = q.device
    _need(k, torch.bfloat16, "k", 4, dev)
    if pooled:
        scores = _out(scores, torch.float32, "scores", (L, H, max(n_cand, 0)), dev)
    elif scores is not None:
        raise ValueError("pooled=False computes no pooled scores")
    if return_raw or raw is not None or not pooled:
        raw = _out(raw, torch.float32, "raw", (L, H, n), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_score
    args = (L, H, G, d, n, W, q_mode, agg, float(scale), pool)
    _check(f(None, None, *args, None, _ptr(raw), None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(q), _ptr(k), *args, _ptr(scores), _ptr(raw), _ptr(ws), ctypes.byref(nbytes),
             _stream(dev)))
    return scores, raw


def kvsel_score_chunked(q, k, k_self, *, G: int, m: int, n_prompt: int,
                        scale: float | None = None, pool: int = 1, return_raw: bool = False,
                        scores=None, raw=None, workspace=None):
    """KVzip chunked scores [L][H_kv][n] (and raw). q bf16 [L][T][H_kv*G][n_in][d],
    k bf16 [L][H_kv][n][d], k_self bf16 [L][T][H_kv][n_in][d], n_in = n_prompt + m."""
    _need(q, torch.bfloat16, "q", 5)
    _need(k, torch.bfloat16, "k", 4)
    _need(k_self, torch.bfloat16, "k_self", 5)
    L, H, n, d = k.shape
    me = min(m, n)
    T, n_in = (n + me - 1) // me, n_prompt + me
    if tuple(q.shape) != (L, T, H * G, n_in, d) or tuple(k_self.shape) != (L, T, H, n_in, d):
        raise ValueError(f"chunked shapes: q {tuple(q.shape)}, k_self {tuple(k_self.shape)}; "
                         f"expected {(L, T, H * G, n_in, d)} and {(L, T, H, n_in, d)}")
    if scale is None:
        scale = 1.0 / d ** 0.5
    dev = k.device
    _need(q, torch.bfloat16, "q", 5, dev)
    _need(k_self, torch.bfloat16, "k_self", 5, dev)
    scores = _out(scores, torch.float32, "scores", (L, H, n), dev)
    if return_raw or raw is not None:
        raw = _out(raw, torch.float32, "raw", (L, H, n), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_score_chunked
    args = (L, H, G, d, n, m, n_prompt, float(scale), pool)
    _check(f(None, None, None, *args, None, _ptr(raw), None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(q), _ptr(k), _ptr(k_self), *args, _ptr(scores), _ptr(raw), _ptr(ws),
             ctypes.byref(nbytes), _stream(dev)))
    return scores, raw


def kvsel_value_weight(v, w_o, *, G: int, n_cand: int | None = None,
                       group_mode: int = GROUP_MEAN_OF_NORMS, weight=None, workspace=None):
    """CriticalKV value weight [L][H_kv][n_cand]. v bf16 [L][H_kv][n][d],
    w_o bf16 [L][D][H_kv*G*d]. group_mode: GROUP_MEAN_OF_NORMS (mean over
    the group of each query head's L1 norm) or GROUP_NORM_OF_SUM (L1 norm of
    the group-summed projection)."""
    _need(v, torch.bfloat16, "v", 4)
    dev = v.device
    _need(w_o, torch.bfloat16, "w_o", 3, dev)
    L, H, n, d = v.shape
    if w_o.shape[0] != L or w_o.shape[2] != H * G * d:
        raise ValueError(f"shape mismatch: v {tuple(v.shape)}, w_o {tuple(w_o.shape)}, G={G}")
    D = w_o.shape[1]
    n_cand = n if n_cand is None else n_cand
    weight = _out(weight, torch.float32, "weight", (L, H, n_cand), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_value_weight
    args = (L, H, G, d, n, D, n_cand, int(group_mode))
    _check(f(None, None, *args, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(v), _ptr(w_o), *args, _ptr(weight), _ptr(ws), ctypes.byref(nbytes),
             _stream(dev)))
    return weight


def kvsel_value_l2_factor(w_o, *, G: int, H_kv: int, factor=None):
    """Per-(layer, query head) factor R (R^T R = W^T W) for the L2 value
    weight: bf16 [L][H_kv*G][2][d][d] (R_hi, R_lo). w_o bf16 [L][D][H_kv*G*d]."""
    _need(w_o, torch.bfloat16, "w_o", 3)
    L, D, cols = w_o.shape
    Hq = H_kv * G
    if cols % Hq:
        raise ValueError(f"w_o has {cols} input columns, not a multiple of H_kv*G={Hq}")
    d = cols // Hq
    factor = _out(factor, torch.bfloat16, "factor", (L, Hq, 2, d, d), w_o.device)
    _check(lib().kvsel_value_l2_factor(_ptr(w_o), L, H_kv, G, d, D, _ptr(factor),
                                       _stream(w_o.device)))
    return factor


def kvsel_value_weight_l2(v, factor, *, G: int, n_cand: int | None = None, weight=None):
    """L2 form of the CriticalKV value weight [L][H_kv][n_cand]. v bf16
    [L][H_kv][n][d], factor from kvsel_value_l2_factor."""
    _need(v, torch.bfloat16, "v", 4)
    _need(factor, torch.bfloat16, "factor", 5, v.device)
    L, H, n, d = v.shape
    if tuple(factor.shape) != (L, H * G, 2, d, d):
        raise ValueError(f"shape mismatch: v {tuple(v.shape)}, factor {tuple(factor.shape)}, G={G}")
    n_cand = n if n_cand is None else n_cand
    weight = _out(weight, torch.float32, "weight", (L, H, n_cand), v.device)
    _check(lib().kvsel_value_weight_l2(_ptr(v), _ptr(factor), L, H, G, d, n, n_cand,
                                       _ptr(weight), _stream(v.device)))
    return weight


def kvsel_select(scores, *, n: int, W: int, budget: int, adaptive: bool = False,
                 weight=None, score_norm: float = 1.0, eps: float = 1e-4,
                 alpha: float = 0.5, return_stage: bool = False, workspace=None):
    """Kept positions. scores f32 [L][H_kv][n-W]; returns (idx, head_offsets,
    stage): idx [L][H_kv][budget] (uniform) or [L][budget] with
    head_offsets [L][H_kv+1] (adaptive)."""
    _need(scores, torch.float32, "scores", 3)
    dev = scores.device
    if weight is not None:
        _need(weight, torch.float32, "weight", 3, dev)
        if weight.shape != scores.shape:
            raise ValueError("weight must match scores")
    L, H, n_cand = scores.shape
    if n_cand != n - W:
        raise ValueError(f"scores has {n_cand} candidates, expected n-W={n - W}")
    shape = (L, budget) if adaptive else (L, H, budget)
    idx = torch.empty(shape, dtype=torch.int32, device=dev)
    offs = torch.empty((L, H + 1), dtype=torch.int32, device=dev) if adaptive else None
    stage = torch.empty(shape, dtype=torch.uint8, device=dev) if return_stage else None
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_select
    args = (L, H, n, W, int(budget), int(adaptive), float(score_norm), float(eps), float(alpha))
    _check(f(None, _ptr(weight), *args, None, None, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(scores), _ptr(weight), *args, _ptr(idx), _ptr(offs), _ptr(stage), _ptr(ws),
             ctypes.byref(nbytes), _stream(dev)))
    return idx, offs, stage


def kvsel_select_pool(raw, *, n: int, W: int, budget: int, pool: int = 7, adaptive: bool = False,
                      weight=None, score_norm: float = 1.0, eps: float = 1e-4,
                      alpha: float = 0.5, return_stage: bool = False, return_pooled: bool = False,
                      workspace=None):
    """kvsel_select on raw [L][H_kv][n] scores max-pooled (width `pool`) by
    the call itself; returns (idx, head_offsets, stage, pooled)."""
    _need(raw, torch.float32, "raw", 3)
    dev = raw.device
    L, H, n_raw = raw.shape
    if n_raw != n:
        raise ValueError(f"raw has {n_raw} positions, expected n={n}")
    if weight is not None:
        _need(weight, torch.float32, "weight", 3, dev)
        if tuple(weight.shape) != (L, H, n - W):
            raise ValueError("weight must be [L][H_kv][n-W]")
    shape = (L, budget) if adaptive else (L, H, budget)
    idx = torch.empty(shape, dtype=torch.int32, device=dev)
    offs = torch.empty((L, H + 1), dtype=torch.int32, device=dev) if adaptive else None
    stage = torch.empty(shape, dtype=torch.uint8, device=dev) if return_stage else None
    pooled = torch.empty((L, H, n - W), dtype=torch.float32, device=dev) if return_pooled else None
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_select_pool
    args = (int(pool), L, H, n, W, int(budget), int(adaptive), float(score_norm), float(eps),
            float(alpha))
    _check(f(None, _ptr(weight), *args, None, None, None, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(raw), _ptr(weight), *args, _ptr(idx), _ptr(offs), _ptr(stage), _ptr(pooled),
             _ptr(ws), ctypes.byref(nbytes), _stream(dev)))
    return idx, offs, stage, pooled


def kvsel_select_static(scores, *, n: int, W: int, budget: int, adaptive: bool = False,
                        weight=None, score_norm: float = 1.0, eps: float = 1e-4,
                        alpha: float = 0.5, idx=None, head_offsets=None, stage=None):
    """kvsel_select through the entry point that takes its scratch from the
    library's static device array (no workspace). Outputs as kvsel_select;
    caller-supplied idx / head_offsets / stage are checked and written."""
    _need(scores, torch.float32, "scores", 3)
    dev = scores.device
    if weight is not None:
        _need(weight, torch.float32, "weight", 3, dev)
        if weight.shape != scores.shape:
            raise ValueError("weight must match scores")
    L, H, n_cand = scores.shape
    if n_cand != n - W:
        raise ValueError(f"scores has {n_cand} candidates, expected n-W={n - W}")
    shape = (L, budget) if adaptive else (L, H, budget)
    idx = _out(idx, torch.int32, "idx", shape, dev)
    offs = _out(head_offsets, torch.int32, "head_offsets", (L, H + 1), dev) if adaptive else None
    if stage is not None:
        stage = _out(stage, torch.uint8, "stage", shape, dev)
    args = (L, H, n, W, int(budget), int(adaptive), float(score_norm), float(eps), float(alpha))
    _check(lib().kvsel_select_static(_ptr(scores), _ptr(weight), *args, _ptr(idx), _ptr(offs),
                                     _ptr(stage), _stream(dev)))
    return idx, offs, stage


def kvsel_static_scratch_bytes() -> int:
    return int(lib().kvsel_static_scratch_bytes())


def kvsel_select_budgets(scores, budgets, *, n: int, W: int, layer_stride: int | None = None,
                         weight=None, score_norm: float = 1.0, eps: float = 1e-4,
                         alpha: float = 0.5, return_stage: bool = False, workspace=None):
    """Kept positions under a per-head budget vector. scores f32 [L][H_kv][n-W];
    budgets i32 [L][H_kv] on the device. Returns (idx [L][layer_stride],
    head_offsets [L][H_kv+1], stage). layer_stride defaults to the largest
    per-layer sum of the budgets clamped into [W, n] (read back from the
    device: a synchronising copy; pass it to avoid that)."""
    _need(scores, torch.float32, "scores", 3)
    _need(budgets, torch.int32, "budgets", 2, scores.device)
    if weight is not None:
        _need(weight, torch.float32, "weight", 3, scores.device)
        if weight.shape != scores.shape:
            raise ValueError("weight must match scores")
    L, H, n_cand = scores.shape
    if n_cand != n - W:
        raise ValueError(f"scores has {n_cand} candidates, expected n-W={n - W}")
    if tuple(budgets.shape) != (L, H):
        raise ValueError(f"budgets must be {(L, H)}, got {tuple(budgets.shape)}")
    if layer_stride is None:
        layer_stride = int(budgets.clamp(W, n).sum(dim=1).max().item())
    dev = scores.device
    idx = torch.empty((L, layer_stride), dtype=torch.int32, device=dev)
    offs = torch.empty((L, H + 1), dtype=torch.int32, device=dev)
    stage = torch.empty((L, layer_stride), dtype=torch.uint8, device=dev) if return_stage else None
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_select_budgets
    args = (L, H, n, W)
    tail = (float(score_norm), float(eps), float(alpha))
    _check(f(None, _ptr(weight), *args, None, int(layer_stride), *tail, None, None, None, None,
             ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(scores), _ptr(weight), *args, _ptr(budgets), int(layer_stride), *tail, _ptr(idx),
             _ptr(offs), _ptr(stage), _ptr(ws), ctypes.byref(nbytes), _stream(dev)))
    return idx, offs, stage


def kvsel_head_score(scores, *, out=None):
    """Head scores [L][H_kv]: max over positions of scores f32 [L][H_kv][n_pos]."""
    _need(scores, torch.float32, "scores", 3)
    L, H, n_pos = scores.shape
    out = _out(out, torch.float32, "out", (L, H), scores.device)
    _check(lib().kvsel_head_score(_ptr(scores), L, H, n_pos, _ptr(out), _stream(scores.device)))
    return out


def kvsel_head_budgets(head_score, *, keep: int, n: int, W: int, out=None, workspace=None):
    """Budgets i32 [L][H_kv] of head-level eviction: n for the `keep` heads
    with the largest head score, W for the others."""
    _need(head_score, torch.float32, "head_score", 2)
    L, H = head_score.shape
    dev = head_score.device
    out = _out(out, torch.int32, "out", (L, H), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_head_budgets
    _check(f(None, L, H, int(keep), n, W, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(head_score), L, H, int(keep), n, W, _ptr(out), _ptr(ws), ctypes.byref(nbytes),
             _stream(dev)))
    return out


def kvsel_anchor_select(scores, rand, *, n: int, W: int, k: int, rho: float = 0.7,
                        out=None, workspace=None):
    """AnchorKV anchor positions i32 [L][H_kv][k] (ascending). scores, rand
    f32 [L][H_kv][n-W]."""
    _need(scores, torch.float32, "scores", 3)
    dev = scores.device
    _need(rand, torch.float32, "rand", 3, dev)
    if rand.shape != scores.shape:
        raise ValueError("rand must match scores")
    L, H, n_cand = scores.shape
    if n_cand != n - W:
        raise ValueError(f"scores has {n_cand} candidates, expected n-W={n - W}")
    out = _out(out, torch.int32, "out", (L, H, k), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_anchor_select
    args = (L, H, n, W, int(k), float(rho))
    _check(f(None, None, *args, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(scores), _ptr(rand), *args, _ptr(out), _ptr(ws), ctypes.byref(nbytes),
             _stream(dev)))
    return out


def kvsel_anchor_assign(x, anchors, *, slot=None, gamma=None, workspace=None):
    """Nearest-anchor slot i32 and gamma f32 [L][H_kv][n] of x bf16
    [L][H_kv][n][d] for anchors i32 [L][H_kv][k]."""
    _need(x, torch.bfloat16, "x", 4)
    dev = x.device
    _need(anchors, torch.int32, "anchors", 3, dev)
    L, H, n, d = x.shape
    if anchors.shape[:2] != (L, H):
        raise ValueError(f"anchors must be [L][H_kv][k], got {tuple(anchors.shape)}")
    k = anchors.shape[2]
    slot = _out(slot, torch.int32, "slot", (L, H, n), dev)
    gamma = _out(gamma, torch.float32, "gamma", (L, H, n), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_anchor_assign
    _check(f(None, None, L, H, d, n, k, None, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(x), _ptr(anchors), L, H, d, n, k, _ptr(slot), _ptr(gamma), _ptr(ws),
             ctypes.byref(nbytes), _stream(dev)))
    return slot, gamma


def kvsel_compact(k, v, idx, head_offsets=None, k_out=None, v_out=None):
    """Gather kept rows: returns (k_out, v_out) bf16 [L][kept_per_layer][d]
    (allocated unless given)."""
    _need(k, torch.bfloat16, "k", 4)
    dev = k.device
    _need(v, torch.bfloat16, "v", 4, dev)
    _need(idx, torch.int32, "idx", None, dev)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    L, H, n, d = k.shape
    if idx.dim() < 2 or idx.shape[0] != L:
        raise ValueError("idx must have a leading L axis")
    kept = idx[0].numel()
    if head_offsets is not None:
        _need(head_offsets, torch.int32, "head_offsets", 2, dev)
        if tuple(head_offsets.shape) != (L, H + 1):
            raise ValueError(f"head_offsets must be {(L, H + 1)}, got {tuple(head_offsets.shape)}")
    elif idx.dim() != 3 or idx.shape[1] != H:
        raise ValueError(f"without head_offsets idx must be [L][H_kv][B], got {tuple(idx.shape)}")
    k_out = _out(k_out, torch.bfloat16, "k_out", (L, kept, d), dev)
    v_out = _out(v_out, torch.bfloat16, "v_out", (L, kept, d), dev)
    _check(lib().kvsel_compact(_ptr(k), _ptr(v), L, H, d, n, _ptr(idx), _ptr(head_offsets),
                               kept, _ptr(k_out), _ptr(v_out), _stream(k.device)))
    return k_out, v_out


def kvsel_decode_attention(q, k_kept, v_kept, *, G: int, scale: float | None = None,
                           head_offsets=None, out=None, workspace=None):
    """One decoding step over the kept rows. q bf16 [L][H_kv*G][d];
    k_kept, v_kept bf16 [L][kept_per_layer][d] (kvsel_compact's output);
    head_offsets i32 [L][H_kv+1] or None (uniform heads). Returns out f32
    [L][H_kv*G][d]."""
    _need(q, torch.bfloat16, "q", 3)
    _need(k_kept, torch.bfloat16, "k_kept", 3, q.device)
    _need(v_kept, torch.bfloat16, "v_kept", 3, q.device)
    if k_kept.shape != v_kept.shape:
        raise ValueError("k_kept and v_kept must have the same shape")
    L, Hq, d = q.shape
    if Hq % G != 0:
        raise ValueError("q must hold H_kv*G query heads")
    H = Hq // G
    if k_kept.shape[0] != L or k_kept.shape[2] != d:
        raise ValueError("k_kept must be [L][kept][d]")
    kept = k_kept.shape[1]
    if head_offsets is not None:
        _need(head_offsets, torch.int32, "head_offsets", 2, q.device)
        if tuple(head_offsets.shape) != (L, H + 1):
            raise ValueError("head_offsets must be [L][H_kv+1]")
    if scale is None:
        scale = 1.0 / d ** 0.5
    dev = q.device
    out = _out(out, torch.float32, "out", (L, Hq, d), dev)
    nbytes = ctypes.c_size_t(0)
    f = lib().kvsel_decode_attention
    args = (L, H, G, d, int(kept), _ptr(head_offsets), float(scale))
    _check(f(None, None, None, *args, None, None, ctypes.byref(nbytes), None))
    ws, wsb = _workspace(nbytes.value, dev, workspace)
    nbytes = ctypes.c_size_t(wsb)
    _check(f(_ptr(q), _ptr(k_kept), _ptr(v_kept), *args, _ptr(out), _ptr(ws), ctypes.byref(nbytes),
             _stream(dev)))
    return out
