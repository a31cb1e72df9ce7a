"""Seeded synthetic KV caches for the prefill-end scoring / selection path.

This module only draws random numbers and shapes them: Gaussian draws, the
heavy-hitter key scaling that gives attention its power-law skew, and
round-to-nearest-even conversion to bf16. It holds no step of the scoring
or selection method, so both the HIP path (tests, bench) and the CPU oracle
can take their inputs from here without sharing any of the method's code.

Layouts (all bf16 stored as uint16 bit patterns):
  q    [H_kv*G][W][d]   query head hq = h*G + g serves KV head h
  k, v [H_kv][n][d]
  w_o  [D][H_kv*G*d]    output projection, torch Linear layout (out, in)

Every tensor of every layer has its own stream:
SeedSequence([seed, workload_code, tensor_code, layer]), so one layer can be
regenerated alone (the oracle checks sampled layers of big workloads).
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

# ----------------------------------------------------------------- bf16 ----

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return bf16_to_f32(b).astype(np.float64)


# ------------------------------------------------------------ workloads ----

@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic scoring workload.

    q_mode 'window': the W scoring queries are the cache's own last W tokens
    (causal, the window is always kept); 'external': W scoring queries that
    sit outside the cache and see all n keys.
    heavy: 'uniform1pct' scales floor(0.01*n) distinct prefix keys by 4;
    'zipf' scales the key of rank r (random order) by 1 + 3 r^-1.1.
    """
    name: str
    L: int
    H_kv: int
    G: int
    d: int
    n: int
    W: int
    q_mode: str = "window"
    agg: str = "sum"             # 'sum', 'max' (softmax weights) or 'logit' (raw logits, external)
    pool: int = 7
    beta: float = 0.2            # kept fraction (window included)
    adaptive: bool = False       # one budget per layer shared by all heads
    budget_vector: bool = False  # one budget per (layer, head), from gen_budgets
    head_keep: float = 0.0       # > 0: head-level eviction keeping this fraction of heads
    anchor_k: int = 0            # > 0: AnchorKV anchor stage with this many anchors per head
    rho: float = 0.7             # AnchorKV: share of the non-window anchors taken by score
    chunk: int = 0               # > 0: KVzip chunked scoring, cached keys per chunk
    n_prompt: int = 0            # chunked scoring: repeat-prompt tokens before each chunk
    value_weight: bool = False   # value-norm weighted two-stage selection
    value_norm: str = "l1"       # norm of the projected value: 'l1' or 'l2'
    D: int = 0                   # model width for w_o
    alpha: float = 0.5
    eps: float = 1e-4
    q_chunk: int = 0
    heavy: str = "zipf"
    compact: bool = True

    @property
    def H_q(self) -> int:
        return self.H_kv * self.G

    @property
    def T(self) -> int:
        """Chunks per layer (chunked scoring)."""
        return (self.n + self.chunk - 1) // self.chunk if self.chunk else 1

    @property
    def n_in(self) -> int:
        """Input tokens per chunk (chunked scoring)."""
        return self.n_prompt + min(self.chunk, self.n)

    def shape(self, tensor: str) -> tuple:
        """Per-layer shape of an input tensor."""
        if tensor == "q":
            if self.chunk:
                return (self.T, self.H_q, self.n_in, self.d)
            return (self.H_q, self.W, self.d)
        if tensor == "kself":
            return (self.T, self.H_kv, self.n_in, self.d)
        if tensor in ("k", "v"):
            return (self.H_kv, self.n, self.d)
        if tensor == "w_o":
            return (self.D, self.H_q * self.d)
        raise ValueError(tensor)

    @property
    def n_cand(self) -> int:
        return self.n - self.W if self.q_mode == "window" else self.n

    @property
    def W_kept(self) -> int:
        return self.W if self.q_mode == "window" else 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def budget(self) -> int:
        """Kept entries incl. the window: per head, or per layer if adaptive."""
        if self.adaptive:
            return int(np.floor(self.beta * self.H_kv * self.n))
        return int(np.floor(self.beta * self.n))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        # one layer, n = 4K, uniform 1% heavy hitters, 20% per head
        Workload("snapkv_L1_n4k", L=1, H_kv=8, G=4, d=128, n=4096, W=32,
                 pool=7, beta=0.20, heavy="uniform1pct"),
        # Llama-3.1-8B-shaped cache, n = 32K, 40% per head (headline)
        Workload("llama8b_n32k", L=32, H_kv=8, G=4, d=128, n=32768, W=32,
                 pool=7, beta=0.40),
        # same shape, head-adaptive: one budget per layer, n = 64K, 20%
        Workload("adakv_llama8b_n64k", L=32, H_kv=8, G=4, d=128, n=65536,
                 W=32, pool=7, beta=0.20, adaptive=True),
        # value-norm weighted two-stage selection, n = 128K, 10%
        Workload("criticalkv_llama8b_n128k", L=32, H_kv=8, G=4, d=128,
                 n=131072, W=32, pool=7, beta=0.10, value_weight=True,
                 D=4096),
        # the same with the L2 norm of the projected value
        Workload("criticalkv_l2_llama8b_n128k", L=32, H_kv=8, G=4, d=128,
                 n=131072, W=32, pool=7, beta=0.10, value_weight=True,
                 value_norm="l2", D=4096),
        # CriticalAdaKV: value-norm weighted two-stage selection over one
        # budget per layer (the flattened candidates of its heads), n = 32K, 20%
        Workload("criticaladakv_llama8b_n32k", L=32, H_kv=8, G=4, d=128, n=32768,
                 W=32, pool=7, beta=0.20, adaptive=True, value_weight=True, D=4096),
        # per-(layer, head) budgets averaging 20% (a HeadKV-style offline
        # allocation), n = 32K
        Workload("headkv_llama8b_n32k", L=32, H_kv=8, G=4, d=128, n=32768, W=32,
                 pool=7, beta=0.20, budget_vector=True),
        # head-level eviction: head score = max over positions of the window
        # score, half of all heads kept whole, the others their window
        Workload("headlevel_llama8b_n32k", L=32, H_kv=8, G=4, d=128, n=32768, W=32,
                 pool=7, head_keep=0.5),
        # AnchorKV's anchor stage: k = n/128 anchors per head (W = 32 recent,
        # 70% of the rest by pooled score, 30% uniform), every key and value
        # assigned to its most cosine-similar anchor
        Workload("anchorkv_llama8b_n32k", L=32, H_kv=8, G=4, d=128, n=32768, W=32,
                 pool=7, anchor_k=256, rho=0.7),
        # H2O-style accumulated attention: window scoring with W = 256, 20%
        Workload("h2o_llama8b_n32k", L=32, H_kv=8, G=4, d=128, n=32768, W=256,
                 pool=7, beta=0.20),
        # KVzip-logit: the same queries, max of the raw logits (no softmax)
        Workload("kvzip_logit_qwen7b_n32k", L=28, H_kv=4, G=7, d=128, n=32768,
                 W=4096, q_mode="external", agg="logit", pool=1, beta=0.25,
                 q_chunk=512),
        # KVzip's chunked scoring: chunks of 2048 cached keys, each scored by
        # a 32-token repeat prompt plus the chunk (own keys in the softmax);
        # W = the 2080 queries of a chunk's input
        Workload("kvzip_chunked_qwen7b_n32k", L=28, H_kv=4, G=7, d=128, n=32768,
                 W=2080, q_mode="external", agg="max", pool=1, beta=0.25, chunk=2048,
                 n_prompt=32),
        # many external queries, max aggregation, Qwen2.5-7B GQA shape
        Workload("kvzip_qwen7b_n32k", L=28, H_kv=4, G=7, d=128, n=32768,
                 W=4096, q_mode="external", agg="max", pool=1, beta=0.25,
                 q_chunk=512),
    ]
}

_TENSOR = {"q": 1, "k": 2, "v": 3, "w_o": 4, "heavy": 5, "budgets": 6, "kself": 7, "rand": 8}


def _rng(seed: int, wl: Workload, tensor: str, layer: int) -> np.random.Generator:
    code = zlib.crc32(wl.name.encode()) & 0x7FFFFFFF
    ss = np.random.SeedSequence([int(seed), code, _TENSOR[tensor], int(layer)])
    return np.random.Generator(np.random.PCG64(ss))


def _heavy_factors(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """Per-(head, position) multiplicative key scale, [H_kv][n] float32."""
    f = np.ones((wl.H_kv, wl.n), dtype=np.float32)
    n_pool = wl.n - wl.W if wl.q_mode == "window" else wl.n
    for h in range(wl.H_kv):
        if wl.heavy == "uniform1pct":
            m = int(np.floor(0.01 * wl.n))
            pos = rng.choice(n_pool, size=m, replace=False)
            f[h, pos] = 4.0
        elif wl.heavy == "zipf":
            perm = rng.permutation(n_pool)
            rank = np.arange(1, n_pool + 1, dtype=np.float64)
            f[h, perm] = (1.0 + 3.0 * rank ** -1.1).astype(np.float32)
        elif wl.heavy == "none":
            pass
        else:
            raise ValueError(wl.heavy)
    return f


def gen_q(wl: Workload, seed: int, layer: int) -> np.ndarray:
    r = _rng(seed, wl, "q", layer)
    x = r.standard_normal(wl.shape("q"), dtype=np.float32)
    return bf16_bits(x)


def gen_kself(wl: Workload, seed: int, layer: int) -> np.ndarray:
    """Chunked scoring: each chunk's own input keys, N(0, 1)."""
    r = _rng(seed, wl, "kself", layer)
    return bf16_bits(r.standard_normal(wl.shape("kself"), dtype=np.float32))


def gen_k(wl: Workload, seed: int, layer: int) -> np.ndarray:
    r = _rng(seed, wl, "k", layer)
    x = r.standard_normal((wl.H_kv, wl.n, wl.d), dtype=np.float32)
    f = _heavy_factors(wl, _rng(seed, wl, "heavy", layer))
    x *= f[:, :, None]
    return bf16_bits(x)


def gen_v(wl: Workload, seed: int, layer: int) -> np.ndarray:
    r = _rng(seed, wl, "v", layer)
    return bf16_bits(r.standard_normal((wl.H_kv, wl.n, wl.d), dtype=np.float32))


def gen_w_o(wl: Workload, seed: int, layer: int) -> np.ndarray:
    r = _rng(seed, wl, "w_o", layer)
    x = r.standard_normal((wl.D, wl.H_q * wl.d), dtype=np.float32)
    x *= np.float32(0.02)
    return bf16_bits(x)


def gen_budgets(wl: Workload, seed: int) -> np.ndarray:
    """Per-(layer, head) budgets [L][H_kv] int32 for a budget-vector workload.

    A stand-in for an offline allocation: every head draws a log-normal
    importance (sigma 0.75), and the candidate budget of all heads together,
    L*H_kv*(floor(beta*n) - W), is shared in proportion to it. Each budget
    counts its W window entries and is capped at n."""
    r = _rng(seed, wl, "budgets", 0)
    imp = r.lognormal(0.0, 0.75, size=(wl.L, wl.H_kv))
    pool = wl.L * wl.H_kv * (int(np.floor(wl.beta * wl.n)) - wl.W_kept)
    b = wl.W_kept + np.floor(imp / imp.sum() * pool)
    return np.minimum(b, wl.n).astype(np.int32)


def gen_rand(wl: Workload, seed: int) -> np.ndarray:
    """Uniform draws in [0, 1) per candidate, [L][H_kv][n_cand] float32 (the
    random anchors of AnchorKV are the candidates with the largest draws)."""
    r = _rng(seed, wl, "rand", 0)
    return r.random((wl.L, wl.H_kv, wl.n_cand), dtype=np.float32)


def gen_layer(wl: Workload, seed: int, layer: int, which=("q", "k", "v", "w_o")) -> dict:
    out = {}
    if "q" in which:
        out["q"] = gen_q(wl, seed, layer)
    if "k" in which:
        out["k"] = gen_k(wl, seed, layer)
    if "v" in which and (wl.value_weight or wl.compact):
        out["v"] = gen_v(wl, seed, layer)
    if "w_o" in which and wl.value_weight:
        out["w_o"] = gen_w_o(wl, seed, layer)
    if "kself" in which and wl.chunk:
        out["kself"] = gen_kself(wl, seed, layer)
    return out


def gen_all(wl: Workload, seed: int, which=("q", "k", "v", "w_o")) -> dict:
    """All layers stacked on a leading L axis (uint16 bf16 bit patterns)."""
    per = [gen_layer(wl, seed, l, which) for l in range(wl.L)]
    return {key: np.stack([p[key] for p in per]) for key in per[0]}


# ------------------------------------------------------- device generator ----

def gen_all_device(wl: Workload, seed: int, which=("q", "k", "v", "w_o"), device="cuda"):
    """Same shapes and distributions as gen_all, drawn on the GPU with torch's
    seeded generator (not bit-identical to the host draws). For workloads
    too large to draw on the host in reasonable time."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + (zlib.crc32(wl.name.encode()) & 0xFFFF))
    out = {}

    def normal(shape, std=1.0):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for l in range(shape[0]):
            t[l] = (torch.randn(shape[1:], generator=g, device=device) * std).to(torch.bfloat16)
        return t

    if "q" in which:
        out["q"] = normal((wl.L, *wl.shape("q")))
    if "kself" in which and wl.chunk:
        out["kself"] = normal((wl.L, *wl.shape("kself")))
    if "k" in which:
        k = torch.empty((wl.L, wl.H_kv, wl.n, wl.d), dtype=torch.bfloat16, device=device)
        n_pool = wl.n - wl.W if wl.q_mode == "window" else wl.n
        for l in range(wl.L):
            x = torch.randn((wl.H_kv, wl.n, wl.d), generator=g, device=device)
            f = torch.ones((wl.H_kv, wl.n), device=device)
            for h in range(wl.H_kv):
                if wl.heavy == "uniform1pct":
                    pos = torch.randperm(n_pool, generator=g, device=device)[: int(0.01 * wl.n)]
                    f[h, pos] = 4.0
                elif wl.heavy == "zipf":
                    perm = torch.randperm(n_pool, generator=g, device=device)
                    rank = torch.arange(1, n_pool + 1, device=device, dtype=torch.float64)
                    f[h, perm] = (1.0 + 3.0 * rank ** -1.1).to(torch.float32)
            k[l] = (x * f[:, :, None]).to(torch.bfloat16)
        out["k"] = k
    if "v" in which and (wl.value_weight or wl.compact):
        out["v"] = normal((wl.L, wl.H_kv, wl.n, wl.d))
    if "w_o" in which and wl.value_weight:
        out["w_o"] = normal((wl.L, wl.D, wl.H_q * wl.d), 0.02)
    return out
