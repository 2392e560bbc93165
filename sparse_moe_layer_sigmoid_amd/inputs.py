"""Seeded synthetic inputs for the MoE layer: the workload shapes and value distributions.

This module holds the configurations and the random generators and nothing of the layer's
arithmetic; the HIP path and the CPU oracle both take their inputs from here.

Every tensor comes from its own NumPy ``Generator(PCG64(SeedSequence(key)))`` stream with
``key = [seed, tensor_id, index...]``, so any one expert's weights (or any chunk of tokens)
can be regenerated on its own.  Normals are drawn in float32, scaled, then rounded to
bfloat16 (round-to-nearest-even, via torch's CPU conversion).

The layer shape follows DeepSeek-V3 as the pages state it ("DeepSeek-V3 Technical Report"
wiki summary, "DeepSeekMoE と補助損失なしの負荷分散" and "事前学習": hidden 7168, 1 shared
+ 256 routed experts, 8 routed per token, expert width 2048).  Weights are random, not
trained: no checkpoint is used.
"""
from __future__ import annotations

import dataclasses
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# tensor ids inside a seed key
_X, _ROUTER, _BIAS, _W13, _W2, _OUTLIER, _ZIPF, _STEP_X = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int = 1
    dtype: str = "bf16"          # compute path: "bf16" or "fp8" ("fp32" inputs run as bf16)
    n_group: int = 1
    topk_group: int = 1
    w_std: float = 0.006
    router_std: float = 0.006
    bias_kind: str = "uniform"   # "zero" | "uniform" (U(-0.01, 0.01)) | "zipf"
    outlier_frac: float = 0.0    # fraction of x entries scaled by outlier_scale
    outlier_scale: float = 100.0
    seed: int = 0                # activations, router bias
    weight_seed: int = 100       # expert and router weights
    steps: int = 1               # decode run: number of bias-update steps
    gamma: float = 0.001

    @property
    def rows(self) -> int:
        return self.T * (self.top_k + self.n_shared)

    @property
    def groups(self) -> int:
        return self.n_experts + self.n_shared


# The five workloads.  The tiny one is fp32 as stated, and runs on the GPU rounded to bf16.
TINY = MoEConfig("tiny_fp32_T64", T=64, d=256, n_experts=16, top_k=2, inter=64, dtype="fp32",
                 w_std=0.02, router_std=0.02, bias_kind="zero", seed=0, weight_seed=0)
V3_BF16 = MoEConfig("v3_bf16_T4096", T=4096, d=7168, n_experts=256, top_k=8, inter=2048,
                    dtype="bf16", seed=1)
V3_GROUP = MoEConfig("v3_group_bf16_T8192", T=8192, d=7168, n_experts=256, top_k=8, inter=2048,
                     dtype="bf16", n_group=8, topk_group=4, seed=2)
V3_FP8 = MoEConfig("v3_fp8_T16384", T=16384, d=7168, n_experts=256, top_k=8, inter=2048,
                   dtype="fp8", outlier_frac=0.001, seed=3)
V3_DECODE = MoEConfig("v3_decode_fp8_T256", T=256, d=7168, n_experts=256, top_k=8, inter=2048,
                      dtype="fp8", bias_kind="zipf", seed=4, steps=100)
CONFIGS = {c.name: c for c in (TINY, V3_BF16, V3_GROUP, V3_FP8, V3_DECODE)}


def small(cfg: MoEConfig, **kw) -> MoEConfig:
    """A reduced copy of a config (for parity tests that the oracle finishes in seconds)."""
    return dataclasses.replace(cfg, **kw)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _to_dtype(a32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t if dtype == "fp32" else t.to(torch.bfloat16)


def _normal(key, shape, std) -> np.ndarray:
    a = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


_ROW_CHUNK = 256


def gen_x(cfg: MoEConfig, step: int | None = None, threads: int = 8) -> torch.Tensor:
    """Activations x [T, d] ~ N(0, 1) (bf16, or fp32 for the tiny config).

    Rows are drawn in chunks of 256 tokens, each from its own stream.  With
    ``outlier_frac`` > 0 a Bernoulli mask (its own stream per chunk) multiplies that
    fraction of the entries by ``outlier_scale``.  ``step`` selects a fresh batch for the
    decode run."""
    T, d = cfg.T, cfg.d
    out = np.empty((T, d), dtype=np.float32)
    tag = (_X,) if step is None else (_STEP_X, step)

    def fill(c):
        r0, r1 = c * _ROW_CHUNK, min(T, (c + 1) * _ROW_CHUNK)
        a = _rng(cfg.seed, *tag, c).standard_normal(size=(r1 - r0, d), dtype=np.float32)
        if cfg.outlier_frac > 0:
            m = _rng(cfg.seed, _OUTLIER, *tag, c).random(size=(r1 - r0, d)) < cfg.outlier_frac
            a[m] *= np.float32(cfg.outlier_scale)
        out[r0:r1] = a

    n_chunks = (T + _ROW_CHUNK - 1) // _ROW_CHUNK
    if n_chunks > 1 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    else:
        for c in range(n_chunks):
            fill(c)
    return _to_dtype(out, "fp32" if cfg.dtype == "fp32" else "bf16")


def gen_router(cfg: MoEConfig) -> torch.Tensor:
    """Router rows e_i [N, d] ~ N(0, router_std)."""
    a = _normal((cfg.weight_seed, _ROUTER), (cfg.n_experts, cfg.d), cfg.router_std)
    return _to_dtype(a, "fp32" if cfg.dtype == "fp32" else "bf16")


def gen_expert(cfg: MoEConfig, e: int):
    """Expert e's weights (e == n_experts is the shared expert):
    w13 [2I, d] (rows [0, I) gate W1, [I, 2I) up W3) and w2 [d, I], ~ N(0, w_std)."""
    dt = "fp32" if cfg.dtype == "fp32" else "bf16"
    w13 = _normal((cfg.weight_seed, _W13, e), (2 * cfg.inter, cfg.d), cfg.w_std)
    w2 = _normal((cfg.weight_seed, _W2, e), (cfg.d, cfg.inter), cfg.w_std)
    return _to_dtype(w13, dt), _to_dtype(w2, dt)


def zipf_beta_file() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias.json")


def gen_bias(cfg: MoEConfig) -> torch.Tensor:
    """Per-expert routing bias b [N] (float32).

    "zero": b = 0.  "uniform": b ~ U(-0.01, 0.01).  "zipf": a seeded permutation gives
    expert i the popularity rank r_i (1-based) and b_i = -beta * ln(r_i), shifted to zero
    mean, with beta read from ``zipf_bias.json`` (written by a calibration script that
    fits the rank/load slope to -1.1 with the CPU oracle's router)."""
    N = cfg.n_experts
    if cfg.bias_kind == "zero":
        return torch.zeros(N, dtype=torch.float32)
    if cfg.bias_kind == "uniform":
        b = _rng(cfg.seed, _BIAS).uniform(-0.01, 0.01, size=N).astype(np.float32)
        return torch.from_numpy(b)
    if cfg.bias_kind == "zipf":
        with open(zipf_beta_file()) as f:
            beta = float(json.load(f)["beta"])
        return zipf_bias(cfg, beta)
    raise ValueError(cfg.bias_kind)


def zipf_bias(cfg: MoEConfig, beta: float) -> torch.Tensor:
    N = cfg.n_experts
    rank = _rng(cfg.seed, _ZIPF).permutation(N) + 1
    b = -beta * np.log(rank.astype(np.float64))
    b -= b.mean()
    return torch.from_numpy(b.astype(np.float32))


def gen_all_weights(cfg: MoEConfig, device, threads: int = 16):
    """All expert weights stacked as W13 [G, 2I, d] and W2 [G, d, I] (bf16) on ``device``,
    generated one expert at a time (so host memory stays bounded) with a thread pool."""
    G, I, d = cfg.groups, cfg.inter, cfg.d
    W13 = torch.empty((G, 2 * I, d), dtype=torch.bfloat16, device=device)
    W2 = torch.empty((G, d, I), dtype=torch.bfloat16, device=device)

    def one(e):
        a, b = gen_expert(cfg, e)
        return e, a.to(torch.bfloat16), b.to(torch.bfloat16)

    with ThreadPoolExecutor(threads) as ex:
        for start in range(0, G, 2 * threads):  # bounded batches keep host memory small
            for e, a, b in ex.map(one, range(start, min(G, start + 2 * threads))):
                W13[e].copy_(a)
                W2[e].copy_(b)
    return W13, W2


# ------------------------------------------------------------------ unit-level test inputs


def gen_routing(seed: int, T: int, K: int, N: int, zipf: float = 0.0):
    """Synthetic routing decisions: idx [T, K] int32 (K distinct experts per token, drawn with
    popularity proportional to rank^-zipf under a seeded permutation) and gates [T, K]
    float32 (positive, each row summing to about one)."""
    r = _rng(seed, 101)
    w = np.arange(1, N + 1, dtype=np.float64) ** (-zipf)
    w = w[r.permutation(N)]
    w /= w.sum()
    idx = np.stack([r.choice(N, size=K, replace=False, p=w) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, K), np.int32)
    g = r.random((T, K)) + 0.05
    g = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    return torch.from_numpy(idx), torch.from_numpy(g)


def gen_normal(seed: int, shape, std: float = 1.0, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std) values rounded to ``dtype`` (bf16 by default)."""
    a = _rng(seed, 102).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return torch.from_numpy(a).to(dtype)


def gen_group_sizes(seed: int, n_groups: int, mean: float, empty_frac: float = 0.1) -> np.ndarray:
    """Ragged group sizes (Poisson around ``mean``, a fraction forced empty)."""
    r = _rng(seed, 103)
    sizes = r.poisson(mean, size=n_groups)
    sizes[r.random(n_groups) < empty_frac] = 0
    return sizes.astype(np.int64)


def gen_e4m3_codes(seed: int, shape, small_int: bool = False) -> torch.Tensor:
    """Random E4M3 codes (never NaN).  small_int: only codes of the integers -15..15."""
    r = _rng(seed, 104)
    if small_int:
        # E4M3 codes of 0..15: 0, 1..7 -> 0x38.., see the format: v = (1+m/8) 2^(E-7)
        ints = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E,
                8: 0x50, 9: 0x51, 10: 0x52, 11: 0x53, 12: 0x54, 13: 0x55, 14: 0x56, 15: 0x57}
        mag = r.integers(0, 16, size=shape)
        code = np.vectorize(ints.get)(mag).astype(np.uint8)
        sign = (r.random(shape) < 0.5) & (mag > 0)
        code = np.where(sign, code | 0x80, code).astype(np.uint8)
    else:
        code = r.integers(0, 0x7F, size=shape).astype(np.uint8)  # 0x00..0x7E
        code = np.where(r.random(shape) < 0.5, code | 0x80, code).astype(np.uint8)
    return torch.from_numpy(code)


def gen_scales(seed: int, shape, pow2: bool = False) -> torch.Tensor:
    """Positive float32 scales (log-uniform), or powers of two."""
    r = _rng(seed, 105)
    e = r.integers(-8, -2, size=shape)
    if pow2:
        return torch.from_numpy(np.exp2(e).astype(np.float32))
    return torch.from_numpy((np.exp2(e) * r.uniform(1.0, 2.0, size=shape)).astype(np.float32))
