"""Seeded synthetic inputs for the MoE-layer workloads.

This module is the one piece shared by the GPU path's callers and the oracle: it draws
random numbers and rounds them to the stored element types, and holds none of the
method's arithmetic. Every tensor comes from its own numpy PCG64 stream, keyed by
(seed, tensor id[, expert]), so results do not depend on thread count or draw order.
fp32 -> bf16 rounding is round-to-nearest-even (torch's conversion).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_TENSOR_ID = {"x": 1, "w_r": 2, "w1": 3, "w2": 4, "w3": 5, "rank": 6, "noise": 7, "logits": 8,
              "s1": 9, "s2": 10, "s3": 11}


def _rng(seed: int, name: str, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), _TENSOR_ID[name], int(sub)])))


def _normal(seed: int, name: str, shape, std: float, sub: int = 0) -> np.ndarray:
    a = _rng(seed, name, sub).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _expert_stack(seed: int, name: str, E: int, shape, std: float, dtype: str) -> torch.Tensor:
    out = torch.empty((E, *shape), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)

    def one(e):
        out[e].copy_(_store(_normal(seed, name, shape, std, sub=e), dtype))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(E)))
    return out


def _int8_stack(seed: int, name: str, E: int, shape) -> torch.Tensor:
    """int8 weights drawn uniformly from [-127, 127] (std about 73.3)."""
    out = torch.empty((E, *shape), dtype=torch.int8)

    def one(e):
        out[e].copy_(torch.from_numpy(_rng(seed, name, e).integers(-127, 128, size=shape, dtype=np.int8)))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(E)))
    return out


def _scales(seed: int, name: str, E: int, n: int, std: float) -> torch.Tensor:
    """Per-(expert, column) scales: std / 73.3 times a factor uniform in [0.5, 1.5], so the
    weights q * s have about the requested std."""
    f = _rng(seed, name).random(size=(E, n), dtype=np.float32) + np.float32(0.5)
    return torch.from_numpy((f * np.float32(std / 73.3)).astype(np.float32))


def zipf_bias(cfg: dict) -> torch.Tensor | None:
    """Per-expert logit bias b_e = -beta * s * ln(r_e), ranks r a seeded permutation."""
    if cfg.get("zipf_s") is None:
        return None
    E = cfg["E"]
    ranks = _rng(cfg["seed"], "rank").permutation(E) + 1
    b = -float(cfg["zipf_beta"]) * float(cfg["zipf_s"]) * np.log(ranks.astype(np.float64))
    return torch.from_numpy(b.astype(np.float32))


def make_inputs(cfg: dict, weights: bool = True) -> dict:
    """Host tensors of one workload: x, w_r, logit_bias, noise, and (if weights) w1, w2, w3."""
    N, D, F, E = cfg["N"], cfg["D"], cfg["F"], cfg["E"]
    s, dt = cfg["seed"], cfg["dtype"]
    out = {"cfg": dict(cfg)}
    out["x"] = _store(_normal(s, "x", (N, D), cfg["x_std"]), dt)
    out["w_r"] = torch.from_numpy(_normal(s, "w_r", (D, E), float(cfg["wr_var"]) ** 0.5))
    if weights and cfg.get("weight_dtype", "same") == "int8":
        # weight-only 8-bit experts: int8 values and fp32 scales per (expert, output column)
        out["w1"] = _int8_stack(s, "w1", E, (D, F))
        out["w2"] = _int8_stack(s, "w2", E, (D, F))
        out["w3"] = _int8_stack(s, "w3", E, (F, D))
        out["s1"] = _scales(s, "s1", E, F, cfg["w_std"])
        out["s2"] = _scales(s, "s2", E, F, cfg["w_std"])
        out["s3"] = _scales(s, "s3", E, D, cfg["w3_std"])
    elif weights:
        out["w1"] = _expert_stack(s, "w1", E, (D, F), cfg["w_std"], dt)
        out["w2"] = _expert_stack(s, "w2", E, (D, F), cfg["w_std"], dt)
        out["w3"] = _expert_stack(s, "w3", E, (F, D), cfg["w3_std"], dt)
    out["logit_bias"] = zipf_bias(cfg)
    out["noise"] = (torch.from_numpy(_normal(s, "noise", (N, E), cfg["noise_std"]))
                    if cfg.get("noise_std") is not None else None)
    return out


def make_logits(N: int, E: int, seed: int, std: float = 1.0, zipf_s=None, zipf_beta=None,
                quantum: float | None = None, hot_expert: int | None = None) -> torch.Tensor:
    """fp32 router logits drawn directly (for routing tests fed identical logits).

    quantum: round logits to multiples of it, which makes exact ties frequent.
    hot_expert: add +50 to that expert, so every token selects it first."""
    a = _normal(seed, "logits", (N, E), std).astype(np.float64)
    if zipf_s is not None:
        ranks = _rng(seed, "rank").permutation(E) + 1
        a += -float(zipf_beta) * float(zipf_s) * np.log(ranks.astype(np.float64))[None, :]
    if quantum is not None:
        a = np.round(a / quantum) * quantum
    if hot_expert is not None:
        a[:, hot_expert] += 50.0
    return torch.from_numpy(a.astype(np.float32))


def make_topk(N: int, E: int, k: int, seed: int, skew: float = 0.0):
    """Random routing records for dispatch tests fed identical inputs: k distinct experts
    per token (drawn with probabilities proportional to rank^-skew over a seeded expert
    order) and positive gates in decreasing order that sum to at most 1."""
    rng = _rng(seed, "logits", 1)
    order = rng.permutation(E)
    w = (np.arange(1, E + 1, dtype=np.float64) ** -float(skew))
    p = np.empty(E)
    p[order] = w / w.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(N)]).astype(np.int32)
    g = rng.random((N, k)) + 0.05
    g = -np.sort(-g, axis=1)
    g = g / (g.sum(axis=1, keepdims=True) * (1.0 + rng.random((N, 1))))
    return torch.from_numpy(idx.reshape(N, k)), torch.from_numpy(g.astype(np.float32))


def make_rows(rows: int, D: int, seed: int, dtype: str, std: float = 1.0) -> torch.Tensor:
    """Random expert-buffer rows [rows, D] in the stored element type."""
    return _store(_normal(seed, "x", (rows, D), std, sub=7), dtype)
