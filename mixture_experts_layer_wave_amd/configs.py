"""The five synthetic MoE-layer workloads (shapes, dtypes, routing options, distributions).

Pure data: no arithmetic of the method. Distributions follow one convention per
symbol: "var" is a variance (std = sqrt(var)), "std" is a standard deviation.

Shapes come from the pages: Mixtral-shaped D=4096, F=14336, E=8, k=2; Grok-1-shaped
D=6144, F=32768, E=8, k=2 ("Grok-1 中文精读" index page, writing conventions; chapter 5
§5.2.1 router shape [6144, 8]); GShard capacity routing with a noisy second choice and
zero-padded buffers ("8.1 MoE 系列" §2-§3).
"""
from __future__ import annotations

import copy

# Keys of one workload:
#   N, D, F, E, k         sizes
#   dtype                 "f32" | "bf16" (x, W1..W3, h, y); router and gates are fp32
#   routing_mode          "softmax_topk" (Grok-1, unnormalised) | "topk_softmax" (Mixtral)
#   second_choice         "topk" | "noisy" (GShard random routing of slots >= 1) |
#                         "noisy_all" (noisy top-k gating: logits + noise everywhere)
#   activation            "silu" | "gelu_erf" | "gelu_tanh"
#   capacity_mode         "none" (ragged, no drops) | "padded" ([E,C,D], drops)
#   capacity_factor, min_capacity
#   capacity_priority     "slot_major" | "token_major" (order records claim positions)
#   capacity_formula      "tokens_k": ceil(CF N k / E) | "tokens": ceil((N / E) CF) (Switch)
#   x_std, wr_var, w_std (W1,W2), w3_std   input distributions (zero mean normal)
#   zipf_s, zipf_beta     per-expert logit bias -beta*s*ln(rank), ranks a seeded
#                         permutation of 1..E (None = no bias)
#   noise_std             std of the routing noise [N,E] (None = no noise)
#   weight_dtype          "same" (W1..W3 in dtype) | "int8" (weight-only 8-bit: int8 W with
#                         fp32 scales per expert and output column; dtype must be bf16)
#   seed                  generator seed

CONFIGS = {
    "tiny_fp32": dict(
        N=64, D=128, F=256, E=4, k=2, dtype="f32",
        routing_mode="topk_softmax", second_choice="topk", activation="silu",
        capacity_mode="none", capacity_factor=0.0, min_capacity=0,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 128, w_std=(1.0 / 128) ** 0.5, w3_std=(1.0 / 256) ** 0.5,
        zipf_s=None, zipf_beta=None, noise_std=None, seed=1001,
    ),
    "mixtral_prefill": dict(
        N=4096, D=4096, F=14336, E=8, k=2, dtype="bf16",
        routing_mode="topk_softmax", second_choice="topk", activation="silu",
        capacity_mode="none", capacity_factor=0.0, min_capacity=0,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 4096, w_std=0.02, w3_std=0.02,
        zipf_s=None, zipf_beta=None, noise_std=None, seed=1002,
    ),
    "grok1_layer": dict(
        N=8192, D=6144, F=32768, E=8, k=2, dtype="bf16",
        routing_mode="softmax_topk", second_choice="topk", activation="gelu_erf",
        capacity_mode="none", capacity_factor=0.0, min_capacity=0,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 6144, w_std=0.02, w3_std=0.02,
        zipf_s=None, zipf_beta=None, noise_std=None, seed=1003,
    ),
    "mixtral_decode": dict(
        N=64, D=4096, F=14336, E=8, k=2, dtype="bf16",
        routing_mode="topk_softmax", second_choice="topk", activation="silu",
        capacity_mode="none", capacity_factor=0.0, min_capacity=0,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 4096, w_std=0.02, w3_std=0.02,
        zipf_s=1.0, zipf_beta=4.0, noise_std=None, seed=1004,
    ),
    "gshard_capacity": dict(
        N=16384, D=2048, F=8192, E=64, k=2, dtype="bf16",
        routing_mode="topk_softmax", second_choice="noisy", activation="silu",
        capacity_mode="padded", capacity_factor=1.25, min_capacity=4,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 2048, w_std=0.02, w3_std=0.02,
        zipf_s=1.2, zipf_beta=1.0, noise_std=1.0, seed=1005,
    ),
    # Switch-style routing ("8.1 MoE 系列" §7: top-1, capacity without k; noisy top-k
    # gating of "第 5 章 ..." §5.2.2), token-major capacity fill. A parity workload of the
    # routing variants; its sizes are chosen here (the pages give none for it).
    "switch_top1": dict(
        N=8192, D=2048, F=8192, E=16, k=1, dtype="bf16",
        routing_mode="softmax_topk", second_choice="noisy_all", activation="silu",
        capacity_mode="padded", capacity_factor=1.0, min_capacity=4,
        capacity_priority="token_major", capacity_formula="tokens",
        x_std=1.0, wr_var=1.0 / 2048, w_std=0.02, w3_std=0.02,
        zipf_s=1.0, zipf_beta=1.0, noise_std=1.0, seed=1006,
    ),
    # Weight-only 8-bit experts ("第 5 章 ..." §5.3.3-5.3.4: Grok-1 dequantises 8-bit expert
    # weights with scales right before the matmul) on the Mixtral decode and prefill
    # shapes; weights of about the same std as the bf16 workloads.
    "mixtral_decode_int8": dict(
        N=64, D=4096, F=14336, E=8, k=2, dtype="bf16", weight_dtype="int8",
        routing_mode="topk_softmax", second_choice="topk", activation="silu",
        capacity_mode="none", capacity_factor=0.0, min_capacity=0,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 4096, w_std=0.02, w3_std=0.02,
        zipf_s=1.0, zipf_beta=4.0, noise_std=None, seed=1004,
    ),
    "mixtral_prefill_int8": dict(
        N=4096, D=4096, F=14336, E=8, k=2, dtype="bf16", weight_dtype="int8",
        routing_mode="topk_softmax", second_choice="topk", activation="silu",
        capacity_mode="none", capacity_factor=0.0, min_capacity=0,
        capacity_priority="slot_major", capacity_formula="tokens_k",
        x_std=1.0, wr_var=1.0 / 4096, w_std=0.02, w3_std=0.02,
        zipf_s=None, zipf_beta=None, noise_std=None, seed=1002,
    ),
}

# Order of the workloads as they are numbered in the documentation (1..5), then the
# routing-variant and int8-weight workloads.
ORDER = ["tiny_fp32", "mixtral_prefill", "grok1_layer", "mixtral_decode", "gshard_capacity", "switch_top1",
         "mixtral_decode_int8", "mixtral_prefill_int8"]


def get_config(workload: str, **overrides) -> dict:
    """A copy of a named workload, with any field overridden (e.g. a smaller N)."""
    cfg = copy.deepcopy(CONFIGS[workload])
    cfg.update(overrides)
    cfg["name"] = overrides.get("name", workload)
    return cfg


def scaled_config(workload: str, N: int, D: int, F: int, **overrides) -> dict:
    """The routing/dtype recipe of a named workload at smaller sizes, with the weight
    distributions rescaled the same way (var 1/D for the router)."""
    base = CONFIGS[workload]
    cfg = get_config(workload, N=N, D=D, F=F, **overrides)
    cfg["wr_var"] = 1.0 / D
    if base["dtype"] == "f32":
        cfg["w_std"] = (1.0 / D) ** 0.5
        cfg["w3_std"] = (1.0 / F) ** 0.5
    cfg["name"] = overrides.get("name", f"{workload}@N{N}D{D}F{F}")
    return cfg
