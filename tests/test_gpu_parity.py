"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Every stage is checked on identical inputs (both sides fed the same logits, the same
routing records, the same expert rows): indices, loads, slots and the drop mask must be
bit-exact; floating-point results within the stated tolerances. The whole layer is then
checked end to end on the five workloads (full sizes, sampled tokens where the oracle
is slow) and on mid-size variants that span several tiles with ragged tails.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mixture_experts_layer_wave_amd import binding as B
from mixture_experts_layer_wave_amd import configs, inputs
from parity_util import MARGIN, TOL_Y, ambiguous_tokens, assert_rows_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(t):
    return None if t is None else t.to(DEV)


NOISE = {False: "topk", "second": "noisy", "all": "noisy_all"}


def _routing_cfg(N, E, k, mode="topk_softmax", noisy=False, dtype="bf16", D=128, F=128, **kw):
    c = dict(N=N, D=D, F=F, E=E, k=k, dtype=dtype, routing_mode=mode, second_choice=NOISE[noisy],
             activation="silu", capacity_mode="none", capacity_factor=0.0, min_capacity=0)
    c.update(kw)
    return c


# ---------------------------------------------------------------------------------------
# Router: selection and gates from identical fp32 logits
# ---------------------------------------------------------------------------------------

ROUTE_CASES = [
    # N, E, k, dist
    (1, 8, 2, "normal"), (63, 8, 2, "normal"), (65, 8, 1, "normal"), (1000, 8, 2, "ties"),
    (1000, 8, 8, "normal"), (777, 4, 2, "zipf"), (300, 16, 4, "ties"), (4097, 64, 2, "zipf"),
    (513, 64, 8, "normal"), (200, 33, 3, "hot"), (129, 1, 1, "normal"), (640, 64, 2, "ties"),
]


@pytest.mark.parametrize("N,E,k,dist", ROUTE_CASES)
@pytest.mark.parametrize("mode", ["softmax_topk", "topk_softmax"])
@pytest.mark.parametrize("noisy", [False, "second", "all"])
def test_route_from_identical_logits(orc, N, E, k, dist, mode, noisy):
    if noisy == "second" and k < 2:
        pytest.skip("noisy second choice needs k >= 2")
    seed = 10 * N + E + k
    kw = {}
    if dist == "ties":
        kw["quantum"] = 0.25
    elif dist == "zipf":
        kw.update(zipf_s=1.2, zipf_beta=1.0)
    elif dist == "hot":
        kw["hot_expert"] = E // 2
    logits = inputs.make_logits(N, E, seed, **kw)
    noise = inputs.make_logits(N, E, seed + 1, quantum=0.25 if dist == "ties" else None) if noisy else None
    d = B.make_desc(_routing_cfg(N, E, k, mode, noisy))
    idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((N, k), dtype=torch.float32, device=DEV)
    probs = torch.empty((N, E), dtype=torch.float32, device=DEV)
    lout = torch.empty((N, E), dtype=torch.float32, device=DEV)
    B.moe_route(d, None, None, None, _dev(noise), _dev(logits), lout, probs, idx, gate)
    torch.cuda.synchronize()
    r = orc.route(logits, k, mode, noise=noise, noise_all=noisy == "all")
    assert np.array_equal(host(idx), r.idx), "selection differs from the oracle on identical logits"
    # logits_out: the logits the routing used (logit + noise, one fp32 rounding, under noisy_all)
    want = logits.numpy() + noise.numpy() if noisy == "all" else logits.numpy()
    assert np.array_equal(host(lout), want)
    np.testing.assert_allclose(host(gate), r.gate, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(host(probs), r.probs, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("N,E,k", [(300, 64, 2), (300, 40, 8), (97, 64, 1), (300, 33, 3), (1000, 16, 2),
                                   (300, 8, 2), (65, 4, 3), (200, 5, 2), (129, 24, 4),
                                   # at most 64 tokens and 16 experts: the token-parallel router
                                   (64, 8, 2), (1, 8, 2), (37, 16, 8), (64, 5, 2), (50, 12, 3), (64, 16, 1)])
@pytest.mark.parametrize("mode", ["softmax_topk", "topk_softmax"])
@pytest.mark.parametrize("noisy", [False, "second", "all"])
def test_route_split_epilogue(orc, N, E, k, mode, noisy):
    """The bf16 router's own epilogue (x bf16 with scratch: the split-K router, or for at
    most 64 tokens and 16 experts the token-parallel one; four lanes per token, each with
    E / 4 experts) against the oracle routing the logits that router produced: identical
    selection, gates and probabilities within fp32 rounding."""
    if noisy == "second" and k < 2:
        pytest.skip("noisy second choice needs k >= 2")
    cfg = _routing_cfg(N, E, k, mode, noisy, D=256)
    d = B.make_desc(cfg)
    seed = 7 * N + E + k
    x = inputs.make_rows(N, 256, seed, "bf16")
    w_r = inputs.make_logits(256, E, seed + 2, std=1.0 / 16)  # N(0, 1/D) router weights
    noise = inputs.make_logits(N, E, seed + 1) if noisy else None
    idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((N, k), dtype=torch.float32, device=DEV)
    probs = torch.empty((N, E), dtype=torch.float32, device=DEV)
    lout = torch.empty((N, E), dtype=torch.float32, device=DEV)
    sc = torch.empty(B.moe_scratch_size(d), dtype=torch.uint8, device=DEV)
    B.moe_route(d, _dev(x), _dev(w_r), None, _dev(noise), None, lout, probs, idx, gate, sc)
    torch.cuda.synchronize()
    # logits_out holds the logits the selection used: fl32(logit + noise) under noisy_all
    used = host(lout)
    r = orc.route(used, k, mode, noise=noise if noisy == "second" else None)
    assert np.array_equal(host(idx), r.idx), "selection differs from the oracle on the router's own logits"
    np.testing.assert_allclose(host(gate), r.gate, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(host(probs), r.probs, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------------------------------
# Router GEMM: fp32 logits against the exact (fp64) logits
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,N,D", [("tiny_fp32", 64, 128), ("mixtral_prefill", 333, 4096),
                                      ("grok1_layer", 129, 6144), ("gshard_capacity", 1000, 2048),
                                      ("mixtral_decode", 64, 4096), ("mixtral_decode", 1, 4096),
                                      ("gshard_capacity", 4097, 128), ("switch_top1", 257, 2048),
                                      ("switch_top1", 33, 2048),
                                      ("mixtral_prefill", 70000, 256)])
@pytest.mark.parametrize("scratch", [False, True], ids=["single_pass", "split_k"])
def test_router_logits(orc, name, N, D, scratch):
    """fp32 router logits against the exact ones: the single-pass fp32 MFMA path (no
    scratch) and, for bf16 x, the split-K path with W_r split into three bf16 pieces, or for
    at most 64 tokens and 16 experts the token-parallel path (fp32 fused multiply-adds)."""
    # clean logits (under noisy top-k gating logits_out would report logit + noise)
    cfg = configs.scaled_config(name, N=N, D=D, F=128, second_choice="topk")
    inp = inputs.make_inputs(cfg, weights=False)
    d = B.make_desc(cfg)
    E, k = cfg["E"], cfg["k"]
    lout = torch.empty((N, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((N, k), dtype=torch.float32, device=DEV)
    sc = torch.empty(B.moe_scratch_size(d), dtype=torch.uint8, device=DEV) if scratch else None
    B.moe_route(d, _dev(inp["x"]), _dev(inp["w_r"]), _dev(inp["logit_bias"]), _dev(inp["noise"]), None, lout, None,
                idx, gate, sc)
    torch.cuda.synchronize()
    exact = orc.router_logits(inp["x"], inp["w_r"], inp["logit_bias"])
    x64 = inp["x"].double().numpy()
    mag = np.abs(x64) @ np.abs(inp["w_r"].double().numpy())   # sum_d |x_d w_de|
    err = np.abs(host(lout).astype(np.float64) - exact)
    tol = 4e-6 * mag + 1e-6
    assert np.all(err <= tol), f"max |dlogit| {err.max():.3e}, worst ratio {(err / tol).max():.2f}"


# ---------------------------------------------------------------------------------------
# Dispatch + gather from identical routing records
# ---------------------------------------------------------------------------------------

DISPATCH_CASES = [
    # N, E, k, skew, capacity_mode, cf, min_cap
    (1, 8, 2, 0.0, "none", 0.0, 0), (255, 8, 2, 0.0, "none", 0.0, 0), (257, 8, 2, 1.0, "none", 0.0, 0),
    (1000, 64, 2, 1.2, "padded", 1.25, 4), (4096, 8, 2, 0.5, "padded", 1.0, 0),
    (700, 16, 4, 2.0, "padded", 0.5, 1), (513, 4, 4, 0.0, "padded", 0.3, 0), (300, 64, 8, 1.0, "none", 0.0, 0),
    (999, 8, 1, 3.0, "padded", 2.0, 0), (128, 2, 2, 0.0, "padded", 0.01, 1), (50, 64, 2, 0.0, "padded", 10.0, 0),
    (2000, 16, 2, 1.0, "padded", 1.0, 0), (1025, 8, 4, 1.5, "padded", 0.7, 2),
    # at most 256 tokens: one fused launch while the buffer has at most 4096 rows, else
    # the three-pass path
    (64, 8, 2, 4.0, "none", 0.0, 0), (256, 64, 8, 1.0, "padded", 2.0, 0), (200, 64, 8, 1.0, "padded", 30.0, 0),
    # more than 512 (segment, 256-token block) entries per expert: the scan's long-sequence
    # loop (slot-major: k segments; token-major: one segment)
    (70000, 64, 2, 1.2, "padded", 1.25, 4),   # slot-major 548 entries; token-major 274
    (20000, 16, 8, 1.0, "padded", 1.0, 0),    # slot-major 632 entries; token-major 79
    (140000, 8, 2, 0.5, "none", 0.0, 0),      # slot-major 1094 entries; token-major 547
]


def _run_dispatch(d, x, idx, gate):
    N, k, E, D = d.N, d.k, d.E, d.D
    rows = B.moe_rows(d)
    out = dict(load=torch.empty(E, dtype=torch.int32, device=DEV), counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               row_of=torch.empty((N, k), dtype=torch.int32, device=DEV),
               dropped=torch.empty((N, k), dtype=torch.uint8, device=DEV),
               gate_eff=torch.empty((N, k), dtype=torch.float32, device=DEV),
               token_of_row=torch.full((rows,), -7, dtype=torch.int32, device=DEV),
               x_perm=torch.full((rows, D), 7.0, dtype=x.dtype, device=DEV))
    scratch = torch.empty(B.moe_scratch_size(d), dtype=torch.uint8, device=DEV)
    B.moe_dispatch(d, x, idx, gate, out["load"], out["counts"], out["offsets"], out["row_of"], out["dropped"],
                   out["gate_eff"], out["token_of_row"], out["x_perm"], scratch)
    torch.cuda.synchronize()
    return out, scratch


@pytest.mark.parametrize("N,E,k,skew,cap,cf,minc", DISPATCH_CASES)
@pytest.mark.parametrize("prio,formula", [("slot_major", "tokens_k"), ("token_major", "tokens_k"),
                                          ("token_major", "tokens")])
def test_dispatch_from_identical_records(orc, N, E, k, skew, cap, cf, minc, prio, formula):
    cfg = _routing_cfg(N, E, k, capacity_mode=cap, capacity_factor=cf, min_capacity=minc, D=128,
                       capacity_priority=prio, capacity_formula=formula)
    d = B.make_desc(cfg)
    idx, gate = inputs.make_topk(N, E, k, seed=N * 7 + E, skew=skew)
    x = inputs.make_rows(N, 128, seed=N, dtype="bf16")
    out, _ = _run_dispatch(d, x.to(DEV), idx.to(DEV), gate.to(DEV))
    padded = cap == "padded"
    C = orc.capacity(N, E, k, cf, minc, formula) if padded else None
    if padded:
        assert B.moe_capacity(d) == C
    o = orc.dispatch(idx, gate.double(), E, C, padded, token_major=prio == "token_major")
    assert np.array_equal(host(out["load"]), o.load)
    assert np.array_equal(host(out["counts"]), o.counts)
    assert np.array_equal(host(out["offsets"]), o.offsets)
    assert np.array_equal(host(out["row_of"]), o.row_of)
    assert np.array_equal(host(out["dropped"]), o.dropped)
    np.testing.assert_allclose(host(out["gate_eff"]), o.gate_eff, rtol=1e-6, atol=1e-7)
    gone = np.all(o.dropped == 1, axis=1)
    assert np.all(host(out["gate_eff"])[gone] == 0.0)
    # gather: every kept record's row holds its token; padding rows are -1 and zero
    tor = host(out["token_of_row"])
    xp = out["x_perm"].cpu()
    kept = o.row_of >= 0
    tok = np.broadcast_to(np.arange(N)[:, None], o.row_of.shape)
    assert np.array_equal(tor[o.row_of[kept]], tok[kept])
    assert torch.equal(xp[torch.from_numpy(o.row_of[kept])], x[torch.from_numpy(tok[kept].copy())])
    filled = np.zeros(len(tor), bool)
    filled[o.row_of[kept]] = True
    assert np.all(tor[~filled] == -1)
    assert torch.all(xp[torch.from_numpy(~filled)] == 0)


def test_route_dispatch_random_tiny(orc):
    """Seeded random sweep of routing and dispatch on tiny shapes: N <= 300, E 2-64, k 1 to
    min(E, 8), both gate modes, clean / GShard-noisy second / noisy top-k, no capacity or
    CF 0.5 / 1 / 1.25 with a minimum capacity, slot- or token-major priority, k or Switch
    capacity formula, fp32 or bf16 rows, logits with frequent exact ties, Zipf skew or a
    hot expert. Selection from identical logits and dispatch from identical records must
    equal the oracle's bit for bit; the first mismatch stops the sweep and names its case."""
    rng = np.random.default_rng(20261203)
    n_cases = 400
    for case in range(n_cases):
        N = int(rng.integers(1, 301))
        E = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        mode = ["softmax_topk", "topk_softmax"][int(rng.integers(2))]
        noisy = [False, "second", "all"][int(rng.integers(3))]
        if noisy == "second" and k < 2:
            noisy = False
        cf = [None, 0.5, 1.0, 1.25][int(rng.integers(4))]
        minc = int(rng.choice([0, 1, 4]))
        prio = ["slot_major", "token_major"][int(rng.integers(2))]
        formula = ["tokens_k", "tokens"][int(rng.integers(2))]
        dt = ["bf16", "f32"][int(rng.integers(2))]
        dist = ["ties", "normal", "zipf", "hot"][int(rng.integers(4))]
        desc = (f"case {case}: N={N} E={E} k={k} {mode} noisy={noisy} cf={cf} min_cap={minc} {prio} {formula} "
                f"{dt} {dist}")
        seed = 1000 + case
        kw = {"ties": dict(quantum=0.25), "normal": {}, "zipf": dict(zipf_s=1.2, zipf_beta=1.0),
              "hot": dict(hot_expert=int(rng.integers(E)))}[dist]
        logits = inputs.make_logits(N, E, seed, **kw)
        noise = inputs.make_logits(N, E, seed + 1, quantum=0.25 if dist == "ties" else None) if noisy else None
        padded = cf is not None
        cfg = _routing_cfg(N, E, k, mode, noisy, dtype=dt, D=128, capacity_mode="padded" if padded else "none",
                           capacity_factor=cf if padded else 0.0, min_capacity=minc if padded else 0,
                           capacity_priority=prio, capacity_formula=formula)
        d = B.make_desc(cfg)
        idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
        gate = torch.empty((N, k), dtype=torch.float32, device=DEV)
        B.moe_route(d, None, None, None, _dev(noise), _dev(logits), None, None, idx, gate)
        x = inputs.make_rows(N, 128, seed, dt)
        out, _ = _run_dispatch(d, x.to(DEV), idx, gate)
        r = orc.route(logits, k, mode, noise=noise, noise_all=noisy == "all")
        g_idx = host(idx)
        assert np.array_equal(g_idx, r.idx), f"selection differs: {desc}"
        assert np.allclose(host(gate), r.gate, rtol=2e-6, atol=1e-7), f"gates differ: {desc}"
        C = orc.capacity(N, E, k, cf, minc, formula) if padded else None
        if padded:
            assert B.moe_capacity(d) == C, desc
        o = orc.dispatch(g_idx, host(gate).astype(np.float64), E, C, padded, token_major=prio == "token_major")
        for name in ("load", "counts", "offsets", "row_of", "dropped"):
            assert np.array_equal(host(out[name]), getattr(o, name)), f"{name} differs: {desc}"
        assert np.allclose(host(out["gate_eff"]), o.gate_eff, rtol=1e-6, atol=1e-7), f"gate_eff differs: {desc}"
        kept = o.row_of >= 0
        tok = np.broadcast_to(np.arange(N)[:, None], o.row_of.shape)
        assert np.array_equal(host(out["token_of_row"])[o.row_of[kept]], tok[kept]), f"token_of_row differs: {desc}"
        assert torch.equal(out["x_perm"].cpu()[torch.from_numpy(o.row_of[kept])],
                           x[torch.from_numpy(tok[kept].copy())]), f"x_perm differs: {desc}"
    print(f"{n_cases} random tiny routing + dispatch cases bit-exact", flush=True)


# ---------------------------------------------------------------------------------------
# Expert FFN from identical expert rows
# ---------------------------------------------------------------------------------------

FFN_CASES = [
    # dtype, act, D, F, E, counts
    ("bf16", "silu", 256, 384, 4, [130, 0, 257, 1]),
    ("bf16", "gelu_erf", 384, 256, 3, [64, 200, 129]),
    ("bf16", "gelu_tanh", 128, 512, 2, [5, 300]),
    ("bf16", "silu", 4096, 1024, 2, [40, 131]),
    ("bf16", "silu", 256, 384, 4, [30, 0, 20, 14]),         # <= 64 rows per expert: stream-K path
    ("bf16", "gelu_erf", 512, 256, 8, [1, 2, 3, 4, 5, 6, 7, 8]),
    ("bf16", "silu", 4096, 512, 3, [64, 0, 0]),
    ("bf16", "gelu_tanh", 384, 256, 3, [17, 64, 0]),        # stream-K, D not a multiple of 256
    # <= 64 rows per expert and enough up-projection tiles to run them whole, no stream-K
    # split: bf16 160 tiles in one round (int8: 80 tiles, stream-K)
    ("bf16", "silu", 512, 2560, 8, [64, 5, 33, 1, 64, 17, 40, 9]),
    # bf16 320 tiles (stream-K); int8 160 tiles in one round
    ("bf16", "gelu_erf", 256, 5120, 8, [3, 64, 0, 22, 64, 64, 1, 50]),
    # bf16 448 tiles in two rounds on 224 workgroups; int8 224 tiles in one round
    ("bf16", "silu", 256, 7168, 8, [10, 20, 30, 40, 50, 60, 64, 2]),
    # bf16: 320 tiles of 64 x (2 x 128) would need stream-K, 160 tiles of 64 x (2 x 256) fill
    # one round whole: the dual-width up-projection takes the wide tiles
    ("bf16", "silu", 256, 5120, 8, [3, 64, 7, 22, 64, 64, 1, 50]),
    # mixed tile heights (bf16): small remainders (1..64 rows past the last whole 256-row
    # block, or all of a small expert) on 64-row tiles beside the 256-row tiles of the rest
    ("bf16", "silu", 256, 512, 8, [300, 17, 520, 64, 65, 256, 0, 700]),
    ("bf16", "gelu_erf", 512, 768, 4, [1, 257, 600, 40]),
    ("bf16", "gelu_tanh", 256, 1024, 3, [320, 512, 129]),
    ("f32", "silu", 128, 256, 4, [30, 33, 0, 65]),
    ("f32", "gelu_erf", 256, 128, 3, [64, 1, 100]),
]


@pytest.mark.parametrize("dt,act,D,F,E,counts", FFN_CASES)
@pytest.mark.parametrize("layout", ["ragged", "padded"])
@pytest.mark.parametrize("wq", ["same", "int8"])
def test_expert_ffn_from_identical_rows(orc, dt, act, D, F, E, counts, layout, wq):
    """Grouped GEMMs against the oracle's expert rows, from identical buffers; wq = int8:
    weight-only 8-bit experts (int8 weights, fp32 column scales)."""
    if wq == "int8" and dt != "bf16":
        pytest.skip("int8 weights go with bf16 activations")
    counts = np.array(counts, np.int64)
    if layout == "ragged":
        N = int(counts.sum())  # k = 1: rows = N
        cfg = dict(N=N, D=D, F=F, E=E, k=1, dtype=dt, routing_mode="topk_softmax", second_choice="topk",
                   activation=act, capacity_mode="none", capacity_factor=0.0, min_capacity=0)
        offsets = np.concatenate([[0], np.cumsum(counts)])
    else:
        C = int(counts.max()) + 3
        N = E * C  # cf = 1 with k = 1 gives C = N / E
        cfg = dict(N=N, D=D, F=F, E=E, k=1, dtype=dt, routing_mode="topk_softmax", second_choice="topk",
                   activation=act, capacity_mode="padded", capacity_factor=1.0, min_capacity=0)
        offsets = np.arange(E + 1) * C
    d = B.make_desc(cfg)
    rows = B.moe_rows(d)
    wcfg = dict(cfg, seed=31 + D + F, x_std=1.0, wr_var=1.0 / D, w_std=0.05 if dt == "bf16" else (1.0 / D) ** 0.5,
                w3_std=0.05 if dt == "bf16" else (1.0 / F) ** 0.5, noise_std=None, zipf_s=None, weight_dtype=wq)
    w = inputs.make_inputs(wcfg)
    sc = (w["s1"], w["s2"], w["s3"]) if wq == "int8" else None
    xp = inputs.make_rows(rows, D, seed=D + rows, dtype=dt)
    x_perm = xp.to(DEV)
    h = torch.full((rows, F), 3.0, dtype=xp.dtype, device=DEV)
    y_perm = torch.full((rows, D), 3.0, dtype=xp.dtype, device=DEV)
    scratch = torch.empty(B.moe_scratch_size(d), dtype=torch.uint8, device=DEV)
    t_off = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    t_cnt = torch.from_numpy(counts.astype(np.int32)).to(DEV)
    if wq == "int8":
        B.moe_expert_ffn_q8(d, x_perm, t_off, t_cnt, w["w1"].to(DEV), sc[0].to(DEV), w["w2"].to(DEV), sc[1].to(DEV),
                            w["w3"].to(DEV), sc[2].to(DEV), h, y_perm, scratch)
    else:
        B.moe_expert_ffn(d, x_perm, t_off, t_cnt, w["w1"].to(DEV), w["w2"].to(DEV), w["w3"].to(DEV), h, y_perm,
                         scratch)
    torch.cuda.synchronize()
    sel = np.concatenate([np.arange(offsets[e], offsets[e] + counts[e]) for e in range(E)])
    experts = np.concatenate([np.full(counts[e], e) for e in range(E)]).astype(np.int32)
    hid, out = orc.expert_rows(xp.float().numpy()[sel], experts, w["w1"], w["w2"], w["w3"], act, scales=sc)
    tol_h = 8e-3 if dt == "bf16" else 1e-5
    assert_rows_close(host(h)[sel], hid, tol_h, "h")
    assert_rows_close(host(y_perm)[sel], out, TOL_Y[dt], "y_perm")
    # rows of other experts' ranges are never written by an expert's tiles
    if layout == "padded":
        for e in range(E):
            lo, hi = offsets[e] + counts[e], offsets[e + 1]
            if hi - lo > 0 and counts[e] % 128 == 0:
                assert torch.all(y_perm[lo:hi].float() == 3.0)


# ---------------------------------------------------------------------------------------
# Combine from identical expert outputs
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("N,E,k,cf", [(1, 4, 2, 0.0), (333, 8, 2, 0.0), (1000, 16, 4, 0.6), (64, 8, 8, 0.0)])
def test_combine_from_identical_rows(orc, dt, N, E, k, cf):
    padded = cf > 0
    cfg = _routing_cfg(N, E, k, dtype=dt, D=256, capacity_mode="padded" if padded else "none",
                       capacity_factor=cf if padded else 0.0)
    d = B.make_desc(cfg)
    idx, gate = inputs.make_topk(N, E, k, seed=5 + N, skew=1.0)
    C = orc.capacity(N, E, k, cf, 0) if padded else None
    o = orc.dispatch(idx, gate.double(), E, C, padded)
    rows = B.moe_rows(d)
    yp = inputs.make_rows(rows, 256, seed=N + 1, dtype=dt)
    y = torch.empty((N, 256), dtype=yp.dtype, device=DEV)
    B.moe_combine(d, yp.to(DEV), torch.from_numpy(o.row_of.astype(np.int32)).to(DEV),
                  torch.from_numpy(o.gate_eff.astype(np.float32)).to(DEV), y)
    torch.cuda.synchronize()
    ref = orc.combine(yp.float().numpy(), o.row_of, o.gate_eff.astype(np.float32))
    tol = 8e-3 if dt == "bf16" else 2e-6
    assert_rows_close(host(y), ref, tol, "y")
    gone = np.all(o.dropped == 1, axis=1)
    assert np.all(host(y)[gone] == 0.0)


# ---------------------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------------------

_CACHE = {}


def _workload(cfg):
    key = cfg["name"]
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = inputs.make_inputs(cfg)
    return _CACHE[key]


def _oracle_routing(orc, cfg, inp, logits=None):
    """The oracle's routing and dispatch of a workload (all N tokens), from its own exact
    logits, or from the given fp32 logits (the logits the selection used: under noisy
    top-k gating these already hold logit + noise)."""
    N, E, k = cfg["N"], cfg["E"], cfg["k"]
    padded = cfg["capacity_mode"] == "padded"
    sc = cfg["second_choice"]
    if logits is None:
        logits = orc.router_logits(inp["x"], inp["w_r"], inp["logit_bias"])
        r = orc.route(logits, k, cfg["routing_mode"], noise=inp["noise"] if sc != "topk" else None,
                      noise_all=sc == "noisy_all")
    else:
        r = orc.route(logits, k, cfg["routing_mode"], noise=inp["noise"] if sc == "noisy" else None)
    C = (orc.capacity(N, E, k, cfg["capacity_factor"], cfg["min_capacity"], cfg.get("capacity_formula", "tokens_k"))
         if padded else None)
    o = orc.dispatch(r.idx, r.gate, E, C, padded, token_major=cfg.get("capacity_priority") == "token_major")
    return r, o


def _gpu_router_logits(orc, cfg, inp, layer):
    """The fp32 logits the forward routed from: moe_route on the same device inputs,
    whose selection and gates must equal the forward's bit for bit. They are checked
    against the exact logits (|dl| <= 4e-6 sum_d |x_d w_de| + 1e-6, plus one fp32 rounding
    of logit + noise under noisy top-k gating) and returned as a host array."""
    d = layer.desc
    N, E, k = cfg["N"], cfg["E"], cfg["k"]
    sc = torch.empty(B.moe_scratch_size(d), dtype=torch.uint8, device=DEV)
    lout = torch.empty((N, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((N, k), dtype=torch.float32, device=DEV)
    B.moe_route(d, layer.x, layer.w_r, layer.bias, layer.noise, None, lout, None, idx, gate, sc)
    torch.cuda.synchronize()
    v = layer.views()
    assert torch.equal(idx, v["topk_idx"]) and torch.equal(gate, v["topk_gate"]), \
        "moe_route and moe_forward route differently from the same inputs"
    g = host(lout).astype(np.float64)
    exact = orc.router_logits(inp["x"], inp["w_r"], inp["logit_bias"])
    mag = np.abs(inp["x"].double().numpy()) @ np.abs(inp["w_r"].double().numpy())
    tol = 4e-6 * mag + 1e-6
    if cfg["second_choice"] == "noisy_all":
        exact = exact + inp["noise"].double().numpy()
        tol = tol + np.abs(g) * 2.0 ** -23
    err = np.abs(g - exact)
    assert np.all(err <= tol), f"router logits: max |dl| {err.max():.3e}, worst ratio {(err / tol).max():.2f}"
    return host(lout)


def _step_values(r, noise, second_noisy):
    """Per selection step, the probabilities that step ranks ([N,k,E]): the softmax of
    the fp32 logits, and for the noisy steps of the GShard second choice the softmax of
    fl32(logit + noise). Used only to check that a near-tie token's GPU selection is a
    valid one."""
    N, k = r.idx.shape
    out = np.repeat(r.probs[:, None, :], k, axis=1)
    if second_noisy and k > 1:
        v = (r.logits.astype(np.float32) + noise.numpy()).astype(np.float64)
        v = np.exp(v - v.max(axis=1, keepdims=True))
        out[:, 1:, :] = (v / v.sum(axis=1, keepdims=True))[:, None, :]
    return out


def _drop_cases(dropped, per_case):
    """Up to per_case tokens of every pattern of kept / dropped slots, evenly spread, and
    the patterns present (k = 1: kept, dropped; k = 2: kk, kd, dk, dd)."""
    k = dropped.shape[1]
    toks, present = [], []
    for pat in np.ndindex(*(2,) * k):
        m = np.nonzero(np.all(dropped == np.array(pat, np.uint8), axis=1))[0]
        if len(m):
            present.append("".join("kd"[b] for b in pat))
            toks += m[:: max(1, len(m) // per_case)][:per_case].tolist()
    return toks, present


def _check_layer(orc, cfg, sample=None, max_amb=16, drop_sample=0, min_frac=0.9):
    """Runs moe_forward and checks routing, dispatch and outputs against the oracle.

    Without capacity the oracle routes from its own exact logits: selections must be
    equal on every token except the near ties (margin < 1e-5), whose GPU selection must
    be a valid one; dispatch, which a flipped near tie shifts, is compared bit for bit
    over all tokens and experts against the oracle's dispatch of the GPU's own selection
    (no other token's output depends on a near tie). With capacity a flipped record moves
    other tokens' slots, so the oracle routes from the GPU's own fp32 logits (checked
    against the exact ones): selection, loads, counts, offsets, slots and the drop mask
    must then be equal over all tokens. Outputs are compared on the sampled tokens (all
    tokens when sample is None), near ties excluded in the first case only; at least
    min_frac of the sample must be compared."""
    inp = _workload(cfg)
    layer = B.MoELayer(cfg, inp)
    layer.forward()
    torch.cuda.synchronize()
    v = layer.views()
    N, E, k = cfg["N"], cfg["E"], cfg["k"]
    padded = cfg["capacity_mode"] == "padded"
    noise = inp["noise"]
    g_idx, g_gate = host(v["topk_idx"]), host(v["topk_gate"])
    g_logits = _gpu_router_logits(orc, cfg, inp, layer)
    r_own, o_own = _oracle_routing(orc, cfg, inp)
    amb_own = ambiguous_tokens(r_own)
    assert len(amb_own) <= max_amb, f"{len(amb_own)} near-tie tokens"

    if padded:
        r, o = _oracle_routing(orc, cfg, inp, logits=g_logits)
        assert np.array_equal(g_idx, r.idx), "routing differs from the oracle's on the GPU's logits"
        np.testing.assert_allclose(g_gate, r.gate, rtol=2e-6, atol=1e-7)
        amb = np.zeros(0, np.int64)
    else:
        r, o_r = r_own, o_own
        amb = amb_own
        clear = np.ones(N, bool)
        clear[amb] = False
        assert np.array_equal(g_idx[clear], r.idx[clear]), "routing differs on tokens with a clear margin"
        np.testing.assert_allclose(g_gate[clear], r.gate[clear], rtol=2e-5, atol=1e-6)
        # a near-tie token's GPU selection must be a valid one: distinct experts, each
        # step's choice within the margin of the best expert the GPU had not yet chosen,
        # in the values that step ranks
        sv = _step_values(r, noise, cfg["second_choice"] == "noisy")
        for t in amb:
            assert len(set(g_idx[t].tolist())) == k and g_idx[t].min() >= 0 and g_idx[t].max() < E
            left = np.ones(E, bool)
            for j in range(k):
                best = sv[t, j, left].max()
                assert sv[t, j, g_idx[t, j]] >= best - MARGIN, \
                    f"token {t}: GPU selection {g_idx[t]} is not a near tie of {r.idx[t]} (step {j})"
                left[g_idx[t, j]] = False
        o = orc.dispatch(g_idx, g_gate.astype(np.float64), E, None, False,
                         token_major=cfg.get("capacity_priority") == "token_major")
        # loads of the oracle's own routing differ only by the records of near-tie tokens
        assert np.abs(host(v["load"]).astype(np.int64) - o_own.load).sum() <= 2 * k * len(amb)

    # dispatch: bit-exact over all tokens and experts
    assert np.array_equal(host(v["load"]), o.load)
    assert np.array_equal(host(v["counts"]), o.counts)
    assert np.array_equal(host(v["offsets"]), o.offsets)
    assert np.array_equal(host(v["row_of"]), o.row_of), "capacity slots differ"
    assert np.array_equal(host(v["dropped"]), o.dropped), "drop mask differs"
    np.testing.assert_allclose(host(v["gate_eff"]), o.gate_eff, rtol=2e-5, atol=1e-6)
    assert int(host(v["load"]).sum()) == N * k

    # outputs
    present = []
    if sample is None:
        sample = np.arange(N)
    sample = np.asarray(sample, np.int64)
    if drop_sample:
        extra, present = _drop_cases(o.dropped, drop_sample)
        sample = np.union1d(sample, np.array(extra, np.int64))
    excl = np.zeros(N, bool)
    excl[amb] = True
    toks = sample[~excl[sample]]
    assert len(toks) >= min_frac * len(sample), f"only {len(toks)} of {len(sample)} sampled tokens compared"
    o_y = o if padded else o_r
    y_ref = orc.layer_tokens(toks, inp["x"], inp["w1"], inp["w2"], inp["w3"], r.idx, o_y.dropped, o_y.gate_eff,
                             cfg["activation"], scales=(inp["s1"], inp["s2"], inp["s3"]) if "s1" in inp else None)
    y = host(layer.y)[toks]
    err = assert_rows_close(y, y_ref, TOL_Y[cfg["dtype"]], "layer output")
    zero = np.all(o_y.dropped[toks] == 1, axis=1)
    assert np.all(y[zero] == 0.0), "fully dropped tokens must have increment exactly 0"
    print(f"[{cfg['name']}] N={N} E={E} k={k}: "
          + ("routing from the GPU's logits, " if padded else "")
          + f"selection equal on {N - len(amb)}/{N} tokens ({len(amb_own)} near ties vs the oracle's own logits), "
          f"dispatch bit-exact on {N} tokens and {E}/{E} experts ({int(o.dropped.sum())} dropped records), "
          f"outputs compared on {len(toks)}/{len(sample)} sampled tokens"
          + (f" (drop cases {present})" if present else "") + f", max normwise error {err:.2e}", flush=True)
    return dict(layer=layer, routing=r, dispatch=o, amb=amb, amb_own=amb_own, err=err, toks=toks, inp=inp,
                present=present, sample=sample)


MID = [
    configs.scaled_config("tiny_fp32", N=64, D=128, F=256),
    configs.scaled_config("tiny_fp32", N=301, D=256, F=384, E=8, k=3),
    configs.scaled_config("mixtral_prefill", N=333, D=256, F=512),
    configs.scaled_config("mixtral_prefill", N=1, D=128, F=128),
    configs.scaled_config("grok1_layer", N=200, D=384, F=640),
    configs.scaled_config("mixtral_decode", N=64, D=512, F=384),
    configs.scaled_config("gshard_capacity", N=1000, D=256, F=384, E=16),
    configs.scaled_config("gshard_capacity", N=777, D=128, F=256, E=64, capacity_factor=0.5, min_capacity=2),
    configs.scaled_config("mixtral_prefill", N=257, D=128, F=256, E=1, k=1),
    configs.scaled_config("mixtral_prefill", N=200, D=128, F=128, E=8, k=8, routing_mode="softmax_topk",
                          activation="gelu_tanh"),
    configs.scaled_config("switch_top1", N=1000, D=256, F=384),
    configs.scaled_config("switch_top1", N=600, D=128, F=256, E=64, capacity_factor=0.5),
    configs.scaled_config("gshard_capacity", N=900, D=128, F=256, E=16, capacity_priority="token_major",
                          capacity_formula="tokens", capacity_factor=1.5, name="gshard_token_major"),
    configs.scaled_config("mixtral_prefill", N=300, D=128, F=256, k=2, second_choice="noisy_all", noise_std=0.5,
                          name="mixtral_noisy_all"),
    configs.scaled_config("mixtral_decode_int8", N=64, D=512, F=384),
    configs.scaled_config("mixtral_prefill_int8", N=700, D=256, F=512),
    configs.scaled_config("gshard_capacity", N=900, D=128, F=256, E=16, weight_dtype="int8", name="gshard_int8"),
    # at most 64 rows per expert, all 8 experts active: wide up-projection tiles, and most
    # down-projection tiles cut by stream-K ranges
    configs.scaled_config("mixtral_prefill", N=64, D=256, F=5120, name="skinny_wide_tiles"),
    # ~275 rows per expert: most experts end in a small remainder past one 256-row block
    # (mixed tile heights); capacity layout with experts of 1..157 rows
    configs.scaled_config("mixtral_prefill", N=1100, D=256, F=512, name="mixed_heights"),
    configs.scaled_config("gshard_capacity", N=1000, D=256, F=512, E=16, name="gshard_mixed"),
]


@pytest.mark.parametrize("cfg", MID, ids=lambda c: c["name"])
def test_layer_mid_size(orc, cfg):
    _check_layer(orc, cfg)


@pytest.mark.parametrize("cfg", [
    configs.scaled_config("gshard_capacity", N=1000, D=256, F=384, E=16),
    configs.scaled_config("gshard_capacity", N=1000, D=256, F=384, E=16, weight_dtype="int8", name="gshard_int8"),
    # at most 256 tokens, E <= 16, bf16: the forward finishes the routing inside the dispatch kernel
    configs.scaled_config("mixtral_decode", N=64, D=512, F=384),
    configs.scaled_config("mixtral_decode_int8", N=64, D=512, F=384),
    configs.scaled_config("gshard_capacity", N=200, D=256, F=384, E=16, name="gshard_small"),
    configs.scaled_config("switch_top1", N=150, D=256, F=384, name="switch_small"),
    configs.scaled_config("mixtral_prefill", N=256, D=256, F=256, routing_mode="softmax_topk", activation="gelu_erf",
                          name="prefill_256"),
    configs.scaled_config("mixtral_prefill", N=257, D=256, F=256, name="prefill_257"),
    configs.scaled_config("mixtral_prefill", N=64, D=256, F=5120, name="skinny_wide_tiles"),
    configs.scaled_config("mixtral_decode_int8", N=64, D=512, F=5120, name="decode_int8_f5120"),
    configs.scaled_config("mixtral_prefill", N=1100, D=256, F=512, name="mixed_heights"),
    configs.scaled_config("gshard_capacity", N=1000, D=256, F=512, E=16, name="gshard_mixed"),
], ids=lambda c: c["name"])
def test_layer_bitwise_reproducible_and_equal_to_steps(orc, cfg):
    inp = inputs.make_inputs(cfg)
    layer = B.MoELayer(cfg, inp)
    sentinel = 0x7F7F if cfg["dtype"] == "bf16" else 0x7F7F7F7F
    xp_bits = layer.views()["x_perm"].view(torch.int16 if cfg["dtype"] == "bf16" else torch.int32)
    xp_bits.fill_(sentinel)
    y1 = layer.forward().clone()
    y2 = layer.forward().clone()
    assert torch.equal(y1, y2)
    d = layer.desc
    N, E, k, D, F = cfg["N"], cfg["E"], cfg["k"], cfg["D"], cfg["F"]
    rows = B.moe_rows(d)
    sc = torch.empty(B.moe_scratch_size(d), dtype=torch.uint8, device=DEV)
    idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((N, k), dtype=torch.float32, device=DEV)
    B.moe_route(d, layer.x, layer.w_r, layer.bias, layer.noise, None, None, None, idx, gate, sc)
    out, _ = _run_dispatch(d, layer.x, idx, gate)
    h = torch.empty((rows, F), dtype=layer.x.dtype, device=DEV)
    yp = torch.empty((rows, D), dtype=layer.x.dtype, device=DEV)
    layer.expert_up(out["x_perm"], out["offsets"], out["counts"], h, sc)
    layer.expert_down(h, out["offsets"], out["counts"], yp, sc)
    y3 = torch.empty_like(y1)
    B.moe_combine(d, yp, out["row_of"], out["gate_eff"], y3)
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)
    # the up-projection reading its rows from x through token_of_row equals the one on the
    # gathered x_perm on every filled row (bf16 weights, experts that may exceed 64 rows)
    may_gather = cfg["dtype"] == "bf16" and cfg.get("weight_dtype", "same") != "int8" and \
        (min(rows // E, N) if cfg["capacity_mode"] == "padded" else N) > 64
    if cfg.get("weight_dtype", "same") != "int8":
        hg = torch.full_like(h, 5.0)
        try:
            B.moe_expert_up_gathered(d, layer.x, out["token_of_row"], out["offsets"], out["counts"], layer.w1,
                                     layer.w2, hg, sc)
            torch.cuda.synchronize()
            assert may_gather, "gathered up-projection accepted for a layer the forward does not gather"
            off, cnt = host(out["offsets"]), host(out["counts"])
            filled = torch.from_numpy(np.concatenate([np.arange(off[e], off[e] + cnt[e]) for e in range(E)]))
            assert torch.equal(hg[filled], h[filled]), "gathered up-projection differs from moe_expert_up"
        except B.MoeError as err:
            assert not may_gather and err.status == B.MOE_E_UNSUPPORTED, err
    # the forward's routing and dispatch intermediates equal the separate calls' bit for bit
    v = layer.views()
    assert torch.equal(v["topk_idx"], idx) and torch.equal(v["topk_gate"], gate)
    for name in ("load", "counts", "offsets", "row_of", "dropped", "gate_eff"):
        assert torch.equal(v[name], out[name]), name
    # Past the single-launch dispatch of small batches (N <= 256), bf16 layers with bf16
    # weights whose up-projection runs 256-row tiles read the token rows of x through
    # token_of_row and leave x_perm unwritten (padding entries of token_of_row unspecified).
    small = N <= 256 and rows <= 4096
    gathered = cfg["dtype"] == "bf16" and cfg.get("weight_dtype", "same") != "int8" and not small and \
        (min(rows // E, N) if cfg["capacity_mode"] == "padded" else N) > 64
    valid = out["token_of_row"] >= 0
    assert torch.equal(v["token_of_row"][valid], out["token_of_row"][valid])
    if gathered:
        assert torch.all(xp_bits == sentinel), "x_perm written by a gathered forward"
    else:
        assert torch.equal(v["token_of_row"], out["token_of_row"])
        assert torch.equal(v["x_perm"], out["x_perm"])
    # and so do the statistics (probability block sums from the router, counts from dispatch)
    B.moe_dispatch(d, layer.x, idx, gate, out["load"], out["counts"], out["offsets"], out["row_of"], out["dropped"],
                   out["gate_eff"], out["token_of_row"], out["x_perm"], sc)
    torch.cuda.synchronize()
    assert layer.stats() == B.moe_read_stats(d, sc)


@pytest.mark.parametrize("cfg", [configs.scaled_config("gshard_capacity", N=1000, D=256, F=384, E=16),
                                 configs.scaled_config("gshard_capacity", N=200, D=256, F=384, E=16,
                                                       name="gshard_capacity_fused_dispatch"),
                                 configs.scaled_config("mixtral_prefill", N=333, D=256, F=512),
                                 configs.scaled_config("switch_top1", N=1000, D=256, F=384),
                                 # token-parallel router: the block sums formed from the
                                 # probabilities it leaves in scratch
                                 configs.scaled_config("mixtral_decode", N=64, D=256, F=384),
                                 configs.scaled_config("gshard_capacity", N=48, D=256, F=384, E=16,
                                                       name="gshard_capacity_n48")],
                         ids=lambda c: c["name"])
def test_stats(orc, cfg):
    res = _check_layer(orc, cfg)
    layer = res["layer"]
    st = layer.stats()
    v = layer.views()
    o, r = res["dispatch"], res["routing"]
    N, k, E = cfg["N"], cfg["k"], cfg["E"]
    # the statistics describe the GPU's own routing exactly
    g_drop = host(v["dropped"])
    assert st["routed_slots"] == N * k
    assert st["dropped_slots"] == int(g_drop.sum())
    assert st["dropped_tokens"] == int(np.all(g_drop == 1, axis=1).sum())
    assert st["drop_rate"] == pytest.approx(g_drop.mean(), rel=1e-12)
    # and the oracle's statistics of the same records (its dispatch of the GPU's selection,
    # or under capacity its routing of the GPU's logits): drops exactly, the balance loss
    # to the rounding of the fp32 probability sums
    assert st["dropped_slots"] == int(o.dropped.sum())
    assert st["dropped_tokens"] == int(np.all(o.dropped == 1, axis=1).sum())
    P, bal, bal_n = orc.balance(r.probs, o.load, k)
    assert abs(st["balance_loss"] - bal) <= 1e-5 * bal
    assert abs(st["balance_loss_div_n"] - bal_n) <= 1e-5 * bal_n


# ---- the five workloads at their full sizes ---------------------------------------------

def _spread(N, n, extra=()):
    s = set(np.linspace(0, N - 1, n).astype(int).tolist()) | set(extra)
    return np.array(sorted(s), np.int64)


@pytest.mark.slow
def test_workload_tiny_fp32(orc):
    _check_layer(orc, configs.get_config("tiny_fp32"))


@pytest.mark.slow
def test_workload_mixtral_prefill(orc):
    cfg = configs.get_config("mixtral_prefill")
    _check_layer(orc, cfg, sample=_spread(cfg["N"], 40, extra=(1, 63, 64, 4095)))


@pytest.mark.slow
def test_workload_mixtral_decode(orc):
    res = _check_layer(orc, configs.get_config("mixtral_decode"))
    load = res["dispatch"].load
    assert (load == 0).sum() >= 1 and (load > 0).sum() >= 2, f"decode workload must leave an expert empty: {load}"


@pytest.mark.slow
def test_workload_gshard_capacity(orc):
    """Capacity slots and drop mask of all 16384 tokens bit-exact (the oracle routes from
    the GPU's fp32 logits); outputs of evenly spread tokens plus 8 of every drop case."""
    cfg = configs.get_config("gshard_capacity")
    res = _check_layer(orc, cfg, sample=_spread(cfg["N"], 16), drop_sample=8)
    assert sorted(res["present"]) == ["dd", "dk", "kd", "kk"], res["present"]
    assert len(res["toks"]) >= 40
    o = res["dispatch"]
    assert (o.load > 640).sum() >= 1
    st = res["layer"].stats()
    assert st["capacity"] == 640
    assert st["dropped_slots"] == int(o.dropped.sum())
    assert st["dropped_tokens"] == int(np.all(o.dropped == 1, axis=1).sum())


@pytest.mark.slow
def test_workload_switch_top1(orc):
    cfg = configs.get_config("switch_top1")
    res = _check_layer(orc, cfg, sample=_spread(cfg["N"], 16), drop_sample=8)
    o = res["dispatch"]
    C = orc.capacity(cfg["N"], cfg["E"], cfg["k"], cfg["capacity_factor"], cfg["min_capacity"], "tokens")
    assert C == 512 and (o.load > C).sum() >= 1, "the workload must overflow an expert"
    assert sorted(res["present"]) == ["d", "k"], res["present"]
    assert res["layer"].stats()["capacity"] == C


@pytest.mark.slow
def test_workload_mixtral_decode_int8(orc):
    res = _check_layer(orc, configs.get_config("mixtral_decode_int8"))
    load = res["dispatch"].load
    assert (load == 0).sum() >= 1 and (load > 0).sum() >= 2, f"decode workload must leave an expert empty: {load}"


@pytest.mark.slow
def test_workload_mixtral_prefill_int8(orc):
    cfg = configs.get_config("mixtral_prefill_int8")
    _check_layer(orc, cfg, sample=_spread(cfg["N"], 24, extra=(1, 4095)))


@pytest.mark.slow
def test_workload_grok1_layer(orc):
    cfg = configs.get_config("grok1_layer")
    res = _check_layer(orc, cfg, sample=_spread(cfg["N"], 12, extra=(8191,)))
    gsum = host(res["layer"].views()["topk_gate"]).sum(axis=1)
    assert np.all(gsum < 1.0)


@pytest.mark.slow
def test_mixtral_shape_eight_times_the_batch(orc):
    # N = 32768 tokens (65536 rows, ~126 persistent rounds of the up-projection, buffers of
    # 0.5-1.9 GB): schedule, row offsets and scratch at the largest batch tested here.
    cfg = configs.scaled_config("mixtral_prefill", N=32768, D=4096, F=14336, name="mixtral_prefill_n32768")
    _check_layer(orc, cfg, sample=_spread(cfg["N"], 10, extra=(1, 32767)))


# ---------------------------------------------------------------------------------------
# Seeded random layers: routing recipe, sizes, expert counts and capacity drawn at random
# (the grouped GEMMs then meet many remainder patterns and splits of the mixed-height
# launch); each checked end to end as above
# ---------------------------------------------------------------------------------------

def _random_layers(n, seed=20261204, budget=1.2e8):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        base = ["mixtral_prefill", "grok1_layer", "gshard_capacity", "switch_top1"][i % 4]
        E = int(rng.choice([2, 4, 8, 16, 32, 64]))
        k = int(rng.integers(1, min(E, 4) + 1))
        if base == "gshard_capacity":
            k = max(k, 2)  # the noisy second choice needs a second slot
        D = int(rng.choice([128, 256, 384]))
        F = int(rng.choice([256, 512, 768, 384]))
        N = int(rng.integers(1, 1500))
        N = max(1, min(N, int(budget // (k * D * F))))
        over = dict(E=E, k=k, seed=70000 + i, name=f"random{i}_{base}_N{N}E{E}k{k}D{D}F{F}")
        if base in ("gshard_capacity", "switch_top1"):
            over["capacity_factor"] = float(rng.choice([0.5, 1.0, 1.25, 2.0]))
            over["min_capacity"] = int(rng.choice([0, 4]))
        if base != "switch_top1" and rng.random() < 0.25:
            over["weight_dtype"] = "int8"
        out.append(configs.scaled_config(base, N=N, D=D, F=F, **over))
    return out


@pytest.mark.parametrize("cfg", _random_layers(40), ids=lambda c: c["name"])
def test_layer_random(orc, cfg):
    _check_layer(orc, cfg)


def _random_small_batches(n, seed=20261205):
    """Seeded layers of at most 64 tokens (the decode regime: token-parallel router for
    E <= 16, one-launch dispatch, skinny GEMM tiles), across the routing recipes."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        base = ["mixtral_decode", "gshard_capacity", "switch_top1", "grok1_layer"][i % 4]
        E = int(rng.choice([2, 4, 5, 8, 12, 16, 16, 32]))
        k = 1 if base == "switch_top1" else int(rng.integers(2 if base == "gshard_capacity" else 1, min(E, 4) + 1))
        D = int(rng.choice([128, 256, 384]))
        F = int(rng.choice([256, 384, 512]))
        N = int(rng.integers(1, 65))
        over = dict(E=E, k=k, seed=80000 + i, name=f"small{i}_{base}_N{N}E{E}k{k}D{D}F{F}")
        if base in ("gshard_capacity", "switch_top1"):
            over["capacity_factor"] = float(rng.choice([0.5, 1.0, 1.25, 2.0]))
            over["min_capacity"] = int(rng.choice([0, 4]))
        if base in ("mixtral_decode", "grok1_layer") and rng.random() < 0.3:
            over["weight_dtype"] = "int8"
        out.append(configs.scaled_config(base, N=N, D=D, F=F, **over))
    return out


@pytest.mark.parametrize("cfg", _random_small_batches(24), ids=lambda c: c["name"])
def test_layer_random_small_batch(orc, cfg):
    _check_layer(orc, cfg)
