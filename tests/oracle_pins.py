"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` takes an ``Oracle`` and raises AssertionError if the oracle disagrees
with a value printed on the pages (fixtures under tests/golden/, each citing its page),
a closed form, an invariant, a library routine, or an independent formulation (subset
enumeration for top-k, Grok-1's dense all-experts + one-hot formula for the layer).
The same pins run against deliberately mutated builds of the oracle
(test_oracle_mutants.py): every plausible mistake must fail at least one of them.

Sources (short keys):
  [GROK5]  "第 5 章 model.py 精读·中：MoE 路由与专家" (yingwang.github.io/grok-1/05-model-2/)
  [BOOK12] "第 12 章 MoE：路由、专家与负载" (book.ozine.me, chapter 12)
  [SERIES] "8.1 MoE 系列：从 GShard 到 Mixtral，再到 Switch Transformer" (gitcode.csdn.net)
  [F2C]    "MoE 公式到源码对照" (jerryiiii.gitbook.io)
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, rtol, atol=0.0):
    np.testing.assert_allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=rtol, atol=atol)


# ---------------------------------------------------------------------------------------
# Independent formulations used by several pins (numpy only; not the oracle's code path)
# ---------------------------------------------------------------------------------------

def dense_all_experts(x, w1, w2, w3, act: str):
    """Every expert on every token with numpy matmuls: [E, N, D]. The activation comes
    from scipy (expit / ndtr) or numpy tanh, not from the oracle."""
    x = np.asarray(x, np.float64)
    out = []
    for e in range(w1.shape[0]):
        h1 = x @ np.asarray(w1[e], np.float64)
        h2 = x @ np.asarray(w2[e], np.float64)
        if act == "silu":
            a = h1 * scipy.special.expit(h1)
        elif act == "gelu_erf":
            a = h1 * scipy.special.ndtr(h1)
        else:
            a = 0.5 * h1 * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (h1 + 0.044715 * h1 ** 3)))
        out.append((a * h2) @ np.asarray(w3[e], np.float64))
    return np.stack(out)


def dense_onehot_layer(all_out, idx, gate_eff, dropped):
    """Grok-1's formulation ([GROK5] §5.3.3-§5.3.5): compute all experts, then select each
    token's outputs with a one-hot weight matrix w[t,e] = sum_j gate_j [idx_j = e]."""
    E, N, D = all_out.shape
    w = np.zeros((N, E))
    for t in range(N):
        for j in range(idx.shape[1]):
            if not dropped[t, j]:
                w[t, idx[t, j]] += gate_eff[t, j]
    return np.einsum("te,etd->td", w, all_out)


def _tiny_case(seed, N=9, D=8, F=12, E=5, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, D)).astype(np.float32)
    w_r = (rng.standard_normal((D, E)) * scale / np.sqrt(D)).astype(np.float32)
    w1 = (rng.standard_normal((E, D, F)) / np.sqrt(D)).astype(np.float32)
    w2 = (rng.standard_normal((E, D, F)) / np.sqrt(D)).astype(np.float32)
    w3 = (rng.standard_normal((E, F, D)) / np.sqrt(F)).astype(np.float32)
    return x, w_r, w1, w2, w3


# ---------------------------------------------------------------------------------------
# Capacity ([SERIES] §2.1; [F2C] §3.1)
# ---------------------------------------------------------------------------------------

def pin_capacity_examples(orc):
    g = golden("capacity_examples.json")
    for c in g["cases"]:
        assert orc.capacity(c["N"], c["E"], c["k"], c["cf"], c["min_capacity"]) == c["C"], c
    for c in g["invalid"]:
        try:
            orc.capacity(c["N"], c["E"], c["k"], c["cf"], 0)
        except ValueError:
            continue
        raise AssertionError(f"invalid capacity inputs accepted: {c}")


def pin_switch_capacity_examples(orc):
    """Switch capacity without k ([SERIES] §7.2); for k = 1 it equals the k form."""
    g = golden("switch_capacity_examples.json")
    for c in g["cases"]:
        assert orc.capacity(c["N"], c["E"], c["k"], c["cf"], c["min_capacity"], "tokens") == c["C"], c
        if c["k"] == 1:
            assert orc.capacity(c["N"], c["E"], 1, c["cf"], c["min_capacity"], "tokens_k") == c["C"], c
    for c in g["invalid"]:
        try:
            orc.capacity(c["N"], c["E"], c["k"], c["cf"], 0, "tokens")
        except ValueError:
            continue
        raise AssertionError(f"invalid capacity inputs accepted: {c}")


# ---------------------------------------------------------------------------------------
# Routing ([GROK5] §5.2.3; [F2C] §1.1-1.2; [SERIES] §1.2, §3; [BOOK12] §12.1)
# ---------------------------------------------------------------------------------------

def pin_worked_example(orc):
    g = golden("worked_example_top2.json")
    logits = np.log(np.array(g["probs"], np.float64))
    for mode, key in (("softmax_topk", "gates_softmax_topk"), ("topk_softmax", "gates_topk_softmax")):
        r = orc.route(logits, g["k"], mode)
        assert r.idx.tolist() == g["top2"], (mode, r.idx)
        _close(r.gate, g[key], rtol=1e-6)
        _close(r.probs, g["probs"], rtol=1e-6)


def pin_mode_equivalence(orc):
    """Softmax over the selected logits == renormalised selected probabilities
    ([BOOK12] §12.1 and [F2C] §1.2 state the two forms are equal)."""
    rng = np.random.default_rng(7)
    for E, k in ((8, 2), (16, 4), (5, 5), (64, 2)):
        lg = rng.standard_normal((50, E)) * 2.0
        rb = orc.route(lg, k, "topk_softmax")
        ra = orc.route(lg, k, "softmax_topk")
        assert np.array_equal(ra.idx, rb.idx)
        sel = np.take_along_axis(rb.probs, rb.idx.astype(np.int64), axis=1)
        _close(rb.gate, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)
        _close(ra.gate, sel, rtol=1e-14)
        _close(rb.gate.sum(axis=1), 1.0, rtol=1e-13)
        assert np.all(ra.gate.sum(axis=1) <= 1.0 + 1e-12)


def pin_softmax_library(orc):
    """Full softmax against scipy.special.softmax on the fp32-rounded logits."""
    rng = np.random.default_rng(11)
    lg = (rng.standard_normal((40, 7)) * 3.0).astype(np.float32).astype(np.float64)
    r = orc.route(lg, 3, "softmax_topk")
    _close(r.probs, scipy.special.softmax(lg, axis=1), rtol=1e-13)


def pin_topk_subset_enumeration(orc):
    """The selected set maximises the sum of logits over all k-subsets (a characterisation
    of top-k that uses no sorting), and slots are in descending logit order."""
    rng = np.random.default_rng(3)
    for E, k in ((4, 2), (5, 3), (6, 2), (6, 4), (3, 1)):
        lg = rng.standard_normal((30, E)).astype(np.float32).astype(np.float64)
        r = orc.route(lg, k, "topk_softmax")
        for t in range(lg.shape[0]):
            best = max(itertools.combinations(range(E), k), key=lambda s: sum(lg[t, list(s)]))
            assert sorted(r.idx[t].tolist()) == sorted(best), (t, r.idx[t], best)
            vals = lg[t, r.idx[t]]
            assert np.all(np.diff(vals) < 0), vals


def pin_tie_rule(orc):
    """Ties on equal fp32 values go to the lower expert index (reading of the pages'
    unspecified top-k order); -0.0 equals +0.0."""
    lg = np.array([[1.0, 2.0, 2.0, 0.0],
                   [3.0, 3.0, 3.0, 3.0],
                   [0.0, -0.0, -1.0, -1.0],
                   [-1.0, 5.0, -1.0, 5.0]])
    r = orc.route(lg, 2, "topk_softmax")
    assert r.idx.tolist() == [[1, 2], [0, 1], [0, 1], [1, 3]], r.idx
    assert r.margin[1] == 0.0 and r.margin[3] == 0.0


def pin_margin(orc):
    """Near-tie margin of a token: the smallest gap, over its k selection steps, between
    the probability of the expert a step chooses and that of the best expert still
    unchosen, the probabilities being the softmax over all E of the values that step
    ranks (clean logits; fl32(logit + noise) for the noisy steps). Each token is built
    from probability vectors that sum to 1 (logits ln p, noise ln q - ln p), so every
    step's probabilities are the printed vectors and each expected margin is a
    difference of two printed entries (up to the fp32 rounding of the logits). The
    smallest gap is placed at a later step, so a margin taken at step 0 only, on
    logits instead of probabilities, on the clean values of a noisy step, or against
    an already chosen runner-up, all fail."""
    def lg(p):
        return np.log(np.array([p], np.float64))

    # plain top-k: step gaps 0.5-0.2 and 0.2-0.19 (experts shuffled so the gaps are
    # between non-adjacent indices)
    r = orc.route(lg([0.19, 0.5, 0.11, 0.2]), 2, "topk_softmax")
    assert r.idx.tolist() == [[1, 3]], r.idx
    _close(r.margin, [0.01], rtol=0, atol=1e-6)
    r = orc.route(lg([0.19, 0.5, 0.11, 0.2]), 1, "softmax_topk")
    _close(r.margin, [0.3], rtol=0, atol=1e-6)
    # k = 3: gaps 0.15, 0.10, 0.01 (the smallest at the last step)
    r = orc.route(lg([0.06, 0.4, 0.14, 0.25, 0.15]), 3, "softmax_topk")
    assert r.idx.tolist() == [[1, 3, 4]], r.idx
    _close(r.margin, [0.01], rtol=0, atol=1e-6)
    # k = E: the last step has no unchosen expert left; gaps 0.2 and 0.1
    r = orc.route(lg([0.3, 0.5, 0.2]), 3, "topk_softmax")
    _close(r.margin, [0.1], rtol=0, atol=1e-6)
    r = orc.route(lg([1.0]), 1, "topk_softmax")
    assert np.isinf(r.margin[0]) and r.margin[0] > 0
    # GShard noisy second choice: step 0 ranks the clean p = (0.4, 0.3, 0.2, 0.1) (gap
    # 0.1), step 1 the noisy q = (0.1, 0.35, 0.33, 0.22) with expert 0 chosen (gap 0.02);
    # on the clean values step 1 would give 0.1
    p = np.array([0.4, 0.3, 0.2, 0.1])
    q = np.array([0.1, 0.35, 0.33, 0.22])
    noise = (np.log(q) - np.log(p)).astype(np.float32)[None, :]
    r = orc.route(lg(p), 2, "topk_softmax", noise=noise)
    assert r.idx.tolist() == [[0, 1]], r.idx
    _close(r.margin, [0.02], rtol=0, atol=1e-6)
    # noisy top-k gating: every step ranks fl32(logit + noise) = ln q; gaps 0.22, 0.01
    q = np.array([0.1, 0.45, 0.23, 0.22])
    noise = (np.log(q) - np.log(p)).astype(np.float32)[None, :]
    r = orc.route(lg(p), 2, "softmax_topk", noise=noise, noise_all=True)
    assert r.idx.tolist() == [[1, 2]], r.idx
    _close(r.margin, [0.01], rtol=0, atol=1e-6)


def pin_uniform_routing(orc):
    """W_r = 0: p = 1/E, slots (0..k-1) by the tie rule, gates 1/E (mode A) or 1/k (mode
    B), and the balance loss equals 1 ([F2C] §2.2; [SERIES] §7.3)."""
    N, D, E, k = 12, 16, 8, 2
    x = np.random.default_rng(0).standard_normal((N, D)).astype(np.float32)
    lg = orc.router_logits(x, np.zeros((D, E), np.float32))
    assert np.all(lg == 0.0)
    for mode, g in (("softmax_topk", 1.0 / E), ("topk_softmax", 1.0 / k)):
        r = orc.route(lg, k, mode)
        assert np.all(r.idx == np.arange(k)[None, :])
        _close(r.gate, g, rtol=1e-15)
        _close(r.probs, 1.0 / E, rtol=1e-15)
        d = orc.dispatch(r.idx, r.gate, E, None, False)
        P, bal, bal_n = orc.balance(r.probs, d.load, k)
        _close(bal, 1.0, rtol=1e-14)
        _close(bal_n, float(k), rtol=1e-14)


def pin_balanced_load(orc):
    """Every expert receives exactly N k / E records -> f = 1/E -> loss = sum_e P_e = 1
    for any router probabilities ([F2C] §2.2)."""
    N, E, k = 16, 8, 2
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((N, E)) * 0.1
    for t in range(N):
        for j in range(k):
            lg[t, (t * k + j) % E] += 10.0 - j
    r = orc.route(lg, k, "softmax_topk")
    d = orc.dispatch(r.idx, r.gate, E, None, False)
    assert np.all(d.load == N * k // E)
    P, bal, _ = orc.balance(r.probs, d.load, k)
    _close(P.sum(), 1.0, rtol=1e-14)
    _close(bal, 1.0, rtol=1e-14)


def pin_balance_closed_form(orc):
    """All tokens on experts (0,1), E=4, k=2: f = (1/2, 1/2, 0, 0), so the loss is
    E (P0 + P1) / 2 with P the column means of the probabilities."""
    lg = np.tile(np.array([[4.0, 3.0, 0.0, -1.0]]), (10, 1))
    r = orc.route(lg, 2, "softmax_topk")
    d = orc.dispatch(r.idx, r.gate, 4, None, False)
    p = scipy.special.softmax(lg[0])
    _, bal, bal_n = orc.balance(r.probs, d.load, 2)
    _close(bal, 4 * (p[0] + p[1]) / 2, rtol=1e-13)
    _close(bal_n, 4 * (p[0] + p[1]), rtol=1e-13)


def pin_gshard_noisy_example(orc):
    g = golden("gshard_noisy_example.json")
    r = orc.route(np.array(g["logits"]), g["k"], "topk_softmax", noise=np.array(g["noise"], np.float32))
    assert r.idx.tolist() == g["idx"], r.idx
    _close(r.gate, g["gates_topk_softmax"], rtol=1e-12)
    clean = orc.route(np.array(g["logits"]), g["k"], "topk_softmax")
    assert clean.idx[0].tolist() == [0, 1] and clean.idx[1].tolist() == [2, 3]


def pin_noisy_topk_example(orc):
    """Noisy top-k gating ([GROK5] §5.2.2): the noisy logits drive selection and gates."""
    g = golden("noisy_topk_example.json")
    lg, nz = np.array(g["logits"]), np.array(g["noise"], np.float32)
    r1 = orc.route(lg, 1, "softmax_topk", noise=nz, noise_all=True)
    assert r1.idx.tolist() == g["top1"], r1.idx
    _close(r1.gate, g["top1_gate_softmax_topk"], rtol=1e-12)
    r2 = orc.route(lg, 2, "topk_softmax", noise=nz, noise_all=True)
    assert r2.idx.tolist() == g["top2"], r2.idx
    _close(r2.gate, g["top2_gates_topk_softmax"], rtol=1e-12)
    clean = orc.route(lg, 1, "softmax_topk")
    assert clean.idx[:, 0].tolist() == [0, 0]


def pin_noisy_topk_invariants(orc):
    """Zero noise reproduces the clean router; otherwise routing the noisy logits equals
    routing fl32(logit + noise) with no noise (the noise replaces the logits everywhere,
    probabilities included), in both gate modes."""
    rng = np.random.default_rng(31)
    lg = rng.standard_normal((64, 8)).astype(np.float32)
    nz = rng.standard_normal((64, 8)).astype(np.float32)
    for mode in ("softmax_topk", "topk_softmax"):
        for k in (1, 2, 3):
            a = orc.route(lg, k, mode, noise=np.zeros_like(nz), noise_all=True)
            b = orc.route(lg, k, mode)
            assert np.array_equal(a.idx, b.idx)
            _close(a.gate, b.gate, rtol=0.0)
            c = orc.route(lg, k, mode, noise=nz, noise_all=True)
            d = orc.route((lg + nz).astype(np.float64), k, mode)
            assert np.array_equal(c.idx, d.idx)
            _close(c.gate, d.gate, rtol=1e-15)
            _close(c.probs, d.probs, rtol=1e-15)


# ---------------------------------------------------------------------------------------
# Dispatch, capacity slots, drop rule ([F2C] §1.3, §3.2-3.3; [SERIES] §2.2; [BOOK12] §12.2)
# ---------------------------------------------------------------------------------------

def pin_drop_cases(orc):
    g = golden("drop_cases.json")
    d = orc.dispatch(np.array(g["idx"], np.int32), np.array(g["gate"]), g["E"], g["capacity"], True)
    assert d.load.tolist() == g["load"]
    assert d.counts.tolist() == g["counts"]
    assert d.offsets.tolist() == g["offsets"]
    assert d.dropped.tolist() == g["dropped"]
    assert d.row_of.tolist() == g["row_of"]
    _close(d.gate_eff, g["gate_eff"], rtol=1e-15, atol=1e-15)


def pin_book_capacity_check(orc):
    g = golden("book_capacity_check.json")
    idx = np.array(g["idx"], np.int32)
    d = orc.dispatch(idx, np.full(idx.shape, 0.5), g["E"], g["capacity"], True)
    assert int(d.load.sum()) == g["dispatches"]
    assert int(d.dropped.sum()) == g["excess"]


def pin_records_and_hard_capacity(orc):
    """sum load = N k; accepted_e = min(load_e, C); dropped = sum max(load_e - C, 0);
    positions fill each expert buffer contiguously from 0 ([F2C] §3.2; [BOOK12] §12.2)."""
    rng = np.random.default_rng(9)
    N, E, k = 200, 6, 2
    lg = rng.standard_normal((N, E))
    lg[:, 0] += 1.5  # a hot expert
    r = orc.route(lg, k, "topk_softmax")
    for C in (1, 7, 40, 75, 1000):
        d = orc.dispatch(r.idx, r.gate, E, C, True)
        assert d.load.sum() == N * k
        assert np.array_equal(d.counts, np.minimum(d.load, C))
        assert d.dropped.sum() == np.maximum(d.load - C, 0).sum()
        assert d.counts.sum() + d.dropped.sum() == N * k
        for e in range(E):
            rows = np.sort(d.row_of[(r.idx == e) & (d.dropped == 0)])
            assert np.array_equal(rows, e * C + np.arange(d.counts[e]))
    dn = orc.dispatch(r.idx, r.gate, E, None, False)
    assert dn.dropped.sum() == 0 and np.array_equal(dn.counts, dn.load)
    assert np.array_equal(np.sort(dn.row_of.ravel()), np.arange(N * k))
    assert np.array_equal(dn.offsets[1:] - dn.offsets[:-1], dn.load)


def pin_slot_major_priority(orc):
    """With capacity, every slot-0 record is placed before any slot-1 record, tokens
    ascending within a slot (reading of [SERIES] §2.2's aim that each token keeps at
    least one expert)."""
    idx = np.array([[1, 0], [0, 1], [0, 1], [1, 0]], np.int32)
    d = orc.dispatch(idx, np.full(idx.shape, 0.5), 2, 2, True)
    # slot 0: t0->e1 pos0, t1->e0 pos0, t2->e0 pos1, t3->e1 pos1; every slot 1 drops.
    assert d.dropped.tolist() == [[0, 1], [0, 1], [0, 1], [0, 1]]
    assert d.row_of.tolist() == [[2, -1], [0, -1], [1, -1], [3, -1]]


def pin_token_major_example(orc):
    """The token-by-token loop of [F2C] §3.2 against its worked outcome, and the
    slot-major order on the same records."""
    g = golden("token_major_example.json")
    idx, gate = np.array(g["idx"], np.int32), np.array(g["gate"])
    for order in ("token_major", "slot_major"):
        d = orc.dispatch(idx, gate, g["E"], g["capacity"], True, token_major=order == "token_major")
        want = g[order]
        assert d.load.tolist() == g["load"]
        assert d.counts.tolist() == want["counts"], order
        assert d.dropped.tolist() == want["dropped"], order
        assert d.row_of.tolist() == want["row_of"], order
        _close(d.gate_eff, want["gate_eff"], rtol=1e-15, atol=1e-15)


def pin_priority_invariants(orc):
    """Both visiting orders keep min(load, C) records per expert and fill each buffer
    from position 0; without a capacity, the token-major rows of an expert follow token
    order, and k = 1 makes the two orders identical."""
    rng = np.random.default_rng(17)
    N, E, k = 150, 5, 2
    lg = rng.standard_normal((N, E))
    lg[:, 1] += 1.0
    r = orc.route(lg, k, "topk_softmax")
    for C in (1, 9, 33, 200):
        for tm in (False, True):
            d = orc.dispatch(r.idx, r.gate, E, C, True, token_major=tm)
            assert np.array_equal(d.counts, np.minimum(d.load, C))
            for e in range(E):
                rows = np.sort(d.row_of[(r.idx == e) & (d.dropped == 0)])
                assert np.array_equal(rows, e * C + np.arange(d.counts[e]))
    d = orc.dispatch(r.idx, r.gate, E, None, False, token_major=True)
    for e in range(E):
        t, j = np.nonzero(r.idx == e)
        assert np.all(np.diff(d.row_of[t, j]) > 0)  # np.nonzero lists tokens ascending
    r1 = orc.route(lg, 1, "softmax_topk")
    for C in (3, 40):
        a = orc.dispatch(r1.idx, r1.gate, E, C, True, token_major=True)
        b = orc.dispatch(r1.idx, r1.gate, E, C, True, token_major=False)
        assert np.array_equal(a.row_of, b.row_of) and np.array_equal(a.dropped, b.dropped)


# ---------------------------------------------------------------------------------------
# Expert FFN, activations, combine ([BOOK12] §12.1-12.2; [GROK5] §5.3.3-5.3.5, §5.8)
# ---------------------------------------------------------------------------------------

def pin_activations(orc):
    zs = np.linspace(-6.0, 6.0, 97)
    for z in zs:
        _close(orc.act("silu", z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
        _close(orc.act("gelu_erf", z), z * scipy.special.ndtr(z), rtol=1e-13, atol=1e-15)
        assert abs(orc.act("gelu_erf", z) - orc.act("gelu_tanh", z)) < 1e-3
        # odd-part identities: act(z) - act(-z) = z
        _close(orc.act("silu", z) - orc.act("silu", -z), z, rtol=1e-13, atol=1e-13)
        _close(orc.act("gelu_erf", z) - orc.act("gelu_erf", -z), z, rtol=1e-13, atol=1e-13)
        _close(orc.act("gelu_tanh", z) - orc.act("gelu_tanh", -z), z, rtol=1e-13, atol=1e-13)
    for kind in ("silu", "gelu_erf", "gelu_tanh"):
        assert orc.act(kind, 0.0) == 0.0
    _close(orc.act("gelu_erf", 1.0), 0.8413447460685429, rtol=1e-15)  # Phi(1)


def pin_expert_ffn_library(orc):
    """One expert on one token equals numpy matmuls with scipy activations, for every
    activation; and bf16 weights give the same result as their exact fp32 widening."""
    import torch
    x, _, w1, w2, w3 = _tiny_case(21, N=3, D=16, F=24, E=3)
    for act in ("silu", "gelu_erf", "gelu_tanh"):
        ref = dense_all_experts(x, w1, w2, w3, act)
        for e in range(3):
            for t in range(3):
                _close(orc.expert_ffn(x[t], w1, w2, w3, e, act), ref[e, t], rtol=1e-12, atol=1e-14)
    b1, b2, b3 = (torch.from_numpy(w).to(torch.bfloat16) for w in (w1, w2, w3))
    f1, f2, f3 = (w.float().numpy() for w in (b1, b2, b3))
    for e in range(3):
        _close(orc.expert_ffn(x[0], b1, b2, b3, e, "silu"), orc.expert_ffn(x[0], f1, f2, f3, e, "silu"),
               rtol=0, atol=0)


def pin_layer_dense_onehot(orc):
    """The layer equals Grok-1's dense all-experts + one-hot selection ([GROK5] §5.3.3),
    in both gate modes and with drops; this is the per-token brute force on tiny inputs
    and catches a wrong gate column (a token's expert may sit in slot 0 or slot 1,
    [BOOK12] §12.2) and overwriting instead of accumulating."""
    x, w_r, w1, w2, w3 = _tiny_case(31, N=10, D=8, F=12, E=4, scale=3.0)
    all_out = dense_all_experts(x, w1, w2, w3, "silu")
    lg = orc.router_logits(x, w_r)
    for mode in ("softmax_topk", "topk_softmax"):
        r = orc.route(lg, 2, mode)
        e_slot0 = set(r.idx[:, 0].tolist())
        e_slot1 = set(r.idx[:, 1].tolist())
        assert e_slot0 & e_slot1, "the case must put one expert in different slots"
        for C in (None, 3):
            d = orc.dispatch(r.idx, r.gate, 4, C, C is not None)
            y = orc.layer_tokens(np.arange(10), x, w1, w2, w3, r.idx, d.dropped, d.gate_eff, "silu")
            ref = dense_onehot_layer(all_out, r.idx, d.gate_eff, d.dropped)
            _close(y, ref, rtol=1e-12, atol=1e-13)
            if C is not None:
                assert d.dropped.sum() > 0
                gone = np.all(d.dropped == 1, axis=1)
                assert np.all(y[gone] == 0.0)


def pin_expert_grouped_equals_per_token(orc):
    """[BOOK12] §12.5 check: grouping tokens by expert (gather, batched matmul,
    index-add) equals the per-token sum; records total N k."""
    x, w_r, w1, w2, w3 = _tiny_case(41, N=5, D=6, F=10, E=3)
    lg = orc.router_logits(x, w_r)
    r = orc.route(lg, 2, "topk_softmax")
    d = orc.dispatch(r.idx, r.gate, 3, None, False)
    assert d.load.sum() == 10
    y = orc.layer_tokens(np.arange(5), x, w1, w2, w3, r.idx, d.dropped, d.gate_eff, "silu")
    out = np.zeros((5, 6))
    for e in np.unique(r.idx):
        sel_t, sel_j = np.nonzero(r.idx == e)
        xe = x[sel_t].astype(np.float64)
        h1 = xe @ w1[e].astype(np.float64)
        h2 = xe @ w2[e].astype(np.float64)
        ye = ((h1 * scipy.special.expit(h1)) * h2) @ w3[e].astype(np.float64)
        np.add.at(out, sel_t, ye * d.gate_eff[sel_t, sel_j][:, None])
    _close(y, out, rtol=1e-12, atol=1e-14)


def pin_special_cases(orc):
    """k = 1 with top-k-then-softmax: gate = 1 and y = f_{s0}(x) ([BOOK12] §12.4, §12.5).
    k = E: both modes give gates = p, and y = sum_e p_e f_e(x), the dense soft mixture."""
    x, w_r, w1, w2, w3 = _tiny_case(51, N=7, D=8, F=8, E=4, scale=2.0)
    all_out = dense_all_experts(x, w1, w2, w3, "gelu_erf")
    lg = orc.router_logits(x, w_r)
    r1 = orc.route(lg, 1, "topk_softmax")
    assert np.all(r1.gate == 1.0)
    d1 = orc.dispatch(r1.idx, r1.gate, 4, None, False)
    y1 = orc.layer_tokens(np.arange(7), x, w1, w2, w3, r1.idx, d1.dropped, d1.gate_eff, "gelu_erf")
    _close(y1, all_out[r1.idx[:, 0], np.arange(7)], rtol=1e-12, atol=1e-14)
    for mode in ("softmax_topk", "topk_softmax"):
        r = orc.route(lg, 4, mode)
        _close(np.take_along_axis(r.probs, r.idx.astype(np.int64), 1), r.gate, rtol=1e-13)
        d = orc.dispatch(r.idx, r.gate, 4, None, False)
        y = orc.layer_tokens(np.arange(7), x, w1, w2, w3, r.idx, d.dropped, d.gate_eff, "gelu_erf")
        _close(y, np.einsum("te,etd->td", r.probs, all_out), rtol=1e-12, atol=1e-14)


def pin_empty_expert(orc):
    """An expert no token selects contributes nothing: replacing its weights changes no
    output ([BOOK12] §12.5 answer 4)."""
    x, w_r, w1, w2, w3 = _tiny_case(61, N=6, D=8, F=8, E=4)
    lg = orc.router_logits(x, w_r)
    lg[:, 3] = -30.0
    r = orc.route(lg, 2, "topk_softmax")
    assert not np.any(r.idx == 3)
    d = orc.dispatch(r.idx, r.gate, 4, None, False)
    y = orc.layer_tokens(np.arange(6), x, w1, w2, w3, r.idx, d.dropped, d.gate_eff, "silu")
    for a in (w1, w2, w3):
        a[3] = 1e3
    y2 = orc.layer_tokens(np.arange(6), x, w1, w2, w3, r.idx, d.dropped, d.gate_eff, "silu")
    assert np.array_equal(y, y2)
    assert d.load[3] == 0


def pin_router_logits_library(orc):
    """Router logits equal a numpy matmul of the exact inputs (fp32 and bf16 x), plus bias."""
    import torch
    rng = np.random.default_rng(71)
    x = rng.standard_normal((13, 32)).astype(np.float32)
    w = (rng.standard_normal((32, 6)) / 6).astype(np.float32)
    b = rng.standard_normal(6).astype(np.float32)
    _close(orc.router_logits(x, w, b), x.astype(np.float64) @ w.astype(np.float64) + b, rtol=1e-13, atol=1e-14)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    _close(orc.router_logits(xb, w), xb.double().numpy() @ w.astype(np.float64), rtol=1e-13, atol=1e-14)


def pin_combine_scatter_matrix(orc):
    """combine(y_perm, row_of, gate_eff) equals S @ y_perm with S[t, row] = gate, a sparse
    matrix formulation of the gate-weighted sum ([GROK5] §5.8; [BOOK12] §12.2)."""
    rng = np.random.default_rng(81)
    N, k, D, rows = 12, 3, 5, 40
    y_perm = rng.standard_normal((rows, D))
    row_of = np.stack([rng.choice(rows, k, replace=False) for _ in range(N)]).astype(np.int64)
    gate = rng.random((N, k))
    row_of[2, 1] = -1
    row_of[5, :] = -1
    S = np.zeros((N, rows))
    for t in range(N):
        for j in range(k):
            if row_of[t, j] >= 0:
                S[t, row_of[t, j]] += gate[t, j]
    y = orc.combine(y_perm, row_of, gate)
    _close(y, S @ y_perm, rtol=1e-13, atol=1e-14)
    assert np.all(y[5] == 0.0)


def pin_expert_rows_library(orc):
    """Row-wise expert evaluation (hidden vector and output) equals numpy matmuls."""
    x, _, w1, w2, w3 = _tiny_case(91, N=6, D=8, F=16, E=3)
    experts = np.array([2, 0, 1, 1, 2, 0], np.int32)
    hid, out = orc.expert_rows(x, experts, w1, w2, w3, "gelu_tanh")
    for i, e in enumerate(experts):
        h1 = x[i].astype(np.float64) @ w1[e].astype(np.float64)
        h2 = x[i].astype(np.float64) @ w2[e].astype(np.float64)
        h = 0.5 * h1 * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (h1 + 0.044715 * h1 ** 3))) * h2
        _close(hid[i], h, rtol=1e-12, atol=1e-14)
        _close(out[i], h @ w3[e].astype(np.float64), rtol=1e-12, atol=1e-14)


def _int8_case(seed, E=3, D=8, F=12):
    rng = np.random.default_rng(seed)
    q1 = rng.integers(-128, 128, (E, D, F)).astype(np.int8)
    q2 = rng.integers(-128, 128, (E, D, F)).astype(np.int8)
    q3 = rng.integers(-128, 128, (E, F, D)).astype(np.int8)
    s1 = (rng.random((E, F)) * 0.02 / 64).astype(np.float32)
    s2 = (rng.random((E, F)) * 0.02 / 64).astype(np.float32)
    s3 = (rng.random((E, D)) * 0.02 / 64).astype(np.float32)
    return (q1, q2, q3), (s1, s2, s3)


def pin_int8_weights_library(orc):
    """Weight-only 8-bit experts ([GROK5] §5.3.3-5.3.4, weight = weight * scales): rows and layer
    outputs equal numpy matmuls with the dequantised weights q[e,k,n] * s[e,n], with
    scipy activations; every int8 value (-128..127) occurs."""
    (q1, q2, q3), (s1, s2, s3) = _int8_case(5)
    assert q1.min() == -128 and q1.max() == 127
    rng = np.random.default_rng(6)
    x = rng.standard_normal((7, 8)).astype(np.float32)
    w1 = q1.astype(np.float64) * s1[:, None, :]
    w2 = q2.astype(np.float64) * s2[:, None, :]
    w3 = q3.astype(np.float64) * s3[:, None, :]
    experts = np.array([2, 0, 1, 1, 2, 0, 1], np.int32)
    hid, out = orc.expert_rows(x, experts, q1, q2, q3, "silu", scales=(s1, s2, s3))
    for i, e in enumerate(experts):
        h1 = x[i].astype(np.float64) @ w1[e]
        h = h1 * scipy.special.expit(h1) * (x[i].astype(np.float64) @ w2[e])
        _close(hid[i], h, rtol=1e-12, atol=1e-16)
        _close(out[i], h @ w3[e], rtol=1e-12, atol=1e-16)
    # the layer: Grok-1's dense all-experts + one-hot formula on the dequantised weights
    lg = rng.standard_normal((7, 3))
    r = orc.route(lg, 2, "softmax_topk")
    d = orc.dispatch(r.idx, r.gate, 3, None, False)
    y = orc.layer_tokens(np.arange(7), x, q1, q2, q3, r.idx, d.dropped, d.gate_eff, "gelu_erf", scales=(s1, s2, s3))
    ref = dense_onehot_layer(dense_all_experts(x, w1, w2, w3, "gelu_erf"), r.idx, d.gate_eff, d.dropped)
    _close(y, ref, rtol=1e-11, atol=1e-15)


def pin_int8_scale_axis(orc):
    """The scale belongs to the output column: scaling column n of W by c_n scales output
    column n of the projection by c_n ((x W) diag(c) = x (W diag(c))), checked by
    doubling one column's scale of W3, and it is per expert."""
    (q1, q2, q3), (s1, s2, s3) = _int8_case(8)
    x = np.random.default_rng(9).standard_normal((1, 8)).astype(np.float32)
    base = orc.expert_ffn(x[0], q1, q2, q3, 1, "silu", scales=(s1, s2, s3))
    t3 = s3.copy()
    t3[1, 5] *= 2.0
    mod = orc.expert_ffn(x[0], q1, q2, q3, 1, "silu", scales=(s1, s2, t3))
    want = base.copy()
    want[5] *= 2.0
    _close(mod, want, rtol=1e-14, atol=0.0)
    t3 = s3.copy()
    t3[0, 5] *= 2.0  # another expert's scale: no change
    _close(orc.expert_ffn(x[0], q1, q2, q3, 1, "silu", scales=(s1, s2, t3)), base, rtol=0.0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
