"""ctypes front end of the fp64 CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each method converts its arguments to contiguous host arrays and calls one C
function; the C file holds every step of the arithmetic. Inputs are the exact stored
values: fp32 arrays, or bf16 tensors passed as their raw 16-bit patterns.

Sources (short keys):
  [GROK5]  "第 5 章 model.py 精读·中：MoE 路由与专家" (yingwang.github.io/grok-1/05-model-2/)
  [BOOK12] "第 12 章 MoE：路由、专家与负载" (book.ozine.me ... 12_moe.html)
  [SERIES] "8.1 MoE 系列：从 GShard 到 Mixtral，再到 Switch Transformer" (gitcode.csdn.net)
  [F2C]    "MoE 公式到源码对照" (jerryiiii.gitbook.io ... moe-formula-to-code-walkthrough)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SOURCE = os.path.join(HERE, "moe_oracle.c")
ORACLE_LIB = os.path.join(HERE, "libmoe_oracle.so")

ACT = {"silu": 0, "gelu_erf": 1, "gelu_tanh": 2}
MODE = {"softmax_topk": 0, "topk_softmax": 1}
CAPF = {"tokens_k": 0, "tokens": 1}

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_dbl = ctypes.c_double
_vp = ctypes.c_void_p


def build_oracle(source: str = ORACLE_SOURCE, out: str = ORACLE_LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp) into a shared library; returns its path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra_flags,
           "-o", out + ".tmp", source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_vp)


def _host(a, dtype=None):
    """Contiguous numpy view of a numpy array or CPU torch tensor; bf16 -> uint16 bits."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach()
            if a.device.type != "cpu":
                raise ValueError("the oracle takes host arrays only")
            if a.dtype == torch.bfloat16:
                a = a.contiguous().view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.contiguous().numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        a = np.ascontiguousarray(a.astype(dtype))
    return a


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.int8:
        return 2
    raise TypeError(f"oracle element type must be fp32, bf16 or int8 (weights), got {a.dtype}")


def _scales(w, s, name):
    """Scales [E, C] of an int8 weight stack [E, R, C] (None for fp32/bf16 weights)."""
    if w.dtype != np.int8:
        return None
    if s is None:
        raise ValueError(f"int8 {name} needs its scales")
    sh = _host(s, np.float32)
    assert sh.shape == (w.shape[0], w.shape[2]), (name, sh.shape, w.shape)
    return sh


@dataclass
class Routing:
    logits: np.ndarray      # [N,E] float64 (the fp32 logits, widened)
    probs: np.ndarray       # [N,E] float64
    idx: np.ndarray         # [N,k] int32
    gate: np.ndarray        # [N,k] float64
    margin: np.ndarray      # [N]   float64


@dataclass
class Dispatch:
    capacity: int           # -1 when unlimited
    load: np.ndarray        # [E] int64
    counts: np.ndarray      # [E] int64
    offsets: np.ndarray     # [E+1] int64
    row_of: np.ndarray      # [N,k] int64
    dropped: np.ndarray     # [N,k] uint8
    gate_eff: np.ndarray    # [N,k] float64


class Oracle:
    """One loaded copy of the oracle library (a path lets tests load a mutated build)."""

    def __init__(self, lib_path: str = ORACLE_LIB):
        self.path = lib_path
        L = ctypes.CDLL(lib_path)
        L.oracle_act.restype = _dbl
        L.oracle_act.argtypes = [_int, _dbl]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [_i64, _i64, _i32, _int, _vp, _vp, _vp, _vp]
        L.oracle_route.restype = _int
        L.oracle_route.argtypes = [_i64, _i32, _i32, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_capacity.restype = _int
        L.oracle_capacity.argtypes = [_i64, _i32, _i32, _dbl, _i32, _int, ctypes.POINTER(_i64)]
        L.oracle_dispatch.restype = _int
        L.oracle_dispatch.argtypes = [_i64, _i32, _i32, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp]
        L.oracle_drop_rule.restype = None
        L.oracle_drop_rule.argtypes = [_i64, _i32, _vp, _vp, _vp]
        L.oracle_expert_ffn.restype = _int
        L.oracle_expert_ffn.argtypes = [_i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp]
        L.oracle_expert_rows.restype = _int
        L.oracle_expert_rows.argtypes = [_i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [_i64, _i64, _i32, _vp, _vp, _vp, _vp]
        L.oracle_layer_tokens.restype = _int
        L.oracle_layer_tokens.argtypes = [_i64, _vp, _i64, _i64, _i64, _i32, _i32, _int, _int, _int,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_set_threads.restype = _int
        L.oracle_set_threads.argtypes = [_int]
        L.oracle_balance.restype = None
        L.oracle_balance.argtypes = [_i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
        self.lib = L

    def set_threads(self, n: int = 0) -> int:
        """Host threads of the parallel loops (n <= 0: leave as is); returns the count in use."""
        return self.lib.oracle_set_threads(int(n))

    # -- activations -------------------------------------------------------------------
    def act(self, kind: str, z: float) -> float:
        return self.lib.oracle_act(ACT[kind], float(z))

    # -- router ------------------------------------------------------------------------
    def router_logits(self, x, w_r, bias=None) -> np.ndarray:
        """fp64 logits x W_r (+ bias), [GROK5] §5.2.1."""
        xh = _host(x)
        wr = _host(w_r, np.float32)
        b = _host(bias, np.float32)
        N, D = xh.shape
        E = wr.shape[1]
        assert wr.shape[0] == D
        out = np.empty((N, E), np.float64)
        self.lib.oracle_router_logits(N, D, E, _dtype_code(xh), _ptr(xh), _ptr(wr), _ptr(b), _ptr(out))
        return out

    def route(self, logits, k: int, mode: str, noise=None, noise_all: bool = False) -> Routing:
        """Softmax, selection and gates from logits (rounded to fp32 for the decisions).

        noise given: GShard second choice (slots >= 1 compare fl32(l + noise)), or, with
        noise_all, noisy top-k gating (every step uses fl32(l + noise)). The returned
        logits are the fp32 values the selection used (noisy ones under noise_all)."""
        lg = _host(logits, np.float64)
        N, E = lg.shape
        nz = _host(noise, np.float32)
        idx = np.empty((N, k), np.int32)
        gate = np.empty((N, k), np.float64)
        probs = np.empty((N, E), np.float64)
        margin = np.empty((N,), np.float64)
        noisy = 0 if nz is None else (2 if noise_all else 1)
        rc = self.lib.oracle_route(N, E, k, MODE[mode], noisy, _ptr(lg), _ptr(nz),
                                   _ptr(idx), _ptr(gate), _ptr(probs), _ptr(margin))
        if rc != 0:
            raise ValueError("oracle_route: invalid inputs")
        l32 = lg.astype(np.float32)
        if noisy == 2:
            l32 = l32 + nz  # fp32 sums, as the oracle compares them
        l32 = l32.astype(np.float64)
        return Routing(l32, probs, idx, gate, margin)

    # -- capacity / dispatch -------------------------------------------------------------
    def capacity(self, N: int, E: int, k: int, cf: float, min_capacity: int = 0, formula: str = "tokens_k") -> int:
        """formula "tokens_k": ceil(CF N k / E) ([F2C] §3.1); "tokens": ceil((N / E) CF) ([SERIES] §7.2)."""
        c = _i64(0)
        rc = self.lib.oracle_capacity(N, E, k, float(cf), int(min_capacity), CAPF[formula], ctypes.byref(c))
        if rc != 0:
            raise ValueError("invalid capacity inputs")
        return c.value

    def dispatch(self, idx, gate, E: int, capacity: int | None, padded: bool, token_major: bool = False) -> Dispatch:
        ih = _host(idx, np.int32)
        gh = _host(gate, np.float64)
        N, k = ih.shape
        C = -1 if capacity is None else int(capacity)
        load = np.empty(E, np.int64)
        counts = np.empty(E, np.int64)
        offsets = np.empty(E + 1, np.int64)
        row_of = np.empty((N, k), np.int64)
        dropped = np.empty((N, k), np.uint8)
        rc = self.lib.oracle_dispatch(N, E, k, _ptr(ih), C, 1 if padded else 0, 1 if token_major else 0,
                                      _ptr(load), _ptr(counts),
                                      _ptr(offsets), _ptr(row_of), _ptr(dropped))
        if rc != 0:
            raise ValueError("oracle_dispatch: invalid inputs")
        gate_eff = np.empty((N, k), np.float64)
        self.lib.oracle_drop_rule(N, k, _ptr(gh), _ptr(dropped), _ptr(gate_eff))
        return Dispatch(C, load, counts, offsets, row_of, dropped, gate_eff)

    # -- experts / layer ------------------------------------------------------------------
    def expert_ffn(self, x_row, w1, w2, w3, e: int, act: str, scales=None) -> np.ndarray:
        """f_e(x) for one row. scales = (s1, s2, s3) when the weights are int8."""
        xr = _host(x_row, np.float64)
        a, b, c = _host(w1), _host(w2), _host(w3)
        s1, s2, s3 = (_scales(a, scales and scales[0], "w1"), _scales(b, scales and scales[1], "w2"),
                      _scales(c, scales and scales[2], "w3"))
        E, D, F = a.shape
        out = np.empty(D, np.float64)
        rc = self.lib.oracle_expert_ffn(D, F, _dtype_code(a), ACT[act], _ptr(xr), _ptr(a), _ptr(s1), _ptr(b), _ptr(s2),
                                        _ptr(c), _ptr(s3), int(e), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_expert_ffn failed")
        return out

    def expert_rows(self, xrows, experts, w1, w2, w3, act: str, want_hidden=True, want_out=True, scales=None):
        """(h, f) for expert-buffer rows: h[i] = act(x_i W1_e) * (x_i W2_e), f[i] = h[i] W3_e.
        scales = (s1, s2, s3) when the weights are int8 (W = q * s[e, column])."""
        xr = _host(xrows, np.float64)
        ex = _host(experts, np.int32)
        a, b, c = _host(w1), _host(w2), _host(w3)
        s1, s2, s3 = (_scales(a, scales and scales[0], "w1"), _scales(b, scales and scales[1], "w2"),
                      _scales(c, scales and scales[2], "w3"))
        n, D = xr.shape
        F = a.shape[2]
        hid = np.empty((n, F), np.float64) if want_hidden else None
        out = np.empty((n, D), np.float64) if want_out else None
        rc = self.lib.oracle_expert_rows(n, D, F, _dtype_code(a), ACT[act], _ptr(xr), _ptr(ex), _ptr(a), _ptr(s1),
                                         _ptr(b), _ptr(s2), _ptr(c), _ptr(s3), _ptr(hid), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_expert_rows failed")
        return hid, out

    def combine(self, y_perm, row_of, gate_eff) -> np.ndarray:
        yp = _host(y_perm, np.float64)
        ro = _host(row_of, np.int64)
        ge = _host(gate_eff, np.float64)
        N, k = ro.shape
        D = yp.shape[1]
        y = np.empty((N, D), np.float64)
        self.lib.oracle_combine(N, D, k, _ptr(yp), _ptr(ro), _ptr(ge), _ptr(y))
        return y

    def layer_tokens(self, tokens, x, w1, w2, w3, idx, dropped, gate_eff, act: str, scales=None) -> np.ndarray:
        """y rows of the listed tokens (fp64). scales = (s1, s2, s3) when the weights are int8."""
        toks = np.ascontiguousarray(np.asarray(tokens, np.int64))
        xh = _host(x)
        a, b, c = _host(w1), _host(w2), _host(w3)
        s1, s2, s3 = (_scales(a, scales and scales[0], "w1"), _scales(b, scales and scales[1], "w2"),
                      _scales(c, scales and scales[2], "w3"))
        ih = _host(idx, np.int32)
        dh = _host(dropped, np.uint8)
        gh = _host(gate_eff, np.float64)
        N, D = xh.shape
        E, D2, F = a.shape
        assert D2 == D and c.shape == (E, F, D)
        k = ih.shape[1]
        if _dtype_code(a) != 2 and _dtype_code(xh) != _dtype_code(a):
            raise TypeError("x and expert weights must share one element type (or the weights are int8)")
        y = np.empty((len(toks), D), np.float64)
        rc = self.lib.oracle_layer_tokens(len(toks), _ptr(toks), N, D, F, E, k, _dtype_code(xh), _dtype_code(a),
                                          ACT[act], _ptr(xh), _ptr(a), _ptr(s1), _ptr(b), _ptr(s2), _ptr(c), _ptr(s3),
                                          _ptr(ih), _ptr(dh), _ptr(gh), _ptr(y))
        if rc != 0:
            raise ValueError("oracle_layer_tokens failed")
        return y

    def balance(self, probs, load, k: int):
        """(P[E], E*sum f P with f = load/(N k), E*sum (load/N) P)."""
        ph = _host(probs, np.float64)
        lh = _host(load, np.int64)
        N, E = ph.shape
        P = np.empty(E, np.float64)
        b = _dbl(0.0)
        bn = _dbl(0.0)
        self.lib.oracle_balance(N, E, k, _ptr(ph), _ptr(lh), _ptr(P), ctypes.byref(b), ctypes.byref(bn))
        return P, b.value, bn.value

    # -- whole layer ------------------------------------------------------------------------
    def forward(self, inputs: dict, tokens=None, logits=None):
        """Run every step for the workload dict produced by the input generator.

        Routing and dispatch cover all N tokens; the expert FFN and combine run for
        ``tokens`` (all tokens when None). ``logits`` overrides the router GEMM (used when
        both sides are fed the same logits). Returns a dict of every intermediate."""
        cfg = inputs["cfg"]
        if logits is None:
            logits = self.router_logits(inputs["x"], inputs["w_r"], inputs.get("logit_bias"))
        sc = cfg["second_choice"]
        r = self.route(logits, cfg["k"], cfg["routing_mode"],
                       inputs.get("noise") if sc in ("noisy", "noisy_all") else None, noise_all=sc == "noisy_all")
        padded = cfg["capacity_mode"] == "padded"
        C = (self.capacity(cfg["N"], cfg["E"], cfg["k"], cfg["capacity_factor"], cfg["min_capacity"],
                           cfg.get("capacity_formula", "tokens_k")) if padded else None)
        d = self.dispatch(r.idx, r.gate, cfg["E"], C, padded, cfg.get("capacity_priority", "slot_major") == "token_major")
        if tokens is None:
            tokens = np.arange(cfg["N"])
        y = self.layer_tokens(tokens, inputs["x"], inputs["w1"], inputs["w2"], inputs["w3"], r.idx, d.dropped,
                              d.gate_eff, cfg["activation"])
        P, bal, bal_n = self.balance(r.probs, d.load, cfg["k"])
        return {"routing": r, "dispatch": d, "tokens": np.asarray(tokens), "y": y,
                "P": P, "balance_loss": bal, "balance_loss_div_n": bal_n}


_DEFAULT: Oracle | None = None


def default_oracle() -> Oracle:
    """The oracle built from ``moe_oracle.c`` (compiled on first use if missing or stale)."""
    global _DEFAULT
    if _DEFAULT is None:
        if (not os.path.exists(ORACLE_LIB)
                or os.path.getmtime(ORACLE_LIB) < os.path.getmtime(ORACLE_SOURCE)):
            build_oracle()
        _DEFAULT = Oracle(ORACLE_LIB)
    return _DEFAULT
