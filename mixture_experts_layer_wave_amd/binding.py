"""ctypes binding of ``libmoe_mi355x.so`` (C ABI in include/moe.h).

Argument marshalling only: each function checks that the torch tensors it is given are
device tensors of the shape and dtype the descriptor implies (so a wrong buffer fails
here on the host instead of faulting the GPU), passes their device pointers and the
current HIP stream, and raises ``MoeError`` on a non-zero status. Every step of the
computation runs in the HIP library. There is no fallback: if the library is missing,
``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK, MOE_E_INVAL, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP = 0, -1, -2, -3, -4
DTYPE = {"f32": 0, "bf16": 1}
ROUTE = {"softmax_topk": 0, "topk_softmax": 1}
SECOND = {"topk": 0, "noisy": 1, "noisy_all": 2}
PRIO = {"slot_major": 0, "token_major": 1}
CAPF = {"tokens_k": 0, "tokens": 1}
ACT = {"silu": 0, "gelu_erf": 1, "gelu_tanh": 2}
CAP = {"none": 0, "padded": 1}
EXPORTED = ["moe_status_string", "moe_capacity", "moe_rows", "moe_scratch_size", "moe_workspace_size",
            "moe_workspace_layout", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_up",
            "moe_expert_down", "moe_combine",
            "moe_forward", "moe_read_stats", "moe_expert_up_q8", "moe_expert_down_q8", "moe_expert_ffn_q8",
            "moe_forward_q8", "moe_forward_noalloc", "moe_expert_up_gathered"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)}")
        self.status = status


class moe_desc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("D", ctypes.c_int64), ("F", ctypes.c_int64),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("routing_mode", ctypes.c_int32), ("second_choice", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("capacity_mode", ctypes.c_int32),
                ("min_capacity", ctypes.c_int32), ("capacity_factor", ctypes.c_double),
                ("capacity_priority", ctypes.c_int32), ("capacity_formula", ctypes.c_int32)]


class moe_stats(ctypes.Structure):
    _fields_ = [("routed_slots", ctypes.c_int64), ("dropped_slots", ctypes.c_int64),
                ("dropped_tokens", ctypes.c_int64), ("capacity", ctypes.c_int64),
                ("drop_rate", ctypes.c_double), ("token_drop_rate", ctypes.c_double),
                ("balance_loss", ctypes.c_double), ("balance_loss_div_n", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class moe_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("scratch", "topk_idx", "topk_gate", "load", "counts", "offsets",
                                               "row_of", "dropped", "gate_eff", "token_of_row", "x_perm", "h",
                                               "y_perm", "total")]


_LIB = None
_vp = ctypes.c_void_p
_dp = ctypes.POINTER(moe_desc)


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build() or python -m mixture_experts_layer_wave_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_capacity.argtypes = [_dp, ctypes.POINTER(ctypes.c_int64)]
        L.moe_rows.argtypes = [_dp, ctypes.POINTER(ctypes.c_int64)]
        L.moe_scratch_size.argtypes = [_dp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_workspace_size.argtypes = [_dp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_workspace_layout.argtypes = [_dp, ctypes.POINTER(moe_ws_layout)]
        L.moe_route.argtypes = [_dp] + [_vp] * 9 + [_vp, ctypes.c_size_t, _vp]
        L.moe_dispatch.argtypes = [_dp] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]
        L.moe_expert_ffn.argtypes = [_dp] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]
        L.moe_expert_up.argtypes = [_dp] + [_vp] * 6 + [_vp, ctypes.c_size_t, _vp]
        L.moe_expert_down.argtypes = [_dp] + [_vp] * 5 + [_vp, ctypes.c_size_t, _vp]
        L.moe_expert_up_gathered.argtypes = [_dp] + [_vp] * 7 + [_vp, ctypes.c_size_t, _vp]
        L.moe_combine.argtypes = [_dp] + [_vp] * 4 + [_vp]
        L.moe_forward.argtypes = [_dp] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]
        L.moe_forward_noalloc.argtypes = [_dp] + [_vp] * 8 + [_vp]
        L.moe_read_stats.argtypes = [_dp, _vp, ctypes.c_size_t, ctypes.POINTER(moe_stats), _vp]
        L.moe_expert_up_q8.argtypes = [_dp] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]
        L.moe_expert_down_q8.argtypes = [_dp] + [_vp] * 6 + [_vp, ctypes.c_size_t, _vp]
        L.moe_expert_ffn_q8.argtypes = [_dp] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]
        L.moe_forward_q8.argtypes = [_dp] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]
        for f in EXPORTED[1:]:
            getattr(L, f).restype = ctypes.c_int
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def make_desc(cfg: dict) -> moe_desc:
    """moe_desc of a workload dict (see configs.py)."""
    return moe_desc(int(cfg["N"]), int(cfg["D"]), int(cfg["F"]), int(cfg["E"]), int(cfg["k"]),
                    DTYPE[cfg["dtype"]], ROUTE[cfg["routing_mode"]], SECOND[cfg["second_choice"]],
                    ACT[cfg["activation"]], CAP[cfg["capacity_mode"]], int(cfg.get("min_capacity", 0)),
                    float(cfg.get("capacity_factor", 0.0)), PRIO[cfg.get("capacity_priority", "slot_major")],
                    CAPF[cfg.get("capacity_formula", "tokens_k")])


def _tdtype(d: moe_desc):
    return torch.bfloat16 if d.dtype == DTYPE["bf16"] else torch.float32


def _ptr(t, shape=None, dtype=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _bytes_ptr(t, nbytes, name):
    if t is None:
        return None, 0
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    size = t.numel() * t.element_size()
    if size < nbytes:
        raise ValueError(f"{name} holds {size} bytes, needs {nbytes}")
    return t.data_ptr(), size


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ---- host queries -------------------------------------------------------------------------

def moe_capacity(d: moe_desc) -> int:
    c = ctypes.c_int64()
    _check(lib().moe_capacity(ctypes.byref(d), ctypes.byref(c)), "moe_capacity")
    return c.value


def moe_rows(d: moe_desc) -> int:
    r = ctypes.c_int64()
    _check(lib().moe_rows(ctypes.byref(d), ctypes.byref(r)), "moe_rows")
    return r.value


def moe_scratch_size(d: moe_desc) -> int:
    b = ctypes.c_size_t()
    _check(lib().moe_scratch_size(ctypes.byref(d), ctypes.byref(b)), "moe_scratch_size")
    return b.value


def moe_workspace_size(d: moe_desc) -> int:
    b = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(d), ctypes.byref(b)), "moe_workspace_size")
    return b.value


def moe_workspace_layout(d: moe_desc) -> moe_ws_layout:
    L = moe_ws_layout()
    _check(lib().moe_workspace_layout(ctypes.byref(d), ctypes.byref(L)), "moe_workspace_layout")
    return L


# ---- compute entry points -------------------------------------------------------------------

def moe_route(d, x, w_r, logit_bias, noise, logits_in, logits_out, probs_out, topk_idx, topk_gate,
              scratch=None, stream=None):
    N, D, E, k = d.N, d.D, d.E, d.k
    f32 = torch.float32
    if logits_in is None:
        px = _ptr(x, (N, D), _tdtype(d), "x")
        pw = _ptr(w_r, (D, E), f32, "w_r")
    else:
        px = pw = None
    pl = _ptr(logits_in, (N, E), f32, "logits_in", optional=True)
    pb = _ptr(logit_bias, (E,), f32, "logit_bias", optional=True)
    pn = _ptr(noise, (N, E), f32, "noise", optional=(d.second_choice == 0))
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_route(ctypes.byref(d), px, pw, pb, pn, pl,
                           _ptr(logits_out, (N, E), f32, "logits_out", optional=True),
                           _ptr(probs_out, (N, E), f32, "probs_out", optional=True),
                           _ptr(topk_idx, (N, k), torch.int32, "topk_idx"),
                           _ptr(topk_gate, (N, k), f32, "topk_gate"), ps, sb, _stream(stream)), "moe_route")


def moe_dispatch(d, x, topk_idx, topk_gate, load, counts, offsets, row_of, dropped, gate_eff, token_of_row,
                 x_perm, scratch, stream=None):
    N, D, E, k = d.N, d.D, d.E, d.k
    rows = moe_rows(d)
    i32, f32 = torch.int32, torch.float32
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_dispatch(ctypes.byref(d), _ptr(x, (N, D), _tdtype(d), "x"),
                              _ptr(topk_idx, (N, k), i32, "topk_idx"), _ptr(topk_gate, (N, k), f32, "topk_gate"),
                              _ptr(load, (E,), i32, "load"), _ptr(counts, (E,), i32, "counts"),
                              _ptr(offsets, (E + 1,), i32, "offsets"), _ptr(row_of, (N, k), i32, "row_of"),
                              _ptr(dropped, (N, k), torch.uint8, "dropped"), _ptr(gate_eff, (N, k), f32, "gate_eff"),
                              _ptr(token_of_row, (rows,), i32, "token_of_row"),
                              _ptr(x_perm, (rows, D), _tdtype(d), "x_perm"), ps, sb, _stream(stream)),
           "moe_dispatch")


def moe_expert_ffn(d, x_perm, offsets, counts, w1, w2, w3, h, y_perm, scratch, stream=None):
    D, F, E = d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_ffn(ctypes.byref(d), _ptr(x_perm, (rows, D), dt, "x_perm"),
                                _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                                _ptr(counts, (E,), torch.int32, "counts"),
                                _ptr(w1, (E, D, F), dt, "w1"), _ptr(w2, (E, D, F), dt, "w2"),
                                _ptr(w3, (E, F, D), dt, "w3"), _ptr(h, (rows, F), dt, "h"),
                                _ptr(y_perm, (rows, D), dt, "y_perm"), ps, sb, _stream(stream)), "moe_expert_ffn")


def moe_expert_up(d, x_perm, offsets, counts, w1, w2, h, scratch, stream=None):
    D, F, E = d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_up(ctypes.byref(d), _ptr(x_perm, (rows, D), dt, "x_perm"),
                               _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                               _ptr(counts, (E,), torch.int32, "counts"),
                               _ptr(w1, (E, D, F), dt, "w1"), _ptr(w2, (E, D, F), dt, "w2"),
                               _ptr(h, (rows, F), dt, "h"), ps, sb, _stream(stream)), "moe_expert_up")


def moe_expert_up_gathered(d, x, token_of_row, offsets, counts, w1, w2, h, scratch, stream=None):
    N, D, F, E = d.N, d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_up_gathered(ctypes.byref(d), _ptr(x, (N, D), dt, "x"),
                                        _ptr(token_of_row, (rows,), torch.int32, "token_of_row"),
                                        _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                                        _ptr(counts, (E,), torch.int32, "counts"),
                                        _ptr(w1, (E, D, F), dt, "w1"), _ptr(w2, (E, D, F), dt, "w2"),
                                        _ptr(h, (rows, F), dt, "h"), ps, sb, _stream(stream)),
           "moe_expert_up_gathered")


def moe_expert_down(d, h, offsets, counts, w3, y_perm, scratch, stream=None):
    D, F, E = d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_down(ctypes.byref(d), _ptr(h, (rows, F), dt, "h"),
                                 _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                                 _ptr(counts, (E,), torch.int32, "counts"),
                                 _ptr(w3, (E, F, D), dt, "w3"), _ptr(y_perm, (rows, D), dt, "y_perm"), ps, sb,
                                 _stream(stream)), "moe_expert_down")


def moe_combine(d, y_perm, row_of, gate_eff, y, stream=None):
    N, D, k = d.N, d.D, d.k
    rows = moe_rows(d)
    dt = _tdtype(d)
    _check(lib().moe_combine(ctypes.byref(d), _ptr(y_perm, (rows, D), dt, "y_perm"),
                             _ptr(row_of, (N, k), torch.int32, "row_of"),
                             _ptr(gate_eff, (N, k), torch.float32, "gate_eff"), _ptr(y, (N, D), dt, "y"),
                             _stream(stream)), "moe_combine")


def moe_forward(d, x, w_r, logit_bias, noise, w1, w2, w3, y, workspace, stream=None):
    N, D, F, E = d.N, d.D, d.F, d.E
    dt = _tdtype(d)
    pw, wb = _bytes_ptr(workspace, moe_workspace_size(d), "workspace")
    _check(lib().moe_forward(ctypes.byref(d), _ptr(x, (N, D), dt, "x"), _ptr(w_r, (D, E), torch.float32, "w_r"),
                             _ptr(logit_bias, (E,), torch.float32, "logit_bias", optional=True),
                             _ptr(noise, (N, E), torch.float32, "noise", optional=(d.second_choice == 0)),
                             _ptr(w1, (E, D, F), dt, "w1"), _ptr(w2, (E, D, F), dt, "w2"),
                             _ptr(w3, (E, F, D), dt, "w3"), _ptr(y, (N, D), dt, "y"), pw, wb, _stream(stream)),
           "moe_forward")


def moe_forward_noalloc(d, x, w_r, logit_bias, noise, w1, w2, w3, y, stream=None):
    """moe_forward with the library's static per-GPU workspace (no workspace argument)."""
    N, D, F, E = d.N, d.D, d.F, d.E
    dt = _tdtype(d)
    _check(lib().moe_forward_noalloc(ctypes.byref(d), _ptr(x, (N, D), dt, "x"), _ptr(w_r, (D, E), torch.float32, "w_r"),
                                     _ptr(logit_bias, (E,), torch.float32, "logit_bias", optional=True),
                                     _ptr(noise, (N, E), torch.float32, "noise", optional=(d.second_choice == 0)),
                                     _ptr(w1, (E, D, F), dt, "w1"), _ptr(w2, (E, D, F), dt, "w2"),
                                     _ptr(w3, (E, F, D), dt, "w3"), _ptr(y, (N, D), dt, "y"), _stream(stream)),
           "moe_forward_noalloc")


# ---- weight-only 8-bit experts: int8 W [E, K, N] with fp32 column scales s [E, N] --------

def _q8(w, s, E, K, N, name):
    return (_ptr(w, (E, K, N), torch.int8, name), _ptr(s, (E, N), torch.float32, "scales of " + name))


def moe_expert_up_q8(d, x_perm, offsets, counts, w1, s1, w2, s2, h, scratch, stream=None):
    D, F, E = d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_up_q8(ctypes.byref(d), _ptr(x_perm, (rows, D), dt, "x_perm"),
                                  _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                                  _ptr(counts, (E,), torch.int32, "counts"), *_q8(w1, s1, E, D, F, "w1"),
                                  *_q8(w2, s2, E, D, F, "w2"), _ptr(h, (rows, F), dt, "h"), ps, sb, _stream(stream)),
           "moe_expert_up_q8")


def moe_expert_down_q8(d, h, offsets, counts, w3, s3, y_perm, scratch, stream=None):
    D, F, E = d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_down_q8(ctypes.byref(d), _ptr(h, (rows, F), dt, "h"),
                                    _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                                    _ptr(counts, (E,), torch.int32, "counts"), *_q8(w3, s3, E, F, D, "w3"),
                                    _ptr(y_perm, (rows, D), dt, "y_perm"), ps, sb, _stream(stream)),
           "moe_expert_down_q8")


def moe_expert_ffn_q8(d, x_perm, offsets, counts, w1, s1, w2, s2, w3, s3, h, y_perm, scratch, stream=None):
    D, F, E = d.D, d.F, d.E
    rows = moe_rows(d)
    dt = _tdtype(d)
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    _check(lib().moe_expert_ffn_q8(ctypes.byref(d), _ptr(x_perm, (rows, D), dt, "x_perm"),
                                   _ptr(offsets, (E + 1,), torch.int32, "offsets"),
                                   _ptr(counts, (E,), torch.int32, "counts"), *_q8(w1, s1, E, D, F, "w1"),
                                   *_q8(w2, s2, E, D, F, "w2"), *_q8(w3, s3, E, F, D, "w3"),
                                   _ptr(h, (rows, F), dt, "h"), _ptr(y_perm, (rows, D), dt, "y_perm"), ps, sb,
                                   _stream(stream)), "moe_expert_ffn_q8")


def moe_forward_q8(d, x, w_r, logit_bias, noise, w1, s1, w2, s2, w3, s3, y, workspace, stream=None):
    N, D, F, E = d.N, d.D, d.F, d.E
    dt = _tdtype(d)
    pw, wb = _bytes_ptr(workspace, moe_workspace_size(d), "workspace")
    _check(lib().moe_forward_q8(ctypes.byref(d), _ptr(x, (N, D), dt, "x"), _ptr(w_r, (D, E), torch.float32, "w_r"),
                                _ptr(logit_bias, (E,), torch.float32, "logit_bias", optional=True),
                                _ptr(noise, (N, E), torch.float32, "noise", optional=(d.second_choice == 0)),
                                *_q8(w1, s1, E, D, F, "w1"), *_q8(w2, s2, E, D, F, "w2"), *_q8(w3, s3, E, F, D, "w3"),
                                _ptr(y, (N, D), dt, "y"), pw, wb, _stream(stream)), "moe_forward_q8")


def moe_read_stats(d, scratch, stream=None) -> dict:
    ps, sb = _bytes_ptr(scratch, moe_scratch_size(d), "scratch")
    st = moe_stats()
    _check(lib().moe_read_stats(ctypes.byref(d), ps, sb, ctypes.byref(st), _stream(stream)), "moe_read_stats")
    return st.as_dict()


# ---- convenience ------------------------------------------------------------------------------

def workspace_views(d: moe_desc, ws: torch.Tensor) -> dict:
    """Typed views of the intermediates inside a moe_forward workspace (uint8 tensor)."""
    L = moe_workspace_layout(d)
    N, D, F, E, k = d.N, d.D, d.F, d.E, d.k
    rows = moe_rows(d)
    dt = _tdtype(d)
    es = 2 if dt == torch.bfloat16 else 4

    def view(off, nbytes, dtype, shape):
        return ws[off:off + nbytes].view(dtype).view(*shape)

    return {
        "scratch": ws[L.scratch:L.scratch + moe_scratch_size(d)],
        "topk_idx": view(L.topk_idx, 4 * N * k, torch.int32, (N, k)),
        "topk_gate": view(L.topk_gate, 4 * N * k, torch.float32, (N, k)),
        "load": view(L.load, 4 * E, torch.int32, (E,)),
        "counts": view(L.counts, 4 * E, torch.int32, (E,)),
        "offsets": view(L.offsets, 4 * (E + 1), torch.int32, (E + 1,)),
        "row_of": view(L.row_of, 4 * N * k, torch.int32, (N, k)),
        "dropped": view(L.dropped, N * k, torch.uint8, (N, k)),
        "gate_eff": view(L.gate_eff, 4 * N * k, torch.float32, (N, k)),
        "token_of_row": view(L.token_of_row, 4 * rows, torch.int32, (rows,)),
        "x_perm": view(L.x_perm, es * rows * D, dt, (rows, D)),
        "h": view(L.h, es * rows * F, dt, (rows, F)),
        "y_perm": view(L.y_perm, es * rows * D, dt, (rows, D)),
    }


class MoELayer:
    """A workload's tensors on the device plus a workspace, calling moe_forward."""

    def __init__(self, cfg: dict, inputs: dict, device="cuda"):
        self.cfg = cfg
        self.desc = make_desc(cfg)
        dev = torch.device(device)
        self.x = inputs["x"].to(dev)
        self.w_r = inputs["w_r"].to(dev)
        self.w1, self.w2, self.w3 = (inputs[n].to(dev) for n in ("w1", "w2", "w3"))
        self.q8 = cfg.get("weight_dtype", "same") == "int8"  # int8 weights + column scales
        self.s1, self.s2, self.s3 = ((inputs[n].to(dev) for n in ("s1", "s2", "s3")) if self.q8 else (None,) * 3)
        self.bias = None if inputs.get("logit_bias") is None else inputs["logit_bias"].to(dev)
        self.noise = None if inputs.get("noise") is None else inputs["noise"].to(dev)
        self.y = torch.empty_like(self.x)
        self.ws = torch.empty(moe_workspace_size(self.desc), dtype=torch.uint8, device=dev)

    def forward(self, stream=None):
        if self.q8:
            moe_forward_q8(self.desc, self.x, self.w_r, self.bias, self.noise, self.w1, self.s1, self.w2, self.s2,
                           self.w3, self.s3, self.y, self.ws, stream)
        else:
            moe_forward(self.desc, self.x, self.w_r, self.bias, self.noise, self.w1, self.w2, self.w3, self.y,
                        self.ws, stream)
        return self.y

    def expert_up(self, x_perm, offsets, counts, h, scratch, stream=None):
        if self.q8:
            moe_expert_up_q8(self.desc, x_perm, offsets, counts, self.w1, self.s1, self.w2, self.s2, h, scratch, stream)
        else:
            moe_expert_up(self.desc, x_perm, offsets, counts, self.w1, self.w2, h, scratch, stream)

    def expert_down(self, h, offsets, counts, y_perm, scratch, stream=None):
        if self.q8:
            moe_expert_down_q8(self.desc, h, offsets, counts, self.w3, self.s3, y_perm, scratch, stream)
        else:
            moe_expert_down(self.desc, h, offsets, counts, self.w3, y_perm, scratch, stream)

    def views(self):
        return workspace_views(self.desc, self.ws)

    def stats(self):
        return moe_read_stats(self.desc, self.views()["scratch"])
