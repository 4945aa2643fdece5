"""The C-ABI library on the host (no GPU work): it loads, exports every entry point that
include/moe.h declares, answers the host-only queries, and rejects invalid arguments
before launching anything."""
import ctypes
import os
import re

import pytest

import oracle_pins
from mixture_experts_layer_wave_amd import binding as B
from mixture_experts_layer_wave_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from mixture_experts_layer_wave_amd.build import build_library
        build_library(verbose=False)
    return B.lib()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^MOE_API\s+[\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_entry_point(L):
    names = declared()
    assert len(names) >= 14
    assert sorted(names) == sorted(B.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    cfg = configs.get_config("mixtral_prefill")
    cfg.update(kw)
    return B.make_desc(cfg)


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4):
        assert B.status_string(code).startswith("MOE_")
    assert "unknown" in B.status_string(7)


def test_capacity_examples_through_abi(L):
    g = oracle_pins.golden("capacity_examples.json")
    for c in g["cases"]:
        if c["N"] < 1:
            continue
        d = _desc(N=c["N"], E=c["E"], k=c["k"], capacity_mode="padded", capacity_factor=c["cf"],
                  min_capacity=c["min_capacity"])
        assert B.moe_capacity(d) == c["C"], c
    for c in g["invalid"]:
        d = _desc(N=c["N"], E=max(c["E"], 0), k=c["k"], capacity_mode="padded", capacity_factor=c["cf"])
        with pytest.raises(B.MoeError) as ei:
            B.moe_capacity(d)
        assert ei.value.status == B.MOE_E_INVAL
    assert B.moe_capacity(_desc(N=100)) == 100  # no capacity limit: C = N


def test_switch_capacity_examples_through_abi(L):
    g = oracle_pins.golden("switch_capacity_examples.json")
    for c in g["cases"]:
        d = _desc(N=c["N"], E=c["E"], k=c["k"], capacity_mode="padded", capacity_factor=c["cf"],
                  min_capacity=c["min_capacity"], capacity_formula="tokens")
        assert B.moe_capacity(d) == c["C"], c
    for c in g["invalid"]:
        d = _desc(N=c["N"], E=max(c["E"], 0), k=c["k"], capacity_mode="padded", capacity_factor=c["cf"],
                  capacity_formula="tokens")
        with pytest.raises(B.MoeError) as ei:
            B.moe_capacity(d)
        assert ei.value.status == B.MOE_E_INVAL


def test_rows_and_sizes(L):
    d5 = B.make_desc(configs.get_config("gshard_capacity"))
    assert B.moe_capacity(d5) == 640
    assert B.moe_rows(d5) == 64 * 640
    d2 = B.make_desc(configs.get_config("mixtral_prefill"))
    assert B.moe_rows(d2) == 4096 * 2
    for d in (d2, d5):
        Lw = B.moe_workspace_layout(d)
        offs = [getattr(Lw, n) for n, _ in Lw._fields_]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert Lw.total == B.moe_workspace_size(d)
        rows = B.moe_rows(d)
        assert Lw.h - Lw.x_perm >= rows * d.D * 2
        assert Lw.total - Lw.y_perm >= rows * d.D * 2
        assert B.moe_scratch_size(d) <= Lw.topk_idx


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), B.MOE_E_INVAL), (dict(k=0), B.MOE_E_INVAL), (dict(k=9, E=8), B.MOE_E_INVAL),
    (dict(E=65, k=2), B.MOE_E_UNSUPPORTED), (dict(E=16, k=9), B.MOE_E_UNSUPPORTED),
    (dict(D=4000), B.MOE_E_UNSUPPORTED), (dict(F=100), B.MOE_E_UNSUPPORTED),
    (dict(capacity_mode="padded", capacity_factor=0.0), B.MOE_E_INVAL),
    (dict(capacity_mode="padded", capacity_factor=1.0, min_capacity=-1), B.MOE_E_INVAL),
])
def test_invalid_desc_rejected(L, kw, status):
    d = _desc(**kw)
    rc = L.moe_scratch_size(ctypes.byref(d), ctypes.byref(ctypes.c_size_t()))
    assert rc == status
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    rc = L.moe_combine(ctypes.byref(d), fake, fake, fake, fake, None)
    assert rc == status


def test_bad_enums_rejected(L):
    for field, val in (("dtype", 5), ("routing_mode", 2), ("second_choice", 3), ("activation", 9),
                       ("capacity_mode", 4), ("capacity_priority", 2), ("capacity_formula", -1),
                       ("second_choice", -1)):
        d = _desc()
        setattr(d, field, val)
        assert L.moe_rows(ctypes.byref(d), ctypes.byref(ctypes.c_int64())) == B.MOE_E_INVAL, field


def test_null_and_misaligned_pointers_rejected(L):
    d = _desc()
    p = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)
    n = None
    # moe_route: idx/gate required
    assert L.moe_route(ctypes.byref(d), p, p, n, n, n, n, n, n, p, n, 0, n) == B.MOE_E_INVAL
    assert L.moe_route(ctypes.byref(d), p, odd, n, n, n, n, n, p, p, n, 0, n) == B.MOE_E_INVAL
    # noisy routing needs noise
    dn = _desc(second_choice="noisy")
    assert L.moe_route(ctypes.byref(dn), p, p, n, n, n, n, n, p, p, n, 0, n) == B.MOE_E_INVAL
    # dispatch: x_perm missing
    assert L.moe_dispatch(ctypes.byref(d), p, p, p, p, p, p, p, p, p, p, n, p, 1 << 30, n) == B.MOE_E_INVAL
    # combine: y missing
    assert L.moe_combine(ctypes.byref(d), p, p, p, n, n) == B.MOE_E_INVAL
    # forward: w3 missing
    assert L.moe_forward(ctypes.byref(d), p, p, n, n, p, p, n, p, p, 1 << 40, n) == B.MOE_E_INVAL


def test_short_workspace_rejected(L):
    d = _desc()
    p = ctypes.c_void_p(0x10000)
    n = None
    need = B.moe_workspace_size(d)
    assert L.moe_forward(ctypes.byref(d), p, p, n, n, p, p, p, p, p, need - 1, n) == B.MOE_E_WORKSPACE
    assert L.moe_forward(ctypes.byref(d), p, p, n, n, p, p, p, p, n, need, n) == B.MOE_E_WORKSPACE
    s = B.moe_scratch_size(d)
    assert L.moe_dispatch(ctypes.byref(d), p, p, p, p, p, p, p, p, p, p, p, p, s - 1, n) == B.MOE_E_WORKSPACE
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, p, p, p, p, p, p, n, s, n) == B.MOE_E_WORKSPACE
    assert L.moe_expert_up(ctypes.byref(d), p, p, p, p, p, p, p, s - 16, n) == B.MOE_E_WORKSPACE
    assert L.moe_expert_down(ctypes.byref(d), p, p, p, p, p, n, s, n) == B.MOE_E_WORKSPACE
    assert L.moe_route(ctypes.byref(d), p, p, n, n, n, n, n, p, p, p, s - 1, n) == B.MOE_E_WORKSPACE
    st = B.moe_stats()
    assert L.moe_read_stats(ctypes.byref(d), p, s - 1, ctypes.byref(st), n) == B.MOE_E_WORKSPACE
