"""The forward without a caller workspace (moe_forward_noalloc, for callers that cannot
allocate: HIP graph capture, tight serving loops) against moe_forward with a workspace
of its own: equal bit for bit on consecutive calls, each later call with a smaller input
than the one before (the static workspace keeps the previous call's contents), and
rejected on the host when the layer's workspace exceeds the static array."""
import ctypes

import pytest
import torch

from mixture_experts_layer_wave_amd import binding as B
from mixture_experts_layer_wave_amd import configs, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(cfg):
    inp = inputs.make_inputs(cfg)
    layer = B.MoELayer(cfg, inp, device=DEV)
    y_ref = layer.forward().clone()
    y = torch.full_like(layer.y, 7.0)
    B.moe_forward_noalloc(layer.desc, layer.x, layer.w_r, layer.bias, layer.noise, layer.w1, layer.w2, layer.w3, y)
    torch.cuda.synchronize()
    return y_ref, y


def test_noalloc_equals_forward_on_consecutive_calls():
    cases = [
        # capacity routing (GShard drops, padded buffers), then the same layer on fewer
        # tokens, then a decode-sized batch through the fused small-batch dispatch
        configs.scaled_config("gshard_capacity", N=1000, D=512, F=1024, E=16, name="gshard_n1000"),
        configs.scaled_config("gshard_capacity", N=300, D=512, F=1024, E=16, name="gshard_n300"),
        configs.scaled_config("mixtral_decode", N=64, D=512, F=384, name="decode_n64"),
        configs.scaled_config("mixtral_prefill", N=40, D=256, F=256, name="prefill_n40"),
    ]
    for cfg in cases:
        need = B.moe_workspace_size(B.make_desc(cfg))
        assert need <= (128 << 20), (cfg["name"], need)
        y_ref, y = _both(cfg)
        assert torch.equal(y, y_ref), f"{cfg['name']}: no-allocation forward differs from moe_forward"
        print(f"[{cfg['name']}] workspace {need / 2 ** 20:.1f} MiB: equal bit for bit", flush=True)


def test_noalloc_rejects_a_workspace_beyond_the_static_array():
    cfg = configs.scaled_config("mixtral_prefill", N=4096, D=4096, F=14336, name="prefill_full")
    d = B.make_desc(cfg)
    assert B.moe_workspace_size(d) > (128 << 20)
    # host-side check: nothing is launched, the (dummy, aligned) pointers are never touched
    buf = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    p = ctypes.c_void_p(buf.data_ptr())
    rc = B.lib().moe_forward_noalloc(ctypes.byref(d), p, p, None, None, p, p, p, p, None)
    assert rc == B.MOE_E_WORKSPACE
