"""The layer's forward captured in a HIP graph and replayed (GPU).

The library launches only kernels on the caller's stream (no allocation, no memset, no
synchronisation), so one moe_forward call can be captured and replayed. Every replay is
checked bit for bit against the eager result, with eager work of the program between the
replays and the output overwritten before each one.
"""
import pytest
import torch

from mixture_experts_layer_wave_amd import binding as B
from mixture_experts_layer_wave_amd import configs, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [
    configs.scaled_config("mixtral_decode", N=64, D=512, F=384),
    configs.scaled_config("mixtral_prefill", N=700, D=256, F=512),
    configs.scaled_config("gshard_capacity", N=900, D=256, F=384, E=16),
    configs.scaled_config("mixtral_decode_int8", N=64, D=512, F=384),
    # mixed tile heights with both shares (small remainders on 64-row tiles)
    configs.scaled_config("mixtral_prefill", N=1100, D=256, F=512, name="mixed_heights"),
], ids=lambda c: c["name"])
def test_forward_graph_replays_equal_eager(cfg):
    inp = inputs.make_inputs(cfg)
    layer = B.MoELayer(cfg, inp)
    y_eager = layer.forward().clone()
    v = layer.views()
    eager_rows = v["row_of"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward()
    torch.cuda.synchronize()
    other = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        layer.y.fill_(float("nan"))
        v["row_of"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, y_eager), f"replay {rep}"
        assert torch.equal(v["row_of"], eager_rows), f"replay {rep}"
        other = other @ other.t() / 512.0  # eager work between replays
        layer.forward()  # and an eager pass on the same buffers
        torch.cuda.synchronize()
        assert torch.equal(layer.y, y_eager)
