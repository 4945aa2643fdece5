"""Host-side logic around the library (CPU): the benchmark's one-GPU contract, the
profile summariser's kernel naming, the seeded inputs, and the binding's argument checks."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mixture_experts_layer_wave_amd import binding as B  # noqa: E402
from mixture_experts_layer_wave_amd import configs, inputs, profiling  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,base,args,stage", [
    ("void moe::(anonymous namespace)::k_gemm_bf16<256, 128, 2, 0, 64, 2, false, false>(moe::GemmParams)",
     "k_gemm_bf16", [256, 128, 2, 0, 64, 2, 0, 0], "expert_up"),
    ("_ZN3moe12_GLOBAL__N_111k_gemm_bf16ILi64ELi256ELi1ELi0ELi64ELi4ELb1ELb0EEEvNS_10GemmParamsE",
     "k_gemm_bf16", [64, 256, 1, 0, 64, 4, 1, 0], "expert_down"),
    ("void moe::(anonymous namespace)::k_gemm_bf16<256, 128, 2, 0, 64, 2, false, false, false>(moe::GemmParams)",
     "k_gemm_bf16", [256, 128, 2, 0, 64, 2, 0, 0, 0], "expert_up"),
    # gathered-row instance: moe_forward and moe_expert_up_gathered
    ("void moe::(anonymous namespace)::k_gemm_bf16<256, 128, 2, 1, 64, 2, false, false, true>(moe::GemmParams)",
     "k_gemm_bf16", [256, 128, 2, 1, 64, 2, 0, 0, 1], "expert_up"),
    ("void moe::(anonymous namespace)::k_gemm_skinny_dual<0>(moe::GemmParams)", "k_gemm_skinny_dual", [0],
     "expert_up"),
    ("k_gemm_streamk_reduce<64, 128, 2, 0, 64, false>", "k_gemm_streamk_reduce", [64, 128, 2, 0, 64, 0], "expert_up"),
    # mixed-height launches: <ACT, NB, BNF_B, BNF_S, BK_S, STAGES_S, GA> and their fix-up
    ("void moe::(anonymous namespace)::k_gemm_mixed<0, 2, 128, 256, 32, 4, true>(moe::GemmParams)", "k_gemm_mixed",
     [0, 2, 128, 256, 32, 4, 1], "expert_up"),
    ("void moe::(anonymous namespace)::k_gemm_mixed<0, 1, 256, 256, 64, 4, false>(moe::GemmParams)", "k_gemm_mixed",
     [0, 1, 256, 256, 64, 4, 0], "expert_down"),
    ("_ZN3moe12_GLOBAL__N_119k_gemm_mixed_reduceILi0ELi1ELi256ELi256ELi64EEEvNS_10GemmParamsEi",
     "k_gemm_mixed_reduce", [0, 1, 256, 256, 64], "expert_down"),
    ("void moe::(anonymous namespace)::k_router_epi<8>(moe::RouterArgs, moe::RouterSplit)", "k_router_epi", [8],
     "route"),
    ("k_route_dispatch_small<8>", "k_route_dispatch_small", [8], "forward"),
    ("void moe::(anonymous namespace)::k_router_tok<8, 2>(moe::RouterArgs)", "k_router_tok", [8, 2], "route"),
    ("k_dispatch_small", "k_dispatch_small", [], "dispatch"),
    ("void moe::(anonymous namespace)::k_combine<__bf16>(moe::CombineArgs, int)", "k_combine", [], "combine"),
    ("__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer", [], "other"),
])
def test_profile_kernel_names(name, base, args, stage):
    assert profiling.parse_kernel(name) == (base, args)
    assert profiling.stage_of(name) == stage


def test_source_hash_is_stable():
    assert profiling.source_hash() == profiling.source_hash()
    assert len(profiling.source_hash()) == 16


def test_inputs_are_seeded_and_shaped():
    cfg = configs.scaled_config("gshard_capacity", N=96, D=128, F=192, E=8)
    a, b = inputs.make_inputs(cfg), inputs.make_inputs(cfg)
    assert set(a) == set(b)
    for k in a:
        if isinstance(a[k], torch.Tensor):
            assert torch.equal(a[k], b[k]), k
    assert tuple(a["x"].shape) == (96, 128) and a["x"].dtype == torch.bfloat16
    assert tuple(a["w1"].shape) == (8, 128, 192) and tuple(a["w3"].shape) == (8, 192, 128)
    assert tuple(a["w_r"].shape) == (128, 8) and a["w_r"].dtype == torch.float32
    assert tuple(a["noise"].shape) == (96, 8)
    c = inputs.make_inputs(dict(cfg, seed=cfg["seed"] + 1))
    assert not torch.equal(a["x"], c["x"])
    q = inputs.make_inputs(dict(cfg, weight_dtype="int8"))
    assert q["w1"].dtype == torch.int8 and int(q["w1"].abs().max()) <= 127
    assert tuple(q["s1"].shape) == (8, 192) and tuple(q["s3"].shape) == (8, 128)
    assert bool(torch.all(q["s1"] > 0))


def test_binding_rejects_host_and_mis_shaped_tensors():
    with pytest.raises(ValueError, match="device tensor"):
        B._ptr(torch.zeros(4), (4,), torch.float32, "x")
    with pytest.raises(ValueError, match="required"):
        B._ptr(None, (4,), torch.float32, "x")
    assert B._ptr(None, (4,), torch.float32, "x", optional=True) is None


def test_configs_scaled_names_and_fields():
    c = configs.scaled_config("mixtral_decode", N=64, D=512, F=384)
    assert c["N"] == 64 and c["D"] == 512 and c["F"] == 384 and c["E"] == 8
    assert "mixtral_decode" in c["name"]
    for name in configs.ORDER:
        g = configs.get_config(name)
        assert g["D"] % 64 == 0 and g["F"] % 64 == 0 and 1 <= g["k"] <= g["E"]
    assert np.isclose(configs.get_config("gshard_capacity")["capacity_factor"], 1.25)


def test_source_hash_ignores_comments_only():
    a = "int f(int x) { return x + 1; }  // add one\n/* block\n comment */"
    b = "int f(int x) {\n  return x + 1;\n}"
    c = "int f(int x) { return x + 2; }"
    assert profiling._code_only(a) == profiling._code_only(b)
    assert profiling._code_only(a) != profiling._code_only(c)
