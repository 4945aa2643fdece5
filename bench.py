"""Benchmark of the MoE-layer forward on one MI355X.

A step is one pass of the whole hot path over one batch of seeded synthetic input that
is already resident in HBM: router (fp32 logits, softmax, top-k, gates) -> dispatch
(histogram, capacity slots, drop rule, gather) -> gated up-projection grouped GEMM ->
down-projection grouped GEMM -> combine, as one moe_forward call. W untimed warm-up steps,
then exactly K timed steps between two device synchronisations give the throughput.
K more steps through the per-stage entry points (the same kernels), with HIP events
recorded on the launch stream between the stages, give each stage's duration.

Prints one JSON line: tokens/s, the roofline of the dominant kernel, the routing
statistics of the last forward (balance loss, drop rates) beside the oracle's, the
weight-streaming decode regime of the same expert shapes (the mixtral_decode workload,
`decode` key), and the fp64 CPU oracle timed on a bounded sample of the same workload on
the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak), Mixtral-shaped"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
STAGES = ["route", "dispatch", "expert_up", "expert_down", "combine"]


def gemm_kernel_of(cfg, stage: str, gathered: bool, capacity) -> str:
    """Name of the grouped-GEMM kernel the library launches for a stage of this workload
    (the launch rules of gemm_bf16.hip: fp32 layers, int8 weights, the skinny regime of at
    most 64 rows per expert, and mixed tile heights when the output width is a multiple of
    256). capacity: the library's C for padded layers, else None."""
    what = "gated up-projection" if stage == "expert_up" else "down-projection"
    if cfg["dtype"] == "f32":
        return f"k_gemm_f32 ({what})"
    max_rows = min(cfg["N"], capacity) if capacity is not None else cfg["N"]
    width = cfg["F"] if stage == "expert_up" else cfg["D"]
    if max_rows <= 64:
        if stage == "expert_up" and width % 256 == 0 and cfg.get("weight_dtype", "same") != "int8":
            return f"k_gemm_skinny_dual ({what}, 64-row tiles of two widths)"
        return f"k_gemm_bf16 ({what}, 64-row stream-K tiles)"
    if cfg.get("weight_dtype", "same") == "int8":
        if stage == "expert_up" and width % 256 == 0:
            return f"k_gemm_mixed ({what}, int8 weights, 256-row tiles, small remainders on 64-row tiles)"
        return f"k_gemm_bf16 ({what}, int8 weights)"
    if width % 256 == 0:
        rows = "rows gathered from x, " if gathered else ""
        return f"k_gemm_mixed ({what}, {rows}256-row tiles, small remainders on 64-row tiles)"
    return f"k_gemm_bf16 ({what})"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral_prefill")
    p.add_argument("--cpu-sample", type=int, default=2048, help="tokens in the oracle's timed FFN sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    p.add_argument("--no-decode", dest="decode", action="store_false",
                   help="skip the decode-regime measurement (the mixtral_decode workload, same run)")
    p.add_argument("--cold-reps", type=int, default=5,
                   help="cold-cache runs of each small stage before the warm-up (0: none)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="instead of the bench: run a device copy of this many MiB `steps` times "
                        "(calibration of the memory-traffic counters)")
    p.add_argument("--copy-kind", choices=("lds", "blit"), default="lds",
                   help="calibration copy: reads by direct-to-LDS copies, the GEMMs' read path (lds), or "
                        "the runtime's blit kernel (blit)")
    return p.parse_args()


def traffic_from_profiles(workload: str, kernel_stage: str):
    """Memory-side bytes per launch (L2 misses and write-backs, Infinity Cache or HBM) from
    the committed rocprofv3 counter summary, if it was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from mixture_experts_layer_wave_amd.profiling import source_hash
    if t.get("source_hash") != source_hash():
        return None
    st = t.get("stages", {}).get(kernel_stage)
    return None if st is None else st.get("memory_bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, sample: int, sample_1t: int = 64):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload, on all
    host threads and (a smaller sample) on one thread."""
    import numpy as np
    from oracle import default_oracle
    orc = default_oracle()
    threads = orc.set_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    N = cfg["N"]
    t0 = time.perf_counter()
    logits = orc.router_logits(inp["x"], inp["w_r"], inp["logit_bias"])
    sc = cfg["second_choice"]
    r = orc.route(logits, cfg["k"], cfg["routing_mode"], inp["noise"] if sc != "topk" else None,
                  noise_all=sc == "noisy_all")
    padded = cfg["capacity_mode"] == "padded"
    C = (orc.capacity(N, cfg["E"], cfg["k"], cfg["capacity_factor"], cfg["min_capacity"], cfg["capacity_formula"])
         if padded else None)
    o = orc.dispatch(r.idx, r.gate, cfg["E"], C, padded, token_major=cfg["capacity_priority"] == "token_major")
    t1 = time.perf_counter()
    scales = (inp["s1"], inp["s2"], inp["s3"]) if "s1" in inp else None
    toks = np.linspace(0, N - 1, min(sample, N)).astype(np.int64)
    orc.layer_tokens(toks, inp["x"], inp["w1"], inp["w2"], inp["w3"], r.idx, o.dropped, o.gate_eff,
                     cfg["activation"], scales=scales)
    t2 = time.perf_counter()
    n = len(toks)
    per_tok = (t1 - t0) / N + (t2 - t1) / n
    # one thread, on the first tokens of the same sample
    orc.set_threads(1)
    toks1 = toks[: min(sample_1t, n)]
    t3 = time.perf_counter()
    orc.layer_tokens(toks1, inp["x"], inp["w1"], inp["w2"], inp["w3"], r.idx, o.dropped, o.gate_eff,
                     cfg["activation"], scales=scales)
    t4 = time.perf_counter()
    orc.set_threads(threads)
    per_tok_1 = (t1 - t0) * threads / N + (t4 - t3) / len(toks1)
    # the oracle's routing statistics of the same workload (its own exact logits)
    _, bal, bal_n = orc.balance(r.probs, o.load, cfg["k"])
    drops = int(o.dropped.sum())
    gone = int(np.all(o.dropped == 1, axis=1).sum())
    stats = {"balance_loss": bal, "balance_loss_div_n": bal_n, "drop_rate": drops / (N * cfg["k"]),
             "token_drop_rate": gone / N, "dropped_slots": drops, "dropped_tokens": gone}
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": _cpu_model(), "nproc": os.cpu_count(),
            "value_1thread": 1.0 / per_tok_1, "routing_stats": stats,
            "sample": f"router+softmax+top-k+dispatch of all {N} tokens ({t1 - t0:.2f} s), expert FFN + combine "
                      f"of {n} evenly spaced tokens ({t2 - t1:.2f} s); rate = 1 / (route time per token + "
                      f"FFN time per token). value_1thread: FFN of the first {len(toks1)} of those tokens on one "
                      f"thread ({t4 - t3:.2f} s), routing time scaled by the thread count"}


def measure_layer(B, cfg, inp, args, dev, cold_reps: int, graph: bool) -> dict:
    """Times one workload on the GPU: K moe_forward calls between two synchronisations (the
    throughput), then K passes through the per-stage entry points running the same kernels
    as the forward (the up-projection through moe_expert_up_gathered wherever the forward
    reads its rows from x), with HIP events recorded on the launch stream between stages."""
    import numpy as np
    import torch
    layer = B.MoELayer(cfg, inp, device=dev)
    d = layer.desc
    N, D, F, E, k = cfg["N"], cfg["D"], cfg["F"], cfg["E"], cfg["k"]
    rows = B.moe_rows(d)
    v = layer.views()
    sc = v["scratch"]
    stream = torch.cuda.current_stream()
    q8 = cfg.get("weight_dtype", "same") == "int8"

    def up_gathered():
        B.moe_expert_up_gathered(d, layer.x, v["token_of_row"], v["offsets"], v["counts"], layer.w1, layer.w2, v["h"],
                                 sc)

    def up_plain():
        layer.expert_up(v["x_perm"], v["offsets"], v["counts"], v["h"], sc)

    def step(ev=None, up=up_plain):
        if ev is not None:
            ev[0].record(stream)
        B.moe_route(d, layer.x, layer.w_r, layer.bias, layer.noise, None, None, None, v["topk_idx"], v["topk_gate"],
                    sc)
        if ev is not None:
            ev[1].record(stream)
        B.moe_dispatch(d, layer.x, v["topk_idx"], v["topk_gate"], v["load"], v["counts"], v["offsets"], v["row_of"],
                       v["dropped"], v["gate_eff"], v["token_of_row"], v["x_perm"], sc)
        if ev is not None:
            ev[2].record(stream)
        up()
        if ev is not None:
            ev[3].record(stream)
        layer.expert_down(v["h"], v["offsets"], v["counts"], v["y_perm"], sc)
        if ev is not None:
            ev[4].record(stream)
        B.moe_combine(d, v["y_perm"], v["row_of"], v["gate_eff"], layer.y)
        if ev is not None:
            ev[5].record(stream)

    step()  # every stage's inputs exist from here on
    # The instance of the up-projection the forward runs: rows read from x through
    # token_of_row (bf16 weights, experts that may exceed 64 rows), else x_perm.
    up = up_plain
    if not q8:
        try:
            up_gathered()
            up = up_gathered
        except B.MoeError as err:
            if err.status != B.MOE_E_UNSUPPORTED:
                raise
    # Small stages alone, each after writing a 512 MB buffer so the last-level cache holds
    # none of their inputs (the timed steps below give the warm numbers). Run before the
    # warm-up so the timed steps are the last calls of every kernel.
    cold_ms = {}
    if cold_reps > 0:
        flush = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        small_fn = {
            "route": lambda: B.moe_route(d, layer.x, layer.w_r, layer.bias, layer.noise, None, None, None,
                                         v["topk_idx"], v["topk_gate"], sc),
            "dispatch": lambda: B.moe_dispatch(d, layer.x, v["topk_idx"], v["topk_gate"], v["load"], v["counts"],
                                               v["offsets"], v["row_of"], v["dropped"], v["gate_eff"],
                                               v["token_of_row"], v["x_perm"], sc),
            "combine": lambda: B.moe_combine(d, v["y_perm"], v["row_of"], v["gate_eff"], layer.y),
        }
        for name, fn in small_fn.items():
            ts = []
            for _ in range(cold_reps):
                flush.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            cold_ms[name] = float(np.median(ts))
        del flush
    for _ in range(args.warmup):
        layer.forward()
        step(up=up)
    # Timed: exactly K passes of the layer, one moe_forward call each, between two device
    # synchronisations (nothing else enqueued in between).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.forward()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The spread of one call: K more calls, each between an event pair.
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        fev[i][0].record(stream)
        layer.forward()
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    fwd_t = np.array([a.elapsed_time(b) for a, b in fev])
    forward_ms = {"mean": float(np.mean(fwd_t)), "p10": float(np.percentile(fwd_t, 10)),
                  "median": float(np.median(fwd_t)), "p90": float(np.percentile(fwd_t, 90))}
    stats = layer.stats()  # routing statistics of the last forward (synchronises)

    # Stage breakdown: K more passes through the per-stage entry points (the same kernels),
    # with events between the stages.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    ts0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i], up=up)
    torch.cuda.synchronize()
    staged_ms_per_step = (time.perf_counter() - ts0) / args.steps * 1e3

    # The same forward captured once in a HIP graph and replayed K times (launch overhead
    # of the individual kernels removed); reported beside the eager throughput.
    graph_res = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layer.forward()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - tg0) / args.steps * 1e3
        graph_res = {"ms_per_step": gms, "tokens_per_s": N / (gms * 1e-3)}
        del g

    stage_t = {s: np.array([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)])
               for j, s in enumerate(STAGES)}
    stage_ms = {s: float(np.mean(t)) for s, t in stage_t.items()}
    stage_pct = {s: {"p10": float(np.percentile(t, 10)), "median": float(np.median(t)),
                     "p90": float(np.percentile(t, 90))} for s, t in stage_t.items()}

    counts = v["counts"].cpu().numpy().astype(np.int64)
    A = int(counts.sum())
    active = int((counts > 0).sum())
    es = 2 if cfg["dtype"] == "bf16" else 4
    ws = 1 if q8 else es  # bytes per weight element (int8 weights also read 4-byte column scales)
    work = {
        "expert_up": dict(flops=4.0 * A * D * F,
                          bytes=ws * 2.0 * active * D * F + (8.0 * active * F if q8 else 0.0) + es * (A * D + A * F)),
        "expert_down": dict(flops=2.0 * A * F * D,
                            bytes=ws * 1.0 * active * D * F + (4.0 * active * D if q8 else 0.0) + es * (A * F + A * D)),
    }
    # Algorithmic HBM bytes of the small stages: router reads x (+ W_r, noise) and writes
    # the selection; dispatch reads the selection and the token rows and writes the expert
    # buffers (padding rows included) and the per-record metadata; combine reads the
    # accepted expert rows and the per-record gates and writes y.
    noisy = cfg["second_choice"] != "topk"
    small_bytes = {
        "route": es * N * D + 4.0 * D * E + (4.0 * N * E if noisy else 0.0) + 8.0 * N * k,
        "dispatch": 8.0 * N * k + es * N * D + es * rows * D + 9.0 * N * k + 4.0 * rows + 12.0 * E,
        "combine": es * A * D + 8.0 * N * k + es * N * D,
    }
    small = {}
    for st_name, b in small_bytes.items():
        warm = b / (stage_ms[st_name] * 1e-3) / 1e9
        small[st_name] = {"bytes": b, "warm_gbs": warm, "warm_frac": warm / PEAK_HBM_GBS}
        if st_name in cold_ms:
            cold = b / (cold_ms[st_name] * 1e-3) / 1e9
            small[st_name].update({"cold_gbs": cold, "cold_frac": cold / PEAK_HBM_GBS})
    dom = max(("expert_up", "expert_down"), key=lambda s_: stage_ms[s_])
    w = work[dom]
    sec = stage_ms[dom] * 1e-3
    peak_f = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_F32_TFLOPS
    if w["flops"] / w["bytes"] >= RIDGE or cfg["dtype"] == "f32":
        roof = {"bound": "mfma", "achieved": w["flops"] / sec / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": w["bytes"] / sec / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    cap = B.moe_capacity(d) if cfg["capacity_mode"] == "padded" else None
    roof["kernel"] = gemm_kernel_of(cfg, dom, dom == "expert_up" and up is up_gathered, cap)
    roof["per_launch"] = {"flops": w["flops"], "algorithmic_bytes": w["bytes"], "avg_ms": stage_ms[dom]}
    return dict(elapsed=elapsed, forward_ms=forward_ms, staged_ms_per_step=staged_ms_per_step, graph=graph_res,
                stage_ms=stage_ms, stage_pct=stage_pct, cold_ms=cold_ms, small=small, work=work, dom=dom, A=A,
                active=active, q8=q8, roofline=roof, stats=stats)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib * 2 ** 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        if args.copy_kind == "lds":
            import ctypes
            from mixture_experts_layer_wave_amd.build import CALIB_LIB
            if not os.path.exists(CALIB_LIB):
                raise RuntimeError(f"calibration library not built: {CALIB_LIB}")
            L = ctypes.CDLL(CALIB_LIB)
            L.moe_calib_copy_lds.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for _ in range(args.steps):
                rc = L.moe_calib_copy_lds(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                          src.numel(), stream)
                if rc != 0:
                    raise RuntimeError(f"moe_calib_copy_lds failed: {rc}")
        else:
            for _ in range(args.steps):
                dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "copies": args.steps, "kind": args.copy_kind}), flush=True)
        return
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd import configs, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = configs.get_config(args.workload)
    inp = inputs.make_inputs(cfg)
    m = measure_layer(B, cfg, inp, args, dev, cold_reps=args.cold_reps, graph=not args.no_graph)
    N, D, F, E, k = cfg["N"], cfg["D"], cfg["F"], cfg["E"], cfg["k"]
    elapsed, stage_ms, work, dom = m["elapsed"], m["stage_ms"], m["work"], m["dom"]
    A, active, q8 = m["A"], m["active"], m["q8"]
    gemm_ms = stage_ms["expert_up"] + stage_ms["expert_down"]
    gemm_tflops = (work["expert_up"]["flops"] + work["expert_down"]["flops"]) / (gemm_ms * 1e-3) / 1e12
    roof = m["roofline"]
    roof["traffic"] = traffic_from_profiles(args.workload, dom)
    roof["traffic_what"] = ("bytes per launch through the L2's memory-side interface (Infinity Cache hits "
                            "included), rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by a direct-to-LDS copy")
    # The weight-streaming decode regime of the same expert shapes, measured in the same run.
    decode = None
    if args.decode and args.workload != "mixtral_decode":
        dcfg = configs.get_config("mixtral_decode")
        dinp = inputs.make_inputs(dcfg)
        dm = measure_layer(B, dcfg, dinp, args, dev, cold_reps=0, graph=False)
        dw = dm["work"]
        dg_ms = dm["stage_ms"]["expert_up"] + dm["stage_ms"]["expert_down"]
        dbytes = dw["expert_up"]["bytes"] + dw["expert_down"]["bytes"]
        decode = {"workload": dcfg["name"], "N": dcfg["N"], "active_experts": dm["active"],
                  "accepted_rows": dm["A"], "ms_per_step": dm["elapsed"] / args.steps * 1e3,
                  "tokens_per_s": dcfg["N"] * args.steps / dm["elapsed"], "forward_ms": dm["forward_ms"],
                  "stages_ms": dm["stage_ms"], "gemm_ms": dg_ms, "gemm_algorithmic_bytes": dbytes,
                  "gemm_gbs": dbytes / (dg_ms * 1e-3) / 1e9, "gemm_frac_hbm": dbytes / (dg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "up_gbs": dw["expert_up"]["bytes"] / (dm["stage_ms"]["expert_up"] * 1e-3) / 1e9,
                  "down_gbs": dw["expert_down"]["bytes"] / (dm["stage_ms"]["expert_down"] * 1e-3) / 1e9,
                  "bytes": "per active expert its W1, W2 and W3 (6 D F bytes, bf16) plus the activation rows "
                           "read and written (x_perm, h, y_perm)"}
        del dm, dinp

    out = {
        "metric": METRIC,
        "value": N * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"] + ("+int8 weights" if q8 else ""),
        "data": "synthetic (seeded normal inputs and random-init expert weights of the workload's shapes)",
        "config": {"workload": cfg["name"], "N": N, "D": D, "F": F, "E": E, "k": k, "routing": cfg["routing_mode"],
                   "second_choice": cfg["second_choice"], "activation": cfg["activation"],
                   "capacity": cfg["capacity_mode"], "parallelism": "single GPU, all experts resident"},
        "grouped_gemm": {"tflops": gemm_tflops, "frac_bf16_peak": gemm_tflops / PEAK_BF16_TFLOPS,
                         "useful_flops": work["expert_up"]["flops"] + work["expert_down"]["flops"],
                         "accepted_rows": A, "active_experts": active},
        "forward_ms": m["forward_ms"],
        "staged_ms_per_step": m["staged_ms_per_step"],
        "graph_replay": m["graph"],
        "stages_ms": stage_ms,
        "stages_ms_pct": m["stage_pct"],
        "stages_ms_cold": m["cold_ms"],
        "small_stages_hbm": m["small"],
        "routing_stats": {"gpu": m["stats"], "oracle": None},
        "decode": decode,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
        out["routing_stats"]["oracle"] = out["cpu_baseline"].pop("routing_stats")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
