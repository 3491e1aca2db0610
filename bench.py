"""Throughput of the MoE-layer forward pass on one MI355X.

One step = one moe_layer_forward call (gate GEMM + top-k, dispatch, tile plan,
grouped FC1 + SiLU*mul, grouped FC2, combine) on one batch of synthetic
inputs already resident in HBM. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The default workload is the Mixtral-8x22B-shaped decode layer (T=256, d=6144,
f=16384, E=8, top-2, bf16, balanced routing). The roofline object covers the
dominant kernel (the grouped FC1), timed with HIP events recorded around each
of its launches inside the timed region; the cpu_baseline object times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral_decode")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0, help="0 = whole batch")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run 5 device copies of 1 GiB (reference kernel for HBM byte counters)")
    return p.parse_args()


def copy_probe():
    """Plain device-to-device copies of a known size; their FETCH_SIZE / WRITE_SIZE
    counter readings scale the counters taken on the layer's kernels."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n, "copies": 5}), flush=True)


def cpu_baseline(cfg, inp, ntok: int):
    """Time the CPU oracle (as it stands) on the first ntok tokens of the same inputs."""
    import numpy as np
    import torch
    import oracle

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(cores)
    except Exception:  # pragma: no cover
        limiter = None
    h = {n: host(v) for n, v in inp.items()}
    x = h["x"][:ntok]
    t0 = time.perf_counter()
    oracle.layer_forward(x, h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], cfg.k, cfg.dtype)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle layer_forward (numpy, fp64 FFN) on the first {ntok} of {cfg.T} tokens "
                      f"of workload {cfg.name}, seed 0 inputs; {dt:.1f} s"}


def kernel_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in ("mixture_experts_layer_gate_amd/csrc/ffn.hip", "mixture_experts_layer_gate_amd/csrc/common.h"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    the counters were taken on a different kernel source or workload."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = kernel_source_sha256()
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        rec = json.loads(line)
        if rec.get("workload") == workload and rec.get("kernel") == kernel and rec.get("source_sha256") == sha:
            return rec["traffic_bytes"]
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer runs on one MI355X)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    import torch
    import moe_inputs
    import mixture_experts_layer_gate_amd as moe
    from mixture_experts_layer_gate_amd import roofline as rf

    cfg = moe_inputs.config(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = moe_inputs.make_layer_inputs(cfg, args.seed, dev)
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    ws = moe.make_workspace(dims)
    out = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], out=out,
                          ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # routing counts of this batch (identical every step) for the work accounting
    _, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                             ws=ws, return_routing=True)
    counts = r["counts"].cpu().tolist()
    torch.cuda.synchronize()

    # Timed region: events only around the dominant kernel (FC1), on the
    # stream it is launched on.
    moe.timing_enable(args.steps, stages=["fc1"])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    moe.timing_disable()
    total_ms = ev0.elapsed_time(ev1)
    ms = total_ms / args.steps
    fc1_rec = moe.timing_read("fc1")
    # Per-stage breakdown from a separate, untimed pass with every stage recorded.
    nbreak = min(args.steps, 5)
    moe.timing_enable(nbreak)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    moe.timing_disable()
    stages = {s: moe.timing_read(s) for s in moe.STAGES}
    stages["fc1"] = fc1_rec

    elt = 2 if cfg.dtype == "bf16" else 4
    n = cfg.T * cfg.k
    fc1_ms = stages["fc1"][0] / max(stages["fc1"][1], 1)
    fc1_flops = rf.fc1_flops(n, cfg.d, cfg.f)
    fc1_bytes = rf.fc1_bytes(cfg.T, cfg.d, cfg.f, cfg.k, counts, elt)
    cls = rf.classify(fc1_flops, fc1_bytes)
    if cls.bound == "hbm":
        achieved = fc1_bytes / (fc1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s"}
    else:
        peak = 2500.0 if cfg.dtype == "bf16" else 157.3
        achieved = fc1_flops / (fc1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(cfg.name, "fc1")
    big_tile = cfg.dtype == "bf16" and os.environ.get("MOE_GEMM_REGIME", "1") != "0"
    roof["kernel"] = ("gemm_dl_kernel<gated, 256x256> (FC1 + SiLU*mul)" if big_tile
                      else "grouped_gemm_kernel<gated, 128x128> (FC1 + SiLU*mul)")
    roof["kernel_ms"] = round(fc1_ms, 4)

    layer_flops = rf.layer_flops(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k)
    layer_bytes = rf.layer_bytes(cfg.T, cfg.d, cfg.f, cfg.E, counts, elt)
    res = {
        "metric": "MoE layer tokens/s at 1 GPU; % bf16 MFMA peak or % HBM peak (roofline)",
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f, "E": cfg.E, "k": cfg.k,
                   "bias_scale": cfg.bias_scale, "seed": args.seed, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"tflops": round(layer_flops / (ms * 1e-3) / 1e12, 1),
                  "gbps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                  "bound": rf.classify(layer_flops, layer_bytes).bound,
                  "floor_ms": round(rf.classify(layer_flops, layer_bytes).floor_s * 1e3, 4),
                  "kappa": round(rf.kappa(counts), 3), "active_experts": rf.active_experts(counts)},
        "stages_ms": {s: round(v[0] / max(v[1], 1), 4) for s, v in stages.items() if v[1] > 0},
    }
    if not args.no_cpu_baseline:
        ntok = cfg.T if args.cpu_sample_tokens <= 0 else min(cfg.T, args.cpu_sample_tokens)
        res["cpu_baseline"] = cpu_baseline(cfg, inp, ntok)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
