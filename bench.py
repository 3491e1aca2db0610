"""Throughput of the MoE-layer forward pass on one MI355X.

One step = one layer call (gate GEMM + top-k, dispatch, tile plan, grouped
FC1 + SiLU*mul, grouped FC2, combine) on one batch of synthetic inputs already
resident in HBM. Prints one JSON line. By default the bf16 layers read expert
weights that moe_pack_weights re-laid once, before the steps, in the order the
grouped FFN streams them (moe_layer_forward_packed: the same arithmetic and
bitwise the same output as moe_layer_forward); --weights stored times
moe_layer_forward on the weights as stored.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-ceilings]
  python bench.py --backward [--workload NAME] ...   (the layer's backward instead)
  python bench.py --backward --saved ...             (with FC1's g|u kept by the forward)
  python bench.py --backward --wgrad-bf16 ...        (weight gradients written as bf16)

The default workload is the Mixtral-8x22B-shaped prefill layer (T=8192,
d=6144, f=16384, E=8, top-2, bf16, routing skewed by the gate-logit bias
1.5*(-ln rank)): the largest single-GPU configuration, MFMA-bound. The
roofline object covers the dominant kernel (the grouped FC1), timed with HIP
events recorded around each of its launches inside the timed region; the
cpu_baseline object times the CPU oracle on a bounded sample of the same
workload. The line also carries, under "decode", the same measurement of the
Mixtral-8x22B-shaped decode layer (T=256, balanced routing, HBM-bound), run
after the main one in the same process (--secondary none skips it).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


DEFAULT_WORKLOAD = "mixtral_prefill_skew"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--secondary", default="mixtral_decode",
                   help="workload measured after the default one and reported under 'decode' "
                        "(only when --workload is the default; 'none' skips it)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="tokens of the CPU-baseline sample (0 = the first 256, the whole batch when smaller)")
    p.add_argument("--protocol", action="store_true",
                   help="median of 2 fresh processes x seeds 0,1,2 per workload, and skew ratios of the twins")
    p.add_argument("--workloads", default="",
                   help="comma-separated workloads for --protocol (default: all)")
    p.add_argument("--seeds", default="", help="comma-separated seeds measured one after another in this process")
    p.add_argument("--expert-curve", choices=sorted(EXPERT_SHAPES), default=None,
                   help="instead of the layer: time one expert's FC1 + FC2 against rows per expert")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured HBM-read and MFMA ceilings (diagnostic, about a second)")
    p.add_argument("--fused", action="store_true",
                   help="time the one-launch layer (moe_layer_forward_fused, or _fused_packed with packed weights)")
    p.add_argument("--weights", choices=["auto", "packed", "stored"], default="auto",
                   help="packed: moe_layer_forward_packed on the expert weights re-laid once in stage order "
                        "(moe_pack_weights, timed apart, not part of a step); stored: moe_layer_forward on the "
                        "weights as stored; auto: packed for bf16 layers without shared experts")
    p.add_argument("--backward", action="store_true",
                   help="time the layer's backward (moe_layer_backward) instead of the forward")
    p.add_argument("--wgrad-bf16", action="store_true",
                   help="with --backward: weight gradients written as bf16 (moe_layer_backward_ex)")
    p.add_argument("--saved", action="store_true",
                   help="with --backward: the forward keeps FC1's g|u (moe_layer_forward_train) and the backward "
                        "reads it (moe_layer_backward_saved); also times forward + backward both ways")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run 5 device copies of 1 GiB (reference kernel for HBM byte counters)")
    return p.parse_args()


# Expert shapes (d, f) of the workloads: Mixtral 8x22B, DBRX, DeepSeek-V3 routed expert.
EXPERT_SHAPES = {"mixtral": (6144, 16384), "dbrx": (6144, 10752), "deepseek": (7168, 2048)}


def expert_curve(shape: str, seed: int):
    """Time T_e(c), the per-expert cost of the grouped FC1 + FC2 at c rows per
    expert, c = 1, 2, 4, ..., 4096: 8 experts of the shape each get exactly c
    rows (round-robin routing, k = 1) in one moe_grouped_ffn call, as experts
    run together in a layer, and T_e = call time / 8. The 8 experts' weights
    exceed the 256 MB last-level cache for every shape, so they stream from
    HBM. Prints one JSON line per c, then the fit T_e = k3 * c + k4 over the
    points with c >= 512 and the floor (mean of c = 1..8)."""
    import numpy as np
    import torch
    import moe_inputs
    import mixture_experts_layer_gate_amd as moe
    from mixture_experts_layer_gate_amd import roofline as rf

    d, f = EXPERT_SHAPES[shape]
    E, cmax = 8, 4096
    cfg = moe_inputs.LayerConfig(f"curve_{shape}", E * cmax, d, f, E, 1, "bf16", 0.0)
    inp = moe_inputs.make_layer_inputs(cfg, seed, torch.device("cuda:0"))
    points = []
    c = 1
    while c <= cmax:
        T = E * c
        dims = moe.Dims(T, d, f, E, 1)
        ws = moe.make_workspace(dims)
        x = inp["x"][:T].contiguous()
        counts = torch.full((E,), c, dtype=torch.int32, device="cuda")
        offsets = torch.arange(0, T + 1, c, dtype=torch.int32, device="cuda")
        # sorted row p = e * c + i holds token i * E + e (routing e = t mod E)
        perm = torch.arange(T, dtype=torch.int32, device="cuda").view(c, E).t().contiguous().view(-1)
        y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        reps = 10
        for _ in range(2):  # warm-up
            moe.grouped_ffn(dims, x, perm, counts, offsets, inp["w1"], inp["w3"], inp["w2"], y, ws)
        torch.cuda.synchronize()
        moe.timing_enable(reps, stages=["fc1", "fc2"])
        for _ in range(reps):
            moe.grouped_ffn(dims, x, perm, counts, offsets, inp["w1"], inp["w3"], inp["w2"], y, ws)
        torch.cuda.synchronize()
        moe.timing_disable()
        fc1 = moe.timing_read("fc1")[0] / reps
        fc2 = moe.timing_read("fc2")[0] / reps
        ms = fc1 + fc2
        flops = rf.ffn_flops(T, d, f)
        wbytes = E * 3 * d * f * 2
        pt = {"shape": shape, "d": d, "f": f, "rows_per_expert": c, "experts": E, "fc1_ms": round(fc1, 4),
              "fc2_ms": round(fc2, 4), "t_e_ms": round(ms / E, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
              "weight_gbps": round(wbytes / (ms * 1e-3) / 1e9, 1),
              "util_e": round(min(c * rf.PEAK_HBM_BYTES_PER_S / rf.PEAK_MFMA_BF16_FLOPS, 1.0), 4)}
        points.append(pt)
        print(json.dumps(pt), flush=True)
        c *= 2
    rows = np.array([p["rows_per_expert"] for p in points], dtype=np.float64)
    t = np.array([p["t_e_ms"] for p in points], dtype=np.float64)
    floor = float(t[:4].mean())  # 1..8 rows per expert: weight streaming
    big = rows >= 512
    k3, k4 = np.polyfit(rows[big], t[big], 1)
    ridge = (floor - k4) / k3 if k3 > 0 else float("nan")
    print(json.dumps({"shape": shape, "fit": "T_e = k3 * rows + k4 over rows >= 512", "k3_ms_per_row": k3,
                      "k4_ms": k4, "floor_ms": floor, "ridge_rows": round(ridge, 1),
                      "datasheet_ridge_rows": round(rf.PEAK_MFMA_BF16_FLOPS / rf.PEAK_HBM_BYTES_PER_S, 1)}),
          flush=True)


SKEW_TWINS = [("mixtral_prefill_skew", "mixtral_prefill_bal"), ("dbrx_zipf", "dbrx_bal"),
              ("deepseek_skew", "deepseek_bal")]


def protocol(args):
    """For each workload, two fresh processes each measure seeds 0, 1 and 2 (the
    usual warm-up and timed steps); prints one JSON line per workload with the
    median of the six layer times, then one line with the skew ratios
    t(skewed) / t(balanced twin). Runs children only: this process never
    touches the GPU."""
    import statistics
    import subprocess
    import moe_inputs
    names = [w for w in args.workloads.split(",") if w] or list(moe_inputs.CONFIGS)
    med = {}
    for w in names:
        runs = []
        for _ in range(2):
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", w, "--seeds", "0,1,2",
                   "--steps", str(args.steps), "--warmup", str(args.warmup), "--no-cpu-baseline", "--no-ceilings", "--secondary", "none",
                   "--weights", args.weights]
            out = subprocess.run(cmd, check=True, capture_output=True, text=True).stdout
            runs += [json.loads(l) for l in out.splitlines() if l.startswith("{")]
        ms = [r["ms_per_step"] for r in runs]
        m = statistics.median(ms)
        med[w] = m
        cfg = moe_inputs.config(w)
        print(json.dumps({"workload": w, "median_ms": round(m, 4), "tokens_per_s": round(cfg.T / (m * 1e-3), 1),
                          "runs_ms": ms, "seeds": [r["config"]["seed"] for r in runs],
                          "fc1_roofline_frac_median": statistics.median(r["roofline"]["frac"] for r in runs),
                          "bound": runs[0]["roofline"]["bound"]}), flush=True)
    ratios = {f"{a}/{b}": round(med[a] / med[b], 3) for a, b in SKEW_TWINS if a in med and b in med}
    print(json.dumps({"skew_ratios": ratios, "target": "<= 1.2"}), flush=True)


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


def stage_rooflines(cfg, kk: int, counts, elt: int, stage_ms: dict) -> dict:
    """Each forward stage against the bound of its own work: the gate's fp32
    multiply-adds against the fp32 matrix-core peak where the library runs them
    there, else the unpacked fp32 vector peak, FC1 and FC2 against
    bf16 MFMA or HBM (whichever their algorithmic work binds), the routing and
    data-movement stages against HBM by the bytes they must move (top-k and
    dispatch move a few MB at most and are bound by launch latency, so their
    fractions are small by nature). Where the gate and top-k run as one launch
    (small batches) the gate entry times both."""
    import torch
    import mixture_experts_layer_gate_amd as moe
    from mixture_experts_layer_gate_amd import roofline as rf
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    n = T * kk
    out = {}

    def put(stage, bound, work, peak, unit, scale):
        ms = stage_ms.get(stage)
        if not ms:
            return
        achieved = work / (ms * 1e-3) / scale
        out[stage] = {"ms": round(ms, 4), "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                      "unit": unit, "frac": round(achieved / peak, 4)}

    hbm = rf.PEAK_HBM_BYTES_PER_S / 1e9
    mfma = (rf.PEAK_MFMA_BF16_FLOPS if cfg.dtype == "bf16" else rf.PEAK_MFMA_FP32_FLOPS) / 1e12
    if moe.gate_on_matrix_cores(moe.Dims(T, d, f, E, kk, torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)) == 1:
        put("gate", "mfma", 2 * T * d * E, round(rf.PEAK_MFMA_FP32_FLOPS / 1e12, 1), "TFLOP/s", 1e12)
    else:
        put("gate", "valu", 2 * T * d * E, round(rf.PEAK_VALU_FP32_UNPACKED_FLOPS / 1e12, 1), "TFLOP/s", 1e12)
    put("topk", "hbm", T * E * 4 + n * 8, hbm, "GB/s", 1e9)
    put("dispatch", "hbm", n * 4 * 2 + n * 8, hbm, "GB/s", 1e9)
    for stage, flops, nbytes in (("fc1", rf.fc1_flops(n, d, f), rf.fc1_bytes(T, d, f, kk, counts, elt)),
                                 ("fc2", rf.fc2_flops(n, d, f), rf.fc2_bytes(T, d, f, kk, counts, elt))):
        if rf.classify(flops, nbytes).bound == "hbm":
            put(stage, "hbm", nbytes, hbm, "GB/s", 1e9)
        else:
            put(stage, "mfma", flops, mfma, "TFLOP/s", 1e12)
    put("combine", "hbm", rf.combine_bytes(T, d, kk, elt), hbm, "GB/s", 1e9)
    # traffic each stage moves beyond its algorithmic bytes (gathered x rows,
    # the h and y round trips), per launch
    ovh = {"fc1": rf.fc1_overhead_bytes(T, d, f, kk, elt), "fc2": rf.fc2_overhead_bytes(T, d, f, kk, elt),
           "combine": rf.combine_overhead_bytes(T, d, kk, elt)}
    for stage, b in ovh.items():
        if stage in out:
            out[stage]["overhead_bytes"] = b
    return out


def cpu_baseline(cfg, inp, ntok: int, seed: int = 0):
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
    # the sample is repeated until it has run for about 10 s (at most 8 passes),
    # so that short samples are timed over a stable stretch of CPU work
    reps, dt = 0, 0.0
    while reps < 8 and (reps == 0 or dt < 10.0):
        t0 = time.perf_counter()
        if cfg.n_shared:
            oracle.layer_forward_shared(x, h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], h["sw1"], h["sw3"],
                                        h["sw2"], cfg.k, cfg.dtype)
        else:
            oracle.layer_forward(x, h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], cfg.k, cfg.dtype)
        dt += time.perf_counter() - t0
        reps += 1
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": ntok * reps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle layer forward (numpy, fp64 FFN) on the first {ntok} of {cfg.T} tokens "
                      f"of workload {cfg.name}, seed {seed} inputs; {reps} pass(es), {dt:.1f} s"}


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
    if args.expert_curve:
        expert_curve(args.expert_curve, args.seed)
        return
    if args.protocol:
        protocol(args)
        return
    seeds = [int(v) for v in args.seeds.split(",") if v] or [args.seed]
    for seed in seeds:
        if args.backward:
            print(json.dumps(run_backward(args, seed)), flush=True)
            continue
        res = run_one(args, seed)
        if args.workload == DEFAULT_WORKLOAD and args.secondary != "none" and not args.seeds:
            res["decode"] = secondary(args, seed)
        print(json.dumps(res), flush=True)


def secondary(args, seed: int) -> dict:
    """The same measurement on a second workload (by default the decode-sized,
    HBM-bound layer), reported beside the main line: its throughput, step time
    and the roofline of its dominant kernel."""
    sub = argparse.Namespace(**vars(args))
    sub.workload, sub.no_cpu_baseline, sub.no_ceilings = args.secondary, True, True
    r = run_one(sub, seed)
    keep = ("metric", "value", "unit", "ms_per_step", "dtype", "config", "roofline", "layer", "stages_ms")
    return {k: r[k] for k in keep}


def cpu_baseline_backward(cfg, inp, dout, ntok: int, seed: int = 0):
    """Time the CPU backward oracle (as it stands) on the first ntok tokens."""
    import numpy as np
    import torch
    import oracle

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    cores = len(os.sched_getaffinity(0))
    h = {n: host(v) for n, v in inp.items()}
    t0 = time.perf_counter()
    oracle.layer_backward(h["x"][:ntok], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], cfg.k, cfg.dtype,
                          host(dout[:ntok]))
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle layer backward (numpy, fp64, routing recomputed) on the first {ntok} of {cfg.T} "
                      f"tokens of workload {cfg.name}, seed {seed} inputs; {dt:.1f} s"}


def run_backward(args, seed: int) -> dict:
    """One measurement of moe_layer_backward on the workload's inputs for `seed`:
    the forward runs once for the routing, then every step computes all
    gradients (dx, dwg, dbias, dw1, dw3, dw2, dlogits, dtopk_w) from dout."""
    import torch
    import moe_inputs
    import mixture_experts_layer_gate_amd as moe
    from mixture_experts_layer_gate_amd import roofline as rf

    cfg = moe_inputs.config(args.workload)
    if cfg.n_shared or cfg.dtype != "bf16":
        raise SystemExit(f"the backward runs on bf16 layers without shared experts; {cfg.name} is not one")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = moe_inputs.make_layer_inputs(cfg, seed, dev)
    dout = moe_inputs.output_grad(cfg.T, cfg.d, cfg.dtype, seed, dev)
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    stream = torch.cuda.current_stream()
    gu = None
    if args.saved:
        _, r, gu = moe.layer_forward_train(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"],
                                           inp["w2"])
    else:
        _, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                 return_routing=True)
    counts = r["counts"].cpu().tolist()
    ws = torch.empty(moe.backward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    wdt = torch.bfloat16 if args.wgrad_bf16 else torch.float32
    grads = moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r, dout, ws=ws,
                               want_dlogits=True, want_dtopk_w=True, gu=gu, wgrad_dtype=wdt)

    def step(keep=gu):
        moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r, dout, ws=ws,
                           stream=stream, want_dlogits=True, want_dtopk_w=True, grads=grads, gu=keep,
                           wgrad_dtype=wdt)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pair = None
    if args.saved:
        # forward + backward both ways, same process and buffers: the plain
        # forward with the FC1 recompute, and the forward keeping g | u
        fws = moe.make_workspace(dims, dev)
        out = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=dev)

        def fwd_plain():
            moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], out=out,
                              ws=fws, stream=stream)

        def fwd_train():
            moe.layer_forward_train(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                    out=out, gu=gu, ws=fws, stream=stream)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps
        pair = {"forward_ms": timed(fwd_plain), "backward_ms": timed(lambda: step(None)),
                "forward_train_ms": timed(fwd_train), "backward_saved_ms": timed(step)}
        pair = {n: round(v, 4) for n, v in pair.items()}
        pair["step_ms_recompute"] = round(pair["forward_ms"] + pair["backward_ms"], 4)
        pair["step_ms_saved"] = round(pair["forward_train_ms"] + pair["backward_saved_ms"], 4)
        pair["gu_bytes"] = gu.numel() * gu.element_size()
        del fws, out
    bwd = [s_ for s_ in moe.STAGES if s_.startswith("bwd_")] + ["plan"]
    # untimed pass with every stage recorded: per-stage times, and the dominant GEMM
    nbreak = min(args.steps, 5)
    moe.timing_enable(nbreak, stages=bwd)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    moe.timing_disable()
    stages = {s_: moe.timing_read(s_) for s_ in bwd}
    stage_ms = {s_: v[0] / max(v[1], 1) for s_, v in stages.items() if v[1] > 0}
    dom = max(rf.BACKWARD_GEMM_FLOPS_PER_ROW, key=lambda s_: stage_ms.get(s_, 0.0))
    # timed region: events only around the dominant GEMM, on its launch stream
    moe.timing_enable(args.steps, stages=[dom])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    moe.timing_disable()
    ms = ev0.elapsed_time(ev1) / args.steps
    rec = moe.timing_read(dom)
    dom_ms = rec[0] / max(rec[1], 1)
    P = cfg.T * cfg.k
    dom_flops = rf.BACKWARD_GEMM_FLOPS_PER_ROW[dom] * cfg.d * cfg.f * P
    roof = {"bound": "mfma", "achieved": round(dom_flops / (dom_ms * 1e-3) / 1e12, 1),
            "peak": rf.PEAK_MFMA_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = {"bwd_fc1": "gemm_dl_kernel<FC1 recompute g|u, 256x256>",
                      "bwd_dh": "gemm_dl_kernel<dout W2, 256x256>",
                      "bwd_dx": "gemm_dl_kernel<[dg|du] [W1;W3], 256x256>",
                      "bwd_wg2": "gemm_dl_kernel<weight gradient dW2, 256x256>",
                      "bwd_wg13": "gemm_dl_kernel<weight gradients dW1|dW3, 256x256>"}[dom]
    roof["kernel_ms"] = round(dom_ms, 4)
    gemm_rates = {s_: round(rf.BACKWARD_GEMM_FLOPS_PER_ROW[s_] * cfg.d * cfg.f * P / (stage_ms[s_] * 1e-3) / 1e12, 1)
                  for s_ in rf.BACKWARD_GEMM_FLOPS_PER_ROW if s_ in stage_ms}
    flops = rf.backward_flops(P, cfg.d, cfg.f, cfg.T, cfg.k)
    res = {
        "metric": "MoE layer backward tokens/s at 1 GPU; % bf16 MFMA peak of the dominant GEMM (roofline)",
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
        "config": {"workload": cfg.name, "pass": "backward (g|u kept by the forward)" if args.saved else "backward",
                   "weight_grads": "bf16" if args.wgrad_bf16 else "fp32", "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E,
                   "k": cfg.k, "bias_scale": cfg.bias_scale, "seed": seed, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"tflops_algorithmic": round(flops / (ms * 1e-3) / 1e12, 1),
                  "recompute_tflop": 0.0 if args.saved else round(rf.fc1_flops(P, cfg.d, cfg.f) / 1e12, 3),
                  "kappa": round(rf.kappa(counts), 3), "active_experts": rf.active_experts(counts)},
        "gemm_tflops": gemm_rates,
        "stages_ms": {s_: round(v, 4) for s_, v in stage_ms.items()},
    }
    if pair is not None:
        res["train_pair"] = pair
    if not args.no_cpu_baseline:
        ntok = min(cfg.T, args.cpu_sample_tokens if args.cpu_sample_tokens > 0 else 32)
        res["cpu_baseline"] = cpu_baseline_backward(cfg, inp, dout, ntok, seed)
    else:
        res["cpu_baseline"] = None
    del inp, ws, grads
    torch.cuda.empty_cache()
    return res


def run_one(args, seed: int) -> dict:
    """One measurement of the layer on the workload's inputs for `seed`."""
    import torch
    import moe_inputs
    import mixture_experts_layer_gate_amd as moe
    from mixture_experts_layer_gate_amd import roofline as rf

    cfg = moe_inputs.config(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = moe_inputs.make_layer_inputs(cfg, seed, dev)
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    ws = moe.make_workspace(dims)
    out = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    S = cfg.n_shared
    use_packed = args.weights == "packed" or (args.weights == "auto" and cfg.dtype == "bf16" and not S)
    if S:
        if args.fused or use_packed:
            raise SystemExit("the fused FFN launch and the packed weights cover layers without shared experts")
        ws = torch.empty(moe.workspace_bytes_shared(dims, S), dtype=torch.uint8, device=dev)
    packed, pack_ms = None, None
    if use_packed:
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pe0.record(stream)
        packed = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"], stream=stream)
        pe1.record(stream)
        torch.cuda.synchronize()
        pack_ms = pe0.elapsed_time(pe1)

    def step():
        if S:
            moe.layer_forward_shared(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                     inp["sw1"], inp["sw3"], inp["sw2"], out=out, ws=ws, stream=stream)
        else:
            moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], out=out,
                              ws=ws, stream=stream, fused=args.fused, packed=packed)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # routing counts of this batch (identical every step) for the work accounting
    if S:
        _, r = moe.layer_forward_shared(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                        inp["sw1"], inp["sw3"], inp["sw2"], ws=ws, return_routing=True)
    else:
        _, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                 ws=ws, return_routing=True, fused=args.fused, packed=packed)
    # shared experts count as S more experts with T rows each
    counts = r["counts"].cpu().tolist() + [cfg.T] * S
    kk = cfg.k + S
    torch.cuda.synchronize()

    # Timed region: events only around the dominant kernel (FC1, or the fused
    # FC1 + FC2 + combine launch), on the stream it is launched on.
    dom = "ffn_fused" if args.fused else "fc1"
    moe.timing_enable(args.steps, stages=[dom])
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
    fc1_rec = moe.timing_read(dom)
    # Per-stage breakdown from a separate, untimed pass with every stage recorded.
    nbreak = min(args.steps, 5)
    moe.timing_enable(nbreak)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    moe.timing_disable()
    stages = {s: moe.timing_read(s) for s in moe.STAGES}
    stages[dom] = fc1_rec

    elt = 2 if cfg.dtype == "bf16" else 4
    n = cfg.T * kk
    fc1_ms = stages[dom][0] / max(stages[dom][1], 1)
    T, d, f = cfg.T, cfg.d, cfg.f
    if args.fused:
        # one launch does FC1, FC2 and the combine: FFN FLOP; all active expert
        # weights, x once and out once (the h and y round trips are overhead)
        fc1_flops = rf.ffn_flops(n, d, f)
        fc1_bytes = (rf.fc1_bytes(T, d, f, kk, counts, elt) + rf.fc2_bytes(T, d, f, kk, counts, elt) +
                     rf.combine_bytes(T, d, kk, elt))
        overhead = (rf.fc1_overhead_bytes(T, d, f, kk, elt) + rf.fc2_overhead_bytes(T, d, f, kk, elt) +
                    rf.combine_overhead_bytes(T, d, kk, elt))
    else:
        fc1_flops = rf.fc1_flops(n, d, f)
        fc1_bytes = rf.fc1_bytes(T, d, f, kk, counts, elt)
        overhead = rf.fc1_overhead_bytes(T, d, f, kk, elt)
    cls = rf.classify(fc1_flops, fc1_bytes)
    if cls.bound == "hbm":
        achieved = fc1_bytes / (fc1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": rf.PEAK_HBM_BYTES_PER_S / 1e9,
                "unit": "GB/s"}
    else:
        peak = (rf.PEAK_MFMA_BF16_FLOPS if cfg.dtype == "bf16" else rf.PEAK_MFMA_FP32_FLOPS) / 1e12
        achieved = fc1_flops / (fc1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["algorithmic"] = {"flop": fc1_flops, "bytes": fc1_bytes, "overhead_bytes": overhead,
                           "per_unit": ("4*d*f FLOP per sorted row (T*k rows); bytes: W1 and W3 of the active "
                                        "experts + x once; overhead: the other T*k - T gathered x rows + h written")
                           if not args.fused else "6*d*f FLOP per sorted row; all active expert weights + x + out"}
    roof["traffic"] = None if args.fused else measured_traffic(cfg.name, "fc1_packed" if use_packed else "fc1")
    big_tile = cfg.dtype == "bf16" and os.environ.get("MOE_GEMM_REGIME", "1") != "0"
    if args.fused:
        roof["kernel"] = ("ffn_fused_kernel (route, dispatch, FC1 + SiLU*mul, FC2, combine; one launch"
                          f"{'; stage-order weights' if use_packed else ''})")
    elif big_tile:
        rows = moe.ffn_block_rows(moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype))
        roof["kernel"] = (f"gemm_dl_kernel<gated, {rows}x256{', stage-order weights' if use_packed else ''}> "
                          "(FC1 + SiLU*mul)")
    else:
        roof["kernel"] = "grouped_gemm_kernel<gated, 128x128> (FC1 + SiLU*mul)"
    roof["kernel_ms"] = round(fc1_ms, 4)

    ceilings = None
    if not args.no_ceilings:
        # measured ceilings of this GPU (diagnostic): the fraction above is against
        # the datasheet peak; this one is against what the library's probes sustain
        hbm = moe.probe_hbm_read_gbps()
        mfma = moe.probe_mfma_tflops()
        ceil = hbm if roof["unit"] == "GB/s" else mfma
        ceilings = {"hbm_read_GBps": round(hbm, 1), "mfma_bf16_TFLOPs": round(mfma, 1),
                    "frac_of_measured": round(roof["achieved"] / ceil, 4),
                    "kind": "library probes: streaming read through LDS; register-only bf16 MFMA chains"}

    layer_flops = rf.layer_flops(cfg.T, cfg.d, cfg.f, cfg.E, kk)
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
                   "n_shared": S, "ffn": "fused" if args.fused else "separate launches",
                   "weights": (f"stage order (packed once in {pack_ms:.2f} ms, outside the steps)" if use_packed
                               else "as stored [E][f][d], [E][d][f]"),
                   "bias_scale": cfg.bias_scale, "seed": seed, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"tflops": round(layer_flops / (ms * 1e-3) / 1e12, 1),
                  "gbps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                  "bound": rf.classify(layer_flops, layer_bytes).bound,
                  "floor_ms": round(rf.classify(layer_flops, layer_bytes).floor_s * 1e3, 4),
                  "kappa": round(rf.kappa(counts), 3), "active_experts": rf.active_experts(counts),
                  "util_pages": round(rf.util(cfg.k, cfg.E, rf.PEAK_HBM_BYTES_PER_S, rf.PEAK_MFMA_BF16_FLOPS, cfg.T), 4)},
        "ceilings": ceilings,
        "stages_ms": {s: round(v[0] / max(v[1], 1), 4) for s, v in stages.items() if v[1] > 0},
    }
    if not args.fused:
        res["stages_roofline"] = stage_rooflines(cfg, kk, counts, elt, res["stages_ms"])
    if not args.no_cpu_baseline:
        ntok = min(cfg.T, args.cpu_sample_tokens if args.cpu_sample_tokens > 0 else 256)
        res["cpu_baseline"] = cpu_baseline(cfg, inp, ntok, seed)
    else:
        res["cpu_baseline"] = None
    del inp, ws, out
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
