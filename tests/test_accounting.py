"""Host-only checks of the roofline accounting and of the bench command line.

The byte and FLOP counts are recomputed here from the shapes by hand
(parameter counts times bytes per element), not through the helpers, so a
dropped term or a wrong factor in the helpers fails a test."""
import json
import os
import subprocess
import sys

import pytest

from mixture_experts_layer_gate_amd import roofline as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Mixtral-8x22B shape: hidden 6144, expert FFN 16384, 8 experts, top-2
D, F, E, K = 6144, 16384, 8, 2


def test_layer_flops_per_token_mixtral():
    # per token: the gate touches d*E weights once (multiply + add), each of
    # the k experts touches its 3*d*f weights once
    per_token = 2 * D * E + K * 3 * D * F * 2
    assert rf.layer_flops(1, D, F, E, K) == per_token
    assert rf.layer_flops(256, D, F, E, K) == 256 * per_token
    assert abs(per_token / 1e9 - 1.208) < 5e-4


def test_fc1_fc2_split_the_ffn():
    rows = 777
    assert rf.fc1_flops(rows, D, F) + rf.fc2_flops(rows, D, F) == rf.ffn_flops(rows, D, F)
    assert rf.fc1_flops(rows, D, F) == 2 * rf.fc2_flops(rows, D, F)


def test_layer_bytes_decode_all_active():
    T = 256
    weights = E * 3 * D * F * 2          # W1, W3, W2 of every expert, bf16
    gate = D * E * 2
    act = 2 * T * D * 2                  # x read once, out written once
    counts = [T * K // E] * E
    assert rf.layer_bytes(T, D, F, E, counts) == weights + gate + act
    assert abs((weights + gate + act) / 1e9 - 4.838) < 1e-3


def test_layer_bytes_skip_idle_experts():
    T = 256
    full = rf.layer_bytes(T, D, F, E, [64] * E)
    three_idle = rf.layer_bytes(T, D, F, E, [128, 128, 64, 64, 128, 0, 0, 0])
    assert full - three_idle == 3 * 3 * D * F * 2
    assert rf.active_experts([0, 3, 0, 1]) == 2


def test_kernel_bytes_add_up_to_the_layer_bytes():
    T = 300
    counts = [75, 0, 150, 75, 0, 0, 0, 300]
    a = 4
    fc1 = rf.fc1_bytes(T, D, F, K, counts)
    fc2 = rf.fc2_bytes(T, D, F, K, counts)
    comb = rf.combine_bytes(T, D, K)
    # algorithmic: W1 and W3 of the active experts plus x read once (FC1), W2
    # (FC2), out written once (combine); with the gate weight, the layer's bytes
    assert fc1 == a * 2 * D * F * 2 + T * D * 2
    assert fc2 == a * D * F * 2
    assert comb == T * D * 2
    assert fc1 + fc2 + comb + D * E * 2 == rf.layer_bytes(T, D, F, E, counts)
    # implementation traffic, reported apart: x gathered T*k times instead of
    # once, h written and read back, y written and read back
    assert rf.fc1_overhead_bytes(T, D, F, K) == (T * K - T) * D * 2 + T * K * F * 2
    assert rf.fc2_overhead_bytes(T, D, F, K) == T * K * F * 2 + T * K * D * 2
    assert rf.combine_overhead_bytes(T, D, K) == T * K * D * 2 + T * K * 8


def test_classify_binding():
    # ridge of the chip in FLOP per byte; bf16 weights give 1 FLOP per byte
    # per row, so the ridge is also the rows per expert where MFMA takes over
    ridge = rf.PEAK_MFMA_BF16_FLOPS / rf.PEAK_HBM_BYTES_PER_S
    assert 300 < ridge < 330
    decode = rf.classify(rf.layer_flops(256, D, F, E, K), rf.layer_bytes(256, D, F, E, [64] * E))
    assert decode.bound == "hbm" and decode.floor_s == decode.t_byte_s
    T = 8192
    prefill = rf.classify(rf.layer_flops(T, D, F, E, K), rf.layer_bytes(T, D, F, E, [T * K // E] * E))
    assert prefill.bound == "mfma" and prefill.floor_s == prefill.t_flop_s


def test_bench_defaults_to_the_largest_single_gpu_workload():
    sys.path.insert(0, ROOT)
    import bench
    import moe_inputs
    cfg = moe_inputs.config(bench.DEFAULT_WORKLOAD)
    # the Mixtral-8x22B prefill layer with skewed routing: T=8192, top-2 of 8
    assert (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.dtype, cfg.bias_scale) == (8192, D, F, E, K, "bf16", 1.5)
    # the largest FLOP count of the single-GPU workloads
    flops = {n: rf.layer_flops(c.T, c.d, c.f, c.E, c.k) for n, c in moe_inputs.CONFIGS.items()}
    assert max(flops, key=flops.get) in ("mixtral_prefill_skew", "mixtral_prefill_bal")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stage_rooflines_by_hand():
    sys.path.insert(0, ROOT)
    import bench
    import moe_inputs
    cfg = moe_inputs.config("mixtral_decode")
    T, k = cfg.T, cfg.k
    counts = [T * k // cfg.E] * cfg.E
    ms = {"gate": 0.01, "fc1": 0.5, "fc2": 0.25, "combine": 0.01, "dispatch": 0.005}
    out = bench.stage_rooflines(cfg, k, counts, 2, ms)
    assert set(out) == set(ms)
    # gate: 2*T*d*E FLOP over 10 us against the unpacked fp32 vector peak
    gate = 2 * T * D * E / 1e-5 / 1e12
    assert out["gate"]["achieved"] == pytest.approx(gate, abs=0.01)
    assert out["gate"]["peak"] == pytest.approx(78.6, abs=0.05)
    # decode FC1 streams W1 and W3 of all 8 experts and reads x: HBM-bound
    fc1 = (8 * 2 * D * F * 2 + T * D * 2) / 0.5e-3 / 1e9
    assert out["fc1"]["bound"] == "hbm"
    assert out["fc1"]["achieved"] == pytest.approx(fc1, abs=0.01)
    assert out["fc1"]["frac"] == pytest.approx(fc1 / 8000.0, abs=1e-4)
    assert out["fc1"]["overhead_bytes"] == (T * K - T) * D * 2 + T * K * F * 2
    fc2 = 8 * D * F * 2 / 0.25e-3 / 1e9
    assert out["fc2"]["bound"] == "hbm"
    assert out["fc2"]["achieved"] == pytest.approx(fc2, abs=0.01)
    # the combine's algorithmic bytes are out written once
    comb = T * D * 2 / 1e-5 / 1e9
    assert out["combine"]["achieved"] == pytest.approx(comb, abs=0.01)
    assert out["combine"]["overhead_bytes"] == T * K * D * 2 + T * K * 8
