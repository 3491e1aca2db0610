"""The fused launch (moe_layer_forward_fused): route and dispatch (for E <= 64),
FC1, FC2 and the combine in one persistent kernel with device-side readiness
counters; MOE_FUSED_FRONT=0 keeps route and dispatch as separate launches before
it, and both forms are tested.

Its tiles do exactly the arithmetic of moe_layer_forward's separate launches:
the same rows per block, FC2 tile width, weight layout and split of K (every
tile of a launch with fewer tiles than compute units; the last partial round
of FC2 tiles at prefill sizes), whose parts the workgroup storing the last one
sums in the separate reduce's order. So the bar is
bitwise equality with that path (itself held to the oracle in
test_gpu_parity.py), checked twice in a row on the same buffers (a missed
wait or a stale read would show up as a difference), plus the oracle bar on
small shapes directly. Shapes with split FC1 and FC2 tiles (FC2 parts then
wait for every split FC1 tile to be summed) run in both tile regimes, and once
with splitting turned off on both sides.
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
import mixture_experts_layer_gate_amd as moe
from conftest import to_numpy
from parity import OUT_TOL, check_plan, gpu_float, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["front", "ffn_only"])
def _front(monkeypatch, request):
    monkeypatch.delenv("MOE_SPLIT_K", raising=False)
    if request.param == "ffn_only":
        monkeypatch.setenv("MOE_FUSED_FRONT", "0")
    else:
        monkeypatch.delenv("MOE_FUSED_FRONT", raising=False)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(cfg_or_shape, seed=0, packed=False):
    if isinstance(cfg_or_shape, str):
        cfg = moe_inputs.config(cfg_or_shape)
        inp = moe_inputs.make_layer_inputs(cfg, seed, "cuda")
        T, d, f, E, k = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k
    else:
        T, d, f, E, k, s = cfg_or_shape
        inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    pk = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"]) if packed else None
    ref, r_ref = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                   return_routing=True, packed=pk)
    ws = moe.make_workspace(dims)
    outs = []
    for _ in range(2):
        out, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], ws=ws,
                                   return_routing=True, fused=True, packed=pk)
        torch.cuda.synchronize()
        # every readiness wait of the launch was met: its outputs are valid
        assert moe.fused_status(dims, ws) == 0
        # the routing arrays (computed in the launch itself, or before it) are the separate launches' bits
        for key in r_ref:
            assert torch.equal(r[key], r_ref[key]), key
        outs.append(out.clone())
    # the tile plan the fused launch used, where a layer call leaves it
    plan = moe.read_plan(dims, ws).numpy()
    check_plan(plan, r_ref["counts"].cpu().numpy(), r_ref["offsets"].cpu().numpy(), moe.ffn_block_rows(dims), T * k)
    return inp, ref, outs, r


FUSED_SHAPES = [
    # T, d, f, E, k, bias scale
    (200, 256, 512, 8, 2, 0.0),
    (300, 512, 768, 4, 2, 1.5),
    (64, 256, 256, 16, 4, 2.0),      # experts without rows
    (40, 128, 256, 8, 8, 0.0),       # k = E
    (1, 256, 256, 4, 2, 0.0),
    (1000, 512, 1024, 8, 2, 0.0),    # several m-blocks per expert
]


@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_fused_small_bitwise_and_oracle(shape):
    _say(f"case fused {shape}")
    inp, ref, outs, r = _both(shape)
    for o in outs:
        assert torch.equal(o, ref)
    T, d, f, E, k, _ = shape
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    want = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")["out"]
    err = rel_err(gpu_float(outs[0]), want)
    _say(f"  bitwise equal to the separate launches; out rel_err={err:.2e}")
    assert err <= OUT_TOL


SPLIT_SHAPES = [
    # T, d, f, E, k, bias scale: fewer tiles than CUs, K of 1024 or more, or a
    # multi-round FC2 whose last partial round is split
    (1, 1024, 1024, 8, 2, 0.0),      # 128-row tiles, FC1 and FC2 split
    (300, 1024, 1024, 4, 2, 1.0),    # 256-row tiles, FC1 and FC2 split
    (16, 2048, 4096, 8, 2, 0.0),     # FC1 whole, FC2 in 4 parts of 16 K steps
    (5, 1536, 1024, 16, 4, 2.0),     # FC1 in 3 parts, FC2 in 2
    (8300, 2048, 1024, 2, 2, 0.0),   # last rounds of 16 tiles (of 528) cut: FC1 in 4 parts, FC2 in 2
]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_fused_split_k_bitwise_and_oracle(shape):
    test_fused_small_bitwise_and_oracle(shape)


def test_fused_whole_k_when_splitting_is_off(monkeypatch):
    """MOE_SPLIT_K=0 turns splitting off for both forms alike."""
    monkeypatch.setenv("MOE_SPLIT_K", "0")
    test_fused_small_bitwise_and_oracle(SPLIT_SHAPES[0])


@pytest.mark.parametrize("shape", [SPLIT_SHAPES[0], SPLIT_SHAPES[1], FUSED_SHAPES[1], FUSED_SHAPES[5]],
                         ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_fused_packed_bitwise(shape):
    """moe_layer_forward_fused_packed against moe_layer_forward_packed."""
    _say(f"case fused packed {shape}")
    _, ref, outs, _ = _both(shape, packed=True)
    for o in outs:
        assert torch.equal(o, ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_decode_t1", "mixtral_decode_t16", "mixtral_prefill_skew",
                                  "dbrx_zipf", "deepseek_skew", "deepseek_bal"])
def test_fused_full_size_bitwise(name):
    _say(f"case fused full {name}")
    _, ref, outs, _ = _both(name)
    for o in outs:
        assert torch.equal(o, ref)
    _say("  bitwise equal to the separate launches, twice")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_decode_t1", "mixtral_prefill_skew"])
def test_fused_packed_full_size_bitwise(name):
    _say(f"case fused packed full {name}")
    _, ref, outs, _ = _both(name, packed=True)
    for o in outs:
        assert torch.equal(o, ref)
    _say("  bitwise equal to the separate packed launches, twice")


def test_fused_reports_a_wait_that_gave_up(monkeypatch):
    """A readiness wait that gives up is reported through moe_fused_status. The failure is
    forced from the host: MOE_FUSED_SPIN_LIMIT=-1 makes every wait that finds its counter
    short give up at once (the kernel then reads operands that may not be stored yet, so
    only the status is checked; with route and dispatch in the launch, a workgroup that gives
    up waiting for the plan leaves the launch at once); a normal call on the same workspace
    clears the word again and gives the separate launches' bits."""
    shape = (1000, 512, 1024, 8, 2, 0.0)
    _say(f"case fused wait failure reported {shape}")
    T, d, f, E, k, s = shape
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, 3, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    ref = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    ws = moe.make_workspace(dims)
    args = (dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    monkeypatch.setenv("MOE_FUSED_SPIN_LIMIT", "-1")
    flags = []
    for _ in range(3):  # some combine block waits on FC2 tiles still running in every launch of this size
        moe.layer_forward(*args, ws=ws, fused=True)
        flags.append(moe.fused_status(dims, ws))
    _say(f"  status words with no waiting: {flags}")
    assert any(v != 0 for v in flags)
    monkeypatch.delenv("MOE_FUSED_SPIN_LIMIT")
    out = moe.layer_forward(*args, ws=ws, fused=True)
    assert moe.fused_status(dims, ws) == 0
    assert torch.equal(out, ref)


def test_fused_rejects_fp32():
    cfg = moe_inputs.config("tiny_fp32")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, torch.float32)
    with pytest.raises(moe.MoeError) as ex:
        moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], fused=True)
    assert ex.value.status == 2
