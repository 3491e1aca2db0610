"""moe_layer_backward_ex through the C ABI: bf16 weight gradients.

Each bf16 element of dw1, dw3 and dw2 must be the round-to-nearest-even bf16 of
the fp32 element moe_layer_backward writes (torch's float32 -> bfloat16
conversion rounds the same way), and every other output must be bitwise
moe_layer_backward's; so this form inherits the fp32 form's parity with the
backward oracle (tests/test_gpu_backward.py) plus one rounding. The same holds
with the g | u rows kept by moe_layer_forward_train, on small shapes, the
empty batch, and the DeepSeek-shaped workload whose weight gradients the bf16
form is for.
"""
import sys

import pytest
import torch

import moe_inputs
import mixture_experts_layer_gate_amd as moe

pytestmark = pytest.mark.gpu

WEIGHT_GRADS = ("dw1", "dw3", "dw2")
OTHER = ("dx", "dwg", "dbias", "dlogits", "dtopk_w")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(inp, dout, dims, tag):
    _, r, gu = moe.layer_forward_train(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    args = (dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r, dout)
    ws = torch.empty(moe.backward_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    g32 = moe.layer_backward(*args, ws=ws, want_dlogits=True, want_dtopk_w=True)
    g16 = moe.layer_backward(*args, ws=ws, want_dlogits=True, want_dtopk_w=True, wgrad_dtype=torch.bfloat16)
    g16s = moe.layer_backward(*args, ws=ws, want_dlogits=True, want_dtopk_w=True, wgrad_dtype=torch.bfloat16,
                              gu=gu)
    torch.cuda.synchronize()
    for n in WEIGHT_GRADS:
        assert g16[n].dtype == torch.bfloat16, n
        assert torch.equal(g16[n], g32[n].to(torch.bfloat16)), (tag, n)
        assert torch.equal(g16s[n], g16[n]), (tag, n)
    for n in OTHER:
        assert torch.equal(g16[n], g32[n]), (tag, n)
        assert torch.equal(g16s[n], g32[n]), (tag, n)


SHAPES = [
    # T, d, f, E, k, bias scale
    (200, 256, 512, 8, 2, 0.0),
    (300, 512, 768, 4, 2, 1.0),
    (64, 256, 256, 16, 4, 2.0),      # experts without rows: zero bf16 gradients
    (1500, 256, 512, 4, 2, 1.0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_bf16_weight_grads(shape):
    T, d, f, E, k, s = shape
    _say(f"case backward_ex bf16 {shape}")
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, 0, device="cuda")
    dout = moe_inputs.output_grad(T, d, "bf16", 0, device="cuda")
    _check(inp, dout, moe.Dims(T, d, f, E, k, torch.bfloat16), shape)


def test_bf16_weight_grads_zero_batch():
    """T = 0: every bf16 weight gradient is written as zeros."""
    d, f, E, k = 256, 256, 8, 2
    _say("case backward_ex bf16 empty batch")
    inp = moe_inputs.random_inputs(1, d, f, E, k, "bf16", 0.0, 0, device="cuda")
    dims0 = moe.Dims(0, d, f, E, k, torch.bfloat16)
    z = {n: torch.empty(0, dtype=torch.int32, device="cuda") for n in ("perm", "inv_perm")}
    z["topk_idx"] = torch.empty((0, k), dtype=torch.int32, device="cuda")
    z["topk_w"] = torch.empty((0, k), dtype=torch.float32, device="cuda")
    z["counts"] = torch.zeros(E, dtype=torch.int32, device="cuda")
    z["offsets"] = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    filled = {n: torch.full((E, f, d), 7.0, dtype=torch.bfloat16, device="cuda") for n in ("dw1", "dw3")}
    filled["dw2"] = torch.full((E, d, f), 7.0, dtype=torch.bfloat16, device="cuda")
    filled["dwg"] = torch.full((E, d), 7.0, dtype=torch.float32, device="cuda")
    filled["dbias"] = torch.full((E,), 7.0, dtype=torch.float32, device="cuda")
    filled["dx"] = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    x0 = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    out = moe.layer_backward(dims0, x0, inp["wg"], inp["w1"], inp["w3"], inp["w2"], z, x0, grads=filled,
                             wgrad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for n in ("dwg", "dbias", "dw1", "dw3", "dw2"):
        assert not torch.any(out[n]), n


@pytest.mark.timeout(600)
def test_bf16_weight_grads_full_size():
    cfg = moe_inputs.config("deepseek_skew")
    _say(f"case backward_ex bf16 full {cfg.name}")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dout = moe_inputs.output_grad(cfg.T, cfg.d, cfg.dtype, 0, device="cuda")
    _check(inp, dout, moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype), cfg.name)
