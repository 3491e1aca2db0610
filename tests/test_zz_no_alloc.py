"""moe_layer_forward_noalloc: the layer with the library's static scratch as workspace.

It runs the launches of moe_layer_forward, so the bar is bitwise equality with
it (itself held to the oracle in test_gpu_parity.py): outputs and every routing
array, on two calls in a row, the second with a smaller batch (the scratch keeps
the first call's contents, which the second must not depend on).
"""
import sys

import pytest
import torch

import moe_inputs
import mixture_experts_layer_gate_amd as moe

pytestmark = pytest.mark.gpu

ROUTING = ("logits", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _routing_buffers(dims, dev="cuda"):
    n = dims.T * dims.k
    return {"logits": torch.empty((dims.T, dims.E), dtype=torch.float32, device=dev),
            "topk_idx": torch.empty((dims.T, dims.k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((dims.T, dims.k), dtype=torch.float32, device=dev),
            "counts": torch.empty(dims.E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(dims.E + 1, dtype=torch.int32, device=dev),
            "perm": torch.empty(n, dtype=torch.int32, device=dev),
            "inv_perm": torch.empty(n, dtype=torch.int32, device=dev)}


def _check(dims, inp, T):
    x = inp["x"][:T].contiguous()
    d = moe.Dims(T, dims.d, dims.f, dims.E, dims.k, dims.dtype)
    ref, r = moe.layer_forward(d, x, inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], return_routing=True)
    out = torch.full_like(ref, float("nan"))
    rb = _routing_buffers(d)
    moe.layer_forward_noalloc(d, x, inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], out, routing=rb)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
    for key in ROUTING:
        assert torch.equal(rb[key], r[key]), key
    # the optional routing outputs may also stay in the scratch
    out2 = torch.full_like(ref, float("nan"))
    moe.layer_forward_noalloc(d, x, inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


SHAPES = [
    # T first call, T second (smaller) call, d, f, E, k, dtype, bias scale
    (300, 37, 1024, 2048, 8, 2, "bf16", 1.0),
    (700, 5, 256, 512, 64, 6, "bf16", 2.0),
    (96, 11, 128, 256, 8, 2, "f32", 0.0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T{}then{}_d{}_f{}_E{}_k{}_{}".format(*s[:7]))
def test_noalloc_matches_layer_forward(shape):
    T1, T2, d, f, E, k, dt, s = shape
    _say(f"case noalloc {shape}")
    inp = moe_inputs.random_inputs(T1, d, f, E, k, dt, s, seed=41, device="cuda")
    dims = moe.Dims(T1, d, f, E, k, torch.bfloat16 if dt == "bf16" else torch.float32)
    _check(dims, inp, T1)
    _check(dims, inp, T2)


@pytest.mark.timeout(600)
def test_noalloc_mixtral_decode_then_single_token():
    """The Mixtral-8x22B decode step (256 tokens) then one token (whose FC2 splits along K
    through the scratch's partial buffer)."""
    cfg = moe_inputs.config("mixtral_decode")
    _say("case noalloc mixtral_decode then T=1")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    assert moe.workspace_bytes(dims) <= moe.NOALLOC_SCRATCH_BYTES
    _check(dims, inp, cfg.T)
    _check(dims, inp, 1)


@pytest.mark.timeout(600)
def test_noalloc_mixtral_shape_700_then_300_tokens():
    """The Mixtral-8x22B layer shape at 700 tokens (256-row blocks; near the largest
    batch the scratch holds), then 300 tokens."""
    _say("case noalloc mixtral shape T=700 then T=300")
    inp = moe_inputs.random_inputs(700, 6144, 16384, 8, 2, "bf16", 1.0, seed=43, device="cuda")
    dims = moe.Dims(700, 6144, 16384, 8, 2, torch.bfloat16)
    assert moe.workspace_bytes(dims) <= moe.NOALLOC_SCRATCH_BYTES
    _check(dims, inp, 700)
    _check(dims, inp, 300)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    cfg = moe_inputs.config("mixtral_prefill_skew")
    _say("case noalloc refuses prefill")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    x = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    wg = torch.empty((cfg.E, cfg.d), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((cfg.E, 64, 64), dtype=torch.bfloat16, device="cuda")
    lib = moe.load_library()
    st = lib.moe_layer_forward_noalloc(moe.api.ctypes.byref(dims.c()), x.data_ptr(), wg.data_ptr(), None,
                                       w.data_ptr(), w.data_ptr(), w.data_ptr(), x.data_ptr(), None, None, None,
                                       None, None, None, None, None)
    assert st == 5
