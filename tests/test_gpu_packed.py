"""Stage-order weights (moe_pack_weights, moe_layer_forward_packed).

The packed tensors hold each expert matrix's bf16 values in the order the
grouped FFN's loads fill an LDS stage, so the packed layer computes exactly
what moe_layer_forward computes: the bar is bitwise equality with it (itself
held to the oracle in test_gpu_parity.py), plus the oracle bar directly on one
shape. The packed values are also compared with the layout written out here
from its definition (16-byte unit (((e*N/64 + g)*K/64 + kt)*64 + rr)*8 + s
holds K elements kt*64 + 8*(s ^ ((rr//2) % 8)) .. +7 of row 64g + rr).
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
import mixture_experts_layer_gate_amd as moe
from conftest import to_numpy
from parity import OUT_TOL, gpu_float, rel_err

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _layout(w):
    """Expected packed tensor (bf16 bit patterns) of w [E][N][K], from the definition."""
    E, N, K = w.shape
    nk = K // 64
    out = np.zeros((E, N // 64, nk, 64, 8, 8), np.uint16)
    chunks = w.reshape(E, N // 64, 64, nk, 8, 8)            # [e, g, rr, kt, chunk, 8]
    for rr in range(64):
        for s in range(8):
            out[:, :, :, rr, s, :] = chunks[:, :, rr, :, s ^ ((rr // 2) % 8), :]
    return out.reshape(E, N, K)


def test_pack_layout_matches_definition():
    E, d, f = 3, 192, 320
    _say(f"case pack layout E{E} d{d} f{f}")
    inp = moe_inputs.random_inputs(8, d, f, E, 1, "bf16", 0.0, seed=21, device="cuda")
    dims = moe.Dims(8, d, f, E, 1, torch.bfloat16)
    packed = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    for name, p in zip(("w1", "w3", "w2"), packed):
        assert p.shape == inp[name].shape and p.dtype == inp[name].dtype
        want = _layout(to_numpy(inp[name], "bf16"))
        assert np.array_equal(to_numpy(p, "bf16"), want), name


PACKED_SHAPES = [
    # T, d, f, E, k, bias scale
    (256, 1024, 2048, 8, 2, 0.0),   # decode-like: 128-row tiles
    (600, 448, 704, 4, 2, 1.5),     # 256-row tiles, hot expert over several blocks; FC1 and FC2 column tails
    (2000, 512, 768, 8, 2, 0.0),    # several m-blocks per expert (FC2 256 columns wide under regime 2)
    (3, 512, 2240, 4, 2, 0.0),      # FC2 split along K
    (1, 2048, 1024, 8, 2, 0.0),     # one token: FC1 and FC2 split
    (97, 256, 192, 64, 6, 1.0),     # many experts, one FC1 column block
]


@pytest.mark.parametrize("regime", ["default", "0", "1", "2", "3"])
@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_packed_layer_bitwise(monkeypatch, shape, regime):
    T, d, f, E, k, s = shape
    _say(f"case packed {shape} regime {regime}")
    if regime == "default":
        monkeypatch.delenv("MOE_GEMM_REGIME", raising=False)
    else:
        monkeypatch.setenv("MOE_GEMM_REGIME", regime)
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed=22, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    packed = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"])
    ref, r0 = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                return_routing=True)
    got, r1 = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, packed=packed,
                                return_routing=True)
    torch.cuda.synchronize()
    for key in r0:
        assert torch.equal(r0[key], r1[key]), key
    if regime == "0":
        # the small-tile kernel reads the weights as stored (different
        # arithmetic order): the packed call uses the large tiles
        h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
        want = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")["out"]
        err = rel_err(gpu_float(got), want)
        _say(f"  packed vs oracle rel_err={err:.2e}")
        assert err <= OUT_TOL
    else:
        assert torch.equal(got, ref)


def test_packed_oracle_bar():
    T, d, f, E, k = 300, 512, 768, 8, 2
    _say("case packed oracle")
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", 1.0, seed=23, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    packed = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"])
    got = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, packed=packed)
    torch.cuda.synchronize()
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    want = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")["out"]
    err = rel_err(gpu_float(got), want)
    _say(f"  rel_err={err:.2e}")
    assert err <= OUT_TOL


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_decode_t1", "deepseek_bal", "dbrx_zipf", "mixtral_prefill_skew"])
def test_packed_full_size_bitwise(name):
    cfg = moe_inputs.config(name)
    _say(f"case packed full {name}")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    packed = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"])
    ref = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    got = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, packed=packed)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


TRANSPOSED_SHAPES = [
    # T, d, f, E, k: d and f of every multiple of 64 the two matrices' blocks can take
    (300, 192, 320, 3, 2),
    (64, 1024, 2048, 8, 2),
    (7, 7168, 2048, 4, 2),    # the DeepSeek-V3 expert shape: W2 blocks from 2048-wide rows
]


@pytest.mark.parametrize("shape", TRANSPOSED_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}".format(*s))
def test_pack_from_input_major_weights(shape):
    """moe_pack_weights_transposed on the d x f / f x d orientation ([E][d][f], [E][f][d]) gives
    the same stage-order bytes as moe_pack_weights on the [out][in] tensors, and the packed
    layer computes the stored-weight layer's bits."""
    T, d, f, E, k = shape
    _say(f"case pack transposed {shape}")
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", 1.0, seed=24, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    a = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"])
    w1t, w3t, w2t = (inp[n].transpose(1, 2).contiguous() for n in ("w1", "w3", "w2"))
    b = moe.pack_weights_transposed(dims, w1t, w3t, w2t)
    torch.cuda.synchronize()
    for name, pa, pb in zip(("w1", "w3", "w2"), a, b):
        assert torch.equal(pa.view(torch.int16), pb.view(torch.int16)), name
    if T * d * f <= 300 * 192 * 320:
        for name, pb in zip(("w1", "w3", "w2"), b):
            assert np.array_equal(to_numpy(pb, "bf16"), _layout(to_numpy(inp[name], "bf16"))), name
    ref = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    got = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, packed=b)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.timeout(600)
def test_pack_from_input_major_weights_full_size():
    """The Mixtral-8x22B prefill layer from input-major weights: packed bytes and layer output
    bitwise equal to those from the [out][in] tensors."""
    cfg = moe_inputs.config("mixtral_prefill_skew")
    _say("case pack transposed full mixtral_prefill_skew")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    a = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"])
    w1t, w3t, w2t = (inp[n].transpose(1, 2).contiguous() for n in ("w1", "w3", "w2"))
    b = moe.pack_weights_transposed(dims, w1t, w3t, w2t)
    torch.cuda.synchronize()
    for name, pa, pb in zip(("w1", "w3", "w2"), a, b):
        assert torch.equal(pa.view(torch.int16), pb.view(torch.int16)), name
    got_a = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, packed=a)
    got_b = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, packed=b)
    torch.cuda.synchronize()
    assert torch.equal(got_a, got_b)
