"""Tile queues of the 256-row forward launches (dynamic tile order).

Where experts' rows span several m-blocks the FC1 and FC2 launches take
their tiles from per-XCD queues in the workspace instead of fixed shares.
Which workgroup computes a tile changes nothing in how it is computed, so the
bar is bitwise equality with the fixed-share order (MOE_TILE_QUEUES=0), on
weights as stored and in stage order, twice in a row on one workspace (the
plan kernel must re-arm the queues), plus the oracle bar on one shape.
"""
import os
import sys

import pytest
import torch

import moe_inputs
import oracle
import mixture_experts_layer_gate_amd as moe
from conftest import to_numpy
from parity import OUT_TOL, gpu_float, rel_err

pytestmark = pytest.mark.gpu

SHAPES = [
    # T, d, f, E, k, bias scale: every one has more than 256 rows per active expert
    (1024, 256, 512, 4, 2, 0.0),    # two m-blocks per expert, a few rounds of tiles
    (3000, 512, 768, 8, 2, 1.5),    # skewed: a hot expert of many m-blocks, partial blocks, K split tail
    (700, 1024, 512, 2, 1, 0.0),    # fewer tiles than CUs: every FC1 tile split along K
    (2048, 1024, 1536, 16, 4, 1.0), # DBRX-like proportions, Zipf-biased
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(dims, inp, ws, packed, queues):
    old = os.environ.get("MOE_TILE_QUEUES")
    os.environ["MOE_TILE_QUEUES"] = "1" if queues else "0"
    try:
        if packed is None:
            out = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], ws=ws)
        else:
            out = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], None, None, None, ws=ws, packed=packed)
        torch.cuda.synchronize()
        return out
    finally:
        if old is None:
            del os.environ["MOE_TILE_QUEUES"]
        else:
            os.environ["MOE_TILE_QUEUES"] = old


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("stage_order", [False, True])
def test_queues_bitwise_equal_fixed_shares(shape, stage_order):
    T, d, f, E, k, s = shape
    _say(f"case tile queues T{T} d{d} f{f} E{E} k{k} s{s} stage_order={stage_order}")
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed=7, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    assert moe.ffn_block_rows(dims) == 256
    packed = moe.pack_weights(dims, inp["w1"], inp["w3"], inp["w2"]) if stage_order else None
    ws = torch.empty(moe.workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    ref = _run(dims, inp, ws, packed, queues=False)
    assert moe.read_plan_multi_block(dims, ws) == 1, "these shapes have experts of several m-blocks"
    for rep in range(2):  # the second call reuses the workspace: the plan re-arms the queues
        got = _run(dims, inp, ws, packed, queues=True)
        assert torch.equal(got, ref), f"call {rep}: queued tile order changed the output bits"


def test_queues_oracle_bar():
    T, d, f, E, k, s = 1500, 256, 384, 4, 2, 1.0
    _say(f"case tile queues vs oracle T{T} d{d} f{f} E{E} k{k} s{s}")
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed=3, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    out = _run(dims, inp, None, None, queues=True)
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    ref = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")
    err = rel_err(gpu_float(out), ref["out"])
    assert err <= OUT_TOL, err
