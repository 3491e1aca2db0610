"""Parity of the HIP path with the CPU oracle, through the C ABI.

Bar: routing indices, counts, offsets, permutations and gate logits bit-exact;
combine weights within 1e-5 relative; outputs within max |g - r| / max(|r|, rms(r))
<= 2e-2. Small shapes are compared element by element over every output; the
full-size workloads compare all routing arrays, check the GPU's tile plan
against its invariants, and compare every output row (decode and DBRX shapes)
or one token per m-block (prefill and DeepSeek shapes).
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
import mixture_experts_layer_gate_amd as moe
from conftest import to_numpy
from parity import (OUT_TOL, LazyExperts, assert_routing_equal, check_plan, gpu_float, host_inputs,
                    oracle_outputs_threaded, oracle_routing, rel_err)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dims(cfg, T=None):
    return moe.Dims(cfg.T if T is None else T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)


def _run_layer(cfg, inp):
    dims = _dims(cfg, inp["x"].shape[0])
    out, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                               return_routing=True)
    torch.cuda.synchronize()
    return out, r


def _full_oracle_check(cfg, inp):
    out, r = _run_layer(cfg, inp)
    h = {n: to_numpy(v, cfg.dtype) for n, v in inp.items()}
    ref = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], cfg.k, cfg.dtype)
    assert_routing_equal(r, ref)
    err = rel_err(gpu_float(out), ref["out"])
    _say(f"  {cfg.name} T={inp['x'].shape[0]} out rel_err={err:.3e}")
    assert err <= OUT_TOL
    return out, r, ref


def test_tiny_fp32_layer():
    cfg = moe_inputs.config("tiny_fp32")
    _say(f"case tiny_fp32 {cfg}")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    _full_oracle_check(cfg, inp)


SMALL = [
    # T, d, f, E, k, dtype, bias scale
    (300, 256, 192, 8, 2, "bf16", 0.0),     # several m-blocks, ragged tails
    (1, 128, 64, 4, 1, "bf16", 0.0),        # one token
    (5, 64, 64, 1, 1, "bf16", 0.0),         # one expert: dense SwiGLU
    (257, 512, 384, 64, 6, "bf16", 1.0),    # many experts, skew
    (130, 192, 128, 16, 4, "bf16", 2.0),    # d not a multiple of 128
    (1000, 128, 256, 256, 8, "bf16", 2.0),  # fine-grained, strong skew: idle experts
    (700, 256, 320, 8, 8, "bf16", 0.0),     # k = E: every expert gets every token
    (96, 128, 256, 8, 2, "f32", 1.5),       # fp32 path with skew
    (9000, 128, 128, 64, 8, "bf16", 1.0),   # > 65536 assignments: multi-kernel dispatch + plan
    (64, 4096, 2048, 8, 2, "bf16", 0.0),    # decode-shaped: wide d and f, few rows per expert
    (200, 64, 64, 1024, 4, "bf16", 1.0),    # the largest expert count
    (40, 64, 128, 1024, 1024, "bf16", 0.0),  # k = E = 1024: every token to every expert
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_{}_s{}".format(*s))
def test_small_shapes(shape):
    T, d, f, E, k, dt, s = shape
    _say(f"case small {shape}")
    cfg = moe_inputs.LayerConfig("small", T, d, f, E, k, dt, s)
    inp = moe_inputs.make_layer_inputs(cfg, 1, "cuda")
    _full_oracle_check(cfg, inp)


def test_forced_skew_all_tokens_to_k_experts():
    cfg = moe_inputs.LayerConfig("forced", 520, 256, 192, 16, 3, "bf16", 0.0)
    _say("case forced skew")
    inp = moe_inputs.make_layer_inputs(cfg, 2, "cuda")
    bias = torch.zeros(cfg.E, dtype=torch.float32)
    bias[:cfg.k] = 1e4
    inp["bias"] = bias.cuda()
    out, r, ref = _full_oracle_check(cfg, inp)
    assert r["counts"].cpu().tolist() == [cfg.T] * cfg.k + [0] * (cfg.E - cfg.k)


# Exactly tied logits: rows of x that are zero give logit = bias exactly, and
# the bias repeats values (and holds both -0.0 and +0.0, equal under IEEE
# comparison). Equal logits go to the lower expert index, on both the one-launch
# gate + top-k (small batches) and the separate launches.
@pytest.mark.parametrize("shape", [(96, 128, 128, 8, 3), (700, 256, 128, 8, 3), (300, 256, 128, 32, 4)],
                         ids=lambda s: "T{}_d{}_f{}_E{}_k{}".format(*s))
def test_tied_logits_take_the_lower_expert(shape):
    T, d, f, E, k = shape
    _say(f"case tied logits {shape}")
    cfg = moe_inputs.LayerConfig("ties", T, d, f, E, k, "bf16", 0.0)
    inp = moe_inputs.make_layer_inputs(cfg, 4, "cuda")
    inp["x"][::3] = 0
    base = [0.5, 1.0, 1.0, -0.0, 0.0, 1.0, 0.25, 0.5]
    bias = torch.tensor([base[e % 8] for e in range(E)], dtype=torch.float32)
    inp["bias"] = bias.cuda()
    out, r, ref = _full_oracle_check(cfg, inp)
    idx = r["topk_idx"].cpu().numpy()[::3]
    want = [e for e in np.argsort(-bias.numpy(), kind="stable")[:k]]
    assert (idx == np.array(want, dtype=idx.dtype)[None, :]).all()
    w = r["topk_w"].cpu().numpy()[::3]
    # tied selected logits: equal weights summing to one
    if len({float(bias[e]) for e in want}) == 1:
        np.testing.assert_allclose(w, 1.0 / k, rtol=1e-6)


def test_all_logits_tied_pick_the_first_k():
    cfg = moe_inputs.LayerConfig("allties", 64, 128, 128, 16, 4, "bf16", 0.0)
    _say("case all logits tied")
    inp = moe_inputs.make_layer_inputs(cfg, 5, "cuda")
    inp["x"].zero_()
    inp["bias"] = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
    out, r, ref = _full_oracle_check(cfg, inp)
    assert (r["topk_idx"].cpu().numpy() == np.arange(cfg.k)[None, :]).all()
    np.testing.assert_allclose(r["topk_w"].cpu().numpy(), 1.0 / cfg.k, rtol=1e-6)
    assert r["counts"].cpu().tolist() == [cfg.T] * cfg.k + [0] * (cfg.E - cfg.k)
    assert float(np.abs(gpu_float(out)).max()) == 0.0


def test_determinism_bitwise():
    cfg = moe_inputs.LayerConfig("det", 777, 256, 256, 32, 4, "bf16", 1.0)
    _say("case determinism")
    inp = moe_inputs.make_layer_inputs(cfg, 3, "cuda")
    o1, r1 = _run_layer(cfg, inp)
    o2, r2 = _run_layer(cfg, inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for n in r1:
        assert torch.equal(r1[n], r2[n]), n


def test_stage_calls_match_layer_forward():
    cfg = moe_inputs.LayerConfig("stages", 333, 256, 192, 8, 2, "bf16", 1.0)
    _say("case stage calls")
    inp = moe_inputs.make_layer_inputs(cfg, 4, "cuda")
    dims = _dims(cfg)
    out_l, r = _run_layer(cfg, inp)
    logits, idx, w = moe.route(dims, inp["x"], inp["wg"], inp["bias"])
    counts, offsets, perm, inv = moe.permute(dims, idx)
    y = moe.grouped_ffn(dims, inp["x"], perm, counts, offsets, inp["w1"], inp["w3"], inp["w2"])
    out = moe.combine(dims, y, inv, w)
    torch.cuda.synchronize()
    for a, b in ((logits, r["logits"]), (idx, r["topk_idx"]), (w, r["topk_w"]), (perm, r["perm"]),
                 (inv, r["inv_perm"]), (counts, r["counts"])):
        assert torch.equal(a, b)
    assert torch.equal(out.view(torch.int16), out_l.view(torch.int16))


def test_permute_on_given_indices():
    """moe_permute on hand-made routing: all assignments to one expert, and a random one."""
    _say("case permute given idx")
    rng = np.random.default_rng(7)
    cases = []
    for T, E, k in ((1500, 64, 4), (20000, 64, 4)):  # single-workgroup path and multi-kernel path
        cases.append((T, E, k, np.tile(np.array([[5, 9, 0, 63]], np.int32), (T, 1))))
        cases.append((T, E, k, np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)))
    for T, E, k, idx_np in cases:
        dims = moe.Dims(T, 128, 128, E, k)
        counts, offsets, perm, inv = moe.permute(dims, torch.from_numpy(idx_np).cuda())
        torch.cuda.synchronize()
        rc, ro, rp, ri = oracle.dispatch(idx_np, E)
        assert np.array_equal(counts.cpu().numpy(), rc) and np.array_equal(offsets.cpu().numpy(), ro)
        assert np.array_equal(perm.cpu().numpy(), rp) and np.array_equal(inv.cpu().numpy(), ri)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_dispatch_paths_bit_exact(monkeypatch, path):
    """Both dispatch implementations (one workgroup, or histogram/scan/scatter kernels) on the
    same skewed routing, 32768 assignments over 256 experts, against the oracle."""
    _say(f"case dispatch path {path}")
    monkeypatch.setenv("MOE_DISPATCH", path)
    rng = np.random.default_rng(11)
    T, E, k = 4096, 256, 8
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    idx_np = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = moe.permute(moe.Dims(T, 128, 128, E, k), torch.from_numpy(idx_np).cuda())
    torch.cuda.synchronize()
    rc, ro, rp, ri = oracle.dispatch(idx_np, E)
    assert np.array_equal(counts.cpu().numpy(), rc) and np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp) and np.array_equal(inv.cpu().numpy(), ri)


def test_grouped_ffn_round_robin_routing():
    """Exactly balanced synthetic routing e = (t*k + j) mod E fed to moe_grouped_ffn."""
    cfg = moe_inputs.LayerConfig("rr", 256, 256, 320, 8, 2, "bf16", 0.0)
    _say("case round robin ffn")
    inp = moe_inputs.make_layer_inputs(cfg, 5, "cuda")
    dims = _dims(cfg)
    idx_np = (np.arange(cfg.T * cfg.k) % cfg.E).reshape(cfg.T, cfg.k).astype(np.int32)
    counts, offsets, perm, inv = oracle.dispatch(idx_np, cfg.E)
    y = moe.grouped_ffn(dims, inp["x"], torch.from_numpy(perm).cuda(), torch.from_numpy(counts).cuda(),
                        torch.from_numpy(offsets).cuda(), inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    h = {n: to_numpy(v, cfg.dtype) for n, v in inp.items()}
    ref = oracle.expert_ffn_sorted(h["x"], perm, offsets, h["w1"], h["w3"], h["w2"], cfg.k, cfg.dtype)
    assert rel_err(gpu_float(y), ref) <= OUT_TOL


REGIME_SHAPES = [
    # T, d, f, E, k, bias scale
    (600, 256, 384, 4, 2, 1.5),   # hot expert spans several 256-row blocks, ragged tails
    (300, 320, 192, 8, 3, 0.0),   # column tails in FC1 (f=192) and FC2 (d=320)
    (64, 128, 128, 2, 1, 0.0),    # one block per expert
]


GEMM_REGIMES = [0, 1, 2, 3]


@pytest.mark.parametrize("regime", GEMM_REGIMES)
@pytest.mark.parametrize("shape", REGIME_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_each_gemm_tile_regime(monkeypatch, regime, shape):
    """Every grouped-GEMM tile configuration (forced through MOE_GEMM_REGIME) matches the oracle."""
    T, d, f, E, k, s = shape
    _say(f"case regime {regime} {shape}")
    monkeypatch.setenv("MOE_GEMM_REGIME", str(regime))
    cfg = moe_inputs.LayerConfig("regime", T, d, f, E, k, "bf16", s)
    inp = moe_inputs.make_layer_inputs(cfg, 6, "cuda")
    _full_oracle_check(cfg, inp)


SPLIT_SHAPES = [
    # T, d, f, E, k, bias scale: launches with fewer tiles than CUs, K cut into parts
    (1, 2048, 1024, 8, 2, 0.0),     # one token: FC1 in 4 parts, FC2 in 2
    (2, 1088, 2112, 8, 2, 0.0),     # column tails in both GEMMs; 17 and 33 K steps in uneven parts
    (3, 512, 2240, 4, 2, 0.0),      # FC2 alone split: 35 K steps in 4 parts
    (600, 2048, 1024, 2, 1, 1.0),   # few experts with many rows: parts of up to 256 rows
    (100, 1024, 1536, 1, 1, 0.0),   # one expert: FC2 in 3 parts
    (1200, 1024, 4096, 4, 2, 0.0),  # 256-row tiles: FC1 unsplit (384 tiles), FC2 (72 tiles of 192) in 3 parts
    # k = E: 33 blocks of 256 rows per expert; FC1 and FC2 have 528 tiles each, two
    # full rounds of 256 CUs and a last round of 16 tiles, which alone are cut
    # (FC1 in 4 parts, FC2 in 2)
    (8300, 2048, 1024, 2, 2, 0.0),
]


@pytest.mark.parametrize("regime", ["default", "1"])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_split_k_launches(monkeypatch, shape, regime):
    """Launches split along K (every tile of a few-tile launch, or the last partial
    round of a multi-round FC2): oracle bar, bitwise repeatable, and within the
    oracle bar of the same layer run unsplit (MOE_SPLIT_K=0); with the tiles the batch
    size picks and with 256-row tiles forced."""
    T, d, f, E, k, s = shape
    _say(f"case split-K {shape} regime {regime}")
    if regime == "default":
        monkeypatch.delenv("MOE_GEMM_REGIME", raising=False)
    else:
        monkeypatch.setenv("MOE_GEMM_REGIME", regime)
    cfg = moe_inputs.LayerConfig("splitk", T, d, f, E, k, "bf16", s)
    inp = moe_inputs.make_layer_inputs(cfg, 13, "cuda")
    out, _, ref = _full_oracle_check(cfg, inp)
    again, _ = _run_layer(cfg, inp)
    assert torch.equal(out, again)
    monkeypatch.setenv("MOE_SPLIT_K", "0")
    whole, _ = _run_layer(cfg, inp)
    err = rel_err(gpu_float(whole), ref["out"])
    diff = rel_err(gpu_float(out), gpu_float(whole))
    _say(f"  unsplit rel_err={err:.3e}; split vs unsplit {diff:.3e}")
    assert err <= OUT_TOL and diff <= OUT_TOL


# Rows per expert chosen so that, in 256-row blocks, the upper and lower 128-row
# halves of a block hold every number (0..4) of non-empty 32-row sub-blocks.
PARTIAL_COUNTS = [1, 40, 70, 100, 128, 129, 170, 200, 255, 256, 300]


@pytest.mark.parametrize("regime", GEMM_REGIMES)
def test_grouped_ffn_partial_blocks(monkeypatch, regime):
    """moe_grouped_ffn on shuffled top-1 routing with the counts above, against the oracle."""
    _say(f"case partial blocks regime {regime}")
    monkeypatch.setenv("MOE_GEMM_REGIME", str(regime))
    E, T = len(PARTIAL_COUNTS), sum(PARTIAL_COUNTS)
    cfg = moe_inputs.LayerConfig("partial", T, 256, 192, E, 1, "bf16", 0.0)
    inp = moe_inputs.make_layer_inputs(cfg, 8, "cuda")
    rng = np.random.default_rng(8)
    idx_np = rng.permutation(np.repeat(np.arange(E), PARTIAL_COUNTS)).astype(np.int32).reshape(T, 1)
    counts, offsets, perm, inv = oracle.dispatch(idx_np, E)
    assert list(counts) == PARTIAL_COUNTS
    y = moe.grouped_ffn(_dims(cfg), inp["x"], torch.from_numpy(perm).cuda(), torch.from_numpy(counts).cuda(),
                        torch.from_numpy(offsets).cuda(), inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    h = {n: to_numpy(v, cfg.dtype) for n, v in inp.items()}
    ref = oracle.expert_ffn_sorted(h["x"], perm, offsets, h["w1"], h["w3"], h["w2"], cfg.k, cfg.dtype)
    err = rel_err(gpu_float(y), ref)
    _say(f"  rel_err={err:.3e}")
    assert err <= OUT_TOL


@pytest.mark.parametrize("gate_cfg", ["8,2,4", "4,4,4", "2,4,8", "lds", "lds2", "mfma", ""])
@pytest.mark.parametrize("shape", [(300, 200, 24), (77, 512, 8), (1000, 1024, 64), (500, 832, 48), (45, 576, 40),
                                   (130, 7168, 256)],
                         ids=lambda s: "T{}_d{}_E{}".format(*s))
def test_gate_tile_configs_bit_exact(monkeypatch, gate_cfg, shape):
    """Every gate register-tile configuration (forced via MOE_GATE_CFG) gives the oracle's logits bit for bit."""
    T, d, E = shape
    _say(f"case gate cfg {gate_cfg} {shape}")
    monkeypatch.setenv("MOE_GATE_CFG", gate_cfg)
    cfg = moe_inputs.LayerConfig("gate", T, d, 64, E, 2, "bf16", 1.0)
    inp = moe_inputs.make_layer_inputs(cfg, 8, "cuda")
    dims = moe.Dims(T, d, 64, E, 2)
    logits, idx, w = moe.route(dims, inp["x"], inp["wg"], inp["bias"])
    torch.cuda.synchronize()
    h = {n: to_numpy(inp[n], "bf16") for n in ("x", "wg", "bias")}
    ref = oracle.gate_logits(h["x"], h["wg"], h["bias"], "bf16")
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), oracle.topk_select(ref, 2))


# ---------------- full-size workloads ----------------
SHARED_SHAPES = [
    # T, d, f, E, k, shared experts, dtype
    (300, 256, 192, 8, 2, 1, "bf16"),   # ragged m-blocks, FC2 column tail
    (97, 128, 128, 16, 4, 2, "bf16"),   # two shared experts
    (64, 128, 256, 8, 2, 1, "f32"),     # fp32 path
]


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("shape", SHARED_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_S{}_{}".format(*s))
def test_shared_experts_layer(monkeypatch, shape, path):
    """moe_layer_forward_shared against the oracle: routing bit-exact, output within tolerance."""
    T, d, f, E, k, S, dt = shape
    _say(f"case shared {shape} {path}")
    monkeypatch.setenv("MOE_DISPATCH", path)
    inp = moe_inputs.random_inputs(T, d, f, E, k, dt, 1.0, seed=12, device="cuda", n_shared=S)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out, r = moe.layer_forward_shared(moe.Dims(T, d, f, E, k, tdt), inp["x"], inp["wg"], inp["bias"], inp["w1"],
                                      inp["w3"], inp["w2"], inp["sw1"], inp["sw3"], inp["sw2"], return_routing=True)
    torch.cuda.synchronize()
    h = {n: to_numpy(v, dt) for n, v in inp.items()}
    ref = oracle.layer_forward_shared(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], h["sw1"], h["sw3"],
                                      h["sw2"], k, dt)
    assert_routing_equal(r, ref)
    err = rel_err(gpu_float(out), ref["out"])
    _say(f"  out rel_err={err:.3e}")
    assert err <= OUT_TOL


# Full-size workloads. Routing arrays and gate logits are compared bit for bit;
# the tile plan the GPU used is read back from the workspace and checked against
# the plan invariants; outputs are compared element by element with the oracle
# on every row where the oracle takes seconds (decode and DBRX shapes), and at the
# prefill and DeepSeek shapes on every column of one token per m-block of the
# GPU's own plan (the token of the block's last row), so that every active
# expert, every m-block and every partial block is checked.
FULL_EVERY_ROW = ["mixtral_decode", "mixtral_decode_t1", "mixtral_decode_t16", "dbrx_bal", "dbrx_zipf"]
FULL_PER_MBLOCK = ["mixtral_prefill_skew", "mixtral_prefill_bal", "deepseek_skew", "deepseek_bal"]


def _host(t, dtype):
    return to_numpy(t, dtype)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL_EVERY_ROW + FULL_PER_MBLOCK)
def test_full_size_workload(name):
    cfg = moe_inputs.config(name)
    _say(f"case full {name}: generating inputs on the GPU")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dims = _dims(cfg)
    ws = moe.make_workspace(dims)
    torch.cuda.synchronize()
    _say("  running the layer")
    out, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], ws=ws,
                               return_routing=True)
    torch.cuda.synchronize()
    plan = moe.read_plan(dims, ws).numpy()
    h = host_inputs(inp, cfg.dtype)
    _say("  oracle routing")
    ref = oracle_routing(h, cfg.k, cfg.dtype)
    assert_routing_equal(r, ref)
    counts = ref["counts"]
    _say(f"  routing bit-exact; counts min {counts.min()} max {counts.max()} active {(counts > 0).sum()}")
    beta = moe.ffn_block_rows(dims)
    check_plan(plan, counts, ref["offsets"], beta, cfg.T * cfg.k)
    assert moe.read_plan_multi_block(dims, ws) == int((counts > beta).any()), "plan's multi-block flag"
    _say(f"  plan: {len(plan)} m-blocks of <= {beta} rows, invariants hold")
    assert torch.isfinite(out.float()).all()
    w1, w3, w2 = (_host(inp[n], cfg.dtype) for n in ("w1", "w3", "w2"))
    if name in FULL_EVERY_ROW:
        toks = None
    else:
        last_rows = plan[:, 1] + plan[:, 2] - 1
        toks = np.unique(ref["perm"][last_rows] // cfg.k)
    want = oracle_outputs_threaded(h, w1, w3, w2, ref["topk_idx"], ref["topk_w"], toks, cfg.k, cfg.dtype)
    got = gpu_float(out) if toks is None else gpu_float(out[torch.from_numpy(toks).cuda()])
    err = rel_err(got, want)
    _say(f"  out rel_err={err:.3e} over {got.shape[0]} of {cfg.T} tokens, all {cfg.d} columns")
    assert err <= OUT_TOL


def test_measurement_probes_run():
    """The ceilings the bench reports come from working probes: rates within physical bounds."""
    _say("case probes")
    gbps = moe.probe_hbm_read_gbps(nbytes=1 << 30, reps=2)
    tflops = moe.probe_mfma_tflops(iters=2000, reps=2)
    _say(f"  hbm read {gbps:.0f} GB/s, mfma {tflops:.0f} TFLOP/s")
    assert 1000 < gbps < 8000 * 1.05
    assert 300 < tflops < 2516.6 * 1.05


@pytest.mark.timeout(600)
def test_full_size_shared_workload():
    """DeepSeek-V3-shaped layer with one shared expert: routing bit-exact, sampled rows."""
    cfg = moe_inputs.config("deepseek_shared")
    _say("case full deepseek_shared: generating inputs on the GPU")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dims = _dims(cfg)
    out, r = moe.layer_forward_shared(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                      inp["sw1"], inp["sw3"], inp["sw2"], return_routing=True)
    torch.cuda.synchronize()
    h = host_inputs(inp, cfg.dtype)
    _say("  oracle routing")
    ref = oracle_routing(h, cfg.k, cfg.dtype)
    assert_routing_equal(r, ref)
    toks = np.unique(np.linspace(0, cfg.T - 1, 8).astype(np.int64))
    w1, w3, w2 = (LazyExperts(inp[n], cfg.dtype) for n in ("w1", "w3", "w2"))
    routed = oracle.token_outputs(h["x"], ref["topk_idx"], ref["topk_w"], w1, w3, w2, toks, cfg.dtype)
    sw = {n: to_numpy(inp[n], cfg.dtype) for n in ("sw1", "sw3", "sw2")}
    shared = oracle.shared_expert_ffn(h["x"][toks], sw["sw1"], sw["sw3"], sw["sw2"], cfg.dtype).sum(axis=0)
    err = rel_err(gpu_float(out[torch.from_numpy(toks).cuda()]), routed + shared)
    _say(f"  sampled out rel_err={err:.3e} over {toks.size} tokens")
    assert err <= OUT_TOL


@pytest.mark.parametrize("path", ["stored", "packed", "fused"])
def test_empty_batch_forward(path):
    """T = 0: every layer entry point returns at once, with nothing to compute."""
    _say(f"case empty batch {path}")
    d, f, E, k = 256, 256, 8, 2
    inp = moe_inputs.random_inputs(4, d, f, E, k, "bf16", 0.0, seed=31, device="cuda")
    dims = moe.Dims(0, d, f, E, k, torch.bfloat16)
    x0 = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    packed = moe.pack_weights(moe.Dims(4, d, f, E, k, torch.bfloat16), inp["w1"], inp["w3"], inp["w2"]) \
        if path == "packed" else None
    out, r = moe.layer_forward(dims, x0, inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                               return_routing=True, fused=path == "fused", packed=packed)
    torch.cuda.synchronize()
    assert out.shape == (0, d) and r["topk_idx"].shape == (0, k) and r["perm"].numel() == 0
