"""Seeded synthetic workloads for the MoE-layer forward pass.

This module only makes inputs; it holds none of the layer's arithmetic. Both
the CPU oracle (``oracle/``) and the HIP path (the package
``mixture_experts_layer_gate_amd``) take their inputs from here, so that both
sides see the same bytes.

Workload shapes follow the models the pages evaluate: Mixtral 8x22B and DBRX
(MegaScale-Infer, "5. Experimental Analysis", model list), DeepSeek-V3 and
Mixtral 8x22B (Piper, Table I). Weights are N(0, 1/fan_in) and activations
N(0, 1). Routing skew comes from a per-expert gate-logit bias
s * (-ln rank), rank = e + 1; it stands in for the production and
Qwen3/OLMoE routing traces the pages measure on (MegaFlux, section 2.2 and
appendix B.1), which are not available here.

Recipe (one generator per tensor, in a fixed order, so every tensor is
reproducible on its own):

* ``torch.Generator(device)`` seeded with ``seed * 1000 + tensor_id``;
  tensor ids: x=1, wg=2, w1=3, w3=4, w2=5, for shared experts sw1=6,
  sw3=7, sw2=8, and the backward's output gradient dout=9 (N(0, 1), [T][d]).
* expert weight tensors are drawn one expert at a time, expert 0 first;
* each draw is fp32 ``torch.randn``, multiplied by fp32 ``1/sqrt(fan_in)``,
  then converted to the activation dtype (bf16 conversion rounds to nearest
  even);
* bias[e] = fp32(-s * ln(e + 1)), computed in fp64.

torch's CPU and GPU generators produce different streams for the same seed;
a GPU parity run therefore generates on the GPU and hands the oracle a host
copy of the very same tensors.

Tensor layouts (row-major):
  x  [T][d]       tokens
  wg [E][d]       gate weight, one row per expert
  w1 [E][f][d]    FC1 gate projection, [out][in] per expert
  w3 [E][f][d]    FC1 up projection,   [out][in] per expert
  w2 [E][d][f]    FC2 down projection, [out][in] per expert
  sw1, sw3 [S][f][d], sw2 [S][d][f]   shared experts (only when S > 0)
  bias [E] fp32
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["LayerConfig", "CONFIGS", "TENSOR_IDS", "make_layer_inputs", "gate_bias", "config", "output_grad"]

TENSOR_IDS = {"x": 1, "wg": 2, "w1": 3, "w3": 4, "w2": 5, "sw1": 6, "sw3": 7, "sw2": 8, "dout": 9}


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens
    d: int            # hidden size
    f: int            # expert FFN size
    E: int            # routed experts
    k: int            # experts per token
    dtype: str        # "bf16" or "f32": x, weights, intermediate and output
    bias_scale: float  # s in bias[e] = -s * ln(e + 1); 0 = no skew
    description: str = ""
    n_shared: int = 0  # shared (always-active) experts, same d and f as the routed ones

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, LayerConfig] = {c.name: c for c in [
    LayerConfig("tiny_fp32", 64, 128, 256, 8, 2, "f32", 0.0,
                "tiny layer, fp32, balanced routing"),
    LayerConfig("mixtral_decode", 256, 6144, 16384, 8, 2, "bf16", 0.0,
                "Mixtral-8x22B-shaped layer, decode batch, balanced routing"),
    LayerConfig("mixtral_decode_t1", 1, 6144, 16384, 8, 2, "bf16", 0.0,
                "Mixtral-8x22B-shaped layer, one token (latency of a single decode step)"),
    LayerConfig("mixtral_decode_t16", 16, 6144, 16384, 8, 2, "bf16", 0.0,
                "Mixtral-8x22B-shaped layer, 16-token decode batch"),
    LayerConfig("mixtral_prefill_skew", 8192, 6144, 16384, 8, 2, "bf16", 1.5,
                "Mixtral-8x22B-shaped layer, prefill batch, Zipf-like skew 1.5"),
    LayerConfig("mixtral_prefill_bal", 8192, 6144, 16384, 8, 2, "bf16", 0.0,
                "balanced twin of mixtral_prefill_skew"),
    LayerConfig("dbrx_bal", 2048, 6144, 10752, 16, 4, "bf16", 0.0,
                "DBRX-shaped layer, balanced routing"),
    LayerConfig("dbrx_zipf", 2048, 6144, 10752, 16, 4, "bf16", 1.0,
                "DBRX-shaped layer, Zipf-like skew 1.0"),
    LayerConfig("deepseek_skew", 4096, 7168, 2048, 256, 8, "bf16", 2.0,
                "DeepSeek-style fine-grained layer, 256 experts top-8, skew 2.0"),
    LayerConfig("deepseek_bal", 4096, 7168, 2048, 256, 8, "bf16", 0.0,
                "balanced twin of deepseek_skew"),
    LayerConfig("deepseek_shared", 4096, 7168, 2048, 256, 8, "bf16", 2.0,
                "DeepSeek-V3-shaped layer: 256 routed experts top-8 plus 1 shared expert, skew 2.0",
                n_shared=1),
]}


def config(name: str) -> LayerConfig:
    return CONFIGS[name]


def gate_bias(E: int, s: float) -> torch.Tensor:
    """bias[e] = fp32(-s * ln(e + 1)) as a CPU fp32 tensor (rank of expert e is e + 1)."""
    vals = [-s * math.log(e + 1) for e in range(E)]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


def _draw(shape, sigma: float, gen: torch.Generator, device, dtype: torch.dtype) -> torch.Tensor:
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if sigma != 1.0:
        z.mul_(torch.tensor(sigma, dtype=torch.float32, device=device))
    return z.to(dtype)


def _expert_tensor(E: int, rows: int, cols: int, sigma: float, seed: int, tid: int,
                   device, dtype: torch.dtype) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + tid)
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    for e in range(E):
        out[e].copy_(_draw((rows, cols), sigma, gen, device, dtype))
    return out


def make_layer_inputs(cfg: LayerConfig, seed: int = 0, device="cpu",
                      T: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """All inputs of one layer call as torch tensors on ``device``.

    ``T`` overrides the token count (the first T rows of the x stream are the
    same for any T, since x is one draw of shape [T, d] per seed only when T is
    fixed; a different T is a different workload).
    """
    T = cfg.T if T is None else T
    dt = cfg.torch_dtype
    dev = torch.device(device)
    gx = torch.Generator(device=dev)
    gx.manual_seed(seed * 1000 + TENSOR_IDS["x"])
    x = _draw((T, cfg.d), 1.0, gx, dev, dt)
    gg = torch.Generator(device=dev)
    gg.manual_seed(seed * 1000 + TENSOR_IDS["wg"])
    wg = _draw((cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d), gg, dev, dt)
    w1 = _expert_tensor(cfg.E, cfg.f, cfg.d, 1.0 / math.sqrt(cfg.d), seed, TENSOR_IDS["w1"], dev, dt)
    w3 = _expert_tensor(cfg.E, cfg.f, cfg.d, 1.0 / math.sqrt(cfg.d), seed, TENSOR_IDS["w3"], dev, dt)
    w2 = _expert_tensor(cfg.E, cfg.d, cfg.f, 1.0 / math.sqrt(cfg.f), seed, TENSOR_IDS["w2"], dev, dt)
    bias = gate_bias(cfg.E, cfg.bias_scale).to(dev)
    out = {"x": x, "wg": wg, "bias": bias, "w1": w1, "w3": w3, "w2": w2}
    if cfg.n_shared > 0:
        S = cfg.n_shared
        out["sw1"] = _expert_tensor(S, cfg.f, cfg.d, 1.0 / math.sqrt(cfg.d), seed, TENSOR_IDS["sw1"], dev, dt)
        out["sw3"] = _expert_tensor(S, cfg.f, cfg.d, 1.0 / math.sqrt(cfg.d), seed, TENSOR_IDS["sw3"], dev, dt)
        out["sw2"] = _expert_tensor(S, cfg.d, cfg.f, 1.0 / math.sqrt(cfg.f), seed, TENSOR_IDS["sw2"], dev, dt)
    return out


def output_grad(T: int, d: int, dtype: str = "bf16", seed: int = 0, device="cpu") -> torch.Tensor:
    """The backward's seeded output gradient dout [T][d], N(0, 1) in the activation dtype."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1000 + TENSOR_IDS["dout"])
    return _draw((T, d), 1.0, gen, dev, dt)


def random_inputs(T: int, d: int, f: int, E: int, k: int, dtype: str = "bf16", bias_scale: float = 0.0,
                  seed: int = 0, device="cpu", n_shared: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs for an arbitrary small shape (edge-case and sweep tests)."""
    cfg = LayerConfig("custom", T, d, f, E, k, dtype, bias_scale, n_shared=n_shared)
    return make_layer_inputs(cfg, seed, device)
