"""Work and roofline accounting for one MoE-layer forward call (host-side, pure Python).

* util(): the expert-FFN utilisation bound of MegaScale-Infer, section 2.3:
  util = min(topk/#expert * B/F * b, 1) for a batch of b tokens, memory
  bandwidth B and compute rate F.
* expert_weight_bytes(): 3*E*d*f parameters per layer (Piper, section III-A,
  Table III), at the element size of the stored weights.
* layer_flops() / layer_bytes(): the algorithmic work of one call, counted
  from the actual per-expert row counts, so a skewed routing that leaves
  experts idle is charged only for the experts it uses.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Sequence

# MI355X published peaks (dense, no sparsity). bf16 MFMA: the published 2.5
# PFLOP/s (256 CUs x 4096 FLOP per clock x 2.4 GHz = 2516.6 TFLOP/s, rounded);
# every fraction this package reports uses these constants.
PEAK_HBM_BYTES_PER_S = 8.0e12
PEAK_MFMA_BF16_FLOPS = 2.5e15
PEAK_MFMA_FP32_FLOPS = 157.3e12
PEAK_VALU_FP32_FLOPS = 157.3e12
# fp32 vector FMA without packed instructions (the library is built with packed
# fp32 off): 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz
PEAK_VALU_FP32_UNPACKED_FLOPS = 256 * 4 * 16 * 2 * 2.4e9


def util(topk: int, experts: int, B: float, F: float, b: float) -> float:
    """Utilisation bound of the expert FFN for a global batch of b tokens."""
    return min(topk / experts * B / F * b, 1.0)


def min_full_util_batch(B: float, F: float) -> float:
    """Tokens one weight matrix needs to be compute-bound (F/B)."""
    return F / B


def expert_weight_bytes(E: int, d: int, f: int, elt_bytes: int = 2) -> int:
    """Bytes of one layer's expert weights: three d x f matrices per expert."""
    return 3 * E * d * f * elt_bytes


def layer_flops(T: int, d: int, f: int, E: int, k: int) -> int:
    """Algorithmic FLOP: gate GEMM 2*T*d*E plus FC1 (4*d*f per row) and FC2 (2*d*f per row)."""
    return 2 * T * d * E + 6 * d * f * T * k


def ffn_flops(rows: int, d: int, f: int) -> int:
    return 6 * d * f * rows


def fc1_flops(rows: int, d: int, f: int) -> int:
    return 4 * d * f * rows


def fc2_flops(rows: int, d: int, f: int) -> int:
    return 2 * d * f * rows


def backward_flops(rows: int, d: int, f: int, T: int = 0, k: int = 0) -> int:
    """Algorithmic FLOP of the layer's backward: DGrad (W2^T dout 2*d*f and
    [W1;W3]^T [dg;du] 4*d*f per row), WGrad (dW2 2*d*f, dW1 and dW3 4*d*f per
    row) and the gate part (dWg and the gate's dx, 2*d each per selected logit).
    The FC1 recompute is implementation work, not counted."""
    return 12 * d * f * rows + 4 * d * T * k


# FLOP of each matrix-product stage of the backward, per sorted row
BACKWARD_GEMM_FLOPS_PER_ROW = {"bwd_fc1": 4, "bwd_dh": 2, "bwd_dx": 4, "bwd_wg2": 2, "bwd_wg13": 4}


def active_experts(counts: Iterable[int]) -> int:
    return sum(1 for c in counts if int(c) > 0)


def layer_bytes(T: int, d: int, f: int, E: int, counts: Sequence[int], elt: int = 2) -> int:
    """Algorithmic HBM bytes of one call: weights of the experts that receive
    at least one row, the gate weight, x read once and out written once."""
    a = active_experts(counts)
    return 3 * d * f * elt * a + d * E * elt + 2 * T * d * elt


def fc1_bytes(T: int, d: int, f: int, k: int, counts: Sequence[int], elt: int = 2) -> int:
    """Algorithmic bytes of the FC1 kernel: W1 and W3 of the active experts and
    x read once. The T*k gathered reads of x beyond the first and the h store
    are implementation traffic (fc1_overhead_bytes)."""
    a = active_experts(counts)
    return 2 * d * f * elt * a + T * d * elt


def fc2_bytes(T: int, d: int, f: int, k: int, counts: Sequence[int], elt: int = 2) -> int:
    """Algorithmic bytes of the FC2 kernel: W2 of the active experts. Reading h
    back and storing y are implementation traffic (fc2_overhead_bytes)."""
    a = active_experts(counts)
    return d * f * elt * a


def fc1_overhead_bytes(T: int, d: int, f: int, k: int, elt: int = 2) -> int:
    """FC1 traffic beyond the algorithmic bytes: x rows gathered T*k times
    instead of once, and h [T*k][f] written."""
    return (T * k - T) * d * elt + T * k * f * elt


def fc2_overhead_bytes(T: int, d: int, f: int, k: int, elt: int = 2) -> int:
    """FC2 traffic beyond the algorithmic bytes: h [T*k][f] read, y [T*k][d] written."""
    return T * k * f * elt + T * k * d * elt


def combine_bytes(T: int, d: int, k: int, elt: int = 2) -> int:
    """Algorithmic bytes of the combine: out [T][d] written."""
    return T * d * elt


def combine_overhead_bytes(T: int, d: int, k: int, elt: int = 2) -> int:
    """Combine traffic beyond out: the T*k rows of y read, inv_perm and topk_w (4 bytes each)."""
    return T * k * d * elt + T * k * 8


def kappa(counts: Sequence[int]) -> float:
    """Routing-skew statistic: max rows per expert over the mean (1 for uniform)."""
    c = [int(v) for v in counts]
    mean = sum(c) / len(c)
    return max(c) / mean if mean > 0 else 0.0


@dataclass
class Roofline:
    bound: str          # "hbm" or "mfma"
    t_flop_s: float
    t_byte_s: float

    @property
    def floor_s(self) -> float:
        return max(self.t_flop_s, self.t_byte_s)


def classify(flops: float, nbytes: float, F: float = PEAK_MFMA_BF16_FLOPS,
             B: float = PEAK_HBM_BYTES_PER_S) -> Roofline:
    tf, tb = flops / F, nbytes / B
    return Roofline("mfma" if tf >= tb else "hbm", tf, tb)
