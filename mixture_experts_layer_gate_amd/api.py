"""Thin ctypes binding of the C ABI in ``include/moe.h``.

Each function takes torch tensors that already live on the GPU, checks their
dtype and shape, and passes ``data_ptr()`` values, the workspace and the
current HIP stream to the library. No step of the layer runs here. The library
is loaded on first use; if it is missing, calls raise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe_amd.so"

STAGES = ["gate", "topk", "hist", "scan", "scatter", "plan", "fc1", "fc2", "combine", "dispatch",
          "bwd_wt", "bwd_fc1", "bwd_dh", "bwd_swiglu", "bwd_route", "bwd_dx", "bwd_dxsum", "bwd_act_t",
          "bwd_wg2", "bwd_wg13", "bwd_gate", "ffn_fused"]
MOE_DTYPE = {torch.float32: 0, torch.bfloat16: 1}

# Every symbol include/moe.h declares.
EXPORTS = ["moe_version", "moe_status_string", "moe_workspace_bytes", "moe_route", "moe_permute",
           "moe_grouped_ffn", "moe_combine", "moe_layer_forward", "moe_timing_enable",
           "moe_timing_disable", "moe_timing_read", "moe_probe_cus", "moe_probe_hbm_read", "moe_probe_mfma",
           "moe_workspace_bytes_shared", "moe_layer_forward_shared", "moe_backward_workspace_bytes",
           "moe_layer_backward", "moe_layer_forward_fused", "moe_ffn_block_rows", "moe_gate_on_matrix_cores", "moe_pack_weights",
           "moe_layer_forward_packed", "moe_fused_status", "moe_layer_plan_layout", "moe_pack_weights_transposed",
           "moe_layer_forward_noalloc", "moe_layer_forward_fused_packed", "moe_layer_forward_train",
           "moe_layer_backward_saved", "moe_layer_backward_ex"]

# Bytes of the static scratch moe_layer_forward_noalloc uses (MOE_NOALLOC_SCRATCH_BYTES in include/moe.h).
NOALLOC_SCRATCH_BYTES = 128 << 20


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32)]


@dataclass(frozen=True)
class Dims:
    T: int
    d: int
    f: int
    E: int
    k: int
    dtype: torch.dtype = torch.bfloat16

    def c(self) -> _Dims:
        return _Dims(self.T, self.d, self.f, self.E, self.k, MOE_DTYPE.get(self.dtype, -1))


def library_path() -> str:
    return os.environ.get("MOE_AMD_LIB", os.path.join(_PKG, _LIB_NAME))


_lib = None
_P = ctypes.c_void_p
_S = ctypes.c_size_t
_DP = ctypes.POINTER(_Dims)


def load_library():
    """Load the built library (and declare its signatures). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.moe_version.restype = ctypes.c_int
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_workspace_bytes.restype = _S
    lib.moe_workspace_bytes.argtypes = [_DP]
    lib.moe_ffn_block_rows.restype = ctypes.c_int
    lib.moe_ffn_block_rows.argtypes = [_DP]
    lib.moe_gate_on_matrix_cores.restype = ctypes.c_int
    lib.moe_gate_on_matrix_cores.argtypes = [_DP]
    lib.moe_route.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _S, _P]
    lib.moe_permute.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _S, _P]
    lib.moe_grouped_ffn.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]
    lib.moe_combine.argtypes = [_DP, _P, _P, _P, _P, _P]
    lib.moe_layer_forward.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]
    lib.moe_layer_forward_fused.argtypes = lib.moe_layer_forward.argtypes
    lib.moe_pack_weights.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P]
    lib.moe_layer_forward_packed.argtypes = lib.moe_layer_forward.argtypes
    lib.moe_layer_forward_fused_packed.argtypes = lib.moe_layer_forward.argtypes
    lib.moe_pack_weights_transposed.argtypes = lib.moe_pack_weights.argtypes
    lib.moe_fused_status.argtypes = [_DP, _P, _S, ctypes.POINTER(ctypes.c_int32), _P]
    lib.moe_layer_plan_layout.argtypes = [_DP, ctypes.c_int, ctypes.POINTER(_S), ctypes.POINTER(_S),
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.moe_layer_forward_noalloc.argtypes = [_DP] + [_P] * 15
    lib.moe_workspace_bytes_shared.restype = _S
    lib.moe_workspace_bytes_shared.argtypes = [_DP, ctypes.c_int]
    lib.moe_layer_forward_shared.argtypes = [_DP, ctypes.c_int] + [_P] * 18 + [_S, _P]
    lib.moe_backward_workspace_bytes.restype = _S
    lib.moe_backward_workspace_bytes.argtypes = [_DP]
    lib.moe_layer_backward.argtypes = [_DP] + [_P] * 21 + [_S, _P]
    lib.moe_layer_forward_train.argtypes = [_DP] + [_P] * 16 + [_S, _P]
    lib.moe_layer_backward_saved.argtypes = [_DP] + [_P] * 22 + [_S, _P]
    lib.moe_layer_backward_ex.argtypes = [_DP] + [_P] * 13 + [ctypes.c_int] + [_P] * 9 + [_S, _P]
    lib.moe_timing_enable.argtypes = [ctypes.c_int, ctypes.c_uint]
    lib.moe_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.moe_probe_cus.restype = ctypes.c_int
    lib.moe_probe_hbm_read.argtypes = [_P, _S, _P, _P]
    lib.moe_probe_mfma.argtypes = [ctypes.c_int, _P, _P]
    for fn in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
               "moe_layer_forward_shared", "moe_layer_backward", "moe_layer_forward_fused", "moe_fused_status",
               "moe_layer_plan_layout", "moe_pack_weights", "moe_pack_weights_transposed",
               "moe_layer_forward_packed", "moe_layer_forward_noalloc", "moe_layer_forward_fused_packed",
               "moe_timing_enable", "moe_timing_disable", "moe_timing_read", "moe_probe_hbm_read", "moe_probe_mfma"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status, load_library().moe_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes(dims: Dims) -> int:
    return int(load_library().moe_workspace_bytes(ctypes.byref(dims.c())))


def ffn_block_rows(dims: Dims) -> int:
    """Rows per m-block of the grouped FFN for these dims (128 or 256; 0 if invalid)."""
    return int(load_library().moe_ffn_block_rows(ctypes.byref(dims.c())))


def gate_on_matrix_cores(dims: Dims) -> int:
    """1 if the gate GEMM of these dims runs on the fp32 matrix cores, 0 on the vector
    ALUs, -1 if the dims are invalid."""
    return int(load_library().moe_gate_on_matrix_cores(ctypes.byref(dims.c())))


def make_workspace(dims: Dims, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(dims), 256), dtype=torch.uint8, device=device)


def _ws(dims: Dims, ws: Optional[torch.Tensor]):
    if ws is None:
        ws = make_workspace(dims)
    return ws, ws.numel()


def route(dims: Dims, x, wg, bias=None, logits=None, topk_idx=None, topk_w=None, ws=None, stream=None):
    """Gate logits, top-k indices and weights. Returns (logits, topk_idx, topk_w)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    _need(wg, "wg", dims.dtype, (dims.E, dims.d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (dims.E,))
    logits = torch.empty((dims.T, dims.E), dtype=torch.float32, device=dev) if logits is None else logits
    topk_idx = torch.empty((dims.T, dims.k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty((dims.T, dims.k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    ws, nws = _ws(dims, ws)
    _check("moe_route", lib.moe_route(ctypes.byref(dims.c()), _ptr(x), _ptr(wg), _ptr(bias), _ptr(logits),
                                      _ptr(topk_idx), _ptr(topk_w), _ptr(ws), nws, _stream(stream)))
    return logits, topk_idx, topk_w


def permute(dims: Dims, topk_idx, ws=None, stream=None):
    """Returns (counts, offsets, perm, inv_perm)."""
    lib = load_library()
    dev = topk_idx.device
    _need(topk_idx, "topk_idx", torch.int32, (dims.T, dims.k))
    n = dims.T * dims.k
    counts = torch.empty(dims.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(dims.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    inv = torch.empty(n, dtype=torch.int32, device=dev)
    ws, nws = _ws(dims, ws)
    _check("moe_permute", lib.moe_permute(ctypes.byref(dims.c()), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                                          _ptr(perm), _ptr(inv), _ptr(ws), nws, _stream(stream)))
    return counts, offsets, perm, inv


def grouped_ffn(dims: Dims, x, perm, counts, offsets, w1, w3, w2, y_sorted=None, ws=None, stream=None):
    """Returns y_sorted [T*k, d]."""
    lib = load_library()
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    _need(perm, "perm", torch.int32, (dims.T * dims.k,))
    _need(counts, "counts", torch.int32, (dims.E,))
    _need(offsets, "offsets", torch.int32, (dims.E + 1,))
    if y_sorted is None:
        y_sorted = torch.empty((dims.T * dims.k, dims.d), dtype=dims.dtype, device=x.device)
    ws, nws = _ws(dims, ws)
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(ctypes.byref(dims.c()), _ptr(x), _ptr(perm), _ptr(counts),
                                                  _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y_sorted),
                                                  _ptr(ws), nws, _stream(stream)))
    return y_sorted


def combine(dims: Dims, y_sorted, inv_perm, topk_w, out=None, stream=None):
    """Returns out [T, d]."""
    lib = load_library()
    _need(y_sorted, "y_sorted", dims.dtype, (dims.T * dims.k, dims.d))
    _need(inv_perm, "inv_perm", torch.int32, (dims.T * dims.k,))
    _need(topk_w, "topk_w", torch.float32, (dims.T, dims.k))
    if out is None:
        out = torch.empty((dims.T, dims.d), dtype=dims.dtype, device=y_sorted.device)
    _check("moe_combine", lib.moe_combine(ctypes.byref(dims.c()), _ptr(y_sorted), _ptr(inv_perm), _ptr(topk_w),
                                          _ptr(out), _stream(stream)))
    return out


def pack_weights(dims: Dims, w1, w3, w2, stream=None):
    """Stage-order copies (w1p, w3p, w2p) of the expert weights for layer_forward(packed=...):
    tensors of the same shapes and dtype whose values are permuted within each expert."""
    lib = load_library()
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    w1p, w3p, w2p = torch.empty_like(w1), torch.empty_like(w3), torch.empty_like(w2)
    _check("moe_pack_weights", lib.moe_pack_weights(ctypes.byref(dims.c()), _ptr(w1), _ptr(w3), _ptr(w2),
                                                    _ptr(w1p), _ptr(w3p), _ptr(w2p), _stream(stream)))
    return w1p, w3p, w2p


def pack_weights_transposed(dims: Dims, w1t, w3t, w2t, stream=None):
    """The stage-order tensors of pack_weights from weights held input-major:
    w1t, w3t [E][d][f] and w2t [E][f][d]. Returns (w1p, w3p, w2p) of shapes
    [E][f][d], [E][f][d], [E][d][f]."""
    lib = load_library()
    for name, w, shp in (("w1t", w1t, (dims.E, dims.d, dims.f)), ("w3t", w3t, (dims.E, dims.d, dims.f)),
                         ("w2t", w2t, (dims.E, dims.f, dims.d))):
        _need(w, name, dims.dtype, shp)
    dev = w1t.device
    w1p = torch.empty((dims.E, dims.f, dims.d), dtype=dims.dtype, device=dev)
    w3p = torch.empty((dims.E, dims.f, dims.d), dtype=dims.dtype, device=dev)
    w2p = torch.empty((dims.E, dims.d, dims.f), dtype=dims.dtype, device=dev)
    _check("moe_pack_weights_transposed", lib.moe_pack_weights_transposed(
        ctypes.byref(dims.c()), _ptr(w1t), _ptr(w3t), _ptr(w2t), _ptr(w1p), _ptr(w3p), _ptr(w2p), _stream(stream)))
    return w1p, w3p, w2p


def fused_status(dims: Dims, ws, stream=None) -> int:
    """Error word of the last fused layer call on workspace ws (0: every readiness wait was met).
    Waits for the stream."""
    v = ctypes.c_int32()
    _check("moe_fused_status", load_library().moe_fused_status(ctypes.byref(dims.c()), _ptr(ws), ws.numel(),
                                                                ctypes.byref(v), _stream(stream)))
    return v.value


def plan_layout(dims: Dims, n_shared: int = 0):
    """(m-block list byte offset, count byte offset, max m-blocks) of the tile plan in a layer workspace."""
    mo, co, mx = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
    _check("moe_layer_plan_layout", load_library().moe_layer_plan_layout(
        ctypes.byref(dims.c()), n_shared, ctypes.byref(mo), ctypes.byref(co), ctypes.byref(mx)))
    return mo.value, co.value, mx.value


def read_plan(dims: Dims, ws, n_shared: int = 0) -> torch.Tensor:
    """The m-blocks [count][4] (int32: expert, first sorted row, rows, group info) that the
    last layer call on ws covered, as a host tensor. Synchronises the device."""
    mo, co, mx = plan_layout(dims, n_shared)
    torch.cuda.synchronize()
    count = int(ws[co:co + 4].cpu().view(torch.int32)[0])
    if not 0 <= count <= mx:
        raise RuntimeError(f"m-block count {count} outside [0, {mx}]")
    return ws[mo:mo + 16 * count].cpu().view(torch.int32).view(count, 4).clone()


def read_plan_multi_block(dims: Dims, ws, n_shared: int = 0) -> int:
    """The plan's flag word after the m-block count (moe_layer_plan_layout): 1 if some expert's
    rows span more than one m-block in the last layer call on ws. Synchronises the device."""
    _, co, _ = plan_layout(dims, n_shared)
    torch.cuda.synchronize()
    return int(ws[co + 4:co + 8].cpu().view(torch.int32)[0])


def layer_forward_noalloc(dims: Dims, x, wg, bias, w1, w3, w2, out, routing=None, stream=None):
    """moe_layer_forward_noalloc: the layer with the library's static scratch as workspace.
    out and the optional routing outputs (a dict of preallocated tensors under the names
    layer_forward(..., return_routing=True) returns) are the caller's; nothing is allocated."""
    lib = load_library()
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    _need(wg, "wg", dims.dtype, (dims.E, dims.d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (dims.E,))
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    _need(out, "out", dims.dtype, (dims.T, dims.d))
    g = (routing or {}).get
    _check("moe_layer_forward_noalloc", lib.moe_layer_forward_noalloc(
        ctypes.byref(dims.c()), _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
        _ptr(g("logits")), _ptr(g("topk_idx")), _ptr(g("topk_w")), _ptr(g("counts")), _ptr(g("offsets")),
        _ptr(g("perm")), _ptr(g("inv_perm")), _stream(stream)))
    return out


def layer_forward(dims: Dims, x, wg, bias, w1, w3, w2, out=None, ws=None, stream=None, return_routing=False,
                  fused=False, packed=None):
    """The whole layer. With return_routing, also returns the routing arrays as a dict.
    fused=True runs the layer as one persistent launch (moe_layer_forward_fused;
    bitwise the same result). packed=(w1p, w3p, w2p) from pack_weights reads the
    stage-order weights instead of w1, w3, w2 (which may then be None;
    moe_layer_forward_packed, or with fused=True moe_layer_forward_fused_packed;
    bitwise the same result)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    _need(wg, "wg", dims.dtype, (dims.E, dims.d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (dims.E,))
    if packed is not None:
        w1, w3, w2 = packed
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    if out is None:
        out = torch.empty((dims.T, dims.d), dtype=dims.dtype, device=dev)
    r = {}
    if return_routing:
        n = dims.T * dims.k
        r = {"logits": torch.empty((dims.T, dims.E), dtype=torch.float32, device=dev),
             "topk_idx": torch.empty((dims.T, dims.k), dtype=torch.int32, device=dev),
             "topk_w": torch.empty((dims.T, dims.k), dtype=torch.float32, device=dev),
             "counts": torch.empty(dims.E, dtype=torch.int32, device=dev),
             "offsets": torch.empty(dims.E + 1, dtype=torch.int32, device=dev),
             "perm": torch.empty(n, dtype=torch.int32, device=dev),
             "inv_perm": torch.empty(n, dtype=torch.int32, device=dev)}
    ws, nws = _ws(dims, ws)
    g = r.get
    fn = {(False, False): "moe_layer_forward", (False, True): "moe_layer_forward_packed",
          (True, False): "moe_layer_forward_fused", (True, True): "moe_layer_forward_fused_packed"}[
        (bool(fused), packed is not None)]
    _check(fn, getattr(lib, fn)(
        ctypes.byref(dims.c()), _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
        _ptr(g("logits")), _ptr(g("topk_idx")), _ptr(g("topk_w")), _ptr(g("counts")), _ptr(g("offsets")),
        _ptr(g("perm")), _ptr(g("inv_perm")), _ptr(ws), nws, _stream(stream)))
    return (out, r) if return_routing else out


def layer_forward_train(dims: Dims, x, wg, bias, w1, w3, w2, out=None, gu=None, ws=None, stream=None):
    """The layer's forward that also keeps FC1's g | u for the backward
    (moe_layer_forward_train). Returns (out, routing, gu): routing as
    layer_forward(..., return_routing=True) gives it, gu [T*k][2f] bf16 with
    g then u of each sorted row; pass gu to layer_backward to skip its FC1
    recompute."""
    lib = load_library()
    dev = x.device
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    _need(wg, "wg", dims.dtype, (dims.E, dims.d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (dims.E,))
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    n = dims.T * dims.k
    if out is None:
        out = torch.empty((dims.T, dims.d), dtype=dims.dtype, device=dev)
    if gu is None:
        gu = torch.empty((n, 2 * dims.f), dtype=dims.dtype, device=dev)
    _need(gu, "gu", dims.dtype, (n, 2 * dims.f))
    r = {"logits": torch.empty((dims.T, dims.E), dtype=torch.float32, device=dev),
         "topk_idx": torch.empty((dims.T, dims.k), dtype=torch.int32, device=dev),
         "topk_w": torch.empty((dims.T, dims.k), dtype=torch.float32, device=dev),
         "counts": torch.empty(dims.E, dtype=torch.int32, device=dev),
         "offsets": torch.empty(dims.E + 1, dtype=torch.int32, device=dev),
         "perm": torch.empty(n, dtype=torch.int32, device=dev),
         "inv_perm": torch.empty(n, dtype=torch.int32, device=dev)}
    ws, nws = _ws(dims, ws)
    _check("moe_layer_forward_train", lib.moe_layer_forward_train(
        ctypes.byref(dims.c()), _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
        _ptr(r["logits"]), _ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
        _ptr(r["perm"]), _ptr(r["inv_perm"]), _ptr(gu), _ptr(ws), nws, _stream(stream)))
    return out, r, gu


def workspace_bytes_shared(dims: Dims, n_shared: int) -> int:
    return int(load_library().moe_workspace_bytes_shared(ctypes.byref(dims.c()), n_shared))


def layer_forward_shared(dims: Dims, x, wg, bias, w1, w3, w2, sw1, sw3, sw2, out=None, ws=None, stream=None,
                         return_routing=False):
    """The layer with shared (always-active) experts sw1, sw3 [S][f][d], sw2 [S][d][f]."""
    lib = load_library()
    dev = x.device
    S = int(sw1.shape[0])
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    _need(wg, "wg", dims.dtype, (dims.E, dims.d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (dims.E,))
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f)), ("sw1", sw1, (S, dims.f, dims.d)),
                         ("sw3", sw3, (S, dims.f, dims.d)), ("sw2", sw2, (S, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    if out is None:
        out = torch.empty((dims.T, dims.d), dtype=dims.dtype, device=dev)
    r = {}
    if return_routing:
        n = dims.T * dims.k
        r = {"logits": torch.empty((dims.T, dims.E), dtype=torch.float32, device=dev),
             "topk_idx": torch.empty((dims.T, dims.k), dtype=torch.int32, device=dev),
             "topk_w": torch.empty((dims.T, dims.k), dtype=torch.float32, device=dev),
             "counts": torch.empty(dims.E, dtype=torch.int32, device=dev),
             "offsets": torch.empty(dims.E + 1, dtype=torch.int32, device=dev),
             "perm": torch.empty(n, dtype=torch.int32, device=dev),
             "inv_perm": torch.empty(n, dtype=torch.int32, device=dev)}
    if ws is None:
        ws = torch.empty(max(workspace_bytes_shared(dims, S), 256), dtype=torch.uint8, device=dev)
    g = r.get
    _check("moe_layer_forward_shared", lib.moe_layer_forward_shared(
        ctypes.byref(dims.c()), S, _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(sw1),
        _ptr(sw3), _ptr(sw2), _ptr(out), _ptr(g("logits")), _ptr(g("topk_idx")), _ptr(g("topk_w")),
        _ptr(g("counts")), _ptr(g("offsets")), _ptr(g("perm")), _ptr(g("inv_perm")), _ptr(ws), ws.numel(),
        _stream(stream)))
    return (out, r) if return_routing else out


def backward_workspace_bytes(dims: Dims) -> int:
    return int(load_library().moe_backward_workspace_bytes(ctypes.byref(dims.c())))


def layer_backward(dims: Dims, x, wg, w1, w3, w2, routing: dict, dout, ws=None, stream=None,
                   want_dlogits=False, want_dtopk_w=False, grads=None, gu=None, wgrad_dtype=torch.float32):
    """Gradients of the layer for output gradient dout [T][d] (bf16).

    routing: the forward's topk_idx, topk_w, counts, offsets, perm, inv_perm
    (layer_forward(..., return_routing=True)). Returns a dict with dx [T][d]
    (bf16), dwg [E][d], dbias [E], dw1, dw3 [E][f][d], dw2 [E][d][f] (fp32) and,
    when asked for, dlogits [T][E] and dtopk_w [T][k]. ``grads`` may hold
    preallocated output tensors under those names. ``gu``: the g | u rows that
    layer_forward_train kept (moe_layer_backward_saved; the same gradients
    without the FC1 recompute). ``wgrad_dtype`` torch.bfloat16 returns dw1,
    dw3, dw2 in bf16, each the rounded fp32 value (moe_layer_backward_ex)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", dims.dtype, (dims.T, dims.d))
    _need(wg, "wg", dims.dtype, (dims.E, dims.d))
    _need(dout, "dout", dims.dtype, (dims.T, dims.d))
    for name, w, shp in (("w1", w1, (dims.E, dims.f, dims.d)), ("w3", w3, (dims.E, dims.f, dims.d)),
                         ("w2", w2, (dims.E, dims.d, dims.f))):
        _need(w, name, dims.dtype, shp)
    n = dims.T * dims.k
    for name, dt, shp in (("topk_idx", torch.int32, (dims.T, dims.k)), ("topk_w", torch.float32, (dims.T, dims.k)),
                          ("counts", torch.int32, (dims.E,)), ("offsets", torch.int32, (dims.E + 1,)),
                          ("perm", torch.int32, (n,)), ("inv_perm", torch.int32, (n,))):
        _need(routing[name], name, dt, shp)
    g = dict(grads or {})
    f32 = torch.float32
    if wgrad_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("wgrad_dtype must be torch.float32 or torch.bfloat16")
    wt = wgrad_dtype
    shapes = {"dx": ((dims.T, dims.d), dims.dtype), "dwg": ((dims.E, dims.d), f32), "dbias": ((dims.E,), f32),
              "dw1": ((dims.E, dims.f, dims.d), wt), "dw3": ((dims.E, dims.f, dims.d), wt),
              "dw2": ((dims.E, dims.d, dims.f), wt)}
    if want_dlogits:
        shapes["dlogits"] = ((dims.T, dims.E), f32)
    if want_dtopk_w:
        shapes["dtopk_w"] = ((dims.T, dims.k), f32)
    for name, (shp, dt) in shapes.items():
        if name not in g:
            g[name] = torch.empty(shp, dtype=dt, device=dev)
        _need(g[name], name, dt, shp)
    if ws is None:
        ws = torch.empty(max(backward_workspace_bytes(dims), 256), dtype=torch.uint8, device=dev)
    head = (ctypes.byref(dims.c()), _ptr(x), _ptr(wg), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(routing["topk_idx"]),
            _ptr(routing["topk_w"]), _ptr(routing["counts"]), _ptr(routing["offsets"]), _ptr(routing["perm"]),
            _ptr(routing["inv_perm"]), _ptr(dout))
    tail = (_ptr(g["dx"]), _ptr(g["dwg"]), _ptr(g["dbias"]), _ptr(g["dw1"]), _ptr(g["dw3"]), _ptr(g["dw2"]),
            _ptr(g.get("dlogits")), _ptr(g.get("dtopk_w")), _ptr(ws), ws.numel(), _stream(stream))
    if gu is not None:
        _need(gu, "gu", dims.dtype, (n, 2 * dims.f))
    if wgrad_dtype == torch.bfloat16:
        _check("moe_layer_backward_ex", lib.moe_layer_backward_ex(*head, _ptr(gu), 1, *tail))
    elif gu is None:
        _check("moe_layer_backward", lib.moe_layer_backward(*head, *tail))
    else:
        _check("moe_layer_backward_saved", lib.moe_layer_backward_saved(*head, _ptr(gu), *tail))
    return g


def timing_enable(capacity: int, stages=None):
    """Record HIP events around the library's kernel launches (stages: names, None = all)."""
    mask = 0 if stages is None else sum(1 << STAGES.index(st) for st in stages)
    _check("moe_timing_enable", load_library().moe_timing_enable(capacity, mask))


def timing_disable():
    _check("moe_timing_disable", load_library().moe_timing_disable())


def timing_read(stage: str):
    """(total kernel ms, launches) recorded for a stage since timing_enable."""
    ms, n = ctypes.c_double(), ctypes.c_int()
    _check("moe_timing_read", load_library().moe_timing_read(STAGES.index(stage), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def probe_hbm_read_gbps(nbytes: int = 2 << 30, reps: int = 5, stream=None) -> float:
    """Best-of-reps read rate (GB/s) of the library's streaming-read probe over a
    fresh device buffer of nbytes (one warm-up launch first)."""
    lib = load_library()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(lib.moe_probe_cus(), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream() if stream is None else stream
    best = None
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        _check("moe_probe_hbm_read", lib.moe_probe_hbm_read(_ptr(buf), nbytes, _ptr(sink), st.cuda_stream))
        e1.record(st)
        e1.synchronize()
        if i:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    slice_bytes = nbytes // lib.moe_probe_cus() // 16 * 16
    return slice_bytes * lib.moe_probe_cus() / (best * 1e-3) / 1e9


def probe_mfma_tflops(iters: int = 100000, reps: int = 3, stream=None) -> float:
    """Best-of-reps bf16 MFMA rate (TFLOP/s) of the library's register-only MFMA probe
    (about 50 ms per launch, long enough for the clock to settle at its power limit)."""
    lib = load_library()
    cus = lib.moe_probe_cus()
    sink = torch.empty(cus * 8, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream() if stream is None else stream
    best = None
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        _check("moe_probe_mfma", lib.moe_probe_mfma(iters, _ptr(sink), st.cuda_stream))
        e1.record(st)
        e1.synchronize()
        if i:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    return 524288 * 8 * iters * cus / (best * 1e-3) / 1e12
