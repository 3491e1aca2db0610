"""The C-ABI library loads, exports every declared symbol and rejects bad arguments
before anything is enqueued. Host-only: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest
import torch

import mixture_experts_layer_gate_amd as moe
from mixture_experts_layer_gate_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.library_path()), reason="HIP library not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(api.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = moe.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = moe.load_library()
    for st in range(6):
        assert lib.moe_status_string(st)
    assert lib.moe_version() >= 100


def _dims(**kw):
    base = dict(T=64, d=128, f=256, E=8, k=2, dtype=1)
    base.update(kw)
    return api._Dims(base["T"], base["d"], base["f"], base["E"], base["k"], base["dtype"])


@pytest.mark.parametrize("bad", [dict(k=0), dict(k=9), dict(E=1025, k=2), dict(d=0), dict(f=0), dict(T=-1),
                                 dict(dtype=7), dict(T=2**30, k=4)])
def test_workspace_bytes_rejects_bad_dims(bad):
    assert moe.load_library().moe_workspace_bytes(ctypes.byref(_dims(**bad))) == 0


def test_ffn_block_rows_choice(monkeypatch):
    """128-row m-blocks for batches with at most 96 rows per active expert (and fp32),
    256 otherwise; the environment switch overrides; invalid dims give 0."""
    monkeypatch.delenv("MOE_GEMM_REGIME", raising=False)
    lib = moe.load_library()

    def rows(**kw):
        return lib.moe_ffn_block_rows(ctypes.byref(_dims(**kw)))
    assert rows(T=256, d=6144, f=16384, E=8, k=2) == 128      # decode: 64 rows per expert
    assert rows(T=1, d=6144, f=16384, E=8, k=2) == 128        # one token: 1 row per active expert
    assert rows(T=384, E=8, k=2) == 128                       # exactly 96 per expert
    assert rows(T=385, E=8, k=2) == 256                       # just above
    assert rows(T=8192, d=6144, f=16384, E=8, k=2) == 256     # prefill
    assert rows(T=4096, d=7168, f=2048, E=256, k=8) == 256    # 128 per expert
    assert rows(T=8192, dtype=0) == 128                       # fp32: the small-tile kernel
    assert rows(k=0) == 0
    monkeypatch.setenv("MOE_GEMM_REGIME", "1")
    assert rows(T=1, d=6144, f=16384, E=8, k=2) == 256
    monkeypatch.setenv("MOE_GEMM_REGIME", "3")
    assert rows(T=8192) == 128


def test_gate_unit_query(monkeypatch):
    """The fp32 matrix cores take bf16 gates with E >= 32 and >= 256 tiles of 32 x 32;
    the environment switch overrides; invalid dims give -1."""
    monkeypatch.delenv("MOE_GATE_CFG", raising=False)
    lib = moe.load_library()

    def mc(**kw):
        return lib.moe_gate_on_matrix_cores(ctypes.byref(_dims(**kw)))
    assert mc(T=4096, d=7168, f=2048, E=256, k=8) == 1       # DeepSeek-V3 shape: 128 x 8 tiles
    assert mc(T=8192, d=6144, f=16384, E=8, k=2) == 0        # 8 experts: the VALU tiles
    assert mc(T=992, d=7168, f=2048, E=256, k=8) == 0        # 31 x 8 tiles
    assert mc(T=1024, d=7168, f=2048, E=256, k=8) == 1       # 32 x 8
    assert mc(T=4096, d=7168, f=2048, E=256, k=8, dtype=0) == 0  # fp32 data
    assert mc(k=0) == -1
    monkeypatch.setenv("MOE_GATE_CFG", "lds")
    assert mc(T=4096, d=7168, f=2048, E=256, k=8) == 0
    monkeypatch.setenv("MOE_GATE_CFG", "mfma")
    assert mc(T=77, d=512, f=64, E=8, k=2) == 1


def test_workspace_bytes_grows_with_shape():
    lib = moe.load_library()
    a = lib.moe_workspace_bytes(ctypes.byref(_dims()))
    b = lib.moe_workspace_bytes(ctypes.byref(_dims(T=128)))
    assert 0 < a < b
    # bf16 mixtral decode: h (512 x 16384) and y (512 x 6144) in bf16 dominate
    c = lib.moe_workspace_bytes(ctypes.byref(_dims(T=256, d=6144, f=16384, E=8, k=2)))
    assert c >= 512 * (16384 + 6144) * 2


# Validation cases: each has one bad argument; the library must return its code
# without launching. Skipped when a GPU is visible, so that a validation bug can
# never turn into a launch with the placeholder pointers below.
needs_no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only validation test")
A = 0x10000  # 16-byte aligned placeholder, never dereferenced


@needs_no_gpu
@pytest.mark.parametrize("case,expect", [
    ("null_x", 1), ("misaligned_x", 1), ("null_idx", 1), ("bad_k", 1), ("small_ws", 3), ("d_not_8", 2),
])
def test_route_validation(case, expect):
    lib = moe.load_library()
    dm = _dims(d=100 if case == "d_not_8" else 128, k=0 if case == "bad_k" else 2)
    x = {"null_x": None, "misaligned_x": A + 2}.get(case, A)
    idx = None if case == "null_idx" else A
    ws, wsb = (A, 16) if case == "small_ws" else (A, 1 << 30)
    st = lib.moe_route(ctypes.byref(dm), x, A, None, None, idx, A, ws, wsb, None)
    assert st == expect


@needs_no_gpu
def test_layer_validation():
    lib = moe.load_library()
    ok = lambda **kw: lib.moe_layer_forward(ctypes.byref(_dims(**kw.pop("dims", {}))), *[kw.get(n, A) for n in (  # noqa: E731
        "x", "wg")], kw.get("bias"), *[kw.get(n, A) for n in ("w1", "w3", "w2", "out")],
        None, None, None, None, None, None, None, kw.get("ws", A), kw.get("wsb", 1 << 40), None)
    assert ok(w2=None) == 1
    assert ok(out=A + 8) == 1
    assert ok(dims=dict(d=96)) == 2            # d % 64 != 0
    assert ok(dims=dict(f=100)) == 2           # f % 64 != 0
    assert ok(wsb=1024) == 3
    assert ok(ws=None) == 3
    assert ok(ws=A + 64) == 1                  # workspace must be 256-byte aligned
    assert ok(dims=dict(T=0)) == 0             # empty batch: nothing to do


@needs_no_gpu
def test_packed_validation():
    lib = moe.load_library()
    dm = _dims()
    assert lib.moe_pack_weights(ctypes.byref(_dims(dtype=0)), A, A, A, A, A, A, None) == 2
    assert lib.moe_pack_weights(ctypes.byref(_dims(f=100)), A, A, A, A, A, A, None) == 2
    assert lib.moe_pack_weights(ctypes.byref(dm), A, A, A, None, A, A, None) == 1
    assert lib.moe_pack_weights(ctypes.byref(dm), A, A + 8, A, A, A, A, None) == 1
    fwd = lambda dims=dm, w1p=A, wsb=1 << 40: lib.moe_layer_forward_packed(  # noqa: E731
        ctypes.byref(dims), A, A, None, w1p, A, A, A, None, None, None, None, None, None, None, A, wsb, None)
    assert fwd(dims=_dims(dtype=0)) == 2
    assert fwd(w1p=None) == 1
    assert fwd(wsb=1024) == 3
    assert fwd(dims=_dims(T=0)) == 0
    ffwd = lambda dims=dm, w1p=A, wsb=1 << 40: lib.moe_layer_forward_fused_packed(  # noqa: E731
        ctypes.byref(dims), A, A, None, w1p, A, A, A, None, None, None, None, None, None, None, A, wsb, None)
    assert ffwd(dims=_dims(dtype=0)) == 2
    assert ffwd(w1p=None) == 1
    assert ffwd(wsb=1024) == 3
    assert ffwd(dims=_dims(T=0)) == 0


@needs_no_gpu
def test_permute_ffn_combine_validation():
    lib = moe.load_library()
    dm = _dims()
    assert lib.moe_permute(ctypes.byref(dm), A, None, A, A, A, A, 1 << 30, None) == 1
    assert lib.moe_permute(ctypes.byref(dm), A, A, A, A, A, A, 4, None) == 3
    assert lib.moe_grouped_ffn(ctypes.byref(dm), A, A, A, A, A, A + 4, A, A, A, 1 << 30, None) == 1
    assert lib.moe_grouped_ffn(ctypes.byref(_dims(f=96)), A, A, A, A, A, A, A, A, A, 1 << 30, None) == 2
    assert lib.moe_combine(ctypes.byref(dm), A, A, A, None, None) == 1
    assert lib.moe_combine(ctypes.byref(_dims(d=12)), A, A, A, A, None) == 2
    assert lib.moe_timing_read(99, None, None) == 1


def test_probe_validation():
    """The measurement probes reject null, misaligned and badly sized arguments on the host."""
    lib = moe.load_library()
    assert lib.moe_probe_hbm_read(None, 1 << 20, 16, None) == 1
    assert lib.moe_probe_hbm_read(16, 1 << 20, None, None) == 1
    assert lib.moe_probe_hbm_read(16, 0, 16, None) == 1
    assert lib.moe_probe_hbm_read(16, 100, 16, None) == 1      # not a multiple of 16
    assert lib.moe_probe_hbm_read(24, 1 << 20, 16, None) == 1  # misaligned
    assert lib.moe_probe_mfma(10, None, None) == 1
    assert lib.moe_probe_mfma(0, 16, None) == 1


def test_layer_shared_validation():
    """moe_layer_forward_shared rejects a bad shared-expert count or missing shared weights
    before anything is launched; an empty batch is a no-op."""
    lib = moe.load_library()

    def call(n_shared=1, sw=A, dims=None):
        return lib.moe_layer_forward_shared(ctypes.byref(_dims(**(dims or {}))), n_shared, A, A, None, A, A, A,
                                            sw, sw, sw, A, None, None, None, None, None, None, None, A, 1 << 40,
                                            None)
    assert call(n_shared=0) == 1
    assert call(n_shared=1017) == 1          # E + n_shared > 1024 with E = 8
    assert call(sw=None) == 1
    assert call(dims=dict(T=0)) == 0
    base = lib.moe_workspace_bytes(ctypes.byref(_dims()))
    assert lib.moe_workspace_bytes_shared(ctypes.byref(_dims()), 1) > 0
    assert lib.moe_workspace_bytes_shared(ctypes.byref(_dims()), 2) > lib.moe_workspace_bytes_shared(
        ctypes.byref(_dims()), 1)
    assert lib.moe_workspace_bytes_shared(ctypes.byref(_dims()), 0) == 0
    assert base > 0


def test_layer_backward_validation():
    """moe_layer_backward rejects fp32 data, shapes off the 256 grid, null gradient
    outputs and a short workspace before anything is launched."""
    lib = moe.load_library()
    good = dict(d=256, f=512)

    def call(dims=None, dw1=A, ws_bytes=1 << 40, dlogits=None):
        dm = _dims(**{**good, **(dims or {})})
        return lib.moe_layer_backward(ctypes.byref(dm), A, A, A, A, A, A, A, A, A, A, A, A, A, A, A, dw1, A, A,
                                      dlogits, None, A, ws_bytes, None)
    assert call(dims=dict(dtype=0)) == 2             # fp32: the backward runs on bf16 only
    assert call(dims=dict(d=192)) == 2               # d % 256 != 0
    assert call(dims=dict(f=320)) == 2               # f % 256 != 0
    assert call(dw1=None) == 1
    assert call(dlogits=A + 2) == 1                  # misaligned optional output
    assert call(ws_bytes=16) == 3
    need = lib.moe_backward_workspace_bytes(ctypes.byref(_dims(**good)))
    assert need > lib.moe_backward_workspace_bytes(ctypes.byref(_dims(**{**good, "T": 1})))
    assert lib.moe_backward_workspace_bytes(ctypes.byref(_dims(k=0))) == 0


@needs_no_gpu
def test_training_pair_validation():
    """moe_layer_forward_train, moe_layer_backward_saved and moe_layer_backward_ex
    check the kept g | u buffer, the weight-gradient type and the backward's
    limits before anything is launched."""
    lib = moe.load_library()
    good = dict(d=256, f=512)

    def fwd(dims=None, gu=A, ws_bytes=1 << 40):
        dm = _dims(**{**good, **(dims or {})})
        return lib.moe_layer_forward_train(ctypes.byref(dm), A, A, None, A, A, A, A, None, None, None, None, None,
                                           None, None, gu, A, ws_bytes, None)
    assert fwd(gu=None) == 1                         # g | u output required
    assert fwd(gu=A + 8) == 1                        # and 16-byte aligned
    assert fwd(dims=dict(dtype=0)) == 2              # bf16 only, as the backward
    assert fwd(dims=dict(d=192)) == 2                # d % 256 != 0
    assert fwd(dims=dict(f=320)) == 2                # f % 256 != 0
    assert fwd(ws_bytes=16) == 3                     # the forward's workspace
    assert fwd(dims=dict(T=0), gu=None) == 0         # empty batch: nothing to do

    def bwd(dims=None, gu=A, ws_bytes=1 << 40):
        dm = _dims(**{**good, **(dims or {})})
        return lib.moe_layer_backward_saved(ctypes.byref(dm), A, A, A, A, A, A, A, A, A, A, A, A, gu, A, A, A, A,
                                            A, A, None, None, A, ws_bytes, None)
    assert bwd(gu=None) == 1
    assert bwd(gu=A + 8) == 1
    assert bwd(dims=dict(dtype=0)) == 2
    assert bwd(dims=dict(f=320)) == 2
    assert bwd(ws_bytes=16) == 3

    def ex(dims=None, gu=None, wdt=1, ws_bytes=1 << 40):
        dm = _dims(**{**good, **(dims or {})})
        return lib.moe_layer_backward_ex(ctypes.byref(dm), A, A, A, A, A, A, A, A, A, A, A, A, gu, wdt, A, A, A,
                                         A, A, A, None, None, A, ws_bytes, None)
    assert ex(wdt=2) == 1                            # weight gradients fp32 or bf16 only
    assert ex(wdt=-1) == 1
    assert ex(gu=A + 8) == 1                         # optional g | u, 16-byte aligned
    assert ex(dims=dict(dtype=0)) == 2
    assert ex(dims=dict(d=192)) == 2
    assert ex(ws_bytes=16) == 3
    assert ex(gu=A, wdt=0, ws_bytes=16) == 3


def test_plan_layout_inside_the_workspace():
    """The tile plan's m-block list and count lie inside the layer workspace, 16- and
    4-byte aligned, and the list holds the most m-blocks any plan of the shape can have:
    ceil(T*k / 128) + min(T*k, E) (at most one partial block per active expert)."""
    lib = moe.load_library()
    for kw, n_shared in ((dict(), 0), (dict(T=8192, d=6144, f=16384, E=8, k=2), 0),
                         (dict(T=4096, d=7168, f=2048, E=256, k=8), 0), (dict(T=300, E=16, k=4), 2)):
        dm = _dims(**kw)
        mo, co, mx = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
        assert lib.moe_layer_plan_layout(ctypes.byref(dm), n_shared, ctypes.byref(mo), ctypes.byref(co),
                                         ctypes.byref(mx)) == 0
        rows = dm.T * dm.k + n_shared * dm.T
        experts = dm.E + n_shared
        assert mx.value == -(-rows // 128) + min(rows, experts)
        size = (lib.moe_workspace_bytes(ctypes.byref(dm)) if n_shared == 0
                else lib.moe_workspace_bytes_shared(ctypes.byref(dm), n_shared))
        assert mo.value % 16 == 0 and co.value % 4 == 0
        assert mo.value + 16 * mx.value <= co.value + 4 <= size
    bad = ctypes.c_size_t()
    assert lib.moe_layer_plan_layout(ctypes.byref(_dims(k=0)), 0, ctypes.byref(bad), ctypes.byref(bad),
                                     ctypes.byref(ctypes.c_int64())) == 1
    assert lib.moe_layer_plan_layout(ctypes.byref(_dims()), 0, None, ctypes.byref(bad),
                                     ctypes.byref(ctypes.c_int64())) == 1
    assert lib.moe_layer_plan_layout(ctypes.byref(_dims()), 1017, ctypes.byref(bad), ctypes.byref(bad),
                                     ctypes.byref(ctypes.c_int64())) == 1


@needs_no_gpu
def test_fused_status_validation():
    """moe_fused_status checks its arguments on the host; an empty batch reads nothing."""
    lib = moe.load_library()
    flags = ctypes.c_int32(7)
    assert lib.moe_fused_status(ctypes.byref(_dims()), A, 1 << 30, None, None) == 1
    assert lib.moe_fused_status(ctypes.byref(_dims()), A, 16, ctypes.byref(flags), None) == 3
    assert lib.moe_fused_status(ctypes.byref(_dims()), A + 64, 1 << 30, ctypes.byref(flags), None) == 1
    assert lib.moe_fused_status(ctypes.byref(_dims(T=0)), None, 0, ctypes.byref(flags), None) == 0
    assert flags.value == 0


@needs_no_gpu
def test_pack_weights_transposed_validation():
    lib = moe.load_library()
    dm = _dims()
    assert lib.moe_pack_weights_transposed(ctypes.byref(_dims(dtype=0)), A, A, A, A, A, A, None) == 2
    assert lib.moe_pack_weights_transposed(ctypes.byref(_dims(d=100)), A, A, A, A, A, A, None) == 2
    assert lib.moe_pack_weights_transposed(ctypes.byref(dm), None, A, A, A, A, A, None) == 1
    assert lib.moe_pack_weights_transposed(ctypes.byref(dm), A, A, A, A, A, A + 2, None) == 1


@needs_no_gpu
def test_noalloc_refuses_shapes_beyond_its_scratch():
    """moe_layer_forward_noalloc refuses, before any device call, a shape whose workspace
    exceeds the static scratch (MOE_ERR_SCRATCH = 5), and bad dims first."""
    lib = moe.load_library()

    def call(**kw):
        return lib.moe_layer_forward_noalloc(ctypes.byref(_dims(**kw)), A, A, None, A, A, A, A, None, None, None,
                                             None, None, None, None, None)
    prefill = dict(T=8192, d=6144, f=16384, E=8, k=2)
    assert lib.moe_workspace_bytes(ctypes.byref(_dims(**prefill))) > api.NOALLOC_SCRATCH_BYTES
    assert call(**prefill) == 5
    assert call(k=0) == 1
    assert call(T=0) == 0
    assert b"static" in lib.moe_status_string(5)
    # a decode step of the Mixtral-8x22B shape fits, and so does a 700-token batch
    for T in (256, 700):
        assert lib.moe_workspace_bytes(ctypes.byref(_dims(T=T, d=6144, f=16384, E=8, k=2))) <= \
            api.NOALLOC_SCRATCH_BYTES
    # the binding's copy of the size is the header's
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", open(HEADER).read())
    assert m and int(m.group(1)) << 20 == api.NOALLOC_SCRATCH_BYTES
