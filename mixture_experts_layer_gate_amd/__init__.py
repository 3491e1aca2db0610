"""MI355X-native forward and backward passes of one Mixture-of-Experts layer.

Route (gate GEMM + top-k softmax), dispatch (histogram, scan, stable
permutation), grouped SwiGLU expert FFN and weighted combine, and the layer's
gradients (DGrad, WGrad, routing-weight and gate gradients), each a
hand-written HIP kernel for gfx950 behind the C-ABI declared in
``include/moe.h``. The Python functions here only marshal torch tensors into
that ABI; the library is loaded on first use and a missing build is an error.
"""
from .api import (  # noqa: F401
    MoeError, Dims, workspace_bytes, route, permute, grouped_ffn, combine, layer_forward,
    library_path, load_library, STAGES, EXPORTS, make_workspace, timing_enable, timing_disable, timing_read,
    probe_hbm_read_gbps, probe_mfma_tflops, workspace_bytes_shared, layer_forward_shared,
    backward_workspace_bytes, layer_backward, layer_forward_train, ffn_block_rows, gate_on_matrix_cores, pack_weights, pack_weights_transposed,
    fused_status, plan_layout, read_plan, read_plan_multi_block, layer_forward_noalloc, NOALLOC_SCRATCH_BYTES,
)
