"""One GPU's MoE-layer forward on MI355X (gfx950): router GEMM and static
top-k gating, counting-sort dispatch queues, grouped SwiGLU expert FFN on
bf16 MFMA, gate-weighted combine; and the layer's backward on the same
queues.

The kernels live in ``libmoe.so`` (C ABI in ``include/moe.h``); this package
only binds them to torch tensors and streams.
"""
from ._lib import MoeError, load  # noqa: F401
from .api import (  # noqa: F401
    backward, backward_weights, combine, dispatch, dispatch_no_alloc, expert_ffn, expert_ffn_fp8, forward, mfma_peak_tflops,
    problem, quantize_rows_fp8, quantize_weights_fp8, route, stream_copy_gbs, workspace_size,
)
