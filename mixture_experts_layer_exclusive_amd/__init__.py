"""One GPU's MoE-layer forward on MI355X (gfx950): router GEMM and static
top-k gating, counting-sort dispatch queues, grouped SwiGLU expert FFN on
bf16 MFMA, gate-weighted combine.

The kernels live in ``libmoe.so`` (C ABI in ``include/moe.h``); this package
only binds them to torch tensors and streams.
"""
from ._lib import MoeError, load  # noqa: F401
from .api import (  # noqa: F401
    combine, dispatch, expert_ffn, forward, problem, route, workspace_size,
)
