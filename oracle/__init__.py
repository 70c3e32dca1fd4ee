"""CPU oracle of the MoE layer (forward and backward): TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and it shares no code
with them.

Parity status: every function in ``moe_oracle`` is pinned by
``tests/test_oracle_pins.py`` (brute force on tiny inputs, library routines
for the special cases, closed forms and invariants), and every function in
``moe_backward`` by ``tests/test_oracle_backward_pins.py`` (finite
differences, an independent automatic differentiation, linearity), and
every function in ``moe_fp8`` by ``tests/test_oracle_fp8_pins.py`` (torch's
float8 conversion, exhaustive code round trip, brute-force nearest code,
exact arithmetic on representable inputs).  No function here is "parity
unpinned".
"""
from .moe_oracle import (  # noqa: F401
    router_logits, topk_route, expert_histogram, exclusive_scan, stable_scatter,
    dispatch, gather_rows, silu, swiglu_expert, expert_ffn, combine, forward,
    forward_tokens,
)
from .moe_backward import (  # noqa: F401
    sigmoid, silu_grad, gate_grad, dispatch_grad, topk_gates_backward,
    swiglu_expert_backward, backward,
)
from .moe_fp8 import (  # noqa: F401
    e4m3_encode, e4m3_decode, pow2_scale_exponent, quantize_rows, dequantize_rows, round_bf16,
    quantize_weights, fp8_expert_ffn,
)
