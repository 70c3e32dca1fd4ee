"""Torch-facing binding of the MoE-layer library.

Argument marshalling only: shapes and dtypes are read from the tensors, the
device pointers and the current HIP stream are handed to the C ABI, and
every step of the layer runs in the library's kernels.  Torch supplies the
device memory (outputs and workspace) and the stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib as L

_DTYPES = {torch.float32: L.MOE_DTYPE_F32, torch.bfloat16: L.MOE_DTYPE_BF16}


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype, device=None, required: bool = True):
    """Checks one tensor argument against the problem before anything reaches
    the C ABI (which sees only pointers: a wrong shape or dtype there would
    make the kernels read or write out of bounds)."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect_ws(ws: Optional[torch.Tensor], device):
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"ws must be a contiguous tensor on {device}")


def _float_dtype(name: str, t: torch.Tensor):
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name}: dtype {t.dtype}, expected float32 or bfloat16")
    return t.dtype


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def problem(T: int, d: int, E: int, k: int, f: int, dtype) -> L.MoeProblem:
    """The problem statement as the ABI struct; dtype is a torch dtype."""
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    return L.MoeProblem(T=int(T), d=int(d), E=int(E), k=int(k), f=int(f), dtype=_DTYPES[dtype])


def workspace_size(p: L.MoeProblem, op: int) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.load().moe_workspace_size(ctypes.byref(p), op, ctypes.byref(n)), "moe_workspace_size")
    return n.value


def _workspace(p: L.MoeProblem, op: int, device, ws: Optional[torch.Tensor]):
    need = workspace_size(p, op)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def route(k: int, x: Optional[torch.Tensor] = None, w_router: Optional[torch.Tensor] = None,
          logits: Optional[torch.Tensor] = None, ids: Optional[torch.Tensor] = None,
          gates: Optional[torch.Tensor] = None, logits_out: Optional[torch.Tensor] = None):
    """Router GEMM (unless ``logits`` [T, E] fp32 is given) and top-k gating.
    Returns (topk_ids int32 [T, k], topk_gates fp32 [T, k], logits fp32 [T, E])."""
    if logits is not None:
        if logits.dim() != 2:
            raise ValueError("logits must be [T, E]")
        T, E = logits.shape
        dev = logits.device
        _expect("logits", logits, (T, E), torch.float32)
        d = x.shape[1] if x is not None and x.dim() == 2 else 64
        dt = _float_dtype("x", x) if x is not None else torch.bfloat16
        logits_out = logits
    else:
        if x is None or w_router is None or x.dim() != 2 or w_router.dim() != 2:
            raise ValueError("without logits, x [T, d] and w_router [E, d] are required")
        T, d = x.shape
        E = w_router.shape[0]
        dev = x.device
        dt = _float_dtype("x", x)
        _expect("w_router", w_router, (E, d), dt, dev)
        _expect("logits_out", logits_out, (T, E), torch.float32, dev, required=False)
        if logits_out is None:
            logits_out = torch.empty(T, E, dtype=torch.float32, device=dev)
    _expect("ids", ids, (T, k), torch.int32, dev, required=False)
    _expect("gates", gates, (T, k), torch.float32, dev, required=False)
    p = problem(T, d, E, k, 64, dt)
    if ids is None:
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty(T, k, dtype=torch.float32, device=dev)
    L.check(L.load().moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(logits),
                               _ptr(logits_out) if logits is None else None, _ptr(ids),
                               _ptr(gates), _stream(dev)), "moe_route")
    return ids, gates, logits_out


def dispatch(topk_ids: torch.Tensor, E: int, x: Optional[torch.Tensor] = None,
             with_x_perm: bool = False, ws: Optional[torch.Tensor] = None,
             out: Optional[dict] = None) -> dict:
    """Dispatch queues of ``topk_ids`` [T, k]: counts, offsets, sorted_assign,
    assign_pos and (with ``with_x_perm``) the gathered rows x_perm.  ``out``
    may supply any of these tensors."""
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k]")
    T, k = topk_ids.shape
    dev = topk_ids.device
    _expect("topk_ids", topk_ids, (T, k), torch.int32)
    if with_x_perm and x is None:
        raise ValueError("with_x_perm needs x")
    if x is not None:
        if x.dim() != 2:
            raise ValueError("x must be [T, d]")
        _expect("x", x, (T, x.shape[1]), _float_dtype("x", x), dev)
    d = x.shape[1] if x is not None else 64
    dt = x.dtype if x is not None else torch.bfloat16
    _expect_ws(ws, dev)
    p = problem(T, d, E, k, 64, dt)
    given = dict(out or {})
    for key, shape, tdt in (("counts", (E,), torch.int32), ("offsets", (E + 1,), torch.int32),
                            ("sorted_assign", (T * k,), torch.int32), ("assign_pos", (T * k,), torch.int32),
                            ("x_perm", (T * k, d), dt)):
        _expect(key, given.get(key), shape, tdt, dev, required=False)
    res = dict(out or {})
    res.setdefault("counts", torch.empty(E, dtype=torch.int32, device=dev))
    res.setdefault("offsets", torch.empty(E + 1, dtype=torch.int32, device=dev))
    res.setdefault("sorted_assign", torch.empty(T * k, dtype=torch.int32, device=dev))
    res.setdefault("assign_pos", torch.empty(T * k, dtype=torch.int32, device=dev))
    if with_x_perm:
        res.setdefault("x_perm", torch.empty(T * k, d, dtype=dt, device=dev))
    else:
        res["x_perm"] = None
    ws, nbytes = _workspace(p, L.MOE_OP_DISPATCH, dev, ws)
    L.check(L.load().moe_dispatch(ctypes.byref(p), _ptr(topk_ids), _ptr(x), _ptr(res["counts"]),
                                  _ptr(res["offsets"]), _ptr(res["sorted_assign"]),
                                  _ptr(res["assign_pos"]), _ptr(res["x_perm"]), _ptr(ws), nbytes,
                                  _stream(dev)), "moe_dispatch")
    return res


def dispatch_no_alloc(topk_ids: torch.Tensor, E: int, x: Optional[torch.Tensor] = None,
                      with_x_perm: bool = False, out: Optional[dict] = None) -> dict:
    """``dispatch`` through ``moe_dispatch_no_alloc``: the library's static
    per-GPU scratch instead of a workspace (no device allocation inside the
    call; outputs are allocated here unless ``out`` supplies them)."""
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k]")
    T, k = topk_ids.shape
    dev = topk_ids.device
    _expect("topk_ids", topk_ids, (T, k), torch.int32)
    if with_x_perm and x is None:
        raise ValueError("with_x_perm needs x")
    if x is not None:
        if x.dim() != 2:
            raise ValueError("x must be [T, d]")
        _expect("x", x, (T, x.shape[1]), _float_dtype("x", x), dev)
    d = x.shape[1] if x is not None else 64
    dt = x.dtype if x is not None else torch.bfloat16
    p = problem(T, d, E, k, 64, dt)
    res = dict(out or {})
    for key, shape, tdt in (("counts", (E,), torch.int32), ("offsets", (E + 1,), torch.int32),
                            ("sorted_assign", (T * k,), torch.int32), ("assign_pos", (T * k,), torch.int32),
                            ("x_perm", (T * k, d), dt)):
        _expect(key, res.get(key), shape, tdt, dev, required=False)
        if key != "x_perm" or with_x_perm:
            res.setdefault(key, torch.empty(shape, dtype=tdt, device=dev))
    if not with_x_perm:
        res["x_perm"] = None
    L.check(L.load().moe_dispatch_no_alloc(ctypes.byref(p), _ptr(topk_ids), _ptr(x), _ptr(res["counts"]),
                                           _ptr(res["offsets"]), _ptr(res["sorted_assign"]),
                                           _ptr(res["assign_pos"]), _ptr(res["x_perm"]), _stream(dev)),
            "moe_dispatch_no_alloc")
    return res


def expert_ffn(offsets: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
               w_down: torch.Tensor, k: int, T: int, x_perm: Optional[torch.Tensor] = None,
               x: Optional[torch.Tensor] = None, sorted_assign: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, y_perm: Optional[torch.Tensor] = None):
    """Grouped SwiGLU FFN over the queues; returns y_perm [T*k, d]."""
    if w_gate.dim() != 3:
        raise ValueError("w_gate must be [E, f, d]")
    E, f, d = w_gate.shape
    src = x_perm if x_perm is not None else x
    if src is None:
        raise ValueError("x_perm, or x with sorted_assign, is required")
    dev = src.device
    dt = _float_dtype("w_gate", w_gate)
    if x_perm is not None:
        _expect("x_perm", x_perm, (T * k, d), dt, dev)
    else:
        _expect("x", x, (T, d), dt, dev)
        _expect("sorted_assign", sorted_assign, (T * k,), torch.int32, dev)
    _expect("offsets", offsets, (E + 1,), torch.int32, dev)
    _expect("w_gate", w_gate, (E, f, d), dt, dev)
    _expect("w_up", w_up, (E, f, d), dt, dev)
    _expect("w_down", w_down, (E, d, f), dt, dev)
    _expect("y_perm", y_perm, (T * k, d), dt, dev, required=False)
    _expect_ws(ws, dev)
    p = problem(T, d, E, k, f, src.dtype)
    if y_perm is None:
        y_perm = torch.empty(T * k, d, dtype=src.dtype, device=dev)
    ws, nbytes = _workspace(p, L.MOE_OP_EXPERT_FFN, dev, ws)
    L.check(L.load().moe_expert_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(x), _ptr(sorted_assign),
                                    _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                    _ptr(y_perm), _ptr(ws), nbytes, _stream(dev)),
            "moe_expert_ffn")
    return y_perm


def combine(y_perm: torch.Tensor, assign_pos: torch.Tensor, gates: torch.Tensor,
            y: Optional[torch.Tensor] = None):
    """Gate-weighted combine back to token order; returns y [T, d]."""
    if gates.dim() != 2 or y_perm.dim() != 2:
        raise ValueError("gates must be [T, k] and y_perm [T*k, d]")
    T, k = gates.shape
    d = y_perm.shape[1]
    dev = y_perm.device
    dt = _float_dtype("y_perm", y_perm)
    _expect("y_perm", y_perm, (T * k, d), dt)
    _expect("assign_pos", assign_pos, (T * k,), torch.int32, dev)
    _expect("gates", gates, (T, k), torch.float32, dev)
    _expect("y", y, (T, d), dt, dev, required=False)
    p = problem(T, d, 1 if k == 1 else k, k, 64, y_perm.dtype)
    if y is None:
        y = torch.empty(T, d, dtype=y_perm.dtype, device=dev)
    L.check(L.load().moe_combine(ctypes.byref(p), _ptr(y_perm), _ptr(assign_pos), _ptr(gates),
                                 _ptr(y), _stream(dev)), "moe_combine")
    return y


def forward(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
            k: int, w_router: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
            intermediates: bool = False, ws: Optional[torch.Tensor] = None,
            y: Optional[torch.Tensor] = None):
    """The whole layer in one call.  Returns y [T, d], or (y, dict of
    intermediates) with ``intermediates=True``; the intermediates include
    the forward state ``backward`` reads."""
    if x.dim() != 2 or w_gate.dim() != 3:
        raise ValueError("x must be [T, d] and w_gate [E, f, d]")
    T, d = x.shape
    E, f, _ = w_gate.shape
    dev = x.device
    dt = _float_dtype("x", x)
    _expect("w_gate", w_gate, (E, f, d), dt, dev)
    _expect("w_up", w_up, (E, f, d), dt, dev)
    _expect("w_down", w_down, (E, d, f), dt, dev)
    if w_router is None and logits is None:
        raise ValueError("w_router or logits is required")
    _expect("w_router", w_router, (E, d), dt, dev, required=False)
    _expect("logits", logits, (T, E), torch.float32, dev, required=False)
    _expect("y", y, (T, d), dt, dev, required=False)
    _expect_ws(ws, dev)
    p = problem(T, d, E, k, f, x.dtype)
    if y is None:
        y = torch.empty(T, d, dtype=x.dtype, device=dev)
    outs = None
    o = None
    if intermediates:
        n = T * k
        outs = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev) if logits is None else logits,
                    topk_ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                    topk_gates=torch.empty(T, k, dtype=torch.float32, device=dev),
                    counts=torch.empty(E, dtype=torch.int32, device=dev),
                    offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                    sorted_assign=torch.empty(n, dtype=torch.int32, device=dev),
                    assign_pos=torch.empty(n, dtype=torch.int32, device=dev),
                    y_perm=torch.empty(n, d, dtype=x.dtype, device=dev))
        o = L.MoeForwardOutputs(**{key: (None if (key == "logits" and logits is not None) else v.data_ptr())
                                   for key, v in outs.items()})
    ws, nbytes = _workspace(p, L.MOE_OP_FORWARD, dev, ws)
    L.check(L.load().moe_forward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(logits),
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y),
                                 ctypes.byref(o) if o is not None else None, _ptr(ws), nbytes,
                                 _stream(dev)), "moe_forward")
    return (y, outs) if intermediates else y


def backward_weights(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                     w_down_t: Optional[torch.Tensor] = None, w_gu_t: Optional[torch.Tensor] = None):
    """The weight layouts the backward GEMMs read: (w_down_t [E, f, d],
    w_gu_t [E, d, 2f]).  Recompute after every change of the weights."""
    if w_gate.dim() != 3:
        raise ValueError("w_gate must be [E, f, d]")
    E, f, d = w_gate.shape
    dev = w_gate.device
    dt = _float_dtype("w_gate", w_gate)
    _expect("w_up", w_up, (E, f, d), dt, dev)
    _expect("w_down", w_down, (E, d, f), dt, dev)
    _expect("w_down_t", w_down_t, (E, f, d), dt, dev, required=False)
    _expect("w_gu_t", w_gu_t, (E, d, 2 * f), dt, dev, required=False)
    p = problem(0, d, E, 1, f, w_gate.dtype)
    if w_down_t is None:
        w_down_t = torch.empty(E, f, d, dtype=w_gate.dtype, device=dev)
    if w_gu_t is None:
        w_gu_t = torch.empty(E, d, 2 * f, dtype=w_gate.dtype, device=dev)
    L.check(L.load().moe_backward_weights(ctypes.byref(p), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                          _ptr(w_down_t), _ptr(w_gu_t), _stream(dev)),
            "moe_backward_weights")
    return w_down_t, w_gu_t


_STATE_KEYS = ("topk_ids", "topk_gates", "offsets", "sorted_assign", "assign_pos", "y_perm")


def backward(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, k: int, state: dict,
             dy: torch.Tensor, weights_t, w_router: Optional[torch.Tensor] = None,
             with_dlogits: bool = False, ws: Optional[torch.Tensor] = None,
             out: Optional[dict] = None) -> dict:
    """Gradients of the layer for dy [T, d], given the forward's state (the
    intermediates of ``forward``) and ``weights_t`` from
    ``backward_weights``.  Returns dx, dw_gate, dw_up, dw_down, dw_router
    (None without a router) and dlogits (None unless ``with_dlogits``).
    ``out`` may supply any of these tensors."""
    if x.dim() != 2 or w_gate.dim() != 3:
        raise ValueError("x must be [T, d] and w_gate [E, f, d]")
    T, d = x.shape
    E, f, _ = w_gate.shape
    dev = x.device
    dt = _float_dtype("x", x)
    w_down_t, w_gu_t = weights_t
    _expect("w_gate", w_gate, (E, f, d), dt, dev)
    _expect("w_up", w_up, (E, f, d), dt, dev)
    _expect("w_down_t", w_down_t, (E, f, d), dt, dev)
    _expect("w_gu_t", w_gu_t, (E, d, 2 * f), dt, dev)
    _expect("w_router", w_router, (E, d), dt, dev, required=False)
    _expect("dy", dy, (T, d), dt, dev)
    n = T * k
    if T > 0:
        for key, shape, tdt in (("topk_ids", (T, k), torch.int32), ("topk_gates", (T, k), torch.float32),
                                ("offsets", (E + 1,), torch.int32), ("sorted_assign", (n,), torch.int32),
                                ("assign_pos", (n,), torch.int32)):
            _expect(f"state[{key!r}]", state.get(key), shape, tdt, dev)
        # (y_perm is not read: the backward needs only the routing)
        _expect("state['y_perm']", state.get("y_perm"), (n, d), dt, dev, required=False)
    given = dict(out or {})
    for key, shape, tdt in (("dx", (T, d), dt), ("dw_gate", (E, f, d), dt), ("dw_up", (E, f, d), dt),
                            ("dw_down", (E, d, f), dt), ("dw_router", (E, d), dt),
                            ("dlogits", (T, E), torch.float32)):
        _expect(key, given.get(key), shape, tdt, dev, required=False)
    _expect_ws(ws, dev)
    p = problem(T, d, E, k, f, x.dtype)
    res = dict(out or {})
    res.setdefault("dx", torch.empty(T, d, dtype=x.dtype, device=dev))
    res.setdefault("dw_gate", torch.empty(E, f, d, dtype=x.dtype, device=dev))
    res.setdefault("dw_up", torch.empty(E, f, d, dtype=x.dtype, device=dev))
    res.setdefault("dw_down", torch.empty(E, d, f, dtype=x.dtype, device=dev))
    if w_router is not None:
        res.setdefault("dw_router", torch.empty(E, d, dtype=x.dtype, device=dev))
    else:
        res["dw_router"] = None
    if with_dlogits:
        res.setdefault("dlogits", torch.empty(T, E, dtype=torch.float32, device=dev))
    else:
        res["dlogits"] = None
    # (with no tokens the forward state is not read)
    fw = L.MoeForwardState(**{key: (_ptr(state.get(key)) if T > 0 else None) for key in _STATE_KEYS})
    o = L.MoeBackwardOutputs(**{key: (_ptr(res[key]) if res[key] is not None and res[key].numel() > 0
                                      else None)
                                for key in ("dx", "dw_gate", "dw_up", "dw_down", "dw_router", "dlogits")})
    ws, nbytes = _workspace(p, L.MOE_OP_BACKWARD, dev, ws)
    L.check(L.load().moe_backward(ctypes.byref(p), _ptr(x) if T > 0 else None, _ptr(w_router),
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down_t), _ptr(w_gu_t),
                                  ctypes.byref(fw), _ptr(dy) if T > 0 else None, ctypes.byref(o),
                                  _ptr(ws), nbytes, _stream(dev)), "moe_backward")
    return res


def quantize_rows_fp8(src: torch.Tensor, codes: Optional[torch.Tensor] = None,
                      exps: Optional[torch.Tensor] = None):
    """Per-row FP8 E4M3 codes (uint8) and power-of-two scale exponents
    (int32) of a bf16 matrix [rows, cols]."""
    if src.dim() != 2:
        raise ValueError("src must be [rows, cols]")
    rows, cols = src.shape
    dev = src.device
    _expect("src", src, (rows, cols), torch.bfloat16)
    _expect("codes", codes, (rows, cols), torch.uint8, dev, required=False)
    _expect("exps", exps, (rows,), torch.int32, dev, required=False)
    if codes is None:
        codes = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
    if exps is None:
        exps = torch.empty(rows, dtype=torch.int32, device=dev)
    L.check(L.load().moe_quantize_rows_fp8(_ptr(src) if rows else None, rows, cols,
                                           _ptr(codes) if rows else None, _ptr(exps) if rows else None,
                                           _stream(dev)), "moe_quantize_rows_fp8")
    return codes, exps


def quantize_weights_fp8(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor) -> dict:
    """The expert weights as FP8 codes with per-row scale exponents (for
    ``expert_ffn_fp8``)."""
    if w_gate.dim() != 3:
        raise ValueError("w_gate must be [E, f, d]")
    E, f, d = w_gate.shape
    dev = w_gate.device
    _expect("w_gate", w_gate, (E, f, d), torch.bfloat16)
    _expect("w_up", w_up, (E, f, d), torch.bfloat16, dev)
    _expect("w_down", w_down, (E, d, f), torch.bfloat16, dev)
    p = problem(1, d, E, 1, f, w_gate.dtype)
    q = dict(w_gate=torch.empty(E, f, d, dtype=torch.uint8, device=dev),
             w_gate_exp=torch.empty(E, f, dtype=torch.int32, device=dev),
             w_up=torch.empty(E, f, d, dtype=torch.uint8, device=dev),
             w_up_exp=torch.empty(E, f, dtype=torch.int32, device=dev),
             w_down=torch.empty(E, d, f, dtype=torch.uint8, device=dev),
             w_down_exp=torch.empty(E, d, dtype=torch.int32, device=dev))
    st = L.MoeFp8Weights(**{key: _ptr(v) for key, v in q.items()})
    L.check(L.load().moe_quantize_weights_fp8(ctypes.byref(p), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                              ctypes.byref(st), _stream(dev)), "moe_quantize_weights_fp8")
    return q


def expert_ffn_fp8(offsets: torch.Tensor, wq: dict, k: int, x: torch.Tensor, sorted_assign: torch.Tensor,
                   ws: Optional[torch.Tensor] = None, y_perm: Optional[torch.Tensor] = None):
    """Grouped SwiGLU FFN on FP8 MFMA (weights from ``quantize_weights_fp8``,
    x bf16 quantised per token inside); returns y_perm [T*k, d] bf16."""
    if x.dim() != 2 or wq.get("w_gate") is None or wq["w_gate"].dim() != 3:
        raise ValueError("x must be [T, d] and wq['w_gate'] [E, f, d]")
    T, d = x.shape
    E, f, _ = wq["w_gate"].shape
    dev = x.device
    _expect("x", x, (T, d), torch.bfloat16)
    for key, shape, tdt in (("w_gate", (E, f, d), torch.uint8), ("w_gate_exp", (E, f), torch.int32),
                            ("w_up", (E, f, d), torch.uint8), ("w_up_exp", (E, f), torch.int32),
                            ("w_down", (E, d, f), torch.uint8), ("w_down_exp", (E, d), torch.int32)):
        _expect(f"wq[{key!r}]", wq.get(key), shape, tdt, dev)
    _expect("offsets", offsets, (E + 1,), torch.int32, dev)
    _expect("sorted_assign", sorted_assign, (T * k,), torch.int32, dev)
    _expect("y_perm", y_perm, (T * k, d), torch.bfloat16, dev, required=False)
    _expect_ws(ws, dev)
    p = problem(T, d, E, k, f, x.dtype)
    if y_perm is None:
        y_perm = torch.empty(T * k, d, dtype=x.dtype, device=dev)
    st = L.MoeFp8Weights(**{key: _ptr(v) for key, v in wq.items()})
    ws, nbytes = _workspace(p, L.MOE_OP_EXPERT_FFN_FP8, dev, ws)
    L.check(L.load().moe_expert_ffn_fp8(ctypes.byref(p), _ptr(x) if T else None,
                                        _ptr(sorted_assign) if T else None, _ptr(offsets), ctypes.byref(st),
                                        _ptr(y_perm) if T else None, _ptr(ws), nbytes, _stream(dev)),
            "moe_expert_ffn_fp8")
    return y_perm


def mfma_peak_tflops(device=None, workgroups: int = 1024, iters: int = 4000, reps: int = 3) -> float:
    """The bf16 MFMA rate this GPU sustains with register operands only
    (``moe_mfma_peak``), in TFLOP/s: the best of ``reps`` timed launches."""
    dev = torch.device(device or "cuda:0")
    sink = torch.empty(workgroups, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for r in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        L.check(L.load().moe_mfma_peak(workgroups, iters, _ptr(sink), _stream(dev)), "moe_mfma_peak")
        b.record(stream)
        torch.cuda.synchronize(dev)
        if r > 0:
            best = max(best, workgroups * 4 * iters * 8 * 32768.0 / (a.elapsed_time(b) * 1e-3) / 1e12)
    return best


def stream_copy_gbs(device=None, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """The streaming bandwidth this GPU sustains in a plain device copy of
    ``nbytes`` (``moe_stream_copy``, read + write bytes), in GB/s: the best of
    ``reps`` timed launches after one warm-up."""
    dev = torch.device(device or "cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.check(L.load().moe_stream_copy(_ptr(a), _ptr(b), nbytes, _stream(dev)), "moe_stream_copy")
        e1.record(stream)
        torch.cuda.synchronize(dev)
        if r > 0:
            best = max(best, 2.0 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    return best
