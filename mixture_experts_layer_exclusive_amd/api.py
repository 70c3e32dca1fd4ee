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
        T, E = logits.shape
        dev = logits.device
        d = x.shape[1] if x is not None else 64
        dt = x.dtype if x is not None else torch.bfloat16
        logits_out = logits
    else:
        T, d = x.shape
        E = w_router.shape[0]
        dev = x.device
        dt = x.dtype
        if logits_out is None:
            logits_out = torch.empty(T, E, dtype=torch.float32, device=dev)
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
    T, k = topk_ids.shape
    dev = topk_ids.device
    d = x.shape[1] if x is not None else 64
    dt = x.dtype if x is not None else torch.bfloat16
    p = problem(T, d, E, k, 64, dt)
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


def expert_ffn(offsets: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
               w_down: torch.Tensor, k: int, T: int, x_perm: Optional[torch.Tensor] = None,
               x: Optional[torch.Tensor] = None, sorted_assign: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, y_perm: Optional[torch.Tensor] = None):
    """Grouped SwiGLU FFN over the queues; returns y_perm [T*k, d]."""
    E, f, d = w_gate.shape
    src = x_perm if x_perm is not None else x
    dev = src.device
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
    T, k = gates.shape
    d = y_perm.shape[1]
    dev = y_perm.device
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
    T, d = x.shape
    E, f, _ = w_gate.shape
    dev = x.device
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
    E, f, d = w_gate.shape
    dev = w_gate.device
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
    T, d = x.shape
    E, f, _ = w_gate.shape
    dev = x.device
    p = problem(T, d, E, k, f, x.dtype)
    w_down_t, w_gu_t = weights_t
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
    fw = L.MoeForwardState(**{key: (_ptr(state[key]) if T > 0 else None) for key in _STATE_KEYS})
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
    rows, cols = src.shape
    dev = src.device
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
    E, f, d = w_gate.shape
    dev = w_gate.device
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
    T, d = x.shape
    E, f, _ = wq["w_gate"].shape
    dev = x.device
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
