"""CPU oracle of the MoE layer's backward pass (test infrastructure only).

Like ``moe_oracle`` this is the plain statement of what the HIP path must
compute, in float64, and only the tests may import it.  It shares no code
with the HIP library.

The pages state the training side only in outline.  The MoEBlaze summary
(euno.news, "MoEBlaze: breaking the memory wall for efficient MoE training
on modern GPUs"), Methodology item 2, has the backward reuse the forward's
compact dispatch queues for the gradients: reverse dispatch of the output
gradient, the expert backward, dispatch of the input gradient.  The
checkpoint bullet of the same item (and Key contributions, bullet 3: smart
activation checkpointing) stores only what the backward needs and recomputes
the rest: here the SwiGLU intermediates are recomputed instead of stored.  Everything else is the derivative
of the forward in ``moe_oracle``, taken by the chain rule:

* slot gradients ``dg[t, j] = <dy[t], y_perm[pos(t, j)]>``;
* the expert rows' output gradient ``dy_perm[pos(t, j)] = g[t, j] dy[t]``;
* per expert, with ``u = x W_gate^T``, ``v = x W_up^T``, ``s = silu(u)``,
  ``h = s v``:
  ``dh = dy_perm W_down``, ``dW_down = dy_perm^T h``,
  ``du = dh v silu'(u)`` with ``silu'(u) = sigma(u) (1 + u (1 - sigma(u)))``,
  ``dv = dh s``, ``dx_perm = du W_gate + dv W_up``,
  ``dW_gate = du^T x_perm``, ``dW_up = dv^T x_perm``;
* ``dx[t] = sum_j dx_perm[pos(t, j)]`` (no gate: it was applied to dy);
* the gates are a softmax over the chosen logits, so for chosen experts
  ``dl_i = g_i (dg_i - sum_j g_j dg_j)``; experts outside the top k get no
  gradient (the selection is piecewise constant in the logits);
* router: ``dW_r = dl^T x`` and ``dx += dl W_r``.

Parity pins: ``tests/test_oracle_backward_pins.py`` (central finite
differences of the float64 forward, an independent automatic
differentiation of the same forward, and linearity in dy).
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import forward, silu


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def sigmoid(u: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-u))


def silu_grad(u: np.ndarray) -> np.ndarray:
    """d silu(u) / du = sigma(u) (1 + u (1 - sigma(u)))."""
    s = sigmoid(u)
    return s * (1.0 + u * (1.0 - s))


def gate_grad(dy: np.ndarray, y_perm: np.ndarray, assign_pos: np.ndarray, k: int) -> np.ndarray:
    """``dg[t, j] = sum_o dy[t, o] y_perm[assign_pos[t*k + j], o]``, float64."""
    dy = _f64(dy)
    T = dy.shape[0]
    pos = np.asarray(assign_pos, dtype=np.int64).reshape(T, k)
    yp = _f64(y_perm)
    return np.stack([np.sum(dy * yp[pos[:, j]], axis=1) for j in range(k)], axis=1)


def dispatch_grad(dy: np.ndarray, gates: np.ndarray, sorted_assign: np.ndarray, k: int) -> np.ndarray:
    """Output gradient of the queue rows: ``dy_perm[pos] = g[a] dy[a // k]``
    with ``a = sorted_assign[pos]`` (the gate-weighted reverse of combine)."""
    sa = np.asarray(sorted_assign, dtype=np.int64)
    g = _f64(gates).reshape(-1)
    return g[sa][:, None] * _f64(dy)[sa // k]


def topk_gates_backward(logits: np.ndarray, ids: np.ndarray, gates: np.ndarray,
                        dgates: np.ndarray) -> np.ndarray:
    """Logit gradient of the renormalised top-k softmax: for each token and
    chosen expert i, ``dl_i = g_i (dg_i - sum_j g_j dg_j)``; 0 elsewhere.
    Returns float64 [T, E]."""
    T, E = np.asarray(logits).shape
    g = _f64(gates)
    dg = _f64(dgates)
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dsel = g * (dg - inner)
    dl = np.zeros((T, E), dtype=np.float64)
    ids64 = np.asarray(ids, dtype=np.int64)
    for j in range(ids64.shape[1]):
        dl[np.arange(T), ids64[:, j]] += dsel[:, j]
    return dl


def swiglu_expert_backward(x_rows: np.ndarray, w_gate_e: np.ndarray, w_up_e: np.ndarray,
                           w_down_e: np.ndarray, dy_rows: np.ndarray, weights: bool = True) -> dict:
    """Backward of one expert ``y = W_down (silu(W_gate x) * (W_up x))`` on
    rows: returns dx [n, d] and (with ``weights``) dw_gate [f, d], dw_up
    [f, d], dw_down [d, f], all float64."""
    xr = _f64(x_rows)
    wg, wu, wd = _f64(w_gate_e), _f64(w_up_e), _f64(w_down_e)
    dyr = _f64(dy_rows)
    u = xr @ wg.T
    v = xr @ wu.T
    s = silu(u)
    h = s * v
    dh = dyr @ wd
    du = dh * v * silu_grad(u)
    dv = dh * s
    if not weights:
        return dict(dx=du @ wg + dv @ wu)
    return dict(dx=du @ wg + dv @ wu, dw_gate=du.T @ xr, dw_up=dv.T @ xr, dw_down=dyr.T @ h)


def backward(x: np.ndarray, k: int, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
             dy: np.ndarray, w_router: np.ndarray | None = None,
             logits: np.ndarray | None = None) -> dict:
    """Gradients of the whole layer for the output gradient ``dy`` [T, d]:
    dx [T, d], dw_gate, dw_up [E, f, d], dw_down [E, d, f], dlogits [T, E],
    dgates [T, k] and (with a router) dw_router [E, d], all float64.  The
    routing (ids, gates, queues) is the forward's.  Given both ``w_router``
    and ``logits``, the logits stand for the router's output as computed
    elsewhere (routing and gates read them) and the router gradients still
    flow through ``w_router``."""
    fw = forward(x, k, w_gate, w_up, w_down, w_router=w_router, logits=logits)
    E = fw["logits"].shape[1]
    T, d = np.asarray(x).shape
    f = np.asarray(w_gate).shape[1]
    dgates = gate_grad(dy, fw["y_perm"], fw["assign_pos"], k)
    dy_perm = dispatch_grad(dy, fw["gates"], fw["sorted_assign"], k)
    sa = np.asarray(fw["sorted_assign"], dtype=np.int64)
    off = fw["offsets"]
    dx_perm = np.zeros((T * k, d), dtype=np.float64)
    dwg = np.zeros((E, f, d), dtype=np.float64)
    dwu = np.zeros((E, f, d), dtype=np.float64)
    dwd = np.zeros((E, d, f), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        r = swiglu_expert_backward(np.asarray(x)[sa[lo:hi] // k], w_gate[e], w_up[e], w_down[e],
                                   dy_perm[lo:hi])
        dx_perm[lo:hi] = r["dx"]
        dwg[e], dwu[e], dwd[e] = r["dw_gate"], r["dw_up"], r["dw_down"]
    pos = np.asarray(fw["assign_pos"], dtype=np.int64).reshape(T, k)
    dx = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        dx += dx_perm[pos[:, j]]
    dlogits = topk_gates_backward(fw["logits"], fw["ids"], fw["gates"], dgates)
    dw_router = None
    if w_router is not None:
        dw_router = dlogits.T @ _f64(x)
        dx += dlogits @ _f64(w_router)
    return dict(dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd, dlogits=dlogits, dgates=dgates,
                dw_router=dw_router, dy_perm=dy_perm, dx_perm=dx_perm, forward=fw)


def backward_tokens(tokens: np.ndarray, x: np.ndarray, logits: np.ndarray, k: int, w_gate, w_up,
                    w_down, dy: np.ndarray, w_router: np.ndarray | None = None) -> dict:
    """Per-token definition of the input and logit gradients on a subset of
    tokens (no queues): for token t with ids e_j and gates g_j from
    ``topk_route`` on its logits row,
    ``dg_j = <dy_t, FFN_{e_j}(x_t)>``, ``dl = topk_gates_backward(dg)``,
    ``dx_t = sum_j J_{e_j}(x_t)^T (g_j dy_t) + sum_j dl_{e_j} W_r[e_j]``
    (the router term only with ``w_router``), where ``J_e^T`` is the
    expert's input gradient.  Expert weights may be callables ``w(e)`` as in
    ``forward_tokens`` (each expert used is widened once).  Returns dx
    [n, d] and dlogits [n, E], float64."""
    from .moe_oracle import swiglu_expert, topk_route
    tokens = np.asarray(tokens, dtype=np.int64)
    l = np.asarray(logits, dtype=np.float32)[tokens]
    ids, gates = topk_route(l, k)
    xs = _f64(np.asarray(x)[tokens])
    dys = _f64(np.asarray(dy)[tokens])

    def get(w, e):
        return w(e) if callable(w) else w[e]

    n, d = xs.shape
    dx = np.zeros((n, d), dtype=np.float64)
    dg = np.zeros((n, k), dtype=np.float64)
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        wg, wu, wd = get(w_gate, e), get(w_up, e), get(w_down, e)
        dg[rows, slots] = np.sum(dys[rows] * swiglu_expert(xs[rows], wg, wu, wd), axis=1)
        g = _f64(gates[rows, slots])[:, None]
        r = swiglu_expert_backward(xs[rows], wg, wu, wd, g * dys[rows], weights=False)
        np.add.at(dx, rows, r["dx"])
    dl = topk_gates_backward(l, ids, gates, dg)
    if w_router is not None:
        dx += dl @ _f64(w_router)
    return dict(dx=dx, dlogits=dl, ids=ids, gates=gates)


def weight_grad_entries(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, e: int, w_gate_e,
                        w_up_e, w_down_e, dy: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> dict:
    """Sampled entries of expert e's weight gradients, each a sum over the
    (token, slot) pairs routed to e (order irrelevant in float64):
    ``dW_down[e][rows][:, cols] = sum g dy_t[rows] h(x_t)[cols]``, and the
    full rows ``dW_gate[e][cols, :] = sum du(x_t)[cols] x_t``,
    ``dW_up[e][cols, :] = sum dv(x_t)[cols] x_t``, with u, v, h, dh, du, dv
    of the expert's SwiGLU for the output gradient g dy_t.  Only the
    requested columns of u, v and dh are formed."""
    ids = np.asarray(ids)
    t, j = np.nonzero(ids == e)
    g = _f64(gates)[t, j]
    xr = _f64(np.asarray(x)[t])
    dyr = g[:, None] * _f64(np.asarray(dy)[t])
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    wg = _f64(np.asarray(w_gate_e)[cols])
    wu = _f64(np.asarray(w_up_e)[cols])
    wd = _f64(np.asarray(w_down_e)[:, cols])
    u = xr @ wg.T
    v = xr @ wu.T
    s = silu(u)
    h = s * v
    dh = dyr @ wd
    du = dh * v * silu_grad(u)
    dv = dh * s
    return dict(dw_down=dyr[:, rows].T @ h, dw_gate=du.T @ xr, dw_up=dv.T @ xr)
