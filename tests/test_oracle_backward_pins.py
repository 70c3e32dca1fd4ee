"""Pins of the backward oracle against what the mathematics fixes:

* central finite differences of the float64 forward (one expert's SwiGLU;
  the renormalised top-k softmax with the chosen set held fixed);
* automatic differentiation (torch, float64, CPU) of the whole layer written
  directly from its definition, independently of the hand-derived formulas
  in ``oracle.moe_backward``;
* linearity in the output gradient, and the closed form of the single-
  expert case (the gate is constant 1, so no logit gradient).
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as O
from oracle import moe_backward as B


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def fd_grad(fun, arr, h=1e-5):
    """Central differences of the scalar fun() over every element of arr
    (modified in place and restored)."""
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h
        fp = fun()
        arr[i] = old - h
        fm = fun()
        arr[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def test_expert_backward_matches_finite_differences():
    rng = np.random.default_rng(3)
    n, d, f = 5, 6, 7
    x = rng.standard_normal((n, d))
    wg, wu = rng.standard_normal((f, d)) * 0.5, rng.standard_normal((f, d)) * 0.5
    wd = rng.standard_normal((d, f)) * 0.5
    dy = rng.standard_normal((n, d))
    loss = lambda: float(np.sum(O.swiglu_expert(x, wg, wu, wd) * dy))  # noqa: E731
    r = B.swiglu_expert_backward(x, wg, wu, wd, dy)
    assert rel(r["dx"], fd_grad(loss, x)) < 1e-7
    assert rel(r["dw_gate"], fd_grad(loss, wg)) < 1e-7
    assert rel(r["dw_up"], fd_grad(loss, wu)) < 1e-7
    assert rel(r["dw_down"], fd_grad(loss, wd)) < 1e-7


def test_silu_grad_closed_form():
    u = np.linspace(-30, 30, 601)
    h = 1e-6
    fd = (O.silu(u + h) - O.silu(u - h)) / (2 * h)
    assert np.max(np.abs(B.silu_grad(u) - fd)) < 1e-8
    assert B.silu_grad(np.array([0.0]))[0] == 0.5  # sigma(0) (1 + 0) = 1/2


def test_topk_gate_backward_matches_finite_differences():
    rng = np.random.default_rng(4)
    T, E, k = 4, 6, 3
    l = rng.standard_normal((T, E))
    ids, gates = O.topk_route(l.astype(np.float32), k)
    dg = rng.standard_normal((T, k))
    idx = ids.astype(np.int64)

    def loss():
        sel = np.take_along_axis(l, idx, axis=1)
        p = np.exp(sel - sel.max(axis=1, keepdims=True))
        return float(np.sum(p / p.sum(axis=1, keepdims=True) * dg))

    fd = fd_grad(loss, l)
    dl = B.topk_gates_backward(l.astype(np.float32), ids, gates, dg)
    # the oracle uses the float32 gates of the forward: agreement to their rounding
    assert rel(dl, fd) < 1e-6
    chosen = np.zeros((T, E), bool)
    chosen[np.arange(T)[:, None], idx] = True
    assert np.all(dl[~chosen] == 0.0)
    # softmax invariance: the logit gradient of each token sums to zero, up to
    # the float32 rounding of the gates (their sum is 1 within a few ulp)
    assert np.max(np.abs(dl.sum(axis=1))) < 1e-6 * np.max(np.abs(dl))


def torch_layer_grads(x, wr, wg, wu, wd, dy, ids):
    """The layer written directly in torch (float64, CPU) with the routing
    held fixed; gradients by autograd."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)  # noqa: E731
    X, WR, WG, WU, WD = t(x), t(wr), t(wg), t(wu), t(wd)
    I = torch.tensor(np.asarray(ids, np.int64))
    logits = X @ WR.T
    g = torch.softmax(logits.gather(1, I), dim=1)
    y = torch.zeros_like(X)
    for j in range(I.shape[1]):
        e = I[:, j]
        u = torch.bmm(WG[e], X[:, :, None])[:, :, 0]
        v = torch.bmm(WU[e], X[:, :, None])[:, :, 0]
        hh = u * torch.sigmoid(u) * v
        y = y + g[:, j:j + 1] * torch.bmm(WD[e], hh[:, :, None])[:, :, 0]
    (y * torch.tensor(np.asarray(dy, np.float64))).sum().backward()
    return dict(dx=X.grad.numpy(), dw_router=WR.grad.numpy(), dw_gate=WG.grad.numpy(),
                dw_up=WU.grad.numpy(), dw_down=WD.grad.numpy())


@pytest.mark.parametrize("T,d,E,k,f,seed", [(7, 8, 4, 2, 5, 0), (9, 6, 5, 3, 4, 1), (6, 5, 3, 3, 6, 2)])
def test_layer_backward_matches_autograd(T, d, E, k, f, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) * 0.5).astype(np.float32)
    wg = (rng.standard_normal((E, f, d)) * 0.5).astype(np.float32)
    wu = (rng.standard_normal((E, f, d)) * 0.5).astype(np.float32)
    wd = (rng.standard_normal((E, d, f)) * 0.5).astype(np.float32)
    dy = rng.standard_normal((T, d))
    r = B.backward(x, k, wg, wu, wd, dy, w_router=wr)
    ref = torch_layer_grads(x, wr, wg, wu, wd, dy, r["forward"]["ids"])
    # the oracle routes on float32 logits and float32 gates (the forward's
    # definition); autograd runs on float64 throughout: agreement to that rounding
    for key in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down"):
        assert rel(r[key], ref[key]) < 2e-6, key


def test_layer_backward_is_linear_in_dy():
    p = mi.Problem(20, 16, 6, 2, 12, "f32")
    L = mi.make_layer(p, seed=5)
    rng = np.random.default_rng(6)
    dy1, dy2 = rng.standard_normal((20, 16)), rng.standard_normal((20, 16))
    args = (L["x"], p.k, L["w_gate"], L["w_up"], L["w_down"])
    r1 = B.backward(*args, dy1, w_router=L["w_router"])
    r2 = B.backward(*args, dy2, w_router=L["w_router"])
    r12 = B.backward(*args, dy1 + 2 * dy2, w_router=L["w_router"])
    for key in ("dx", "dw_gate", "dw_up", "dw_down", "dlogits", "dw_router"):
        assert rel(r12[key], r1[key] + 2 * r2[key]) < 1e-12, key


def test_single_expert_has_no_logit_gradient():
    # E = k = 1: the gate is exp(0)/exp(0) = 1 for every token, whatever the logit
    p = mi.Problem(10, 8, 1, 1, 6, "f32")
    L = mi.make_layer(p, seed=7)
    dy = np.random.default_rng(8).standard_normal((10, 8))
    r = B.backward(L["x"], 1, L["w_gate"], L["w_up"], L["w_down"], dy, w_router=L["w_router"])
    assert np.all(r["dlogits"] == 0.0) and np.all(r["dw_router"] == 0.0)
    # and the layer reduces to one SwiGLU expert on every token
    e = B.swiglu_expert_backward(L["x"], L["w_gate"][0], L["w_up"][0], L["w_down"][0], dy)
    assert rel(r["dx"], e["dx"]) < 1e-12
    assert rel(r["dw_down"][0], e["dw_down"]) < 1e-12


def test_dispatch_grad_rows():
    # queue row pos holds slot a = sorted_assign[pos]: g[a] times dy of token a // k
    rng = np.random.default_rng(9)
    T, E, k, d = 11, 5, 2, 3
    ids, gates = O.topk_route(rng.standard_normal((T, E)).astype(np.float32), k)
    q = O.dispatch(ids, E)
    dy = rng.standard_normal((T, d))
    dyp = B.dispatch_grad(dy, gates, q["sorted_assign"], k)
    for t in range(T):
        for j in range(k):
            pos = q["assign_pos"][t * k + j]
            assert np.array_equal(dyp[pos], np.float64(gates[t, j]) * dy[t])


def test_sampled_backward_functions_match_the_whole_backward():
    # the per-token and per-entry statements agree with the queue-based
    # backward (itself pinned by autograd and finite differences above)
    p = mi.Problem(40, 16, 5, 2, 12, "f32")
    L = mi.make_layer(p, seed=12)
    dy = np.random.default_rng(13).standard_normal((40, 16))
    r = B.backward(L["x"], p.k, L["w_gate"], L["w_up"], L["w_down"], dy, w_router=L["w_router"])
    l = r["forward"]["logits"]
    tok = np.array([0, 7, 21, 39])
    s = B.backward_tokens(tok, L["x"], l, p.k, L["w_gate"], L["w_up"], L["w_down"], dy, w_router=L["w_router"])
    assert rel(s["dx"], r["dx"][tok]) < 1e-12
    assert rel(s["dlogits"], r["dlogits"][tok]) < 1e-12
    ids, gates = r["forward"]["ids"], r["forward"]["gates"]
    rows, cols = np.array([1, 5, 15]), np.array([0, 3, 11])
    for e in range(p.E):
        w = B.weight_grad_entries(L["x"], ids, gates, e, L["w_gate"][e], L["w_up"][e], L["w_down"][e], dy,
                                  rows, cols)
        assert np.allclose(w["dw_down"], r["dw_down"][e][np.ix_(rows, cols)], rtol=1e-12, atol=1e-14)
        assert np.allclose(w["dw_gate"], r["dw_gate"][e][cols], rtol=1e-12, atol=1e-14)
        assert np.allclose(w["dw_up"], r["dw_up"][e][cols], rtol=1e-12, atol=1e-14)
