"""The layer under HIP graph capture: moe_forward and moe_backward issue only
kernel launches on the caller's stream (no allocation, no memset, no host
synchronisation), so a captured graph replays them.  Each replay, with eager
work of the program between replays, must equal the eager result bitwise."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_layer_exclusive_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def test_forward_and_backward_replay_in_a_graph():
    p = mi.Problem(1500, 256, 16, 4, 512, "bf16")
    L = mi.make_layer(p, seed=21)
    x, wr = dev(L["x"]), dev(L["w_router"])
    wg, wu, wd = dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"])
    dy = dev(mi.make_grad_output(p, seed=21))
    prob = moe.problem(p.T, p.d, p.E, p.k, p.f, torch.bfloat16)
    ws_f = torch.empty(moe.workspace_size(prob, 3), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(moe.workspace_size(prob, 4), dtype=torch.uint8, device=DEV)
    wt = moe.backward_weights(wg, wu, wd)
    y = torch.empty(p.T, p.d, dtype=torch.bfloat16, device=DEV)
    _, st = moe.forward(x, wg, wu, wd, p.k, w_router=wr, intermediates=True, ws=ws_f, y=y)
    grads = moe.backward(x, wg, wu, p.k, st, dy, wt, w_router=wr, ws=ws_b)
    out = {key: v for key, v in grads.items() if v is not None}
    torch.cuda.synchronize()
    y_ref = y.clone()
    g_ref = {key: v.clone() for key, v in out.items()}

    def step():
        y_, st_ = moe.forward(x, wg, wu, wd, p.k, w_router=wr, intermediates=True, ws=ws_f, y=y)
        moe.backward(x, wg, wu, p.k, st_, dy, wt, w_router=wr, ws=ws_b, out=out)
        return st_

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for it in range(3):
        y.zero_()
        for v in out.values():
            v.zero_()
        _ = (x.float() * 2).sum().item()  # eager work and a synchronisation between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), it
        for key, v in out.items():
            assert torch.equal(v, g_ref[key]), (it, key)
