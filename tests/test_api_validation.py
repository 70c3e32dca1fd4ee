"""The torch binding checks every tensor argument against the problem before
anything reaches the C ABI, which sees only pointers and sizes.

Runs on the CPU with tensors on torch's ``meta`` device (shapes and dtypes,
no storage): a call whose tensors all agree passes every check and stops only
at the binding's refusal of non-GPU memory; a call with one tensor of the
wrong shape, dtype or device stops earlier, at a ValueError that names that
tensor.  No kernel is launched in either case."""
import pytest
import torch

import mixture_experts_layer_exclusive_amd as moe

META = "meta"
BF = torch.bfloat16
NOT_ON_GPU = "live on the GPU"

T, d, E, k, f = 48, 128, 8, 2, 192


def t(*shape, dtype=BF, device=META):
    return torch.empty(*shape, dtype=dtype, device=device)


def layer():
    return dict(x=t(T, d), w_gate=t(E, f, d), w_up=t(E, f, d), w_down=t(E, d, f), w_router=t(E, d),
                logits=t(T, E, dtype=torch.float32))


def state():
    n = T * k
    return dict(topk_ids=t(T, k, dtype=torch.int32), topk_gates=t(T, k, dtype=torch.float32),
                offsets=t(E + 1, dtype=torch.int32), sorted_assign=t(n, dtype=torch.int32),
                assign_pos=t(n, dtype=torch.int32), y_perm=t(n, d))


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


# ---- forward ----------------------------------------------------------------

def call_forward(**over):
    a = layer()
    a.update(over)
    return moe.forward(a["x"], a["w_gate"], a["w_up"], a["w_down"], k, w_router=a["w_router"],
                       logits=a.get("logits_in"), y=a.get("y"))


def test_forward_consistent_arguments_reach_the_device_check():
    raises(call_forward, NOT_ON_GPU)


@pytest.mark.parametrize("over,name", [
    (dict(w_up=t(E, f, d + 64)), "w_up"),
    (dict(w_down=t(E, f, d)), "w_down"),             # [E, f, d] instead of [E, d, f]
    (dict(w_gate=t(E, f, d, dtype=torch.float32)), "w_gate"),
    (dict(w_router=t(E + 1, d)), "w_router"),
    (dict(w_router=t(E, d, dtype=torch.float32)), "w_router"),
    (dict(logits_in=t(T, E + 1, dtype=torch.float32)), "logits"),
    (dict(logits_in=t(T, E)), "logits"),             # bf16 logits
    (dict(y=t(T - 1, d)), "y"),
    (dict(w_up=t(E, f, d, device="cpu")), "w_up"),   # another device
])
def test_forward_rejects_mismatched_tensor(over, name):
    raises(lambda: call_forward(**over), name)


def test_forward_needs_router_or_logits():
    a = layer()
    raises(lambda: moe.forward(a["x"], a["w_gate"], a["w_up"], a["w_down"], k), "w_router or logits")


def test_forward_rejects_non_float_activations():
    a = layer()
    raises(lambda: moe.forward(t(T, d, dtype=torch.float16), a["w_gate"], a["w_up"], a["w_down"], k,
                               w_router=a["w_router"]), "float32 or bfloat16")


# ---- route, dispatch, expert FFN, combine -----------------------------------

def test_route_checks():
    a = layer()
    raises(lambda: moe.route(k, x=a["x"], w_router=a["w_router"]), NOT_ON_GPU)
    raises(lambda: moe.route(k, logits=a["logits"]), NOT_ON_GPU)
    raises(lambda: moe.route(k, x=a["x"], w_router=t(E, d + 64)), "w_router")
    raises(lambda: moe.route(k, logits=a["logits"], ids=t(T, k + 1, dtype=torch.int32)), "ids")
    raises(lambda: moe.route(k, logits=a["logits"], gates=t(T, k)), "gates")
    raises(lambda: moe.route(k, x=a["x"], w_router=a["w_router"], logits_out=t(T, E)), "logits_out")
    raises(lambda: moe.route(k, logits=t(T, E)), "logits")


def test_dispatch_checks():
    a = layer()
    ids = t(T, k, dtype=torch.int32)
    raises(lambda: moe.dispatch(ids, E, x=a["x"], with_x_perm=True), NOT_ON_GPU)
    raises(lambda: moe.dispatch(t(T, k, dtype=torch.int64), E), "topk_ids")
    raises(lambda: moe.dispatch(ids, E, with_x_perm=True), "needs x")
    raises(lambda: moe.dispatch(ids, E, x=t(T + 1, d), with_x_perm=True), "x")
    raises(lambda: moe.dispatch(ids, E, out=dict(offsets=t(E, dtype=torch.int32))), "offsets")
    raises(lambda: moe.dispatch(ids, E, out=dict(counts=t(E + 1, dtype=torch.int32))), "counts")
    raises(lambda: moe.dispatch(ids, E, out=dict(sorted_assign=t(T, dtype=torch.int32))), "sorted_assign")
    raises(lambda: moe.dispatch(ids, E, out=dict(assign_pos=t(T * k))), "assign_pos")
    raises(lambda: moe.dispatch(ids, E, x=a["x"], with_x_perm=True, out=dict(x_perm=t(T * k, d + 64))),
           "x_perm")
    raises(lambda: moe.dispatch(ids, E, ws=t(1024, dtype=torch.uint8, device="cpu")), "ws")


def test_expert_ffn_checks():
    a = layer()
    st = state()
    off, sa = st["offsets"], st["sorted_assign"]

    def ffn(**over):
        b = dict(offsets=off, w_gate=a["w_gate"], w_up=a["w_up"], w_down=a["w_down"], x=a["x"],
                 sorted_assign=sa)
        b.update(over)
        return moe.expert_ffn(b["offsets"], b["w_gate"], b["w_up"], b["w_down"], k, T, x_perm=b.get("x_perm"),
                              x=b["x"], sorted_assign=b["sorted_assign"], y_perm=b.get("y_perm"))

    raises(ffn, NOT_ON_GPU)
    raises(lambda: ffn(x=None, x_perm=t(T * k, d)), NOT_ON_GPU)
    raises(lambda: ffn(x=None, x_perm=t(T * k - 1, d)), "x_perm")
    raises(lambda: ffn(offsets=t(E, dtype=torch.int32)), "offsets")
    raises(lambda: ffn(sorted_assign=None), "sorted_assign")
    raises(lambda: ffn(sorted_assign=t(T * k - 1, dtype=torch.int32)), "sorted_assign")
    raises(lambda: ffn(w_up=t(E, f, d, dtype=torch.float32)), "w_up")
    raises(lambda: ffn(w_down=t(E, d, f + 64)), "w_down")
    raises(lambda: ffn(x=t(T, d, dtype=torch.float32)), "x")
    raises(lambda: ffn(y_perm=t(T * k, d + 64)), "y_perm")


def test_combine_checks():
    n = T * k
    yp, ap, g = t(n, d), t(n, dtype=torch.int32), t(T, k, dtype=torch.float32)
    raises(lambda: moe.combine(yp, ap, g), NOT_ON_GPU)
    raises(lambda: moe.combine(t(n + 1, d), ap, g), "y_perm")
    raises(lambda: moe.combine(yp, t(n - 1, dtype=torch.int32), g), "assign_pos")
    raises(lambda: moe.combine(yp, ap, t(T, k)), "gates")
    raises(lambda: moe.combine(yp, ap, g, y=t(T, d, dtype=torch.float32)), "y")


# ---- backward ---------------------------------------------------------------

def test_backward_checks():
    a = layer()
    wt = (t(E, f, d), t(E, d, 2 * f))
    dy = t(T, d)

    def bwd(st=None, **over):
        b = dict(x=a["x"], w_gate=a["w_gate"], w_up=a["w_up"], dy=dy, wt=wt, w_router=a["w_router"], out=None)
        b.update(over)
        return moe.backward(b["x"], b["w_gate"], b["w_up"], k, st or state(), b["dy"], b["wt"],
                            w_router=b["w_router"], out=b["out"])

    raises(bwd, NOT_ON_GPU)
    raises(lambda: bwd(dy=t(T, d + 64)), "dy")
    raises(lambda: bwd(wt=(t(E, d, f), wt[1])), "w_down_t")
    raises(lambda: bwd(wt=(wt[0], t(E, d, f))), "w_gu_t")
    raises(lambda: bwd(w_router=t(E, d + 64)), "w_router")
    for key, bad in (("offsets", t(E, dtype=torch.int32)), ("y_perm", t(T * k, d, dtype=torch.float32)),
                     ("topk_gates", t(T, k)), ("assign_pos", None)):
        st = state()
        st[key] = bad
        raises(lambda: bwd(st=st), key)
    raises(lambda: bwd(out=dict(dw_down=t(E, f, d))), "dw_down")
    raises(lambda: bwd(out=dict(dlogits=t(T, E))), "dlogits")


def test_backward_weights_checks():
    a = layer()
    raises(lambda: moe.backward_weights(a["w_gate"], a["w_up"], a["w_down"]), NOT_ON_GPU)
    raises(lambda: moe.backward_weights(a["w_gate"], a["w_up"], t(E, f, d)), "w_down")
    raises(lambda: moe.backward_weights(a["w_gate"], a["w_up"], a["w_down"], w_gu_t=t(E, 2 * f, d)), "w_gu_t")


# ---- fp8 --------------------------------------------------------------------

def test_fp8_checks():
    a = layer()
    u8 = torch.uint8
    raises(lambda: moe.quantize_rows_fp8(t(16, 128)), NOT_ON_GPU)
    raises(lambda: moe.quantize_rows_fp8(t(16, 128, dtype=torch.float32)), "src")
    raises(lambda: moe.quantize_rows_fp8(t(16, 128), codes=t(16, 64, dtype=u8)), "codes")
    raises(lambda: moe.quantize_rows_fp8(t(16, 128), exps=t(15, dtype=torch.int32)), "exps")
    raises(lambda: moe.quantize_weights_fp8(a["w_gate"], a["w_up"], a["w_down"]), NOT_ON_GPU)
    raises(lambda: moe.quantize_weights_fp8(a["w_gate"], a["w_up"], t(E, f, d)), "w_down")
    wq = dict(w_gate=t(E, f, d, dtype=u8), w_gate_exp=t(E, f, dtype=torch.int32), w_up=t(E, f, d, dtype=u8),
              w_up_exp=t(E, f, dtype=torch.int32), w_down=t(E, d, f, dtype=u8), w_down_exp=t(E, d, dtype=torch.int32))
    st = state()
    raises(lambda: moe.expert_ffn_fp8(st["offsets"], wq, k, a["x"], st["sorted_assign"]), NOT_ON_GPU)
    bad = dict(wq, w_down_exp=t(E, f, dtype=torch.int32))
    raises(lambda: moe.expert_ffn_fp8(st["offsets"], bad, k, a["x"], st["sorted_assign"]), "w_down_exp")
    bad = dict(wq, w_up=t(E, f, d))
    raises(lambda: moe.expert_ffn_fp8(st["offsets"], bad, k, a["x"], st["sorted_assign"]), "w_up")
    raises(lambda: moe.expert_ffn_fp8(st["offsets"], wq, k, a["x"], t(T, dtype=torch.int32)), "sorted_assign")
