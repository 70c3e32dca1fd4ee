"""Parity of the HIP backward against the CPU oracle (``oracle.backward``,
float64), element by element.

The forward runs on the GPU (its state feeds the backward); the oracle runs
the whole layer in float64 from the same bf16 inputs.  Routing is held
identical by supplying logits: either seeded ones, or, with the router on
the GPU, the GPU's own logits handed to the oracle (the router's gradient
then still flows through W_r in both).  The HIP path stores every
intermediate (dh, du|dv, g h, dx_perm) in bf16 with fp32 accumulation,
so each gradient must agree with the oracle within
max|err| / max|ref| <= 1e-2, the bf16 tolerance of the forward tests;
the weight layouts of the backward are bit-exact transposes.
Outputs are poisoned before each call so that an unwritten element fails.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as O
import mixture_experts_layer_exclusive_amd as moe
from oracle import moe_backward as B
from routing_helpers import exact_count_logits

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("poison_workspaces")]
DEV = "cuda:0"
TOL = 1e-2


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def poisoned_outputs(p, router):
    nan = float("nan")
    bf = torch.bfloat16
    out = dict(dx=torch.full((p.T, p.d), nan, dtype=bf, device=DEV),
               dw_gate=torch.full((p.E, p.f, p.d), nan, dtype=bf, device=DEV),
               dw_up=torch.full((p.E, p.f, p.d), nan, dtype=bf, device=DEV),
               dw_down=torch.full((p.E, p.d, p.f), nan, dtype=bf, device=DEV),
               dlogits=torch.full((p.T, p.E), nan, dtype=torch.float32, device=DEV))
    if router:
        out["dw_router"] = torch.full((p.E, p.d), nan, dtype=bf, device=DEV)
    return out


def run_layer(L, dy, logits=None):
    """GPU forward (router unless logits are given), then the backward."""
    p = L["problem"]
    x = dev(L["x"])
    wg, wu, wd = dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"])
    wr = dev(L["w_router"]) if logits is None else None
    _, st = moe.forward(x, wg, wu, wd, p.k, w_router=wr, logits=None if logits is None else dev(logits),
                        intermediates=True)
    wt = moe.backward_weights(wg, wu, wd)
    g = moe.backward(x, wg, wu, p.k, st, dev(dy), wt, w_router=wr, with_dlogits=True,
                     out=poisoned_outputs(p, wr is not None))
    torch.cuda.synchronize()
    return st, g


def oracle_grads(L, dy, logits, router):
    f = lambda n: mi.as_f32(L[n], "bf16")  # noqa: E731
    return O.backward(f("x"), L["problem"].k, f("w_gate"), f("w_up"), f("w_down"), mi.as_f32(dy, "bf16"),
                      w_router=f("w_router") if router else None, logits=logits)


def check(g, ref, router):
    for key in ("dx", "dw_gate", "dw_up", "dw_down", "dlogits") + (("dw_router",) if router else ()):
        r = rel(host(g[key]), ref[key])
        assert r <= TOL, (key, r)


BWD_CASES = [
    # T, d, E, k, f, logits
    (600, 256, 8, 2, 512, "gauss"),
    (1000, 192, 16, 4, 320, "zipf"),     # skewed: empty and tiny experts; column tails
    (333, 128, 64, 6, 192, "gauss"),     # many experts with a few rows each
    (64, 128, 128, 8, 64, "gauss"),
    (1, 64, 8, 2, 64, "gauss"),          # one token
    (70, 64, 1, 1, 128, "gauss"),        # one expert: the gate is 1, no logit gradient
    (700, 320, 8, 2, 1088, "gauss"),     # K of the weight GEMMs spans several slices and a padded tail
    (160, 64, 256, 32, 128, "gauss"),    # the largest E and k: 256 experts, padded queues of 64
]


@pytest.mark.parametrize("T,d,E,k,f,kind", BWD_CASES)
def test_backward_supplied_logits(T, d, E, k, f, kind):
    print(f"backward logits T={T} d={d} E={E} k={k} f={f} {kind}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    L = mi.make_layer(p, seed=T + f)
    l = mi.make_gaussian_logits(p, seed=d) if kind == "gauss" else mi.make_zipf_logits(p, seed=d)
    dy = mi.make_grad_output(p, seed=T)
    _, g = run_layer(L, dy, logits=l)
    ref = oracle_grads(L, dy, l, router=False)
    check(g, ref, router=False)
    if E == 1:
        assert np.all(host(g["dlogits"]) == 0.0)


@pytest.mark.parametrize("T,d,E,k,f", [(512, 256, 8, 2, 256), (300, 128, 32, 4, 192)])
def test_backward_with_router(T, d, E, k, f):
    print(f"backward router T={T} d={d} E={E} k={k} f={f}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    L = mi.make_layer(p, seed=E + f)
    dy = mi.make_grad_output(p, seed=E)
    st, g = run_layer(L, dy)
    # the oracle routes on the GPU's logits (routing on equal fp32 logits is
    # bit-exact), and the router gradient flows through W_r on both sides
    ref = oracle_grads(L, dy, host(st["logits"]), router=True)
    assert np.array_equal(host(st["topk_ids"]), ref["forward"]["ids"])
    check(g, ref, router=True)


def run_layer_supplied_with_router(L, dy, logits):
    """GPU forward on supplied logits, then the backward with the router
    weight as well (the logits stand for the router's output: routing reads
    them, the router gradient flows through W_r)."""
    p = L["problem"]
    x = dev(L["x"])
    wg, wu, wd, wr = dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]), dev(L["w_router"])
    _, st = moe.forward(x, wg, wu, wd, p.k, logits=dev(logits), intermediates=True)
    wt = moe.backward_weights(wg, wu, wd)
    g = moe.backward(x, wg, wu, p.k, st, dev(dy), wt, w_router=wr, with_dlogits=True,
                     out=poisoned_outputs(p, True))
    torch.cuda.synchronize()
    return st, g


# rows per expert around the 64-row slices of the weight-gradient GEMMs and
# the 64-row blocks of the router gradient's partial sums: empty, one row,
# one short of, at and one past a slice, and a few slices with a ragged end
EXACT_COUNTS = [0, 1, 63, 64, 65, 127, 128, 129, 191, 193, 256, 3]


def test_backward_exact_expert_counts():
    """Top-2 logits that give every expert an exact row count (EXACT_COUNTS),
    with the router gradient: the queue-order operands of the weight
    gradients end at every offset within a 64-row slice, and so do the
    64-row blocks of the router gradient's partial sums."""
    E, k, d, f = len(EXACT_COUNTS), 2, 128, 192
    T = sum(EXACT_COUNTS) // 2
    print(f"backward exact counts T={T} d={d} E={E} k={k} f={f}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    L = mi.make_layer(p, seed=11)
    logits = exact_count_logits(EXACT_COUNTS, seed=5)
    dy = mi.make_grad_output(p, seed=3)
    st, g = run_layer_supplied_with_router(L, dy, logits)
    assert np.array_equal(host(st["counts"]), np.array(EXACT_COUNTS))
    ref = oracle_grads(L, dy, logits, router=True)
    check(g, ref, router=True)
    # an expert with no rows gets exactly zero weight gradients
    for key in ("dw_gate", "dw_up", "dw_down", "dw_router"):
        assert np.all(host(g[key])[0] == 0.0), key


@pytest.mark.parametrize("T,d,E,k,f", [(400, 640, 16, 2, 128), (257, 1088, 4, 3, 64)])
def test_backward_with_router_wide_rows(T, d, E, k, f):
    """Router gradient with d above one 512-column strip of its partial-sum
    kernel, the last strip ragged (and d not a multiple of 256: the weight
    gradients' last channel range passes the end of the token-major x and
    dy rows)."""
    print(f"backward router wide T={T} d={d} E={E} k={k} f={f}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    L = mi.make_layer(p, seed=d)
    dy = mi.make_grad_output(p, seed=d)
    st, g = run_layer(L, dy)
    ref = oracle_grads(L, dy, host(st["logits"]), router=True)
    assert np.array_equal(host(st["topk_ids"]), ref["forward"]["ids"])
    check(g, ref, router=True)


def test_backward_weight_layouts_are_exact_transposes():
    p = mi.Problem(1, 192, 3, 1, 320, "bf16")
    L = mi.make_layer(p, seed=11)
    wdt, wgut = moe.backward_weights(dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]))
    torch.cuda.synchronize()
    wg, wu, wd = (mi.as_f32(L[n], "bf16") for n in ("w_gate", "w_up", "w_down"))
    assert np.array_equal(host(wdt), np.transpose(wd, (0, 2, 1)))
    assert np.array_equal(host(wgut), np.concatenate([np.transpose(wg, (0, 2, 1)),
                                                      np.transpose(wu, (0, 2, 1))], axis=2))


def test_backward_twice_is_bitwise_identical():
    p = mi.Problem(2000, 256, 16, 4, 256, "bf16")
    L = mi.make_layer(p, seed=3)
    dy = mi.make_grad_output(p, seed=3)
    _, g1 = run_layer(L, dy)
    _, g2 = run_layer(L, dy)
    for key in g1:
        assert torch.equal(g1[key], g2[key]), key


def test_backward_long_weight_gradient_k():
    """Weight gradients over long K ranges: experts of 33000 queue rows (516
    slices of 64, the last of 40 rows), 32768 rows (exactly 512 slices),
    4232 rows and none; top-1 routing on supplied logits.  Checked against
    the oracle, and bitwise on a repeat."""
    counts = [33000, 32768, 4232, 0]
    T = sum(counts)
    print(f"backward long weight-gradient K T={T} counts={counts}", flush=True)
    p = mi.Problem(T, 64, 4, 1, 128, "bf16")
    rng = np.random.default_rng(21)
    owner = rng.permutation(np.repeat(np.arange(4), counts))
    logits = (rng.standard_normal((T, 4)) * 0.5).astype(np.float32)
    logits[np.arange(T), owner] = 4.0
    L = mi.make_layer(p, seed=21)
    dy = mi.make_grad_output(p, seed=21)
    st, g = run_layer(L, dy, logits=logits)
    assert host(st["counts"]).tolist() == counts
    check(g, oracle_grads(L, dy, logits, router=False), router=False)
    _, g2 = run_layer(L, dy, logits=logits)
    for key in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert torch.equal(g[key], g2[key]), key


def test_backward_needs_only_the_routing():
    """The backward reads from the forward state only its routing: with
    y_perm left out of the state, or filled with NaN, every gradient is
    bitwise the same as with the forward's y_perm (the slot gradients come
    from the recompute)."""
    p = mi.Problem(700, 320, 16, 4, 192, "bf16")
    L = mi.make_layer(p, seed=11)
    dy = dev(mi.make_grad_output(p, seed=11))
    x = dev(L["x"])
    wg, wu, wd, wr = (dev(L[n]) for n in ("w_gate", "w_up", "w_down", "w_router"))
    _, st = moe.forward(x, wg, wu, wd, p.k, w_router=wr, intermediates=True)
    wt = moe.backward_weights(wg, wu, wd)
    ref = moe.backward(x, wg, wu, p.k, st, dy, wt, w_router=wr, with_dlogits=True)
    routing = {key: v for key, v in st.items() if key != "y_perm"}
    nan_state = dict(routing, y_perm=torch.full_like(st["y_perm"], float("nan")))
    for state in (routing, nan_state):
        g = moe.backward(x, wg, wu, p.k, state, dy, wt, w_router=wr, with_dlogits=True,
                         out=poisoned_outputs(p, True))
        torch.cuda.synchronize()
        for key in ("dx", "dw_gate", "dw_up", "dw_down", "dw_router", "dlogits"):
            assert torch.equal(g[key], ref[key]), key


def test_backward_zero_tokens_gives_zero_weight_gradients():
    p = mi.Problem(1, 128, 8, 2, 64, "bf16")
    L = mi.make_layer(p, seed=1)
    x = dev(L["x"])[:0]
    wg, wu, wd, wr = (dev(L[n]) for n in ("w_gate", "w_up", "w_down", "w_router"))
    wt = moe.backward_weights(wg, wu, wd)
    # no forward state exists for zero tokens: none is read
    st = {key: None for key in ("topk_ids", "topk_gates", "offsets", "sorted_assign", "assign_pos", "y_perm")}
    out = poisoned_outputs(mi.Problem(0, 128, 8, 2, 64, "bf16"), True)
    g = moe.backward(x, wg, wu, 2, st, x, wt, w_router=wr, out=out)
    torch.cuda.synchronize()
    for key in ("dw_gate", "dw_up", "dw_down", "dw_router"):
        assert torch.count_nonzero(g[key]) == 0, key
    assert g["dx"].shape == (0, 128)


# --------------------------------------------------------------------------
# full-size workloads: every gradient element against the oracle's whole
# backward, routed from the GPU's own logits (router workloads) or from the
# supplied ones
# --------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_8x_bf16", "deepseek_moe_bf16", "qwen3_moe_bf16", "zipf_skewed_bf16"])
def test_full_size_backward(name):
    print(f"full-size backward {name}: generating inputs", flush=True)
    L = mi.make_layer(name, seed=0)
    p = L["problem"]
    dy = mi.make_grad_output(p, seed=0)
    x = dev(L["x"])
    wg, wu, wd = dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"])
    router = L["w_router"] is not None
    wr = dev(L["w_router"]) if router else None
    lg = None if router else dev(L["logits"])
    print(f"full-size backward {name}: forward + backward", flush=True)
    _, st = moe.forward(x, wg, wu, wd, p.k, w_router=wr, logits=lg, intermediates=True)
    wt = moe.backward_weights(wg, wu, wd)
    del wd
    g = moe.backward(x, wg, wu, p.k, st, dev(dy), wt, w_router=wr, with_dlogits=True,
                     out=poisoned_outputs(p, router))
    torch.cuda.synchronize()
    del wt, wg, wu, x
    l_used = host(st["logits"]) if router else L["logits"]
    ids = host(st["topk_ids"])
    del st
    got = {key: host(v) for key, v in g.items() if v is not None}
    del g
    torch.cuda.empty_cache()

    print(f"full-size backward {name}: oracle on all {p.T} tokens", flush=True)
    ref = oracle_grads(L, dy, l_used, router)
    assert np.array_equal(ref["forward"]["ids"], ids)
    errs = {key: rel(got[key], ref[key])
            for key in ("dx", "dlogits", "dw_gate", "dw_up", "dw_down") + (("dw_router",) if router else ())}
    print(f"full-size backward {name}: max|err|/max|ref| " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()),
          flush=True)
    assert max(errs.values()) <= TOL, errs


def bwd_fuzz_cases(n=24, seed=77):
    """Seeded random backward shapes: T in [1, 400], E in {1, 2, 3, 5, 8, 16,
    64, 128}, k in [1, min(E, 8)], d and f multiples of 64 (some above one
    512-column strip of the router's partial sums, some with several 64-row
    weight-gradient slices), Gaussian, Zipf-skewed or tie-heavy supplied
    logits, or the router on the GPU."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 64, 128]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 401))
        d = int(rng.choice([64, 128, 192, 320, 576]))
        f = int(rng.choice([64, 128, 192, 320, 1088]))
        kind = str(rng.choice(["gauss", "zipf", "ties", "router"]))
        cases.append((T, d, E, k, f, kind))
    return cases


@pytest.mark.parametrize("T,d,E,k,f,kind", bwd_fuzz_cases())
def test_fuzz_backward(T, d, E, k, f, kind):
    print(f"backward fuzz T={T} d={d} E={E} k={k} f={f} {kind}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    L = mi.make_layer(p, seed=T * 7 + E)
    dy = mi.make_grad_output(p, seed=T + d)
    if kind == "router":
        st, g = run_layer(L, dy)
        ref = oracle_grads(L, dy, host(st["logits"]), router=True)
        assert np.array_equal(host(st["topk_ids"]), ref["forward"]["ids"])
        check(g, ref, router=True)
        return
    if kind == "gauss":
        logits = mi.make_gaussian_logits(p, seed=d)
    elif kind == "zipf":
        logits = mi.make_zipf_logits(p, seed=d)
    else:
        logits = mi.make_tie_logits(p, seed=d)
    _, g = run_layer(L, dy, logits=logits)
    check(g, oracle_grads(L, dy, logits, router=False), router=False)
