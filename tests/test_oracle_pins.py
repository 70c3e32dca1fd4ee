"""Pins of the CPU oracle against things other than itself.

Each oracle function is checked against at least one of: a pure-Python
brute force written from the definition on tiny inputs, a library routine
for a special case, a closed form computed by hand, or an invariant of the
layer.  A plausible slip in the oracle (a dropped term, a wrong sign, a
swapped index or a transposed operand) fails at least one test here.
"""
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as O


# --------------------------------------------------------------------------
# pure-Python brute force (no numpy arithmetic, no oracle code)
# --------------------------------------------------------------------------

def bf_select(row, k):
    """k largest of a list of floats by repeated scan; ties go to the lower
    index because only a strictly larger value replaces the running best."""
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


def bf_gates(row, chosen):
    """Full softmax over all experts, then restricted and renormalised."""
    m = max(row)
    p = [math.exp(v - m) for v in row]
    s = sum(p)
    probs = [q / s for q in p]
    sel = [probs[e] for e in chosen]
    z = sum(sel)
    return [q / z for q in sel]


def bf_expert(xrow, wg, wu, wd):
    f = len(wg)
    d = len(xrow)
    h = []
    for i in range(f):
        u = sum(float(xrow[c]) * float(wg[i][c]) for c in range(d))
        v = sum(float(xrow[c]) * float(wu[i][c]) for c in range(d))
        h.append(u * (1.0 / (1.0 + math.exp(-u))) * v)
    return [sum(h[i] * float(wd[o][i]) for i in range(f)) for o in range(d)]


def bf_layer(x, wr, wg, wu, wd, k):
    T, d = len(x), len(x[0])
    E = len(wr)
    logits = []
    ys = []
    ids_all = []
    for t in range(T):
        row = [sum(float(x[t][c]) * float(wr[e][c]) for c in range(d)) for e in range(E)]
        row = [float(np.float32(v)) for v in row]  # routing is defined on fp32 logits
        logits.append(row)
        chosen = bf_select(row, k)
        # gates are a float32 output of routing; the combine uses those values
        g = [float(np.float32(v)) for v in bf_gates(row, chosen)]
        y = [0.0] * d
        for j, e in enumerate(chosen):
            ye = bf_expert(x[t], wg[e], wu[e], wd[e])
            for o in range(d):
                y[o] += g[j] * ye[o]
        ys.append(y)
        ids_all.append(chosen)
    return logits, ids_all, ys


def tiny(T=7, d=5, E=4, k=2, f=3, seed=3):
    p = mi.Problem(T, d, E, k, f, "f32")
    L = mi.make_layer(p, seed)
    # scale the router so that routing is not near-uniform
    L["w_router"] = (L["w_router"] * np.float32(50.0)).astype(np.float32)
    return p, L


# --------------------------------------------------------------------------
# P8: whole layer against the brute force on tiny inputs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(7, 5, 4, 2, 3), (6, 3, 5, 3, 4), (4, 6, 3, 1, 2), (5, 4, 4, 4, 5), (3, 2, 1, 1, 3)])
def test_layer_matches_bruteforce(shape):
    T, d, E, k, f = shape
    p, L = tiny(T, d, E, k, f, seed=sum(shape))
    x, wr, wg, wu, wd = (L[n] for n in ("x", "w_router", "w_gate", "w_up", "w_down"))
    bl, bids, by = bf_layer(x.tolist(), wr.tolist(), wg.tolist(), wu.tolist(), wd.tolist(), k)
    out = O.forward(x, k, wg, wu, wd, w_router=wr)
    assert np.array_equal(out["logits"], np.array(bl, dtype=np.float32))
    assert out["ids"].tolist() == bids
    by = np.array(by)
    assert np.max(np.abs(out["y"] - by)) <= 1e-12 * max(1.0, np.max(np.abs(by)))
    # sampled per-token form agrees with the queue form
    tok = np.arange(T)[::2]
    ft = O.forward_tokens(tok, x, out["logits"], k, wg, wu, wd)
    assert np.max(np.abs(ft["y"] - out["y"][tok])) <= 1e-12 * max(1.0, np.max(np.abs(by)))


def test_router_logits_bruteforce():
    p, L = tiny(9, 6, 5, 2, 3)
    x, wr = L["x"], L["w_router"]
    ref = [[float(np.float32(sum(float(x[t, c]) * float(wr[e, c]) for c in range(6)))) for e in range(5)] for t in range(9)]
    assert np.array_equal(O.router_logits(x, wr), np.array(ref, dtype=np.float32))


def test_router_logits_not_transposed():
    # a non-square case where x @ W (instead of x @ W^T) would not even fit
    x = np.arange(6, dtype=np.float32).reshape(2, 3)
    w = np.array([[1, 0, 0], [0, 0, 2], [1, 1, 1], [0, 1, 0]], dtype=np.float32)
    assert O.router_logits(x, w).tolist() == [[0, 4, 3, 1], [3, 10, 12, 4]]


# --------------------------------------------------------------------------
# P1/P2: selection and gates
# --------------------------------------------------------------------------

def test_hand_worked_gates():
    # logits (ln 3, 0, -5): top-2 is experts 0, 1 with gates 3/4, 1/4
    l = np.array([[math.log(3.0), 0.0, -5.0]], dtype=np.float32)
    ids, g = O.topk_route(l, 2)
    assert ids.tolist() == [[0, 1]]
    assert abs(float(g[0, 0]) - 0.75) < 1e-7 and abs(float(g[0, 1]) - 0.25) < 1e-7
    # descending slot order is by logit, not by expert id
    l = np.array([[-1.0, 2.0, 0.5, 3.0]], dtype=np.float32)
    ids, g = O.topk_route(l, 3)
    assert ids.tolist() == [[3, 1, 2]]
    e = [math.exp(0.0), math.exp(-1.0), math.exp(-2.5)]
    s = sum(e)
    assert np.allclose(g[0], [v / s for v in e], rtol=0, atol=1e-7)


def test_gates_shift_invariant_and_finite_for_large_logits():
    # adding a constant to every logit of a token changes neither the choice
    # nor the gates; the closed form for a gap of 1 is 1/(1+e^-1), e^-1/(1+e^-1)
    l = np.array([[1000.0, 999.0, -3.0], [-1000.0, -999.0, -2000.0]], dtype=np.float32)
    ids, g = O.topk_route(l, 2)
    assert ids.tolist() == [[0, 1], [1, 0]]
    a = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(g, [[a, 1 - a], [a, 1 - a]], rtol=0, atol=1e-7)


def test_k1_gate_is_exactly_one():
    p = mi.Problem(50, 4, 6, 1, 2, "f32")
    ids, g = O.topk_route(mi.make_gaussian_logits(p, 1), 1)
    assert np.all(g == np.float32(1.0))


def test_ties_lowest_id_and_signed_zero():
    l = np.zeros((3, 5), dtype=np.float32)
    l[1] = [-0.0, 0.0, -0.0, 0.0, -0.0]
    l[2] = [1.0, 2.0, 2.0, 1.0, 2.0]
    ids, g = O.topk_route(l, 3)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2], [1, 2, 4]]
    assert np.all(np.abs(g - np.float32(1 / 3)) < 1e-7)


def test_selection_bruteforce_tie_heavy():
    p = mi.Problem(300, 4, 9, 4, 2, "f32")
    l = mi.make_tie_logits(p, 5, step=0.5)
    ids, g = O.topk_route(l, p.k)
    for t in range(p.T):
        row = l[t].tolist()
        assert ids[t].tolist() == bf_select(row, p.k)
        bg = bf_gates(row, bf_select(row, p.k))
        assert max(abs(a - b) for a, b in zip(g[t].tolist(), bg)) < 2e-7


def test_k_equals_E_is_full_order_and_gates_are_softmax():
    p = mi.Problem(40, 4, 7, 7, 2, "f32")
    l = mi.make_gaussian_logits(p, 2)
    ids, g = O.topk_route(l, 7)
    # every expert exactly once; library softmax over all experts
    assert all(sorted(r) == list(range(7)) for r in ids.tolist())
    sm = torch.softmax(torch.from_numpy(l).double(), dim=1).numpy()
    assert np.max(np.abs(g - np.take_along_axis(sm, ids.astype(np.int64), 1))) < 1e-7


def test_gate_invariants():
    for seed, (E, k) in enumerate([(8, 2), (64, 6), (128, 8)]):
        p = mi.Problem(500, 4, E, k, 2, "f32")
        ids, g = O.topk_route(mi.make_gaussian_logits(p, seed), k)
        s = g.astype(np.float64).sum(1)
        assert np.max(np.abs(s - 1.0)) <= k * 2.0 ** -24 * 2
        assert np.all(np.diff(g, axis=1) <= 0)  # non-increasing over slots
        assert np.all((ids >= 0) & (ids < E))
        assert all(len(set(r)) == k for r in ids.tolist())


# --------------------------------------------------------------------------
# P3-P6: dispatch queues
# --------------------------------------------------------------------------

@pytest.mark.parametrize("E,k,T", [(8, 2, 256), (64, 6, 333), (128, 8, 200), (1, 1, 17), (5, 5, 9)])
def test_dispatch_against_library_routines(E, k, T):
    p = mi.Problem(T, 4, E, k, 2, "f32")
    ids, _ = O.topk_route(mi.make_tie_logits(p, E + k), k)
    q = O.dispatch(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(q["counts"], np.bincount(flat, minlength=E))
    assert int(q["counts"].sum()) == T * k
    assert q["offsets"][0] == 0 and q["offsets"][-1] == T * k
    assert np.array_equal(np.diff(q["offsets"]), q["counts"])
    # stable counting sort == Python's stable sort by expert id
    assert q["sorted_assign"].tolist() == sorted(range(T * k), key=flat.__getitem__)
    sa, ap = q["sorted_assign"], q["assign_pos"]
    assert np.array_equal(ap[sa], np.arange(T * k))
    assert np.array_equal(np.sort(sa), np.arange(T * k))
    for e in range(E):
        seg = sa[q["offsets"][e]:q["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)  # tokens strictly increase in a queue


def test_dispatch_hand_worked():
    ids = np.array([[2, 0], [0, 1], [2, 1]], dtype=np.int32)  # a = 0..5
    q = O.dispatch(ids, 4)
    assert q["counts"].tolist() == [2, 2, 2, 0]
    assert q["offsets"].tolist() == [0, 2, 4, 6, 6]
    assert q["sorted_assign"].tolist() == [1, 2, 3, 5, 0, 4]
    assert q["assign_pos"].tolist() == [4, 0, 1, 2, 5, 3]


def test_gather_rows_bitwise():
    x = mi.make_x(mi.Problem(6, 8, 3, 2, 2, "bf16"), 0)
    ids = np.array([[2, 0], [0, 1], [2, 1], [1, 0], [2, 0], [1, 2]], dtype=np.int32)
    q = O.dispatch(ids, 3)
    xp = O.gather_rows(x, q["sorted_assign"], 2)
    for pos, a in enumerate(q["sorted_assign"].tolist()):
        assert xp[pos].tobytes() == x[a // 2].tobytes()


def test_zipf_skew_histogram():
    p = mi.Problem(65536, 8, 128, 8, 2, "f32")
    ids, _ = O.topk_route(mi.make_zipf_logits(p, 0), 8)
    counts = O.expert_histogram(ids, 128)
    assert counts.sum() == p.T * p.k
    assert counts.max() <= p.T  # an expert takes each token at most once
    assert counts[0] == counts.max() and counts.max() > 0.12 * p.T * p.k
    assert (counts == 0).sum() > 40  # many experts receive nothing
    w = np.arange(1, 129, dtype=np.float64) ** -1.2
    assert abs(w[0] / w.sum() - 0.27) < 0.01  # Zipf weight of rank 1


# --------------------------------------------------------------------------
# P7: FFN and combine
# --------------------------------------------------------------------------

def dense_swiglu_torch(x, wg, wu, wd):
    """Dense SwiGLU FFN with torch's own silu, float64 on the CPU."""
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    u = xt @ torch.from_numpy(np.asarray(wg, np.float64)).T
    v = xt @ torch.from_numpy(np.asarray(wu, np.float64)).T
    return (torch.nn.functional.silu(u) * v @ torch.from_numpy(np.asarray(wd, np.float64)).T).numpy()


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3), (1, 1), (4, 4)])
def test_identical_experts_equal_dense_ffn(E, k):
    p = mi.Problem(64, 24, E, k, 40, "f32")
    L = mi.make_layer(p, 11)
    wg = np.repeat(L["w_gate"][:1], E, 0)
    wu = np.repeat(L["w_up"][:1], E, 0)
    wd = np.repeat(L["w_down"][:1], E, 0)
    out = O.forward(L["x"], k, wg, wu, wd, w_router=L["w_router"])
    ref = dense_swiglu_torch(L["x"], wg[0], wu[0], wd[0])
    assert np.max(np.abs(out["y"] - ref)) <= 8 * k * 2.0 ** -24 * np.max(np.abs(ref))


def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([math.log(3)]))[0] - 0.75 * math.log(3)) < 1e-15
    assert abs(O.silu(np.array([-math.log(3)]))[0] + 0.25 * math.log(3)) < 1e-15


def test_down_projection_is_linear_and_oriented():
    p = mi.Problem(10, 6, 3, 2, 9, "f32")  # d != f catches a transposed operand
    L = mi.make_layer(p, 4)
    a = O.forward(L["x"], 2, L["w_gate"], L["w_up"], L["w_down"], w_router=L["w_router"])
    b = O.forward(L["x"], 2, L["w_gate"], L["w_up"], 2 * L["w_down"], w_router=L["w_router"])
    assert np.allclose(b["y"], 2 * a["y"], rtol=1e-14, atol=0)
    assert a["y"].shape == (10, 6) and a["y_perm"].shape == (20, 6)


def test_combine_bruteforce():
    rng = np.random.default_rng(7)
    T, k, d = 9, 3, 5
    yp = rng.standard_normal((T * k, d))
    ap = rng.permutation(T * k).astype(np.int32)
    g = rng.random((T, k)).astype(np.float32)
    y = O.combine(yp, ap, g)
    for t in range(T):
        for o in range(d):
            ref = sum(float(g[t, j]) * yp[ap[t * k + j], o] for j in range(k))
            assert abs(y[t, o] - ref) < 1e-13


def test_expert_relabeling_invariance():
    p = mi.Problem(30, 8, 6, 2, 5, "f32")
    L = mi.make_layer(p, 9)
    l = mi.make_gaussian_logits(p, 9)
    a = O.forward(L["x"], 2, L["w_gate"], L["w_up"], L["w_down"], logits=l)
    perm = np.array([3, 0, 5, 1, 4, 2])
    inv = np.argsort(perm)
    # expert e is now called inv[e]: permute logit columns and weights alike
    b = O.forward(L["x"], 2, L["w_gate"][perm], L["w_up"][perm], L["w_down"][perm], logits=l[:, perm])
    assert np.array_equal(inv[b["ids"]], a["ids"]) or np.array_equal(perm[b["ids"]], a["ids"])
    assert np.max(np.abs(a["y"] - b["y"])) < 1e-12


def test_token_batch_invariance():
    p = mi.Problem(40, 8, 5, 2, 6, "f32")
    L = mi.make_layer(p, 12)
    full = O.forward(L["x"], 2, L["w_gate"], L["w_up"], L["w_down"], w_router=L["w_router"])
    part = O.forward(L["x"][10:25], 2, L["w_gate"], L["w_up"], L["w_down"], w_router=L["w_router"])
    assert np.max(np.abs(full["y"][10:25] - part["y"])) < 1e-12


# --------------------------------------------------------------------------
# the input generator
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    v = mi.standard_normal_f32(0, 99, 100000) * np.float32(3.7)
    v[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 65504.0]  # exact ties
    ours = mi.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = mi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_chunked():
    a = mi.standard_normal_f32(1, 2, mi.CHUNK + 1000)
    b = mi.standard_normal_f32(1, 2, mi.CHUNK + 1000)
    assert np.array_equal(a, b)
    c = np.random.default_rng([1, 2, 1]).standard_normal(1000, dtype=np.float32)
    assert np.array_equal(a[mi.CHUNK:], c)
    p = mi.Problem(64, 128, 8, 2, 256, "bf16")
    x = mi.make_x(p, 0)
    assert x.dtype == np.uint16 and x.shape == (64, 128)
    s = mi.as_f32(mi.make_expert_weights(p, 0)[0], "bf16").std()
    assert abs(s - 1 / math.sqrt(128)) < 0.01
