"""Parity of the HIP path against the CPU oracle, element by element.

* Routing and dispatch are bit-exact when both sides route from the same
  supplied fp32 logits (ids, counts, offsets, sorted_assign, assign_pos,
  x_perm); gates within 1e-6.
* Router logits within max|dl| / max|l| <= 1e-5.
* Expert FFN, combine and the whole layer within max|dy| / max|y_ref| <=
  1e-5 (fp32) and 1e-2 (bf16), with the oracle in float64.
* With the router on the GPU, GPU and oracle logits differ by rounding, so a
  token whose k-th and (k+1)-th oracle logits lie closer than twice that
  difference may legitimately pick another expert: such tokens are checked
  for a valid choice instead of an identical one.
* Full-size workloads run in the benchmark's launch configuration and are
  checked on a seeded token sample the oracle computes one token at a time,
  plus properties that hold at any size.
Outputs are poisoned before each call so that an unwritten element fails.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as O
import mixture_experts_layer_exclusive_amd as moe

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("poison_workspaces")]
DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 1e-2}


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def poison_i32(*shape):
    return torch.full(shape, -7, dtype=torch.int32, device=DEV)


def poison_f32(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def poison(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def logits_for(p, kind, seed=0):
    if kind == "gauss":
        return mi.make_gaussian_logits(p, seed)
    if kind == "zipf":
        return mi.make_zipf_logits(p, seed)
    if kind == "ties":
        return mi.make_tie_logits(p, seed)
    raise ValueError(kind)


def f32_of(a, dtype):
    return mi.as_f32(a, dtype)


# --------------------------------------------------------------------------
# routing and dispatch: bit-exact on supplied logits
# --------------------------------------------------------------------------

ROUTE_CASES = [
    (256, 8, 2, "gauss"), (8192, 8, 2, "gauss"), (16384, 64, 6, "gauss"),
    (32768, 128, 8, "gauss"), (65536, 128, 8, "zipf"), (4099, 128, 8, "ties"),
    (1000, 256, 32, "gauss"), (333, 3, 3, "ties"), (17, 1, 1, "gauss"), (1, 64, 5, "gauss"),
    (777, 65, 7, "ties"), (2049, 200, 4, "zipf"),
    # k <= 8 runs the lane-group top-k: k = E, E not a multiple of 4 (scalar
    # loads), the largest E, and k = 1
    (4096, 8, 8, "ties"), (999, 16, 3, "ties"), (513, 255, 8, "ties"), (300, 256, 8, "zipf"),
    (100, 7, 1, "ties"), (64, 9, 9, "gauss"), (123, 5, 5, "ties"), (5000, 32, 4, "gauss"),
]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_and_dispatch_bit_exact(T, E, k, kind):
    print(f"route/dispatch T={T} E={E} k={k} {kind}", flush=True)
    p = mi.Problem(T, 64, E, k, 64, "bf16")
    l = logits_for(p, kind, seed=T + E)
    ids_ref, g_ref = O.topk_route(l, k)
    ids = poison_i32(T, k)
    gates = poison_f32(T, k)
    moe.route(k, logits=dev(l), ids=ids, gates=gates)
    torch.cuda.synchronize()
    assert np.array_equal(host(ids), ids_ref)
    assert np.max(np.abs(host(gates) - g_ref)) <= 1e-6

    q = O.dispatch(ids_ref, E)
    x = mi.make_x(p, seed=T)
    out = dict(counts=poison_i32(E), offsets=poison_i32(E + 1), sorted_assign=poison_i32(T * k),
               assign_pos=poison_i32(T * k), x_perm=poison((T * k, 64), torch.bfloat16))
    moe.dispatch(dev(ids_ref), E, x=dev(x), with_x_perm=True, out=out)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "sorted_assign", "assign_pos"):
        assert np.array_equal(host(out[key]), q[key]), key
    xp = out["x_perm"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(xp, O.gather_rows(x, q["sorted_assign"], k))


@pytest.mark.parametrize("T,E,k,with_x", [(100, 8, 2, True), (5000, 8, 2, True), (5000, 8, 2, False),
                                          (30000, 16, 2, True), (700, 40, 7, True), (10000, 128, 4, True),
                                          (1100, 200, 4, True), (1030, 256, 4, False)])
def test_dispatch_skips_ids_outside_range(T, E, k, with_x):
    """Ids outside [0, E) take no queue row (assign_pos = -1) and leave the
    other assignments' stable order as it is, on every dispatch path (one
    workgroup; histogram + scatter; histogram + one-pass scatter and gather).
    The oracle defines only valid ids, so the expectation is the counting
    sort of the valid assignments alone: pos(a) = offsets[e] + the number of
    valid a' < a with the same expert."""
    print(f"dispatch with out-of-range ids T={T} E={E} k={k} x_perm={with_x}", flush=True)
    p = mi.Problem(T, 64, E, k, 64, "bf16")
    ids, _ = O.topk_route(mi.make_gaussian_logits(p, seed=T), k)
    rng = np.random.default_rng(T)
    bad = rng.random(ids.shape) < 0.03
    ids = np.where(bad, rng.choice(np.array([-1, E, E + 7, -1000], dtype=np.int32), ids.shape), ids).astype(np.int32)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    apos = np.full(T * k, -1, dtype=np.int32)
    seen = offsets[:-1].copy()
    for a in np.nonzero(valid)[0]:
        apos[a] = seen[flat[a]]
        seen[flat[a]] += 1
    nv = int(valid.sum())
    x = mi.make_x(p, seed=1)
    out = dict(counts=poison_i32(E), offsets=poison_i32(E + 1), sorted_assign=poison_i32(T * k),
               assign_pos=poison_i32(T * k), x_perm=poison((T * k, 64), torch.bfloat16) if with_x else None)
    moe.dispatch(dev(ids), E, x=dev(x) if with_x else None, with_x_perm=with_x, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["counts"]), counts)
    assert np.array_equal(host(out["offsets"]), offsets)
    assert np.array_equal(host(out["assign_pos"]), apos)
    sa = host(out["sorted_assign"])[:nv]
    assert np.array_equal(sa, np.nonzero(valid)[0][np.argsort(apos[valid], kind="stable")])
    if with_x:
        xp = out["x_perm"].view(torch.int16).cpu().numpy().view(np.uint16)[:nv]
        assert np.array_equal(xp, np.asarray(x)[sa // k])


@pytest.mark.parametrize("T,E,k,d", [(5000, 8, 2, 64), (3000, 16, 3, 100)])
def test_dispatch_f32_rows_one_pass(T, E, k, d):
    """fp32 rows whose width is a multiple of 16 bytes take the one-pass
    scatter and gather too (the copy is of raw 16-byte words)."""
    p = mi.Problem(T, d, E, k, 64, "f32")
    ids_ref, _ = O.topk_route(mi.make_gaussian_logits(p, 4), k)
    q = O.dispatch(ids_ref, E)
    x = mi.make_x(p, 4)
    out = moe.dispatch(dev(ids_ref), E, x=dev(x), with_x_perm=True,
                       out=dict(x_perm=poison((T * k, d), torch.float32), sorted_assign=poison_i32(T * k),
                                assign_pos=poison_i32(T * k), counts=poison_i32(E), offsets=poison_i32(E + 1)))
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "sorted_assign", "assign_pos"):
        assert np.array_equal(host(out[key]), q[key]), key
    assert np.array_equal(host(out["x_perm"]).view(np.uint32), O.gather_rows(x, q["sorted_assign"], k).view(np.uint32))


def test_dispatch_f32_rows_and_odd_width():
    p = mi.Problem(300, 3, 5, 2, 7, "f32")
    ids_ref, _ = O.topk_route(mi.make_tie_logits(p, 3), 2)
    q = O.dispatch(ids_ref, 5)
    x = mi.make_x(p, 3)
    out = moe.dispatch(dev(ids_ref), 5, x=dev(x), with_x_perm=True,
                       out=dict(x_perm=poison((600, 3), torch.float32)))
    torch.cuda.synchronize()
    assert np.array_equal(host(out["sorted_assign"]), q["sorted_assign"])
    assert np.array_equal(host(out["x_perm"]).view(np.uint32), O.gather_rows(x, q["sorted_assign"], 2).view(np.uint32))


# --------------------------------------------------------------------------
# router GEMM
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,d,E,dtype", [(256, 128, 8, "f32"), (1000, 4096, 8, "bf16"),
                                         (777, 2048, 128, "bf16"), (300, 2048, 64, "bf16"),
                                         (65, 100, 7, "f32"), (129, 192, 256, "bf16"),
                                         # one and two K chunks, E past the last full block,
                                         # 5 and 7 expert blocks (K steps split over the waves)
                                         (100, 64, 3, "bf16"), (513, 128, 40, "bf16"),
                                         (260, 320, 100, "bf16"), (97, 256, 200, "bf16"),
                                         (33, 1024, 160, "bf16"), (211, 384, 96, "bf16"),
                                         (77, 192, 190, "bf16"),
                                         # 64 tokens per workgroup (128 and 256 experts): one
                                         # token, one and two K chunks on the 3-stage ring
                                         (1, 128, 128, "bf16"), (65, 64, 256, "bf16"),
                                         (190, 128, 128, "bf16")])
def test_router_logits(T, d, E, dtype):
    p = mi.Problem(T, d, E, min(2, E), 64, dtype)
    x = mi.make_x(p, 5)
    wr = mi.make_router_weight(p, 5)
    ref = O.router_logits(f32_of(x, dtype), f32_of(wr, dtype))
    lo = poison_f32(T, E)
    ids, gates, _ = moe.route(p.k, x=dev(x), w_router=dev(wr), logits_out=lo)
    torch.cuda.synchronize()
    assert rel(host(lo), ref) <= 1e-5


# --------------------------------------------------------------------------
# expert FFN and combine, from the oracle's queues
# --------------------------------------------------------------------------

FFN_CASES = [
    (2000, 192, 4, 2, 320, "bf16", "gauss"),   # column tails in both GEMMs, many row tiles
    (300, 256, 8, 2, 384, "bf16", "gauss"),
    (1500, 512, 16, 4, 256, "bf16", "zipf"),   # skewed: empty and tiny experts
    (64, 128, 128, 8, 64, "bf16", "gauss"),    # many experts, a few rows each
    (256, 128, 8, 2, 256, "f32", "gauss"),
    (200, 100, 6, 3, 70, "f32", "ties"),
    (1, 64, 8, 2, 64, "bf16", "gauss"),
    (1024, 256, 4, 2, 2048, "bf16", "gauss"),  # few tiles: the down projection splits K (S = 4)
    (700, 320, 8, 2, 1088, "bf16", "gauss"),   # uneven split ranges (17 slices), column tail
    (160, 64, 256, 32, 128, "bf16", "gauss"),  # the largest E and k: 256 experts of about 20 rows
    # long K in both GEMMs, the down projection's tail split (72 tiles: S = 3)
    (1024, 2112, 4, 2, 4096, "bf16", "gauss"),
    (600, 2176, 8, 2, 2240, "bf16", "zipf"),   # full tiles, skewed, column tails
    (900, 2048, 16, 4, 2112, "bf16", "gauss"),  # the down projection at K = 2112: 33 slices
    # pairs of column tiles: an odd number of them (the last pair has one
    # tile) and a ragged last column tile, in both GEMMs
    (700, 1216, 8, 2, 704, "bf16", "zipf"),
    (500, 1280, 16, 4, 384, "bf16", "gauss"),
]


@pytest.mark.parametrize("T,d,E,k,f,dtype,kind", FFN_CASES)
@pytest.mark.parametrize("fused_gather", [True, False])
def test_expert_ffn_and_combine(T, d, E, k, f, dtype, kind, fused_gather):
    print(f"ffn T={T} d={d} E={E} k={k} f={f} {dtype} {kind} fused={fused_gather}", flush=True)
    p = mi.Problem(T, d, E, k, f, dtype)
    L = mi.make_layer(p, seed=T + d)
    x32 = f32_of(L["x"], dtype)
    wg, wu, wd = (f32_of(L[n], dtype) for n in ("w_gate", "w_up", "w_down"))
    ids, gates = O.topk_route(logits_for(p, kind, T), k)
    q = O.dispatch(ids, E)
    yp_ref = O.expert_ffn(x32, q["sorted_assign"], q["offsets"], k, wg, wu, wd)

    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xd = dev(L["x"])
    sa = dev(q["sorted_assign"])
    offs = dev(q["offsets"])
    y_perm = poison((T * k, d), tdt)
    if fused_gather:
        moe.expert_ffn(offs, dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]), k, T, x=xd,
                       sorted_assign=sa, y_perm=y_perm)
    else:
        xp = dev(O.gather_rows(L["x"], q["sorted_assign"], k))
        moe.expert_ffn(offs, dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]), k, T, x_perm=xp,
                       y_perm=y_perm)
    torch.cuda.synchronize()
    assert rel(host(y_perm), yp_ref) <= TOL[dtype]

    # combine from the oracle's expert outputs rounded to the storage dtype
    yp_in = yp_ref.astype(np.float32)
    if dtype == "bf16":
        yp_in = mi.f32_to_bf16_bits(yp_in)
    y_ref = O.combine(f32_of(yp_in, dtype), q["assign_pos"], gates)
    y = poison((T, d), tdt)
    moe.combine(dev(yp_in), dev(q["assign_pos"]), dev(gates), y=y)
    torch.cuda.synchronize()
    assert rel(host(y), y_ref) <= (1e-6 if dtype == "f32" else 4e-3)


# rows per expert around the 256-row tiles of the grouped GEMMs: empty, one
# row, one short of, at and one past one, two and three tiles
FFN_EXACT_COUNTS = [0, 1, 255, 256, 257, 511, 512, 513, 767, 4]


@pytest.mark.parametrize("fused_gather", [True, False])
def test_expert_ffn_exact_tile_counts(fused_gather):
    from routing_helpers import exact_count_logits
    E, k, d, f = len(FFN_EXACT_COUNTS), 2, 192, 320
    T = sum(FFN_EXACT_COUNTS) // 2
    print(f"ffn exact counts T={T} d={d} E={E} k={k} f={f} fused={fused_gather}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    L = mi.make_layer(p, seed=17)
    ids, gates = O.topk_route(exact_count_logits(FFN_EXACT_COUNTS, seed=7), k)
    q = O.dispatch(ids, E)
    assert np.array_equal(q["counts"], np.array(FFN_EXACT_COUNTS))
    wg, wu, wd = (f32_of(L[n], "bf16") for n in ("w_gate", "w_up", "w_down"))
    yp_ref = O.expert_ffn(f32_of(L["x"], "bf16"), q["sorted_assign"], q["offsets"], k, wg, wu, wd)
    y_perm = poison((T * k, d), torch.bfloat16)
    if fused_gather:
        moe.expert_ffn(dev(q["offsets"]), dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]), k, T,
                       x=dev(L["x"]), sorted_assign=dev(q["sorted_assign"]), y_perm=y_perm)
    else:
        xp = dev(O.gather_rows(L["x"], q["sorted_assign"], k))
        moe.expert_ffn(dev(q["offsets"]), dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]), k, T, x_perm=xp,
                       y_perm=y_perm)
    torch.cuda.synchronize()
    assert rel(host(y_perm), yp_ref) <= TOL["bf16"]


def test_expert_ffn_gather_from_x_beyond_4gib():
    # x with 2^31 or more elements: the fused gather addresses its rows with
    # 64-bit offsets.  x repeats a seeded block of R rows, so the oracle
    # knows every row; the sample includes tokens past the 4 GiB mark.
    T, d, E, k, f, R = (1 << 31) // 4096 + 256, 4096, 4, 1, 64, 4096
    print(f"ffn beyond 4 GiB: T={T} d={d} E={E} k={k} f={f}", flush=True)
    p = mi.Problem(T, d, E, k, f, "bf16")
    block = mi.make_x(mi.Problem(R, d, E, k, f, "bf16"), seed=5)
    W = dict(zip(("w_gate", "w_up", "w_down"), mi.make_expert_weights(p, seed=5)))
    ids, _ = O.topk_route(mi.make_gaussian_logits(p, 5), k)
    q = O.dispatch(ids, E)
    xb = dev(block)
    x = xb.repeat((T + R - 1) // R, 1)[:T].contiguous()
    del xb
    y_perm = poison((T * k, d), torch.bfloat16)
    moe.expert_ffn(dev(q["offsets"]), dev(W["w_gate"]), dev(W["w_up"]), dev(W["w_down"]), k, T, x=x,
                   sorted_assign=dev(q["sorted_assign"]), y_perm=y_perm)
    torch.cuda.synchronize()
    del x
    tok = np.unique(np.concatenate([[0, R - 1, T // 2, T - 256, T - 1],
                                    mi.sample_tokens(T, 24, seed=5)]))
    assert tok.max() * d >= (1 << 31)
    wf = {n: f32_of(W[n], "bf16") for n in W}
    x32 = f32_of(block, "bf16")
    for t in tok:
        for j in range(k):
            e = int(ids[t, j])
            ref = O.swiglu_expert(x32[t % R][None], wf["w_gate"][e], wf["w_up"][e], wf["w_down"][e])[0]
            pos = int(q["assign_pos"][t * k + j])
            assert rel(host(y_perm[pos]), ref) <= TOL["bf16"], (t, j)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def run_forward(L, logits=None, k=None):
    p = L["problem"]
    y, inter = moe.forward(dev(L["x"]), dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]),
                           k or p.k, w_router=None if logits is not None else dev(L["w_router"]),
                           logits=None if logits is None else dev(logits), intermediates=True)
    torch.cuda.synchronize()
    return y, inter


@pytest.mark.parametrize("T,d,E,k,f,dtype,kind", [
    (600, 256, 8, 2, 512, "bf16", "gauss"), (1000, 128, 64, 6, 192, "bf16", "zipf"),
    (256, 128, 8, 2, 256, "f32", "ties"), (50, 64, 4, 4, 128, "bf16", "gauss"),
    (33, 64, 1, 1, 64, "bf16", "gauss"), (1, 128, 128, 8, 64, "bf16", "gauss"),
])
def test_forward_supplied_logits(T, d, E, k, f, dtype, kind):
    print(f"forward logits T={T} d={d} E={E} k={k} f={f} {dtype}", flush=True)
    p = mi.Problem(T, d, E, k, f, dtype)
    L = mi.make_layer(p, seed=d + E)
    l = logits_for(p, kind, seed=f)
    ref = O.forward(f32_of(L["x"], dtype), k, *(f32_of(L[n], dtype) for n in ("w_gate", "w_up", "w_down")),
                    logits=l)
    y, inter = run_forward(L, logits=l)
    for key, rkey in (("topk_ids", "ids"), ("counts", "counts"), ("offsets", "offsets"),
                      ("sorted_assign", "sorted_assign"), ("assign_pos", "assign_pos")):
        assert np.array_equal(host(inter[key]).reshape(ref[rkey].shape), ref[rkey]), key
    assert np.max(np.abs(host(inter["topk_gates"]) - ref["gates"])) <= 1e-6
    assert rel(host(y), ref["y"]) <= TOL[dtype]


def fuzz_cases(n=40, seed=2024):
    """Seeded random shapes: T in [1, 300], E in {1, 2, 3, 8, 64, 128},
    k in [1, min(E, 8)]; bf16 with d, f multiples of 64, fp32 with any d, f;
    Gaussian or tie-heavy supplied logits."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 8, 64, 128]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 301))
        dtype = "f32" if i % 4 == 0 else "bf16"
        if dtype == "bf16":
            d, f = int(rng.choice([64, 128, 192])), int(rng.choice([64, 128, 320]))
        else:
            d, f = int(rng.integers(1, 100)), int(rng.integers(1, 100))
        kind = "ties" if rng.random() < 0.5 else "gauss"
        cases.append((T, d, E, k, f, dtype, kind))
    return cases


@pytest.mark.parametrize("T,d,E,k,f,dtype,kind", fuzz_cases())
def test_fuzz_forward_supplied_logits(T, d, E, k, f, dtype, kind):
    test_forward_supplied_logits(T, d, E, k, f, dtype, kind)


def margins(l, k):
    """Gap between the k-th and (k+1)-th largest logit per token (inf if k == E)."""
    s = -np.sort(-l.astype(np.float64), axis=1)
    if k >= l.shape[1]:
        return np.full(l.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def check_routing_with_router(l_gpu, ids_gpu, l_ref, k):
    """Router parity, then ids equal wherever the oracle's top-k margin exceeds
    twice the logit difference; elsewhere the GPU choice must be a valid top-k
    of the oracle logits within that difference.  Returns the safe-token mask."""
    assert rel(l_gpu, l_ref) <= 1e-5
    dl = np.max(np.abs(l_gpu.astype(np.float64) - l_ref), axis=1)
    ids_ref, _ = O.topk_route(l_ref, k)
    safe = margins(l_ref, k) > 2 * dl + 1e-12
    assert np.array_equal(ids_gpu[safe], ids_ref[safe])
    kth = -np.sort(-l_ref.astype(np.float64), axis=1)[:, k - 1]
    chosen = np.take_along_axis(l_ref.astype(np.float64), ids_gpu.astype(np.int64), 1)
    assert np.all(chosen >= kth[:, None] - 2 * dl[:, None] - 1e-12)
    return safe


def test_forward_tiny_f32_with_router():
    L = mi.make_layer("tiny_f32", seed=0)
    p = L["problem"]
    ref = O.forward(L["x"], p.k, L["w_gate"], L["w_up"], L["w_down"], w_router=L["w_router"])
    y, inter = run_forward(L)
    safe = check_routing_with_router(host(inter["logits"]), host(inter["topk_ids"]), ref["logits"], p.k)
    assert safe.mean() > 0.99
    assert rel(host(y)[safe], ref["y"][safe]) <= 1e-5
    # run twice: bitwise identical
    y2, _ = run_forward(L)
    assert torch.equal(y, y2)


def test_identical_experts_give_dense_ffn():
    p = mi.Problem(512, 256, 8, 2, 384, "bf16")
    L = mi.make_layer(p, seed=2)
    for n in ("w_gate", "w_up", "w_down"):
        L[n] = np.ascontiguousarray(np.repeat(L[n][:1], p.E, 0))
    dense = O.swiglu_expert(f32_of(L["x"], "bf16"), *(f32_of(L[n][0], "bf16") for n in ("w_gate", "w_up", "w_down")))
    y, _ = run_forward(L)
    assert rel(host(y), dense) <= 1e-2


def test_forward_twice_is_bitwise_identical():
    p = mi.Problem(3000, 512, 64, 6, 256, "bf16")
    L = mi.make_layer(p, seed=4)
    y1, i1 = run_forward(L)
    y2, i2 = run_forward(L)
    assert torch.equal(y1, y2)
    for key in i1:
        assert torch.equal(i1[key], i2[key]), key


def test_zero_tokens_noop():
    p = mi.Problem(1, 128, 8, 2, 64, "bf16")
    L = mi.make_layer(p, seed=1)
    x = dev(L["x"])[:0]
    y = moe.forward(x, dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"]), 2, w_router=dev(L["w_router"]))
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


# --------------------------------------------------------------------------
# full-size workloads, in the benchmark's launch configuration
# --------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_8x_bf16", "deepseek_moe_bf16", "qwen3_moe_bf16", "zipf_skewed_bf16"])
def test_full_size_workload(name):
    """The whole layer at full size, in the benchmark's launch configuration,
    with every workspace filled with 0xFF first: routing (bit-exact on
    supplied logits, else the margin protocol), the queues (bit-exact), the
    materialised row gather x_perm at the full width (bitwise), and y for
    every token against the oracle's whole layer."""
    print(f"full-size {name}: generating inputs", flush=True)
    L = mi.make_layer(name, seed=0)
    p = L["problem"]
    dt = p.dtype
    n = p.T * p.k
    xg = dev(L["x"])
    wg, wu, wd = dev(L["w_gate"]), dev(L["w_up"]), dev(L["w_down"])
    wr = dev(L["w_router"]) if L["w_router"] is not None else None
    lg = dev(L["logits"]) if L["logits"] is not None else None
    prob = moe.problem(p.T, p.d, p.E, p.k, p.f, torch.bfloat16)
    ws = torch.full((moe.workspace_size(prob, 3),), 0xFF, dtype=torch.uint8, device=DEV)
    y = poison((p.T, p.d), torch.bfloat16)
    print(f"full-size {name}: forward", flush=True)
    _, inter = moe.forward(xg, wg, wu, wd, p.k, w_router=wr, logits=lg, intermediates=True, ws=ws, y=y)
    torch.cuda.synchronize()
    del wg, wu, wd, ws
    ids_gpu = host(inter["topk_ids"])
    yh = host(y)
    del y
    assert np.all(np.isfinite(yh))

    # routing: exact on supplied logits, else the margin protocol over all tokens
    x32 = f32_of(L["x"], dt)
    if L["logits"] is not None:
        l_ref = L["logits"]
        ids_ref, g_ref = O.topk_route(l_ref, p.k)
        assert np.array_equal(ids_gpu, ids_ref)
        assert np.max(np.abs(host(inter["topk_gates"]) - g_ref)) <= 1e-6
        safe = np.ones(p.T, dtype=bool)
    else:
        l_ref = O.router_logits(x32, f32_of(L["w_router"], dt))
        safe = check_routing_with_router(host(inter["logits"]), ids_gpu, l_ref, p.k)
        ids_ref, _ = O.topk_route(l_ref, p.k)
    print(f"full-size {name}: {int((~safe).sum())} near-tie tokens", flush=True)
    assert (~safe).mean() < 0.01

    # dispatch: bit-exact when routing agrees everywhere, else valid for the GPU's own ids
    counts = host(inter["counts"])
    offsets = host(inter["offsets"])
    sa = host(inter["sorted_assign"])
    ap = host(inter["assign_pos"])
    if np.array_equal(ids_gpu, ids_ref):
        q = O.dispatch(ids_ref, p.E)
        for key, v in (("counts", counts), ("offsets", offsets), ("sorted_assign", sa), ("assign_pos", ap)):
            assert np.array_equal(v, q[key]), key
    else:
        flat = ids_gpu.reshape(-1)
        assert counts.sum() == n and offsets[-1] == n
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(ap[sa], np.arange(n))
        for e in range(p.E):
            seg = sa[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)

    # moe_dispatch with the row gather, as the benchmark times it: the same
    # queues, and x_perm a bitwise copy of the source rows at the full width
    print(f"full-size {name}: dispatch with x_perm", flush=True)
    dws = torch.full((max(256, moe.workspace_size(prob, 1)),), 0xFF, dtype=torch.uint8, device=DEV)
    out = dict(counts=poison_i32(p.E), offsets=poison_i32(p.E + 1), sorted_assign=poison_i32(n),
               assign_pos=poison_i32(n), x_perm=poison((n, p.d), torch.bfloat16))
    moe.dispatch(inter["topk_ids"], p.E, x=xg, with_x_perm=True, ws=dws, out=out)
    torch.cuda.synchronize()
    del xg, dws
    for key, v in (("counts", counts), ("offsets", offsets), ("sorted_assign", sa), ("assign_pos", ap)):
        assert np.array_equal(host(out[key]), v), key
    xp = out["x_perm"].view(torch.int16).cpu().numpy().view(np.uint16)
    del out
    assert np.array_equal(xp, O.gather_rows(L["x"], sa, p.k))
    del xp

    # y of every token against the oracle's whole layer, routed from the
    # oracle's logits (tokens on a near tie excluded)
    print(f"full-size {name}: oracle on all {p.T} tokens", flush=True)
    wf = {nm: f32_of(L[nm], dt) for nm in ("w_gate", "w_up", "w_down")}
    ref = O.forward(x32, p.k, wf["w_gate"], wf["w_up"], wf["w_down"], logits=l_ref)
    err = rel(yh[safe], ref["y"][safe])
    print(f"full-size {name}: max|dy|/max|y| over {int(safe.sum())} of {p.T} tokens = {err:.3e}", flush=True)
    assert err <= TOL[dt]


def test_stream_copy_is_exact():
    # the measurement copy kernel: ragged tail past the last whole 32 KB block
    import ctypes
    from mixture_experts_layer_exclusive_amd import _lib as LB
    nbytes = (3 << 20) + 16 * 777
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    st = LB.load().moe_stream_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == LB.MOE_OK
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0
