"""Pins of the fp8 oracle against what the format and the mathematics fix:

* torch's own float8_e4m3fn conversion (round to nearest even) on a sweep
  of float32 values, all the neighbour midpoints included;
* the 254 finite codes decode and re-encode to themselves, and the decoded
  values are the OCP E4M3 table (closed forms: 1.0, 448, 2^-6, 2^-9);
* a brute-force nearest-code search (ties to the even code) on random and
  boundary values;
* the power-of-two scale is the smallest that fits, by brute force;
* the fp8 FFN equals exact arithmetic when every input is already an E4M3
  value times its scale, is independent of which other tokens share the
  batch, and scales exactly with a power of two on W_down.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as O
from oracle import moe_fp8 as F

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def torch_codes(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_closed_forms():
    val = dict(zip(FINITE.tolist(), F.e4m3_decode(FINITE).tolist()))
    assert val[0x38] == 1.0 and val[0x7E] == 448.0 and val[0x08] == 2.0 ** -6
    assert val[0x01] == 2.0 ** -9 and val[0x07] == 7 * 2.0 ** -9 and val[0x00] == 0.0
    assert val[0xB8] == -1.0 and val[0xFE] == -448.0
    assert np.signbit(val[0x80])
    pos = sorted(v for c, v in val.items() if c < 0x80)
    assert len(pos) == 127 and len(set(pos)) == 127  # strictly increasing, no duplicates


def test_round_trip_every_finite_code():
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(FINITE)), FINITE)


def test_matches_torch_float8_conversion():
    pos = np.sort(F.e4m3_decode(FINITE[FINITE < 0x80]))
    mids = (pos[:-1] + pos[1:]) / 2                      # exact ties
    rng = np.random.default_rng(0)
    rand = rng.uniform(-448, 448, 20000)
    small = rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000)   # subnormal range
    v = np.concatenate([pos, -pos, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), rand, small])
    v = v.astype(np.float32).astype(np.float64)
    assert np.array_equal(F.e4m3_encode(v), torch_codes(v))


def brute_force_code(x):
    best, best_d = None, None
    for c in FINITE[FINITE < 0x80] if x >= 0 else FINITE[FINITE >= 0x80]:
        d = abs(F.e4m3_decode(np.array([c]))[0] - x)
        if best is None or d < best_d or (d == best_d and (c & 1) == 0 and (best & 1) == 1):
            best, best_d = c, d
    return best


def test_encode_is_the_nearest_code_ties_to_even():
    rng = np.random.default_rng(1)
    pos = np.sort(F.e4m3_decode(FINITE[FINITE < 0x80]))
    vals = list(rng.uniform(-448, 448, 300)) + list(rng.uniform(-0.02, 0.02, 200)) + \
        list((pos[:-1] + pos[1:]) / 2) + [448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10]
    for x in vals:
        assert F.e4m3_encode(np.array([x]))[0] == brute_force_code(x), x


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([448.5]))
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([np.nan]))


def test_pow2_scale_is_the_smallest_that_fits():
    rng = np.random.default_rng(2)
    amax = np.concatenate([np.ldexp(rng.uniform(0.5, 1, 500), rng.integers(-140, 120, 500)),
                           [448.0, 449.0, 224.0, 896.0, 897.0, 0.875, 1e-40]])
    for m in amax:
        a = F.pow2_scale_exponent(m)
        assert m <= 448.0 * 2.0 ** a and not m <= 448.0 * 2.0 ** (a - 1), m
    assert F.pow2_scale_exponent(0.0) == 0
    assert F.pow2_scale_exponent(448.0) == 0 and F.pow2_scale_exponent(449.0) == 1


def test_quantize_rows_scale_invariance():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((7, 33))
    c, e = F.quantize_rows(a)
    for j in (-5, 3, 40):
        c2, e2 = F.quantize_rows(np.ldexp(a, j))
        assert np.array_equal(c, c2) and np.array_equal(e2, e + j)
    # zero rows: exponent 0, codes 0
    c0, e0 = F.quantize_rows(np.zeros((2, 5)))
    assert np.all(c0 == 0) and np.all(e0 == 0)
    # the dequantised value is within half a code step of the input
    dq = F.dequantize_rows(c, e)
    assert np.all(np.abs(dq - a) <= np.ldexp(np.abs(a), -4) + np.ldexp(1.0, e[:, None] - 10))


def test_vector_scale_exponents_match_the_scalar_rule():
    rng = np.random.default_rng(11)
    amax = np.concatenate([[0.0, 448.0, 449.0, 2.0 ** -133, 3.0e38], np.abs(rng.standard_normal(2000)) *
                           2.0 ** rng.integers(-140, 120, 2000).astype(np.float64)])
    assert np.array_equal(F.pow2_scale_exponents(amax), [F.pow2_scale_exponent(m) for m in amax])


def test_quantize_blocks_is_the_row_rule_on_each_block():
    # every block of 32 columns (and the shorter last one) quantised as a row
    # of its own gives the same codes and exponents
    rng = np.random.default_rng(12)
    a = rng.standard_normal((9, 32 * 3 + 7)) * 2.0 ** rng.integers(-20, 20, (9, 1))
    a[2, 32:64] = 0.0                       # one all-zero block: exponent 0, codes 0
    a[4, :32] *= 2.0 ** 30                  # blocks of one row far apart in scale
    c, e = F.quantize_blocks(a)
    assert c.shape == a.shape and e.shape == (9, 4)
    for b in range(4):
        cb, eb = F.quantize_rows(a[:, 32 * b:32 * (b + 1)])
        assert np.array_equal(c[:, 32 * b:32 * (b + 1)], cb) and np.array_equal(e[:, b], eb)
    assert e[2, 1] == 0 and np.all(c[2, 32:64] == 0)
    # dequantised within half a code step of the input
    dq = F.dequantize_blocks(c, e)
    step = np.ldexp(1.0, np.repeat(e, 32, axis=1)[:, :a.shape[1]] - 10)
    assert np.all(np.abs(dq - a) <= np.ldexp(np.abs(a), -4) + step)


def test_quantize_blocks_floor_of_the_e8m0_range():
    # blocks below about 2^-118 would want an exponent under -127: they take
    # -127, and their codes are those of the values times 2^127 (0.125 is
    # E4M3 0x20, -0.0625 is 0x98, 2^-9 the smallest subnormal 0x01)
    a = np.zeros((1, 64))
    a[0, :4] = [2.0 ** -130, -(2.0 ** -131), 0.0, 2.0 ** -136]
    a[0, 32] = 1.0
    c, e = F.quantize_blocks(a)
    assert e[0, 0] == -127 and e[0, 1] == F.pow2_scale_exponent(1.0) == -8
    assert list(c[0, :4]) == [0x20, 0x98, 0x00, 0x01]
    assert np.array_equal(F.e4m3_decode(c[0, :4]) * 2.0 ** -127, a[0, :4])


def test_round_bf16_matches_torch():
    v = np.random.default_rng(4).standard_normal(5000) * 10.0 ** np.random.default_rng(5).integers(-5, 5, 5000)
    ref = torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.array_equal(F.round_bf16(v), ref)


def representable_layer(seed, T=12, d=32, E=3, k=2, f=24):
    """Inputs whose rows are already E4M3 codes times a power of two."""
    rng = np.random.default_rng(seed)
    codes = lambda *s: FINITE[FINITE != 0x80][rng.integers(0, 253, s)]  # noqa: E731
    x = F.e4m3_decode(codes(T, d)) * 2.0 ** -4
    wg = F.e4m3_decode(codes(E, f, d)) * 2.0 ** -9
    wu = F.e4m3_decode(codes(E, f, d)) * 2.0 ** -9
    wd = F.e4m3_decode(codes(E, d, f)) * 2.0 ** -9
    ids, _ = O.topk_route(rng.standard_normal((T, E)).astype(np.float32), k)
    return x, wg, wu, wd, O.dispatch(ids, E)


def test_fp8_ffn_is_exact_on_representable_inputs():
    x, wg, wu, wd, q = representable_layer(6)
    r = F.fp8_expert_ffn(x, q["sorted_assign"], q["offsets"], 2, wg, wu, wd)
    # GEMM1 sees its inputs unchanged: h is the exact SwiGLU rounded to bf16
    sa, off = q["sorted_assign"], q["offsets"]
    for e in range(3):
        lo, hi = off[e], off[e + 1]
        xr = x[sa[lo:hi] // 2]
        h = F.round_bf16(O.silu(xr @ wg[e].T) * (xr @ wu[e].T))
        assert np.array_equal(r["h"][lo:hi], h)
        # and GEMM2 is exact on the quantised h
        hq = F.dequantize_blocks(r["h_codes"][lo:hi], r["h_exp"][lo:hi])
        assert np.allclose(r["y_perm"][lo:hi], hq @ wd[e].T, rtol=1e-14, atol=0)
    # every x code equals the input's own code (no rounding happened)
    assert np.array_equal(F.dequantize_rows(r["x_codes"], r["x_exp"]), x)


def test_fp8_ffn_token_independence_and_wdown_scaling():
    p = mi.Problem(40, 64, 4, 2, 48, "f32")
    L = mi.make_layer(p, seed=8)
    ids, _ = O.topk_route(mi.make_gaussian_logits(p, 8), 2)
    q = O.dispatch(ids, 4)
    args = (L["x"], q["sorted_assign"], q["offsets"], 2, L["w_gate"], L["w_up"])
    r = F.fp8_expert_ffn(*args, L["w_down"])
    # W_down times 2^3: identical codes, y exactly 8x
    r8 = F.fp8_expert_ffn(*args, L["w_down"] * 8.0)
    assert np.array_equal(r8["y_perm"], 8.0 * r["y_perm"])
    # the first 20 tokens alone give the same rows
    q20 = O.dispatch(ids[:20], 4)
    r20 = F.fp8_expert_ffn(L["x"][:20], q20["sorted_assign"], q20["offsets"], 2, L["w_gate"], L["w_up"],
                           L["w_down"])
    a20 = np.arange(40)
    pos_full = q["assign_pos"][a20]
    pos_sub = q20["assign_pos"][a20]
    assert np.array_equal(r20["y_perm"][pos_sub], r["y_perm"][pos_full])
    # and close to the exact layer (E4M3 keeps 4 significant bits)
    exact = O.expert_ffn(L["x"], q["sorted_assign"], q["offsets"], 2, L["w_gate"], L["w_up"], L["w_down"])
    assert np.max(np.abs(r["y_perm"] - exact)) / np.max(np.abs(exact)) < 0.1


def test_fp8_rows_match_the_queue_ffn():
    p = mi.Problem(30, 64, 5, 2, 48, "f32")
    L = mi.make_layer(p, seed=10)
    ids, _ = O.topk_route(mi.make_gaussian_logits(p, 10), 2)
    q = O.dispatch(ids, 5)
    r = F.fp8_expert_ffn(L["x"], q["sorted_assign"], q["offsets"], 2, L["w_gate"], L["w_up"], L["w_down"])
    tok = np.array([0, 3, 17, 29])
    rows = F.fp8_ffn_rows(np.repeat(L["x"][tok], 2, axis=0), ids[tok].reshape(-1), L["w_gate"], L["w_up"],
                          L["w_down"])
    pos = q["assign_pos"][(tok[:, None] * 2 + np.arange(2)).reshape(-1)]
    assert np.array_equal(rows, r["y_perm"][pos])
