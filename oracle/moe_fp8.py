"""CPU oracle of the fp8 expert FFN (test infrastructure only).

The MoEBlaze summary (euno.news, "MoEBlaze: breaking the memory wall for
efficient MoE training on modern GPUs"), Limitations and future work, names
quantised experts as a next step without fixing a scheme.  The reading taken
here (every step is a definition, written out below):

* the 8-bit format is OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3
  mantissa bits; subnormals; largest finite value 448; no infinities), and a
  real value becomes a code by rounding to nearest, ties to even;
* each row of a quantised matrix carries one power-of-two scale 2^a, the
  smallest with max|row| <= 448 * 2^a (a = 0 for an all-zero row), so that
  dividing by the scale is exact and the code rounding is the only error;
* x is quantised per token, each expert weight matrix per output row
  (W_gate and W_up per h column, W_down per output column);
* GEMM1 sums code products exactly (float64 here) and applies the two
  scales: u = 2^(a_t + b_j) sum_c q(x)[t, c] q(W_gate)[j, c], likewise v;
* h = silu(u) * v is rounded to bf16 (round to nearest even), then
  quantised per block of 32 consecutive columns of each queue row: each
  block takes the smallest power-of-two scale that fits it, as above, but
  not below 2^-127, the smallest scale an E8M0 byte (OCP MX) holds;
* GEMM2 gives y_perm the same way, each code product scaled by its h
  block's and its W_down row's scales.

The combine and the routing are those of ``moe_oracle``.

Parity pins: ``tests/test_oracle_fp8_pins.py`` (torch's own float8_e4m3fn
conversion, an exhaustive round trip over the 254 finite codes, ties between
neighbouring codes, a brute-force nearest-code search, closed forms, and
the FFN against exact arithmetic where inputs are representable).
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import silu

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6       # smallest normal: 2^-6
_MANT_BITS = 3


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of E4M3 codes; the two NaN codes (0x7F, 0xFF) are
    rejected."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("NaN code")
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, _MIN_NORMAL_EXP)
    return sign * np.where(e == 0, sub, normal)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """E4M3 codes of finite values with |v| <= 448, rounded to nearest, ties
    to even (the sign of zero kept)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("values must be finite with |v| <= 448")
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = m 2^ex, m in [0.5, 1) (ex = 0 for a = 0)
    # exponent of the binade: a normal one, or the subnormal range (zero included)
    e_unb = np.where(a == 0, _MIN_NORMAL_EXP, np.maximum(ex - 1, _MIN_NORMAL_EXP))
    quantum = np.ldexp(1.0, e_unb - _MANT_BITS)
    n = np.rint(a / quantum)                 # numpy rounds half to even
    # n in [0, 16]; 16 means the value rounded up into the next binade
    up = n >= 16
    e_unb = np.where(up, e_unb + 1, e_unb)
    n = np.where(up, n / 2, n)
    is_sub = (e_unb == _MIN_NORMAL_EXP) & (n < 8)
    exp_field = np.where(is_sub, 0, e_unb + 7)
    mant = np.where(is_sub, n, n - 8)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


def pow2_scale_exponent(amax: float) -> int:
    """Smallest integer a with amax <= 448 * 2^a (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, e = np.frexp(amax)                    # amax = m 2^e, m in [0.5, 1); 448 = 0.875 * 2^9
    return int(e - 9) if m <= 0.875 else int(e - 8)


def quantize_rows(a: np.ndarray):
    """Per-row power-of-two scaled E4M3 codes of a 2-D array.  Returns
    (codes uint8 [R, C], exponents int32 [R]) with
    a[r] ~= 2^exp[r] * decode(codes[r])."""
    a = np.asarray(a)
    R, C = a.shape
    codes = np.zeros((R, C), dtype=np.uint8)
    exps = np.zeros(R, dtype=np.int32)
    for r0 in range(0, R, 256):  # blocks of rows (the rows are independent)
        blk = np.asarray(a[r0:r0 + 256], dtype=np.float64)
        ex = np.array([pow2_scale_exponent(m) for m in np.max(np.abs(blk), axis=1)], dtype=np.int32)
        codes[r0:r0 + 256] = e4m3_encode(np.ldexp(blk, -ex[:, None]))
        exps[r0:r0 + 256] = ex
    return codes, exps


H_BLOCK = 32        # h columns per scale
E8M0_MIN_EXP = -127  # the smallest scale exponent an E8M0 byte holds


def pow2_scale_exponents(amax: np.ndarray) -> np.ndarray:
    """``pow2_scale_exponent`` of every element of ``amax`` (int64)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)
    a = np.where(m <= 0.875, e - 9, e - 8)
    return np.where(amax == 0.0, 0, a).astype(np.int64)


def quantize_blocks(a: np.ndarray, block: int = H_BLOCK):
    """Power-of-two scaled E4M3 codes of each block of ``block``
    consecutive columns of each row of a 2-D array (a row's last block may
    be shorter): the block's exponent is the row rule of ``quantize_rows``
    applied to the block alone, raised to at least -127.  Returns (codes
    uint8 [R, C], exponents int32 [R, ceil(C / block)]) with
    a[r, c] ~= 2^exp[r, c // block] * decode(codes[r, c])."""
    a = np.asarray(a)
    R, C = a.shape
    nb = -(-C // block)
    codes = np.zeros((R, C), dtype=np.uint8)
    exps = np.zeros((R, nb), dtype=np.int32)
    for r0 in range(0, R, 256):  # blocks of rows (the rows are independent)
        rows = np.asarray(a[r0:r0 + 256], dtype=np.float64)
        for b in range(nb):
            c0, c1 = b * block, min(C, (b + 1) * block)
            sub = rows[:, c0:c1]
            ex = np.maximum(pow2_scale_exponents(np.max(np.abs(sub), axis=1)), E8M0_MIN_EXP)
            codes[r0:r0 + 256, c0:c1] = e4m3_encode(np.ldexp(sub, -ex[:, None]))
            exps[r0:r0 + 256, b] = ex
    return codes, exps


def dequantize_blocks(codes: np.ndarray, exps: np.ndarray, block: int = H_BLOCK) -> np.ndarray:
    """2^exps[r, c // block] * value(codes[r, c]), float64."""
    codes = np.asarray(codes)
    exps = np.asarray(exps, dtype=np.int64)
    cols = np.arange(codes.shape[1]) // block
    out = np.empty(codes.shape, dtype=np.float64)
    for r0 in range(0, codes.shape[0], 256):
        out[r0:r0 + 256] = np.ldexp(e4m3_decode(codes[r0:r0 + 256]), exps[r0:r0 + 256][:, cols])
    return out


def dequantize_rows(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """2^exps[r] * value(codes[r, c]), float64 (in blocks of rows)."""
    codes = np.asarray(codes)
    exps = np.asarray(exps, dtype=np.int64)
    out = np.empty(codes.shape, dtype=np.float64)
    for r0 in range(0, codes.shape[0], 256):
        out[r0:r0 + 256] = np.ldexp(e4m3_decode(codes[r0:r0 + 256]), exps[r0:r0 + 256, None])
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Values rounded to bf16 (8 significant bits), to nearest, ties to even
    (normal range)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def quantize_weights(w: np.ndarray):
    """Per-output-row quantisation of expert weights [E, out, in]:
    (codes [E, out, in], exponents [E, out])."""
    E, o, i = w.shape
    c, x = quantize_rows(np.asarray(w).reshape(E * o, i))
    return c.reshape(E, o, i), x.reshape(E, o)


def fp8_expert_ffn(x: np.ndarray, sorted_assign: np.ndarray, offsets: np.ndarray, k: int,
                   w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> dict:
    """The fp8 expert FFN over the dispatch queues (definition above).
    Returns y_perm (float64 [T*k, d]), h (the bf16-rounded values, float64
    [T*k, f]) and the codes and exponents of x, h (one exponent per block of
    32 columns) and the weights."""
    sa = np.asarray(sorted_assign, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    xq, xe = quantize_rows(x)
    wg, ge = quantize_weights(w_gate)
    wu, ue = quantize_weights(w_up)
    wd, de = quantize_weights(w_down)
    E = off.shape[0] - 1
    n, d = sa.shape[0], np.asarray(x).shape[1]
    f = wg.shape[1]
    h = np.zeros((n, f), dtype=np.float64)
    xdq = dequantize_rows(xq, xe)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        xr = xdq[sa[lo:hi] // k]
        u = xr @ dequantize_rows(wg[e], ge[e]).T
        v = xr @ dequantize_rows(wu[e], ue[e]).T
        h[lo:hi] = round_bf16(silu(u) * v)
    hq, he = quantize_blocks(h)
    hdq = dequantize_blocks(hq, he)
    y = np.zeros((n, d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            y[lo:hi] = hdq[lo:hi] @ dequantize_rows(wd[e], de[e]).T
    return dict(y_perm=y, h=h, x_codes=xq, x_exp=xe, h_codes=hq, h_exp=he,
                w_gate=(wg, ge), w_up=(wu, ue), w_down=(wd, de))


def fp8_ffn_rows(x_rows: np.ndarray, experts: np.ndarray, w_gate, w_up, w_down) -> np.ndarray:
    """The fp8 FFN of single queue rows (every quantisation above is per
    row or per block of a row, so a row's output depends only on its token
    and expert): row i is
    token row x_rows[i] through expert experts[i].  Weights may be callables
    ``w(e)`` returning one expert's matrix; each expert used is quantised
    once.  Returns float64 [n, d]."""
    def get(w, e):
        return w(e) if callable(w) else w[e]

    xq, xe = quantize_rows(x_rows)
    xdq = dequantize_rows(xq, xe)
    experts = np.asarray(experts, dtype=np.int64)
    out = None
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        wg = dequantize_rows(*quantize_rows(get(w_gate, e)))
        wu = dequantize_rows(*quantize_rows(get(w_up, e)))
        wd = dequantize_rows(*quantize_rows(get(w_down, e)))
        xr = xdq[rows]
        h = round_bf16(silu(xr @ wg.T) * (xr @ wu.T))
        y = dequantize_blocks(*quantize_blocks(h)) @ wd.T
        if out is None:
            out = np.zeros((len(experts), y.shape[1]), dtype=np.float64)
        out[rows] = y
    return out
