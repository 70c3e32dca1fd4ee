"""Analytic resource model of one GPU's MoE layer on MI355X.

The structure follows Piper's resource model (Piper summary, euno.news,
"Piper: efficient large-scale MoE training via resource modeling and
pipelined hybrid parallelism", Methodology 1 and 2): closed-form per-GPU
memory (expert weights, activations, routing tables), compute (router,
expert FFN) and communication (the all-to-all an expert-parallel layout
would exchange), from the expert count, batch, top-k and layer widths, and
a check of its predictions against micro-benchmarks, skinny GEMM kernels
among them, to within 10 %.

Here, for this library on one MI355X:

* ``memory``: every buffer of the layer and of each entry point's
  workspace, byte for byte as the library sizes them (checked against
  ``moe_workspace_size``).
* ``flops`` and ``hbm_bytes``: algorithmic work per call.
* ``predict_times``: kernel times from a tile-wave model.  A grouped GEMM is
  a list of 256-row x 256-weight-row tiles, one workgroup per CU, so it runs
  in ``ceil(tiles / CUs)`` waves of ``slice_us * K/64 + tile_us`` each; a
  tail that leaves most CUs idle is split along K as the library splits it.
  The weight-gradient tiles differ in K (their expert's row count), so that
  launch is list-scheduled as the hardware deals it: workgroup i to XCD
  i mod 8, then to the first free CU of that XCD.
  Bandwidth-bound kernels take ``launch_us + bytes / stream_bw``.  The
  constants come from ``calibrate`` (micro-benchmarks of skinny expert
  GEMMs, least squares).
* ``all_to_all_bytes``: the expert-parallel exchange volume per GPU (a
  formula only: one GPU cannot measure it).

Nothing here launches work on the GPU except ``calibrate``'s measurement
callback, which the caller supplies.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, replace
from typing import Dict, Optional, Sequence

# ---- the library's tiling and workspace constants --------------------------

ALIGN = 256            # workspace sub-buffer alignment (bytes)
TM = 256               # queue rows per GEMM tile
GATEUP_COLS = 128      # h columns per GEMM1 tile (gate and up rows each)
DOWN_COLS = 256        # output columns per tile of the other GEMMs
BK = 64                # K columns per slice
SPLIT_WGS = 256        # partial tiles the split-K workspace holds
SPLIT_MAX = 8
SPLIT_MIN_SLICES = 8
MAX_DISPATCH_CHUNK = 8192

OP_DISPATCH, OP_EXPERT_FFN, OP_FORWARD, OP_BACKWARD = 1, 2, 3, 4


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _align(b: int, a: int = ALIGN) -> int:
    return _cdiv(b, a) * a


@dataclass(frozen=True)
class Layer:
    """One call's shape: T tokens, hidden d, E experts, top-k, SwiGLU width
    f, storage bytes per element s (2 for bf16, 4 for fp32)."""

    T: int
    d: int
    E: int
    k: int
    f: int
    s: int = 2

    @property
    def n(self) -> int:
        return self.T * self.k


# ---- memory -----------------------------------------------------------------

def _dispatch_chunk(n: int) -> int:
    return min(max(_cdiv(_cdiv(n, 256), 256) * 256, 256), MAX_DISPATCH_CHUNK)


def _dispatch_ws(L: Layer) -> int:
    return _align(_cdiv(L.n, _dispatch_chunk(L.n)) * L.E * 4)


def dispatch_launches(L: Layer) -> int:
    """Kernel launches of a dispatch with x_perm: one workgroup for up to 4096
    assignments, plus the gather; histogram and one pass of scatter and
    gather for chunks of 256 ids with at most 4096 block counts; else
    histogram, scatter and gather."""
    if L.n <= 4096:
        return 2
    if _dispatch_chunk(L.n) == 256 and _cdiv(L.n, 256) * L.E <= 4096 and (L.d * L.s) % 16 == 0:
        return 2
    return 3


def _split_bytes(K: int, s: int) -> int:
    return SPLIT_WGS * TM * DOWN_COLS * 4 if (s == 2 and K // BK >= 2 * SPLIT_MIN_SLICES) else 0


def _ffn_ws(L: Layer) -> int:
    return _align(L.n * L.f * L.s) + _split_bytes(L.f, L.s)


def kpad(L: Layer) -> int:
    """Rows of the backward's padded queue (each expert's queue rounded up to
    64 rows): the router gradient's partial sums take one row per 64."""
    return _align(L.n + 63 * L.E, 64)


# Rows after each queue-order operand of the weight-gradient GEMMs.
WGRAD_PAD_ROWS = 65


def workspace(L: Layer, op: int) -> int:
    """Workspace bytes of an entry point, as the library sizes it."""
    if op == OP_DISPATCH:
        return _dispatch_ws(L)
    if op == OP_EXPERT_FFN:
        return _ffn_ws(L)
    if op == OP_FORWARD:
        return (_align(L.T * L.E * 4) + 4 * _align(L.n * 4) + _align(L.E * 4) + _align((L.E + 1) * 4)
                + _dispatch_ws(L) + _ffn_ws(L) + _align(L.n * L.d * L.s))
    if op == OP_BACKWARD:
        kp = kpad(L)
        npad = L.n + WGRAD_PAD_ROWS
        # dsel, the queue rows' tokens and gates, the slot gradients' partial
        # sums, dx_perm, dh_raw, g h, du|dv, poff, order, router partial
        # sums, split-K partials (x and dy are read by token, not copied into
        # queue order; y_perm is not read)
        parts = 2 * _cdiv(L.f, GATEUP_COLS)
        return (_align(L.n * 4) + _align(npad * 4) + _align(L.n * 4) + _align(L.n * parts * 4)
                + _align(L.n * L.d * 2)
                + _align(L.n * L.f * 2) + _align(npad * L.f * 2) + _align(npad * 2 * L.f * 2)
                + _align((L.E + 1) * 4) + _align(L.E * 4) + _align(kp // 64 * L.d * 4)
                + _align(_split_bytes(2 * L.f, 2)))
    raise ValueError(f"unknown op {op}")


def memory(L: Layer, backward: bool = False) -> Dict[str, int]:
    """Per-GPU bytes of one layer call, by kind (Piper's memory terms).

    weights: W_gate, W_up, W_down and the router; activations: x and y;
    routing_tables: logits, ids, gates, both permutations, counts, offsets
    and the dispatch block counts; expert_buffers: h and y_perm (and the
    split-K partial tiles); with ``backward``: the transposed weight
    layouts, the gradients and the backward workspace."""
    m = {
        "weights": 3 * L.E * L.d * L.f * L.s + L.E * L.d * L.s,
        "activations": 2 * L.T * L.d * L.s,
        "routing_tables": (_align(L.T * L.E * 4) + 4 * _align(L.n * 4) + _align(L.E * 4) + _align((L.E + 1) * 4)
                           + _dispatch_ws(L)),
        "expert_buffers": _ffn_ws(L) + _align(L.n * L.d * L.s),
    }
    if backward:
        m["weight_layouts"] = 3 * L.E * L.d * L.f * L.s
        m["gradients"] = 3 * L.E * L.d * L.f * L.s + L.E * L.d * L.s + 2 * L.T * L.d * L.s + L.T * L.E * 4
        m["backward_workspace"] = workspace(L, OP_BACKWARD)
    m["total"] = sum(m.values())
    return m


def max_tokens(d: int, E: int, k: int, f: int, budget: int, s: int = 2, backward: bool = False) -> int:
    """Largest T whose layer call fits in ``budget`` bytes (capacity planning)."""
    lo, hi = 0, 1
    while memory(Layer(hi, d, E, k, f, s), backward)["total"] <= budget:
        lo, hi = hi, hi * 2
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if memory(Layer(mid, d, E, k, f, s), backward)["total"] <= budget:
            lo = mid
        else:
            hi = mid
    return lo


# ---- compute and bytes ---------------------------------------------------------

def flops(L: Layer, router: bool = True) -> Dict[str, float]:
    """Algorithmic FLOPs per call (Piper's compute terms, for this layer)."""
    return {
        "router": 2.0 * L.T * L.d * L.E if router else 0.0,
        "expert_ffn": 6.0 * L.n * L.d * L.f,
        "backward_gemms": 16.0 * L.n * L.d * L.f,
        "backward_router": 4.0 * L.T * L.d * L.E if router else 0.0,
    }


def hbm_bytes(L: Layer) -> Dict[str, float]:
    """Algorithmic HBM bytes per call of the bandwidth-bound steps."""
    s = L.s
    return {
        "dispatch_with_x_perm": (1 + L.k) * L.T * L.d * s + 12.0 * L.n,
        "combine": (L.k + 1) * L.T * L.d * s + 8.0 * L.n,
        "router_read": L.T * L.d * s + L.E * L.d * s + 4.0 * L.T * L.E,
        # the queue rows' tokens and gates, and the slot and logit gradients
        # from the recompute's partial sums (y_perm is not read)
        "backward_dy": L.n * (8.0 + 8.0 + 4.0 * 2 * _cdiv(L.f, GATEUP_COLS)) + 4.0 * L.T * L.E,
        "backward_dx": (L.k + 1) * L.T * L.d * 2.0,
        # the router gradient's partial sums: every queue row's x row read
        "backward_router_partials": L.n * L.d * 2.0,
    }


def all_to_all_bytes(L: Layer, G: int) -> float:
    """Bytes each GPU sends (and receives) per direction when E experts are
    sharded over G GPUs in contiguous blocks and tokens are spread evenly:
    the rows whose expert lives elsewhere, (G-1)/G of T*k rows."""
    return L.n * L.d * L.s * (G - 1) / G


# ---- time ----------------------------------------------------------------------

@dataclass(frozen=True)
class Hardware:
    """MI355X and the model's calibrated constants.

    ``slice_us`` and ``tile_us``: one 64-column K slice of a 256 x 256 tile,
    and the fixed cost of a tile (start, epilogue); ``upbwd_tile_us``: the
    extra epilogue of the backward's recompute tile; ``stream_bw``: bytes
    per microsecond of the bandwidth-bound kernels; ``launch_us``: their
    fixed cost.  The defaults were fitted by ``calibrate`` on one MI355X
    (the micro-benchmarks of ``tests/test_gpu_resource_model.py``)."""

    cus: int = 256
    slice_us: float = 1.374
    tile_us: float = 10.81
    upbwd_tile_us: float = 17.19
    stream_bw: float = 5.09e6
    launch_us: float = 4.0


def row_tiles(counts: Sequence[int]) -> int:
    return sum(_cdiv(int(c), TM) for c in counts)


def gemm_terms(hw: Hardware, tiles: int, nk: float, split: bool = False, extra_us: float = 0.0,
               out_cols: int = DOWN_COLS):
    """(a, b, c) with time = a * slice_us + b * tile_us + c microseconds for
    one grouped GEMM launch of ``tiles`` tiles of ``nk`` K slices; with
    ``split`` the library's split-K tail (its reduction in c)."""
    if tiles == 0:
        return 0.0, 0.0, 0.0
    slots = hw.cus
    r = tiles % slots
    if split and r > 0:
        S = min(slots // r, min(SPLIT_MAX, int(nk) // SPLIT_MIN_SLICES))
        if S >= 2:
            w = (tiles - r) // slots
            reduce_bytes = r * S * TM * out_cols * 4 + r * TM * out_cols * 2
            return (w * nk + math.ceil(nk / S), w + 1.0,
                    w * extra_us + hw.launch_us + reduce_bytes / hw.stream_bw)
    w = _cdiv(tiles, slots)
    return w * nk, float(w), w * extra_us


def gemm_time(hw: Hardware, tiles: int, nk: float, split: bool = False, extra_us: float = 0.0,
              out_cols: int = DOWN_COLS) -> float:
    """Microseconds of one grouped GEMM launch (see ``gemm_terms``)."""
    a, b, c = gemm_terms(hw, tiles, nk, split, extra_us, out_cols)
    return a * hw.slice_us + b * hw.tile_us + c


def ffn_terms(L: Layer, counts: Sequence[int], hw: Hardware):
    """(a, b, c) of the expert-FFN call: GEMM1 plus GEMM2."""
    R = row_tiles(counts)
    g1 = gemm_terms(hw, R * _cdiv(L.f, GATEUP_COLS), L.d / BK)
    g2 = gemm_terms(hw, R * _cdiv(L.d, DOWN_COLS), L.f / BK, split=_split_bytes(L.f, L.s) > 0)
    return tuple(x + y for x, y in zip(g1, g2))


def list_time(hw: Hardware, tile_us: Sequence[float], xcds: int = 8) -> float:
    """Makespan of tiles dealt in order: tile i to XCD i mod ``xcds``, then
    to the CU of that XCD that frees first."""
    per = hw.cus // xcds
    worst = 0.0
    for x in range(xcds):
        heap = [0.0] * per
        for t in tile_us[x::xcds]:
            heapq.heappush(heap, heapq.heappop(heap) + t)
        worst = max(worst, max(heap))
    return worst


def xcd_list_time(hw: Hardware, lists: Sequence[Sequence[float]]) -> float:
    """Makespan when XCD x runs the tiles of lists[x] in order, each on the
    CU of that XCD that frees first."""
    per = hw.cus // len(lists)
    worst = 0.0
    for tiles in lists:
        heap = [0.0] * per
        for t in tiles:
            heapq.heappush(heap, heapq.heappop(heap) + t)
        worst = max(worst, max(heap))
    return worst


def wgrad_time(hw: Hardware, counts: Sequence[int], M: int, N: int, xcds: int = 8) -> float:
    """One weight-gradient launch: per expert ceil(M/256) * ceil(N/256) tiles
    of K = its padded row count.  Whole experts go to XCDs, heaviest first
    (ties: lower id) in a snake order (XCD 0 to 7, then 7 to 0, ...), and
    each XCD runs its experts' tiles in that order on its CUs."""
    per_e = _cdiv(M, TM) * _cdiv(N, DOWN_COLS)
    nks = [_cdiv(int(c), BK) for c in counts]
    order = sorted(range(len(counts)), key=lambda e: (-nks[e], e))
    lists = [[] for _ in range(xcds)]
    for r, e in enumerate(order):
        j, i = divmod(r, xcds)
        lists[xcds - 1 - i if j % 2 else i].extend([hw.slice_us * nks[e] + hw.tile_us] * per_e)
    return xcd_list_time(hw, lists)


def _backward_parts(L: Layer, counts: Sequence[int], hw: Hardware) -> Dict[str, float]:
    R = row_tiles(counts)
    t = {}
    t["bwd_dh"] = gemm_time(hw, R * _cdiv(L.f, DOWN_COLS), L.d / BK)
    t["bwd_recompute"] = gemm_time(hw, R * _cdiv(L.f, GATEUP_COLS), L.d / BK, extra_us=hw.upbwd_tile_us)
    t["bwd_dx_perm"] = gemm_time(hw, R * _cdiv(L.d, DOWN_COLS), 2 * L.f / BK, split=_split_bytes(2 * L.f, 2) > 0)
    t["bwd_wgrad"] = wgrad_time(hw, counts, L.d, L.f) + 2 * wgrad_time(hw, counts, L.f, L.d)
    # (launches: offsets and order, the queue rows' tokens and gates, the
    # slot and logit gradients, dx; no router)
    t["bwd_streaming"] = 4 * hw.launch_us + backward_stream_bytes(L) / hw.stream_bw
    return t


def backward_stream_bytes(L: Layer, router: bool = False) -> float:
    """Bytes of the backward's bandwidth-bound kernels: the slot gradients,
    the dx sum and, with a router, its gradient's partial sums."""
    b = hbm_bytes(L)
    return b["backward_dy"] + b["backward_dx"] + (b["backward_router_partials"] if router else 0.0)


def predict_times(L: Layer, counts: Sequence[int], hw: Optional[Hardware] = None) -> Dict[str, float]:
    """Predicted microseconds per kernel of the forward call and of the
    backward call (bf16), given the routing's expert counts."""
    hw = hw or Hardware()
    R = row_tiles(counts)
    b = hbm_bytes(L)
    t = {}
    t["gemm1"] = gemm_time(hw, R * _cdiv(L.f, GATEUP_COLS), L.d / BK)
    t["gemm2"] = gemm_time(hw, R * _cdiv(L.d, DOWN_COLS), L.f / BK, split=_split_bytes(L.f, L.s) > 0)
    t["expert_ffn"] = t["gemm1"] + t["gemm2"]
    t["combine"] = hw.launch_us + b["combine"] / hw.stream_bw
    t["dispatch_with_x_perm"] = dispatch_launches(L) * hw.launch_us + b["dispatch_with_x_perm"] / hw.stream_bw
    bw = _backward_parts(L, counts, hw)
    t.update(bw)
    t["backward"] = sum(bw.values())
    return t


def _lstsq2(rows):
    """Least squares of t = a x + b y over rows (a, b, t)."""
    sxx = sum(a * a for a, _, _ in rows)
    sxy = sum(a * b for a, b, _ in rows)
    syy = sum(b * b for _, b, _ in rows)
    sxt = sum(a * t for a, _, t in rows)
    syt = sum(b * t for _, b, t in rows)
    det = sxx * syy - sxy * sxy
    return (sxt * syy - syt * sxy) / det, (syt * sxx - sxt * sxy) / det


def calibrate(measure, shapes: Optional[Sequence[Layer]] = None, hw: Optional[Hardware] = None,
              measure_backward=None) -> Hardware:
    """Fit the model's constants from micro-benchmarks, by least squares.

    ``measure(layer) -> (microseconds, counts)`` times one expert-FFN call of
    a layer (the caller runs it on the GPU, with whatever routing it likes)
    and returns the routing's expert counts: each call is one linear
    equation in ``slice_us`` and ``tile_us`` (``ffn_terms``).  With
    ``measure_backward(layer) -> (microseconds, counts)``, the backward calls
    then fit ``upbwd_tile_us`` and ``stream_bw`` (linear in the epilogue
    cost and in 1 / bandwidth, the GEMM terms taken from the first fit)."""
    hw = hw or Hardware()
    shapes = shapes or CALIBRATION_SHAPES
    fwd = [(L,) + tuple(measure(L)) for L in shapes]
    bwd = [(L,) + tuple(measure_backward(L)) for L in shapes] if measure_backward is not None else []
    # the two fits share the split-K reduction's bandwidth term: refit a few
    # times on the stored measurements until the constants settle
    for _ in range(8 if bwd else 1):
        rows = []
        for L, us, counts in fwd:
            a, b, c = ffn_terms(L, counts, hw)
            rows.append((a, b, us - c))
        slice_us, tile_us = _lstsq2(rows)
        hw = replace(hw, slice_us=slice_us, tile_us=tile_us)
        if not bwd:
            break
        rows = []
        for L, us, counts in bwd:
            # the backward is linear in both constants: read the coefficients off
            def total(upbwd, inv_bw):
                h = replace(hw, upbwd_tile_us=upbwd, stream_bw=1.0 / inv_bw if inv_bw else float("inf"))
                return sum(_backward_parts(L, counts, h).values())
            known = total(0.0, 0.0)
            rows.append((total(1.0, 0.0) - known, total(0.0, 1.0) - known, us - known))
        upbwd, inv_bw = _lstsq2(rows)
        hw = replace(hw, upbwd_tile_us=upbwd, stream_bw=1.0 / inv_bw)
    return hw


# Micro-benchmark shapes for ``calibrate``: skinny expert GEMMs with short and
# long K in both projections, none of them one of the validated workloads.
CALIBRATION_SHAPES = (Layer(8192, 2048, 16, 2, 2048), Layer(16384, 1024, 32, 4, 1024),
                      Layer(8192, 4096, 8, 2, 2048), Layer(8192, 2048, 8, 2, 8192))
