"""The analytic resource model on the CPU: its memory terms equal what the
library sizes (moe_workspace_size, no GPU call), and its FLOP and tile
counts equal the per-expert GEMM shapes they summarise."""
import ctypes

import numpy as np
import pytest

from mixture_experts_layer_exclusive_amd import _lib as Lb
from mixture_experts_layer_exclusive_amd import resource_model as RM

SHAPES = [(8192, 4096, 8, 2, 14336), (16384, 2048, 64, 6, 1408), (32768, 2048, 128, 8, 768),
          (65536, 2048, 128, 8, 768), (1, 64, 8, 2, 64), (777, 192, 16, 4, 320), (4096, 128, 3, 3, 512),
          (5000, 512, 256, 32, 1024), (0, 256, 8, 2, 512)]


def lib_ws(T, d, E, k, f, dtype, op):
    p = Lb.MoeProblem(T=T, d=d, E=E, k=k, f=f, dtype=dtype)
    n = ctypes.c_size_t(0)
    st = Lb.load().moe_workspace_size(ctypes.byref(p), op, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("T,d,E,k,f", SHAPES)
def test_workspace_model_equals_library(T, d, E, k, f):
    for dtype, s in ((Lb.MOE_DTYPE_BF16, 2), (Lb.MOE_DTYPE_F32, 4)):
        L = RM.Layer(T, d, E, k, f, s)
        for op in (RM.OP_DISPATCH, RM.OP_EXPERT_FFN, RM.OP_FORWARD) + ((RM.OP_BACKWARD,) if s == 2 else ()):
            st, nb = lib_ws(T, d, E, k, f, dtype, op)
            assert st == Lb.MOE_OK
            assert RM.workspace(L, op) == nb, (dtype, op)


def test_memory_terms_add_up():
    L = RM.Layer(8192, 4096, 8, 2, 14336)
    m = RM.memory(L)
    # the forward's workspace is the routing tables plus the expert buffers
    assert m["routing_tables"] + m["expert_buffers"] == RM.workspace(L, RM.OP_FORWARD)
    assert m["weights"] == 3 * 8 * 4096 * 14336 * 2 + 8 * 4096 * 2
    mb = RM.memory(L, backward=True)
    assert mb["total"] == sum(v for key, v in mb.items() if key != "total")
    assert mb["backward_workspace"] == RM.workspace(L, RM.OP_BACKWARD)


def test_max_tokens_is_the_largest_that_fits():
    budget = 288 * 10**9
    for d, E, k, f in ((4096, 8, 2, 14336), (2048, 128, 8, 768)):
        for bwd in (False, True):
            t = RM.max_tokens(d, E, k, f, budget, backward=bwd)
            assert RM.memory(RM.Layer(t, d, E, k, f), bwd)["total"] <= budget
            assert RM.memory(RM.Layer(t + 1, d, E, k, f), bwd)["total"] > budget


def test_flops_equal_the_sum_of_per_expert_gemms():
    rng = np.random.default_rng(0)
    T, d, E, k, f = 3000, 256, 16, 4, 384
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    counts = np.bincount(ids.ravel(), minlength=E)
    fw = sum(2 * c * (2 * f) * d + 2 * c * d * f for c in counts)  # GEMM1 (gate and up), GEMM2
    bw = sum(2 * c * f * d                 # dh
             + 2 * c * (2 * f) * d         # recompute of gate and up
             + 2 * c * d * (2 * f)         # dx_perm
             + 2 * c * d * f + 2 * 2 * c * f * d for c in counts)  # dW_down, dW_gate, dW_up
    fl = RM.flops(RM.Layer(T, d, E, k, f))
    assert fl["expert_ffn"] == fw and fl["backward_gemms"] == bw


def test_tile_wave_model():
    hw = RM.Hardware(slice_us=1.0, tile_us=10.0)
    # whole waves: time = waves * (slices + tile cost)
    assert RM.gemm_time(hw, 512, 64) == 2 * 74.0
    # a partial last wave still takes a whole tile time without a split
    assert RM.gemm_time(hw, 513, 64) == 3 * 74.0
    # with the split: 64 leftover tiles on 256 slots split 4 ways (64 slices -> 16 each)
    t = RM.gemm_time(hw, 512 + 64, 64, split=True)
    assert 2 * 74.0 + 16 + 10.0 < t < 2 * 74.0 + 16 + 10.0 + 30.0
    assert RM.row_tiles([0, 1, 256, 257, 512]) == 0 + 1 + 1 + 2 + 2


def test_calibration_recovers_known_constants():
    true = RM.Hardware(slice_us=1.4, tile_us=9.0)
    rng = np.random.default_rng(1)

    def measure(L):
        counts = rng.multinomial(L.n, np.ones(L.E) / L.E)  # uneven counts: partial waves, split tails
        return RM.predict_times(L, counts, true)["expert_ffn"], counts

    hw = RM.calibrate(measure)
    assert abs(hw.slice_us - 1.4) < 1e-9 and abs(hw.tile_us - 9.0) < 1e-9
    # all four constants together (the split-K reduction couples the fits)
    true2 = RM.Hardware(slice_us=1.4, tile_us=9.0, upbwd_tile_us=7.0, stream_bw=4.5e6)

    def measure2(L):
        counts = rng.multinomial(L.n, np.ones(L.E) / L.E)
        return RM.predict_times(L, counts, true2)["expert_ffn"], counts

    def measure_bwd(L):
        counts = rng.multinomial(L.n, np.ones(L.E) / L.E)
        return RM.predict_times(L, counts, true2)["backward"], counts

    hw = RM.calibrate(measure2, measure_backward=measure_bwd)
    assert abs(hw.slice_us - 1.4) < 1e-6 and abs(hw.tile_us - 9.0) < 1e-4
    assert abs(hw.upbwd_tile_us - 7.0) < 1e-3 and abs(hw.stream_bw / 4.5e6 - 1) < 1e-6


def test_all_to_all_volume():
    L = RM.Layer(8192, 4096, 8, 2, 14336)
    assert RM.all_to_all_bytes(L, 1) == 0
    assert RM.all_to_all_bytes(L, 8) == 16384 * 4096 * 2 * 7 / 8


def test_list_schedule():
    hw = RM.Hardware(cus=16, slice_us=1.0, tile_us=0.0)
    # equal tiles: whole waves per XCD (2 CUs each)
    assert RM.list_time(hw, [1.0] * 32) == 2.0
    # one long tile bounds its XCD; the others finish earlier
    assert RM.list_time(hw, [10.0] + [1.0] * 15) == 10.0
    # whole experts per XCD: the heavy expert's one tile bounds its XCD
    t = RM.wgrad_time(RM.Hardware(slice_us=1.0, tile_us=0.0), [64 * 100] + [64] * 15, 256, 256)
    assert t == 100.0
    # snake order: 16 experts of 16 tiles each on 16 CUs (2 per XCD); ranks 0
    # and 15 share XCD 0, ranks 7 and 8 XCD 7: 16 tiles of 8 slices per CU pair
    counts = [64 * (16 - e) for e in range(16)]
    t = RM.wgrad_time(RM.Hardware(cus=16, slice_us=1.0, tile_us=0.0), counts, 4 * 256, 4 * 256)
    assert t == (16 + 1) * 16 / 2
    # one expert's tiles (16 here) never leave its XCD
    t = RM.wgrad_time(RM.Hardware(cus=16, slice_us=1.0, tile_us=0.0), [64] + [0] * 7, 4 * 256, 4 * 256)
    assert t == 16 / 2


def test_dispatch_launches_follow_the_library_paths():
    # one workgroup (+ gather) up to 4096 assignments; histogram + one pass of
    # scatter and gather for chunks of 256 ids and at most 4096 block counts;
    # else histogram, scatter, gather
    L = lambda T, E, k, d=4096: RM.Layer(T, d, E, k, 1024, 2)  # noqa: E731
    assert RM.dispatch_launches(L(2048, 8, 2)) == 2
    assert RM.dispatch_launches(L(8192, 8, 2)) == 2          # 64 blocks x 8 experts
    assert RM.dispatch_launches(L(2048, 64, 6)) == 2         # 48 blocks x 64 experts
    assert RM.dispatch_launches(L(32768, 16, 2)) == 2        # 256 blocks x 16 experts
    assert RM.dispatch_launches(L(32768, 32, 2)) == 3        # 8192 block counts
    assert RM.dispatch_launches(L(40000, 8, 2)) == 3         # chunks of 512 ids
    assert RM.dispatch_launches(L(16384, 64, 6)) == 3
