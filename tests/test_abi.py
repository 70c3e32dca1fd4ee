"""The C ABI on the CPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments before any HIP call (so
these tests need no GPU and never launch a kernel)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_exclusive_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

# Plausible-looking device addresses that are never dereferenced: every call
# below fails validation before the library touches the GPU.
A = 0x10000
MIS = 0x10004  # not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def prob(T=64, d=128, E=8, k=2, f=256, dtype=L.MOE_DTYPE_BF16):
    return L.MoeProblem(T=T, d=d, E=E, k=k, f=f, dtype=dtype)


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
            "moe_workspace_size", "moe_status_string", "moe_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define MOE_MAX_EXPERTS (\d+)", text).group(1)) == L.MOE_MAX_EXPERTS
    assert int(re.search(r"#define MOE_MAX_TOPK (\d+)", text).group(1)) == L.MOE_MAX_TOPK
    assert 1 << int(re.search(r"#define MOE_NO_ALLOC_SCRATCH_BYTES \(1u << (\d+)\)", text).group(1)) == \
        L.MOE_NO_ALLOC_SCRATCH_BYTES
    for name in ("MOE_OK", "MOE_ERR_INVALID_ARGUMENT", "MOE_ERR_UNSUPPORTED",
                 "MOE_ERR_WORKSPACE_TOO_SMALL", "MOE_ERR_HIP", "MOE_DTYPE_F32", "MOE_DTYPE_BF16",
                 "MOE_OP_DISPATCH", "MOE_OP_EXPERT_FFN", "MOE_OP_FORWARD", "MOE_OP_BACKWARD",
                 "MOE_OP_EXPERT_FFN_FP8"):
        assert int(re.search(name + r"\s*=\s*(\d+)", text).group(1)) == getattr(L, name)


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moe_status_string(99) == b"MOE_ERR_UNKNOWN"
    assert lib.moe_abi_version() >= 1


def ws_size(lib, p, op):
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(p), op, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("bad,status", [
    (dict(k=9), L.MOE_ERR_INVALID_ARGUMENT),        # k > E
    (dict(T=-1), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(d=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(f=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=0, k=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=300), L.MOE_ERR_UNSUPPORTED),           # above MOE_MAX_EXPERTS
    (dict(E=64, k=33), L.MOE_ERR_UNSUPPORTED),      # above MOE_MAX_TOPK
    (dict(d=100), L.MOE_ERR_UNSUPPORTED),           # bf16 needs d % 64 == 0
    (dict(f=96), L.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 30, k=2), L.MOE_ERR_UNSUPPORTED),  # T*k >= 2^31
    # one 256-lane workgroup per token would exceed the 32-bit work-item count
    (dict(T=2 ** 25, d=64, E=8, k=1), L.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 24, d=64, E=8, k=1), L.MOE_ERR_UNSUPPORTED),
    (dict(d=65536, f=32768), L.MOE_ERR_UNSUPPORTED),  # bf16 d*f >= 2^31
])
def test_problem_validation(lib, bad, status):
    p = prob(**bad)
    assert ws_size(lib, p, L.MOE_OP_FORWARD)[0] == status
    assert lib.moe_route(ctypes.byref(p), A, A, None, A, A, A, None) == status
    assert lib.moe_dispatch(ctypes.byref(p), A, None, A, A, A, A, None, A, 1 << 40, None) == status
    assert lib.moe_expert_ffn(ctypes.byref(p), A, None, A, A, A, A, A, A, A, 1 << 40, None) == status
    assert lib.moe_combine(ctypes.byref(p), A, A, A, A, None) == status
    assert lib.moe_forward(ctypes.byref(p), A, A, None, A, A, A, A, None, A, 1 << 40, None) == status


def test_largest_token_count_is_accepted(lib):
    # 2^24 - 1 tokens: 256 lanes per token still fit the 32-bit work-item count
    assert ws_size(lib, prob(T=2 ** 24 - 1, d=64, E=8, k=1), L.MOE_OP_FORWARD)[0] == L.MOE_OK


def test_f32_allows_any_width(lib):
    assert ws_size(lib, prob(d=100, f=70, dtype=L.MOE_DTYPE_F32), L.MOE_OP_FORWARD)[0] == L.MOE_OK


def test_null_and_misaligned_pointers(lib):
    p = ctypes.byref(prob())
    E = L.MOE_ERR_INVALID_ARGUMENT
    U = L.MOE_ERR_UNSUPPORTED
    assert lib.moe_workspace_size(p, L.MOE_OP_FORWARD, None) == E
    assert lib.moe_workspace_size(p, 99, ctypes.byref(ctypes.c_size_t())) == E
    # route: without logits_in, x, w_router and logits_out are all required
    assert lib.moe_route(p, None, A, None, A, A, A, None) == E
    assert lib.moe_route(p, A, None, None, A, A, A, None) == E
    assert lib.moe_route(p, A, A, None, None, A, A, None) == E
    assert lib.moe_route(p, None, None, A, None, None, A, None) == E
    assert lib.moe_route(p, None, None, MIS, None, A, A, None) == U
    assert lib.moe_route(p, None, None, A, None, A, MIS, None) == U
    # dispatch
    assert lib.moe_dispatch(p, None, None, A, A, A, A, None, A, 1 << 40, None) == E
    assert lib.moe_dispatch(p, A, None, A, A, A, A, A, A, 1 << 40, None) == E  # x_perm needs x
    assert lib.moe_dispatch(p, A, None, A, A, MIS, A, None, A, 1 << 40, None) == U
    assert lib.moe_dispatch(p, A, None, A, A, A, A, None, None, 1 << 40, None) == E
    # expert ffn: the fused gather needs x and sorted_assign
    assert lib.moe_expert_ffn(p, None, None, A, A, A, A, A, A, A, 1 << 40, None) == E
    assert lib.moe_expert_ffn(p, None, A, None, A, A, A, A, A, A, 1 << 40, None) == E
    assert lib.moe_expert_ffn(p, A, None, None, A, A, A, MIS, A, A, 1 << 40, None) == U
    # combine
    assert lib.moe_combine(p, A, A, None, A, None) == E
    assert lib.moe_combine(p, A, A, A, MIS, None) == U
    # forward
    assert lib.moe_forward(p, A, None, None, A, A, A, A, None, A, 1 << 40, None) == E
    assert lib.moe_forward(p, A, A, None, A, A, A, None, None, A, 1 << 40, None) == E
    outs = L.MoeForwardOutputs(counts=MIS)
    assert lib.moe_forward(p, A, A, None, A, A, A, A, ctypes.byref(outs), A, 1 << 40, None) == U


def test_workspace_too_small(lib):
    p = prob()
    for op in (L.MOE_OP_DISPATCH, L.MOE_OP_EXPERT_FFN, L.MOE_OP_FORWARD):
        st, need = ws_size(lib, p, op)
        assert st == L.MOE_OK and need > 0
    pp = ctypes.byref(p)
    W = L.MOE_ERR_WORKSPACE_TOO_SMALL
    _, nd = ws_size(lib, p, L.MOE_OP_DISPATCH)
    _, nf = ws_size(lib, p, L.MOE_OP_EXPERT_FFN)
    _, nw = ws_size(lib, p, L.MOE_OP_FORWARD)
    assert lib.moe_dispatch(pp, A, None, A, A, A, A, None, A, nd - 1, None) == W
    assert lib.moe_expert_ffn(pp, A, None, None, A, A, A, A, A, A, nf - 1, None) == W
    assert lib.moe_forward(pp, A, A, None, A, A, A, A, None, A, nw - 1, None) == W


def test_zero_tokens_is_a_noop(lib):
    p = ctypes.byref(prob(T=0))
    # no tensor is touched, so NULL pointers are fine
    assert lib.moe_route(p, None, None, None, None, None, None, None) == L.MOE_OK
    assert lib.moe_dispatch(p, None, None, None, None, None, None, None, None, 0, None) == L.MOE_OK
    assert lib.moe_expert_ffn(p, None, None, None, None, None, None, None, None, None, 0, None) == L.MOE_OK
    assert lib.moe_combine(p, None, None, None, None, None) == L.MOE_OK
    assert lib.moe_forward(p, None, None, None, None, None, None, None, None, None, 0, None) == L.MOE_OK


def test_workspace_has_no_dense_routing_matrix(lib):
    # The dispatch queues replace a dense token-by-expert matrix: the dispatch
    # workspace holds per-block expert counts only (about 256 blocks).
    for T, d, E, k, f in [(65536, 2048, 128, 8, 768), (8192, 4096, 8, 2, 14336), (16384, 2048, 64, 6, 1408)]:
        p = prob(T, d, E, k, f)
        _, nd = ws_size(lib, p, L.MOE_OP_DISPATCH)
        assert nd <= E * 256 * 4 + 256  # at most 256 blocks
        assert nd * 16 < T * E * 4
        # forward: logits, ids/gates/permutations, counts, h, y_perm and the
        # split-K partial tiles of the down projection (256 tiles of 256 x 256
        # fp32) only
        _, nw = ws_size(lib, p, L.MOE_OP_FORWARD)
        s = 2
        split = 256 * 256 * 256 * 4 if f >= 1024 else 0
        expect = T * E * 4 + 4 * T * k * 4 + T * k * f * s + T * k * d * s + nd + split
        assert expect <= nw <= expect + 16 * 256
        _, nf = ws_size(lib, p, L.MOE_OP_EXPERT_FFN)
        assert T * k * f * s + split <= nf <= T * k * f * s + split + 256


def bwd_args(fw=True, out=True, w_router=A, dw_router=A, ws_bytes=1 << 40, **fields):
    st = L.MoeForwardState(topk_ids=A, topk_gates=A, offsets=A, sorted_assign=A, assign_pos=A, y_perm=A)
    o = L.MoeBackwardOutputs(dx=A, dw_gate=A, dw_up=A, dw_down=A, dw_router=dw_router, dlogits=None)
    for key, v in fields.items():
        setattr(st if key in dict(L.MoeForwardState._fields_) else o, key, v)
    return (A, w_router, A, A, A, A, ctypes.byref(st) if fw else None, A,
            ctypes.byref(o) if out else None, A, ws_bytes, None)


def test_backward_validation(lib):
    U = L.MOE_ERR_UNSUPPORTED
    E = L.MOE_ERR_INVALID_ARGUMENT
    good = prob(T=64, d=256, E=8, k=2, f=512)
    st, need = ws_size(lib, good, L.MOE_OP_BACKWARD)
    assert st == L.MOE_OK and need > 0
    for bad, status in [(dict(dtype=L.MOE_DTYPE_F32), U),       # bf16 only
                        (dict(d=32768, f=32768), U),            # d*f >= 2^30
                        (dict(T=2 ** 20, d=2048, k=1), U),      # T*d >= 2^31: 32-bit gather offsets
                        (dict(k=9), E)]:
        p = prob(T=64, d=256, E=8, k=2, f=512)
        for key, v in bad.items():
            setattr(p, key, v)
        assert ws_size(lib, p, L.MOE_OP_BACKWARD)[0] == status
        assert lib.moe_backward_weights(ctypes.byref(p), A, A, A, A, A, None) == status
        assert lib.moe_backward(ctypes.byref(p), *bwd_args()) == status
    pp = ctypes.byref(good)
    assert lib.moe_backward_weights(pp, A, A, None, A, A, None) == E
    assert lib.moe_backward_weights(pp, A, A, A, MIS, A, None) == U
    assert lib.moe_backward(pp, *bwd_args(fw=False)) == E
    assert lib.moe_backward(pp, *bwd_args(out=False)) == E
    assert lib.moe_backward(pp, *bwd_args(dw_router=None)) == E      # a router needs its gradient
    assert lib.moe_backward(pp, *bwd_args(w_router=None)) == E       # a gradient needs the router
    assert lib.moe_backward(pp, *bwd_args(assign_pos=None)) == E
    # y_perm is not read: its absence passes the checks (up to the workspace's)
    assert lib.moe_backward(pp, *bwd_args(y_perm=None, ws_bytes=need - 1)) == L.MOE_ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_backward(pp, *bwd_args(offsets=MIS)) == U
    assert lib.moe_backward(pp, *bwd_args(dw_down=None)) == E
    assert lib.moe_backward(pp, *bwd_args(dlogits=MIS)) == U
    assert lib.moe_backward(pp, *bwd_args(ws_bytes=need - 1)) == L.MOE_ERR_WORKSPACE_TOO_SMALL


def test_backward_workspace_size(lib):
    # dsel; each queue row's token (with 65 entries of padding) and gate; the
    # slot gradients' partial sums (one per 64 columns of each 128-column
    # recompute tile); the weight gradients' queue-order operands g h and
    # du|dv, each with 65 rows
    # of padding (whole 64-row slices past an expert's end, one row for a
    # channel range past a row's end); dx_perm and dh; the padded offsets and
    # expert order; the router gradient's partial sums per 64-row block of
    # the padded queue (Kpad = 64-aligned T*k + 63 E); and the split-K partial
    # tiles of the dx_perm GEMM.  No transposed copy, and no copy of x or dy
    # in queue order: the weight gradients read them by token.
    for T, d, E, k, f in [(8192, 4096, 8, 2, 14336), (16384, 2048, 64, 6, 1408), (64, 256, 8, 2, 512)]:
        n = T * k
        np_ = n + 65
        kp = -(-(n + 63 * E) // 64) * 64
        split = 256 * 256 * 256 * 4 if 2 * f // 64 >= 16 else 0
        parts = 2 * -(-f // 128)
        expect = n * 4 + np_ * 4 + n * 4 + n * parts * 4 + n * d * 2 + n * f * 2 + np_ * f * 2 + \
            np_ * 2 * f * 2 + (E + 1) * 4 + E * 4 + kp // 64 * d * 4 + split
        st, nb = ws_size(lib, prob(T, d, E, k, f), L.MOE_OP_BACKWARD)
        assert st == L.MOE_OK
        assert expect <= nb <= expect + 12 * 256


def test_fp8_validation(lib):
    U = L.MOE_ERR_UNSUPPORTED
    E = L.MOE_ERR_INVALID_ARGUMENT
    good = prob(T=64, d=256, E=8, k=2, f=512)
    st, need = ws_size(lib, good, L.MOE_OP_EXPERT_FFN_FP8)
    assert st == L.MOE_OK
    n = 64 * 2
    # x codes and exponents, h codes and one scale byte per 32 columns
    assert need >= 64 * 256 + 64 * 4 + n * 512 + n * 512 // 32
    w = L.MoeFp8Weights(w_gate=A, w_gate_exp=A, w_up=A, w_up_exp=A, w_down=A, w_down_exp=A)
    for bad in (dict(d=192), dict(f=320), dict(dtype=L.MOE_DTYPE_F32), dict(T=2 ** 22, d=2048)):
        p = prob(T=64, d=256, E=8, k=2, f=512)
        for key, v in bad.items():
            setattr(p, key, v)
        assert ws_size(lib, p, L.MOE_OP_EXPERT_FFN_FP8)[0] == U, bad
        assert lib.moe_quantize_weights_fp8(ctypes.byref(p), A, A, A, ctypes.byref(w), None) == U
        assert lib.moe_expert_ffn_fp8(ctypes.byref(p), A, A, A, ctypes.byref(w), A, A, 1 << 40, None) == U
    pp = ctypes.byref(good)
    assert lib.moe_quantize_weights_fp8(pp, A, A, A, None, None) == E
    assert lib.moe_expert_ffn_fp8(pp, A, A, A, None, A, A, 1 << 40, None) == E
    w.w_down_exp = None
    assert lib.moe_expert_ffn_fp8(pp, A, A, A, ctypes.byref(w), A, A, 1 << 40, None) == E
    w.w_down_exp = MIS
    assert lib.moe_expert_ffn_fp8(pp, A, A, A, ctypes.byref(w), A, A, 1 << 40, None) == U
    w.w_down_exp = A
    assert lib.moe_expert_ffn_fp8(pp, A, A, A, ctypes.byref(w), A, A, need - 1, None) == \
        L.MOE_ERR_WORKSPACE_TOO_SMALL
    # quantize rows: cols a positive multiple of 16
    assert lib.moe_quantize_rows_fp8(A, 4, 24, A, A, None) == U
    assert lib.moe_quantize_rows_fp8(A, 4, 0, A, A, None) == E
    assert lib.moe_quantize_rows_fp8(A, -1, 16, A, A, None) == E
    assert lib.moe_quantize_rows_fp8(None, 0, 16, None, None, None) == L.MOE_OK
    assert lib.moe_quantize_rows_fp8(A, 4, 16, MIS, A, None) == U
    # one workgroup per row: 2^24 rows of 256 lanes exceed the 32-bit work-item count
    assert lib.moe_quantize_rows_fp8(A, 2 ** 24, 4096, A, A, None) == U


def test_mfma_peak_validation(lib):
    assert lib.moe_mfma_peak(0, 10, A, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_mfma_peak(4, 0, A, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_mfma_peak(4, 10, None, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_mfma_peak(4, 10, MIS, None) == L.MOE_ERR_UNSUPPORTED


def test_stream_copy_validation(lib):
    assert lib.moe_stream_copy(A, A, 24, None) == L.MOE_ERR_UNSUPPORTED   # not a multiple of 16
    assert lib.moe_stream_copy(None, A, 32, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_stream_copy(A, MIS, 32, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_stream_copy(None, None, 0, None) == L.MOE_OK


def test_dispatch_no_alloc_validation(lib):
    def call(p, *ptrs):
        return lib.moe_dispatch_no_alloc(ctypes.byref(p), *ptrs, None)

    good = prob(T=4096, d=64, E=128, k=8)
    assert call(prob(k=9), A, None, A, A, A, A, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert call(good, None, None, A, A, A, A, None) == L.MOE_ERR_INVALID_ARGUMENT
    assert call(good, A, None, A, MIS, A, A, None) == L.MOE_ERR_UNSUPPORTED
    assert call(good, A, None, A, A, A, A, A) == L.MOE_ERR_INVALID_ARGUMENT  # x_perm without x
    assert call(prob(T=0), None, None, None, None, None, None, None) == L.MOE_OK
    # the count table of the largest problems does not fit the static scratch:
    # rejected before any HIP call (the workspace size says how large it is)
    big = prob(T=2 ** 21, d=64, E=256, k=8)
    st, table = ws_size(lib, big, L.MOE_OP_DISPATCH)
    assert st == L.MOE_OK and table > L.MOE_NO_ALLOC_SCRATCH_BYTES
    assert call(big, A, None, A, A, A, A, None) == L.MOE_ERR_UNSUPPORTED
    st, table = ws_size(lib, prob(T=65536, d=2048, E=128, k=8), L.MOE_OP_DISPATCH)
    assert st == L.MOE_OK and table <= L.MOE_NO_ALLOC_SCRATCH_BYTES
