"""moe_dispatch_no_alloc, the dispatch for callers that cannot allocate,
against moe_dispatch, through the C ABI: the queues (counts, offsets,
sorted_assign, assign_pos) and the gathered rows x_perm must be identical,
bit for bit, on two calls in a row, the second on a smaller problem (the
static scratch then still holds the first call's larger count table).
Outputs and the reference call's workspace are poisoned first."""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle as O
from mixture_experts_layer_exclusive_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def outputs(T, d, E, k):
    n = T * k
    return dict(counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
                offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
                sorted_assign=torch.full((n,), -7, dtype=torch.int32, device=DEV),
                assign_pos=torch.full((n,), -7, dtype=torch.int32, device=DEV),
                x_perm=torch.full((n, d), float("nan"), dtype=torch.bfloat16, device=DEV))


def call(lib, p, ids, x, out, ws=None):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [ctypes.byref(p), ptr(ids), ptr(x), ptr(out["counts"]), ptr(out["offsets"]),
            ptr(out["sorted_assign"]), ptr(out["assign_pos"]), ptr(out["x_perm"])]
    if ws is None:
        st = lib.moe_dispatch_no_alloc(*args, stream)
    else:
        st = lib.moe_dispatch(*args, ptr(ws), ws.numel(), stream)
    assert st == L.MOE_OK, lib.moe_status_string(st)


@pytest.mark.parametrize("first,second", [
    # (T, d, E, k, logits): the second call is smaller in every count
    ((65536, 64, 128, 8, "zipf"), (20000, 128, 64, 6, "gauss")),
    ((16384, 2048, 64, 6, "gauss"), (3000, 64, 8, 2, "gauss")),
])
def test_no_alloc_dispatch_matches_dispatch(first, second):
    lib = L.load()
    for T, d, E, k, kind in (first, second):
        print(f"no-alloc dispatch T={T} d={d} E={E} k={k} {kind}", flush=True)
        p = mi.Problem(T, d, E, k, 64, "bf16")
        lg = mi.make_zipf_logits(p, 3) if kind == "zipf" else mi.make_gaussian_logits(p, 3)
        ids_h, _ = O.topk_route(lg, k)
        ids = torch.from_numpy(ids_h).to(DEV)
        x = torch.from_numpy(mi.make_x(p, 3).view(np.int16)).view(torch.bfloat16).to(DEV)
        prob = L.MoeProblem(T=T, d=d, E=E, k=k, f=64, dtype=L.MOE_DTYPE_BF16)
        n = ctypes.c_size_t(0)
        assert lib.moe_workspace_size(ctypes.byref(prob), L.MOE_OP_DISPATCH, ctypes.byref(n)) == L.MOE_OK
        assert n.value <= L.MOE_NO_ALLOC_SCRATCH_BYTES
        ws = torch.full((max(256, n.value),), 0xFF, dtype=torch.uint8, device=DEV)
        ref = outputs(T, d, E, k)
        got = outputs(T, d, E, k)
        call(lib, prob, ids, x, ref, ws)
        call(lib, prob, ids, x, got)
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "sorted_assign", "assign_pos"):
            assert torch.equal(got[key], ref[key]), key
        assert torch.equal(got["x_perm"].view(torch.int16), ref["x_perm"].view(torch.int16))
        # and the reference itself is the oracle's counting sort
        q = O.dispatch(ids_h, E)
        assert np.array_equal(ref["sorted_assign"].cpu().numpy(), q["sorted_assign"])
