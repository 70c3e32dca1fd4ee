"""The resource model's time predictions against measured calls on the GPU.

As in Piper's validation (micro-benchmarks first, then real workloads): the
model's constants are fitted on skinny-GEMM micro-benchmark layers
(``resource_model.CALIBRATION_SHAPES``), then it predicts the expert-FFN
call and the backward call of the four full-size workloads, whose shapes it
has not seen.  Inputs are random (timing does not depend on values); the
routing comes from Gaussian logits, or Zipf-skewed ones for the skewed
workload, and the model is given the resulting expert counts.  Each
prediction must land within 10 % of the measured time (Piper's validation
bound); the errors are printed.  Every measured time is the median of
several timed blocks of calls, so that one slow block does not decide it.
"""
import statistics

import pytest
import torch

import mixture_experts_layer_exclusive_amd as moe
from mixture_experts_layer_exclusive_amd import resource_model as RM

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def event_us(fn, reps, blocks=5):
    """Median over `blocks` timed blocks of `reps` calls, in us per call."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(blocks):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        per_call.append(a.elapsed_time(b) * 1e3 / reps)
    return statistics.median(per_call)


class Bench:
    """Random tensors of one layer shape and its routing on the GPU."""

    def __init__(self, L: RM.Layer, zipf: bool = False, seed: int = 0):
        g = torch.Generator(device=DEV)
        g.manual_seed(seed)
        self.L = L
        s = L.d ** -0.5
        self.x = torch.randn(L.T, L.d, device=DEV, generator=g).to(BF)
        self.wg = (torch.randn(L.E, L.f, L.d, device=DEV, generator=g) * s).to(BF)
        self.wu = (torch.randn(L.E, L.f, L.d, device=DEV, generator=g) * s).to(BF)
        self.wd = (torch.randn(L.E, L.d, L.f, device=DEV, generator=g) * s).to(BF)
        lg = torch.randn(L.T, L.E, device=DEV, generator=g)
        if zipf:
            r = torch.arange(1, L.E + 1, device=DEV, dtype=torch.float64) ** -1.2
            lg = lg + (2 * torch.log(r / r.sum())).float()
        self.logits = lg
        _, self.st = moe.forward(self.x, self.wg, self.wu, self.wd, L.k, logits=lg, intermediates=True)
        torch.cuda.synchronize()
        self.counts = self.st["counts"].cpu().tolist()

    def ffn_us(self):
        L = self.L
        p = moe.problem(L.T, L.d, L.E, L.k, L.f, BF)
        ws = torch.empty(moe.workspace_size(p, 2), dtype=torch.uint8, device=DEV)
        yp = torch.empty(L.n, L.d, dtype=BF, device=DEV)
        st = self.st
        return event_us(lambda: moe.expert_ffn(st["offsets"], self.wg, self.wu, self.wd, L.k, L.T, x=self.x,
                                               sorted_assign=st["sorted_assign"], ws=ws, y_perm=yp), 10)

    def backward_us(self):
        L = self.L
        wt = moe.backward_weights(self.wg, self.wu, self.wd)
        dy = torch.randn(L.T, L.d, device=DEV).to(BF)
        p = moe.problem(L.T, L.d, L.E, L.k, L.f, BF)
        ws = torch.empty(moe.workspace_size(p, 4), dtype=torch.uint8, device=DEV)
        out = {key: v for key, v in moe.backward(self.x, self.wg, self.wu, L.k, self.st, dy, wt, ws=ws).items()
               if v is not None}
        return event_us(lambda: moe.backward(self.x, self.wg, self.wu, L.k, self.st, dy, wt, ws=ws, out=out), 3)


WORKLOADS = [("mixtral", RM.Layer(8192, 4096, 8, 2, 14336), False),
             ("deepseek", RM.Layer(16384, 2048, 64, 6, 1408), False),
             ("qwen3", RM.Layer(32768, 2048, 128, 8, 768), False),
             ("zipf_skewed", RM.Layer(65536, 2048, 128, 8, 768), True)]


def test_time_model_predicts_unseen_workloads():
    cache = {}

    def bench(L):
        if L not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[L] = Bench(L, seed=7)
        return cache[L]

    def measure(L):
        b = bench(L)
        us = b.ffn_us()
        print(f"calibration {L}: expert FFN {us:.1f} us", flush=True)
        return us, b.counts

    def measure_backward(L):
        b = bench(L)
        us = b.backward_us()
        print(f"calibration {L}: backward {us:.1f} us", flush=True)
        return us, b.counts

    hw = RM.calibrate(measure, measure_backward=measure_backward)
    cache.clear()
    print(f"calibrated: {hw}", flush=True)
    errs = {}
    for name, L, zipf in WORKLOADS:
        torch.cuda.empty_cache()
        b = Bench(L, zipf=zipf, seed=1)
        pred = RM.predict_times(L, b.counts, hw)
        ffn, bwd = b.ffn_us(), b.backward_us()
        errs[name] = (pred["expert_ffn"] / ffn - 1, pred["backward"] / bwd - 1)
        print(f"{name}: expert FFN measured {ffn:.0f} us, predicted {pred['expert_ffn']:.0f} us "
              f"({errs[name][0]:+.1%}); backward measured {bwd:.0f} us, predicted {pred['backward']:.0f} us "
              f"({errs[name][1]:+.1%})", flush=True)
        del b
    for name, (e1, e2) in errs.items():
        assert abs(e1) <= 0.10 and abs(e2) <= 0.10, (name, e1, e2)
