"""Seeded synthetic inputs for one GPU's MoE-layer forward.

This module is shared by the CPU oracle tests and by the HIP-path tests and
bench. It holds no arithmetic of the MoE layer itself: it only draws random
numbers, scales them to the stated standard deviations, rounds them to the
storage dtype and widens bf16 bit patterns back to float32.

Recipe (the same for every caller):

* Tensor ``i`` of a problem (0 = x, 1 = router weight, 2 = W_gate,
  3 = W_up, 4 = W_down, 5 = router-logit noise, 6 = tie-heavy logits,
  7 = token sample, 8 = output gradient dy) is drawn in row-major order in chunks of ``CHUNK``
  elements; chunk ``c`` comes from ``numpy.random.default_rng([seed, i, c])``
  as ``standard_normal(dtype=float32)``.  Chunks are independent streams, so
  they are drawn in parallel threads and the result does not depend on the
  thread count.
* Each draw is multiplied by its standard deviation (computed in fp64 and
  rounded once to fp32): x 1, router weight 0.02, all three expert matrices
  ``1/sqrt(d)``, output gradient dy 1.  The second parameter of ``N(0, s)`` is read as a standard
  deviation.
* bf16 problems round the scaled fp32 values to bf16 with round-to-nearest-
  even and store the 16-bit patterns as ``uint16``.
* Skewed routing logits: ``z[t, e] + fp32(2 * ln w_e)`` with ``z ~ N(0, 1)``
  fp32 and ``w_e = (e + 1)^-s / sum_r r^-s`` (Zipf, s = 1.2, rank = expert id
  + 1), added in fp32.

The workloads are the MoE layer shapes the pages discuss (Mixtral-,
DeepSeek-MoE- and Qwen3-MoE-shaped layers; a Zipf-skewed load), with random
weights in place of trained ones.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22

# stream ids
S_X, S_WR, S_WG, S_WU, S_WD, S_LOGIT, S_TIES, S_SAMPLE, S_DY = range(9)


@dataclass(frozen=True)
class Problem:
    """Shape of one MoE layer call: T tokens, hidden size d, E experts,
    top-k, SwiGLU width f, storage dtype ("f32" or "bf16")."""

    T: int
    d: int
    E: int
    k: int
    f: int
    dtype: str = "bf16"

    @property
    def n_assign(self) -> int:
        return self.T * self.k


# The five workloads.  Names say what they are; sizes follow the MoE layer
# shapes of the models the pages name.
WORKLOADS = {
    "tiny_f32": dict(problem=Problem(256, 128, 8, 2, 256, "f32"), logits="router"),
    "mixtral_8x_bf16": dict(problem=Problem(8192, 4096, 8, 2, 14336, "bf16"), logits="router"),
    "deepseek_moe_bf16": dict(problem=Problem(16384, 2048, 64, 6, 1408, "bf16"), logits="router"),
    "qwen3_moe_bf16": dict(problem=Problem(32768, 2048, 128, 8, 768, "bf16"), logits="router"),
    "zipf_skewed_bf16": dict(problem=Problem(65536, 2048, 128, 8, 768, "bf16"), logits="zipf"),
}

ZIPF_S = 1.2
SIGMA_ROUTER = 0.02


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def standard_normal_f32(seed: int, stream: int, n: int) -> np.ndarray:
    """n float32 N(0,1) draws of tensor ``stream`` under ``seed`` (chunked
    independent streams, see the module docstring)."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        out[lo:hi] = np.random.default_rng([seed, stream, c]).standard_normal(hi - lo, dtype=np.float32)

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)

    def conv(c: int) -> None:
        lo = c * step
        hi = min(flat_u.size, lo + step)
        v = flat_u[lo:hi]
        bias = ((v >> 16) & 1) + np.uint32(0x7FFF)
        flat_o[lo:hi] = ((v + bias) >> 16).astype(np.uint16)

    n = (flat_u.size + step - 1) // step
    if n <= 1:
        if flat_u.size:
            conv(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(n)))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _sigma_f32(s: float) -> np.float32:
    return np.float32(s)


def _draw(seed: int, stream: int, shape, sigma: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    v = standard_normal_f32(seed, stream, n)
    if sigma != 1.0:
        v *= _sigma_f32(sigma)
    v = v.reshape(shape)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_x(p: Problem, seed: int = 0) -> np.ndarray:
    """Activations x[T, d]: N(0, 1)."""
    return _draw(seed, S_X, (p.T, p.d), 1.0, p.dtype)


def make_grad_output(p: Problem, seed: int = 0) -> np.ndarray:
    """Output gradient dy[T, d] for the backward: N(0, 1)."""
    return _draw(seed, S_DY, (p.T, p.d), 1.0, p.dtype)


def make_router_weight(p: Problem, seed: int = 0) -> np.ndarray:
    """Router weight W_r[E, d] (nn.Linear [out, in] layout): N(0, 0.02)."""
    return _draw(seed, S_WR, (p.E, p.d), SIGMA_ROUTER, p.dtype)


def make_expert_weights(p: Problem, seed: int = 0):
    """Expert SwiGLU weights, all N(0, 1/sqrt(d)):
    W_gate[E, f, d], W_up[E, f, d], W_down[E, d, f]."""
    s = 1.0 / math.sqrt(p.d)
    wg = _draw(seed, S_WG, (p.E, p.f, p.d), s, p.dtype)
    wu = _draw(seed, S_WU, (p.E, p.f, p.d), s, p.dtype)
    wd = _draw(seed, S_WD, (p.E, p.d, p.f), s, p.dtype)
    return wg, wu, wd


def zipf_bias_f32(E: int, s: float = ZIPF_S) -> np.ndarray:
    """Per-expert logit bias fp32(2 ln w_e), w_e = (e+1)^-s / sum_r r^-s."""
    r = np.arange(1, E + 1, dtype=np.float64)
    w = r ** (-s)
    w /= w.sum()
    return (2.0 * np.log(w)).astype(np.float32)


def make_gaussian_logits(p: Problem, seed: int = 0) -> np.ndarray:
    """Supplied router logits l[T, E] ~ N(0, 1) fp32."""
    return standard_normal_f32(seed, S_LOGIT, p.T * p.E).reshape(p.T, p.E)


def make_zipf_logits(p: Problem, seed: int = 0, s: float = ZIPF_S) -> np.ndarray:
    """Skewed supplied logits: N(0, 1) noise plus the Zipf bias, in fp32."""
    z = make_gaussian_logits(p, seed)
    return z + zipf_bias_f32(p.E, s)[None, :]


def make_tie_logits(p: Problem, seed: int = 0, step: float = 0.25) -> np.ndarray:
    """Tie-heavy logits: N(0, 1) rounded to multiples of ``step`` (exact in
    fp32), so many tokens hold equal logits for different experts."""
    z = standard_normal_f32(seed, S_TIES, p.T * p.E).reshape(p.T, p.E)
    return (np.round(z / np.float32(step)) * np.float32(step)).astype(np.float32)


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """A sorted seeded sample of n distinct token indices in [0, T)."""
    n = min(n, T)
    rng = np.random.default_rng([seed, S_SAMPLE])
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """View any generated tensor as float32 values (bf16 patterns widened)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def make_layer(name_or_problem, seed: int = 0, with_experts: bool = True):
    """All inputs of one workload as a dict of numpy arrays.

    Keys: problem, x, w_router (None when logits are supplied), logits
    (None when the router runs), w_gate, w_up, w_down (None unless
    ``with_experts``)."""
    if isinstance(name_or_problem, str):
        spec = WORKLOADS[name_or_problem]
        p, mode = spec["problem"], spec["logits"]
    else:
        p, mode = name_or_problem, "router"
    out = dict(problem=p, x=make_x(p, seed), w_router=None, logits=None,
               w_gate=None, w_up=None, w_down=None)
    if mode == "router":
        out["w_router"] = make_router_weight(p, seed)
    elif mode == "zipf":
        out["logits"] = make_zipf_logits(p, seed)
    else:
        raise ValueError(mode)
    if with_experts:
        out["w_gate"], out["w_up"], out["w_down"] = make_expert_weights(p, seed)
    return out
