"""CPU oracle for one GPU's MoE-layer forward (test infrastructure only).

This is the plain, slow, obviously-correct statement of what the layer
computes.  It is test infrastructure: only the tests, the smoke check and
the CPU-baseline leg of the benchmark may import it.  The product path never
calls it, and it shares no code with the HIP library (its only common input
is the seeded generator module, which holds none of the layer's arithmetic).

Arithmetic: inputs arrive as float32 arrays (bf16 data widened exactly);
every sum, exponential and product is taken in float64.  Router logits and
gates are returned rounded once to float32, because the routing decision is
defined on float32 logits.  Expert outputs and the layer output are returned
in float64.

Sources (the pages are summaries of three papers; they give the structure,
not the formulas):

* MoEBlaze summary (euno.news, "MoEBlaze: breaking the memory wall for
  efficient MoE training on modern GPUs"), Methodology item 1: tokens reach
  their experts through compact per-expert dispatch queues built during the
  forward pass and dropped afterwards; the dense token-by-expert routing
  matrix is never built.  Methodology item 2: dispatch and reverse dispatch
  (scatter/gather) around the expert feed-forward.  Limitations: the routing
  policy is static top-k.
* Piper technical summary (gist.science, Dutch), section 1 (problem
  statement): fine-grained MoE layers give tall-and-skinny expert GEMMs and
  skewed expert loads.
* DisagMoE technical summary (gist.science, Korean), section 2.2 (AF-Pipe):
  k is the number of experts each token is routed to.

Where the pages are silent the plainest reading is taken: softmax gating
over the router logits, the k largest logits selected (ties to the lower
expert id, slots in descending order), gates renormalised over the k chosen
experts, dropless queues, and a bias-free SwiGLU expert
``W_down (silu(W_gate x) * (W_up x))``.  The dispatch queues are a stable
counting sort of the flattened assignments ``a = t*k + j`` by expert id.

Parity pins for every function here live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Router GEMM: ``l[t, e] = sum_c x[t, c] * W_r[e, c]`` in float64,
    rounded once to float32.  The router is the part of the layer that picks
    a few experts per token (Piper, Japanese explainer, opening section;
    Piper Korean summary, Methodology 1: routing FLOPs)."""
    return (_f64(x) @ _f64(w_router).T).astype(np.float32)


def topk_route(logits: np.ndarray, k: int):
    """Static top-k gating (MoEBlaze summary, Limitations: static top-k).

    Selection: per token, experts ordered by the key (-l[t, e], e) on the
    float32 logits (-0.0 equals +0.0), the first k kept, so ties go to the
    lower expert id and slots run in descending logit order.  Selecting on
    logits equals selecting on softmax probabilities because softmax is
    strictly increasing.

    Gates: softmax restricted to the chosen experts (the full-softmax
    denominator cancels after renormalisation):
    ``g[t, j] = exp(l_j - m) / sum_i exp(l_i - m)``, m = l of slot 0, in
    float64, rounded once to float32.

    Returns (ids int32 [T, k], gates float32 [T, k])."""
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # A stable sort of -l keeps equal logits in ascending expert order.
    order = np.argsort(-l32, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(_f64(l32), ids.astype(np.int64), axis=1)
    m = sel[:, :1]
    p = np.exp(sel - m)
    gates = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, gates


# --------------------------------------------------------------------------
# dispatch queues: counting sort (histogram, exclusive scan, stable scatter)
# --------------------------------------------------------------------------

def expert_histogram(ids: np.ndarray, E: int) -> np.ndarray:
    """``counts[e]`` = number of assignments routed to expert e, over the
    flattened assignments ``a = t*k + j`` (MoEBlaze summary, Methodology 1:
    per-expert queue lengths instead of a dense routing matrix)."""
    counts = [0] * E
    for e in np.asarray(ids).reshape(-1).tolist():
        counts[e] += 1
    return np.array(counts, dtype=np.int32)


def exclusive_scan(counts: np.ndarray) -> np.ndarray:
    """``offsets[0] = 0``, ``offsets[e+1] = offsets[e] + counts[e]``: where
    each expert's queue starts in the permuted order."""
    offsets = [0]
    for c in np.asarray(counts).tolist():
        offsets.append(offsets[-1] + c)
    return np.array(offsets, dtype=np.int32)


def stable_scatter(ids: np.ndarray, offsets: np.ndarray):
    """Place each assignment in its expert's queue, visiting assignments in
    ascending ``a`` so that each queue keeps assignment order (stable).

    Returns ``sorted_assign`` (queue position -> assignment a) and its
    inverse ``assign_pos`` (a -> queue position), both int32 [T*k]."""
    flat = np.asarray(ids).reshape(-1).tolist()
    cursor = np.asarray(offsets).tolist()[:-1]
    n = len(flat)
    sorted_assign = [0] * n
    assign_pos = [0] * n
    for a, e in enumerate(flat):
        pos = cursor[e]
        cursor[e] = pos + 1
        sorted_assign[pos] = a
        assign_pos[a] = pos
    return np.array(sorted_assign, dtype=np.int32), np.array(assign_pos, dtype=np.int32)


def dispatch(ids: np.ndarray, E: int) -> dict:
    """The dispatch queues of one layer call: counts, offsets and the two
    directions of the permutation (MoEBlaze summary, Methodology 1)."""
    counts = expert_histogram(ids, E)
    offsets = exclusive_scan(counts)
    sorted_assign, assign_pos = stable_scatter(ids, offsets)
    return dict(counts=counts, offsets=offsets, sorted_assign=sorted_assign,
                assign_pos=assign_pos)


def gather_rows(x: np.ndarray, sorted_assign: np.ndarray, k: int) -> np.ndarray:
    """Dispatch gather: queue row ``pos`` holds token ``sorted_assign[pos] // k``
    (a bitwise copy of that token's row of x)."""
    return np.asarray(x)[np.asarray(sorted_assign, dtype=np.int64) // k]


# --------------------------------------------------------------------------
# expert feed-forward and combine
# --------------------------------------------------------------------------

def silu(u: np.ndarray) -> np.ndarray:
    """silu(u) = u / (1 + exp(-u)), float64."""
    return u / (1.0 + np.exp(-u))


def swiglu_expert(x_rows: np.ndarray, w_gate_e: np.ndarray, w_up_e: np.ndarray,
                  w_down_e: np.ndarray) -> np.ndarray:
    """One expert's SwiGLU FFN on rows of x, float64 throughout, no biases:
    ``y = W_down (silu(W_gate x) * (W_up x))`` with weights in
    [out, in] layout.  x_rows [n, d] -> [n, d]."""
    xr = _f64(x_rows)
    u = xr @ _f64(w_gate_e).T
    v = xr @ _f64(w_up_e).T
    h = silu(u) * v
    return h @ _f64(w_down_e).T


def expert_ffn(x: np.ndarray, sorted_assign: np.ndarray, offsets: np.ndarray, k: int,
               w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """Expert FFN over the dispatch queues: for each expert e, the rows
    ``pos`` in ``[offsets[e], offsets[e+1])`` hold token
    ``sorted_assign[pos] // k`` and get ``y_perm[pos] = FFN_e(x[token])``.
    The per-expert products are the tall-and-skinny GEMMs of the Piper
    summary (section 1).  Returns y_perm float64 [T*k, d]."""
    E = len(offsets) - 1
    d = np.asarray(x).shape[1]
    sa = np.asarray(sorted_assign, dtype=np.int64)
    y_perm = np.zeros((len(sa), d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = np.asarray(x)[sa[lo:hi] // k]
        y_perm[lo:hi] = swiglu_expert(rows, w_gate[e], w_up[e], w_down[e])
    return y_perm


def combine(y_perm: np.ndarray, assign_pos: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """Reverse dispatch with gate weighting (MoEBlaze summary, Methodology 2):
    ``y[t] = sum_j g[t, j] * y_perm[assign_pos[t*k + j]]``, float64, summed
    over ascending slot j."""
    g = _f64(gates)
    T, k = g.shape
    pos = np.asarray(assign_pos, dtype=np.int64).reshape(T, k)
    yp = _f64(y_perm)
    y = np.zeros((T, yp.shape[1]), dtype=np.float64)
    for j in range(k):
        y += g[:, j:j + 1] * yp[pos[:, j]]
    return y


def forward(x: np.ndarray, k: int, w_gate: np.ndarray, w_up: np.ndarray,
            w_down: np.ndarray, w_router: np.ndarray | None = None,
            logits: np.ndarray | None = None) -> dict:
    """The whole layer: router GEMM (unless logits are supplied), top-k
    gating, dispatch queues, expert FFN, combine.  Returns every
    intermediate and ``y`` (float64 [T, d])."""
    if logits is None:
        if w_router is None:
            raise ValueError("need w_router or logits")
        logits = router_logits(x, w_router)
    logits = np.asarray(logits, dtype=np.float32)
    E = logits.shape[1]
    ids, gates = topk_route(logits, k)
    q = dispatch(ids, E)
    y_perm = expert_ffn(x, q["sorted_assign"], q["offsets"], k, w_gate, w_up, w_down)
    y = combine(y_perm, q["assign_pos"], gates)
    return dict(logits=logits, ids=ids, gates=gates, y_perm=y_perm, y=y, **q)


def forward_tokens(tokens: np.ndarray, x: np.ndarray, logits: np.ndarray, k: int,
                   w_gate, w_up, w_down) -> dict:
    """Per-token definition of the layer on a subset of tokens:
    ``y_t = sum_j g[t, j] * FFN_{ids[t, j]}(x_t)`` with ids and gates from
    ``topk_route`` on the given logits rows (no queues).  Used to check
    sampled outputs of full-size runs.  Expert weights may be given as
    callables ``w(e) -> [out, in]`` so that only the experts a sample uses
    are widened to float64.  Returns ids, gates and y (float64)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, gates = topk_route(np.asarray(logits, dtype=np.float32)[tokens], k)
    xs = np.asarray(x)[tokens]
    y = np.zeros((len(tokens), xs.shape[1]), dtype=np.float64)

    def get(w, e):
        return w(e) if callable(w) else w[e]

    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        ye = swiglu_expert(xs[rows], get(w_gate, e), get(w_up, e), get(w_down, e))
        y[rows] += _f64(gates[rows, slots])[:, None] * ye
    return dict(ids=ids, gates=gates, y=y)
