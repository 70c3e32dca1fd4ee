"""Seeded routings with exact per-expert row counts, for tests that must hit
the kernels' tile and slice boundaries (plain numpy; no layer arithmetic)."""
import numpy as np


def exact_count_logits(counts, seed):
    """Top-2 logits [T, E] (T = sum(counts) / 2) that give expert e exactly
    counts[e] assignments: the multiset of expert slots is shuffled and
    paired into tokens with two distinct experts, which get logits 4.0 and
    3.5 (every other logit N(0, 0.25), far below)."""
    if sum(counts) % 2:
        raise ValueError("the counts of a top-2 routing add up to an even number")
    rng = np.random.default_rng(seed)
    slots = rng.permutation(np.repeat(np.arange(len(counts)), counts))
    for i in range(0, len(slots), 2):
        if slots[i] == slots[i + 1]:
            # swap in a slot of another pair that keeps both pairs distinct
            j = next(j for j in range(len(slots)) if j // 2 != i // 2 and slots[j] != slots[i] and
                     slots[j ^ 1] != slots[i + 1])
            slots[i + 1], slots[j] = slots[j], slots[i + 1]
    pairs = slots.reshape(-1, 2)
    assert np.all(pairs[:, 0] != pairs[:, 1])
    T = len(pairs)
    logits = (rng.standard_normal((T, len(counts))) * 0.5).astype(np.float32)
    logits[np.arange(T), pairs[:, 0]] = 4.0
    logits[np.arange(T), pairs[:, 1]] = 3.5
    return logits
