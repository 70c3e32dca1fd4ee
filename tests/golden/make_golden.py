"""Writes oracle_tiny_layer.json from the oracle alone (see README.md)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402


def build():
    p = mi.Problem(T=12, d=8, E=5, k=2, f=6, dtype="f32")
    L = mi.make_layer(p, seed=7)
    logits = mi.make_tie_logits(p, seed=7, step=0.5)
    out = oracle.forward(L["x"], p.k, L["w_gate"], L["w_up"], L["w_down"], logits=logits)
    return {
        "problem": dict(T=p.T, d=p.d, E=p.E, k=p.k, f=p.f, dtype=p.dtype, seed=7, logits="tie_heavy_step_0.5"),
        "ids": out["ids"].tolist(),
        "gates": [[float(g) for g in row] for row in out["gates"]],
        "counts": out["counts"].tolist(),
        "offsets": out["offsets"].tolist(),
        "sorted_assign": out["sorted_assign"].tolist(),
        "assign_pos": out["assign_pos"].tolist(),
        "y": [[float(v) for v in row] for row in out["y"]],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_tiny_layer.json"), "w") as fh:
        json.dump(build(), fh, indent=1)
