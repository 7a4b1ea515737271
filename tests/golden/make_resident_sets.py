"""Write tests/golden/resident_sets.json: the calibrated resident (hot) set of
each workload shape, as the "Luce Spark" page, sec. 1, picks it -- the experts
that calibration traffic routes to most.

Calibration traffic: 1024 tokens drawn like the workload's activations with
seed + 1 (moe_inputs.make_activations), routed by the workload's router
(seed).  Everything else is the oracle: router logits, top-k, the per-expert
counts of its permutation, the counters, and the hot set (most used first,
equal counts to the lower id).  Run from the repository root:
    python tests/golden/make_resident_sets.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402

CAL_TOKENS = 1024
SEED = 0


def calibrate(shape, seed=SEED, tokens=CAL_TOKENS):
    Wr, bias = mi.make_router(shape, seed)
    x, _ = mi.make_activations(shape.H, tokens, seed + 1)
    ids, _ = oracle.topk(oracle.router_logits(x, Wr, bias), shape.k, True)
    counts = oracle.permute(ids, shape.E)["counts"]
    freq = oracle.freq_update(counts, np.zeros(shape.E, np.uint32))
    return freq, oracle.hot_set(freq, shape.n_resident)


def main():
    out = {"source": "the 'Luce Spark' page, sec. 1 (calibrated placement); written by "
                     "tests/golden/make_resident_sets.py from the oracle",
           "calibration_tokens": CAL_TOKENS, "router_seed": SEED, "activation_seed": SEED + 1, "shapes": {}}
    for name in mi.CONFIG_ORDER:
        shape = mi.CONFIGS[name]
        freq, hot = calibrate(shape)
        out["shapes"][name] = dict(E=shape.E, k=shape.k, n_resident=shape.n_resident, hot=hot.tolist(),
                                   counts=freq.tolist())
        print(name, "hot:", hot[:12].tolist(), "...", file=sys.stderr)
    with open(os.path.join(HERE, "resident_sets.json"), "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
