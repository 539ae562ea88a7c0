"""Writes tests/golden/oracle_rollouts.json: regression fixtures of the oracle.

The pages print no worked numeric example of a Domino rollout, so no stored
value here comes from them.  These are the outputs of the oracle (and only of
the oracle) on small seeded synthetic models, kept so that an unintended
change to the oracle's arithmetic shows up as a changed fixture.  What pins
the oracle to the pages and to the mathematics is tests/test_oracle.py (float64
brute force, torch.nn.GRUCell, closed forms, invariants); these fixtures only
freeze it.  Regenerate with `python tests/golden/make_fixtures.py` and justify
the change in the commit message.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from gru_corrected_draft_amd import synth  # noqa: E402

# (vocabulary, hidden, emb, gru, proj, dtype, weight seed), batch, input seed, K values
CASES = [
    ((64, 16, 8, 8, 8, "fp32", 601), 2, 611, (0, 5)),
    ((97, 32, 16, 16, 16, "bf16", 602), 3, 612, (0, 1, 40, 97)),
]
SCALES = {"embed": 16.0, "gru_w_ih": 3.0, "gru_w_hh": 3.0, "fc1_w": 3.0}


def fixtures():
    out = []
    for dims, B, seed, ks in CASES:
        shape = synth.custom_shape(*dims, name="golden")
        w = synth.make_weights(shape, SCALES)
        f32 = {n: w.f32(n) for n in ("lm_head", "embed", "gru_w_ih", "gru_w_hh", "fc1_w", "fc2_w",
                                     "fc2_b")}
        inp = synth.make_inputs(shape, B, seed, 0)
        for K in ks:
            r = oracle.rollout(f32, inp.hidden_f32(), inp.step_s, inp.verified, K)
            out.append({
                "shape": list(dims), "batch": B, "input_seed": seed, "K": K,
                "scales": SCALES,
                "tokens": r["tokens"].tolist(),
                "top1": [[float(x) for x in row] for row in r["top1"]],
                "margin": [[float(x) for x in row] for row in r["margin"]],
                "pools": [None if p is None else [int(i) for i in p] for p in r["pools"]],
            })
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_rollouts.json")
    with open(path, "w") as f:
        json.dump({"source": "oracle.rollout on seeded synthetic models (tests/golden/make_fixtures.py)",
                   "cases": fixtures()}, f, indent=1)
    print(path)
