"""The oracle against its stored regression fixtures (tests/golden/).

The pages print no worked numeric example, so the fixtures are the oracle's
own outputs on small seeded models, written by tests/golden/make_fixtures.py
(which calls only the oracle).  They freeze the oracle; the pins that tie it
to the pages and to the mathematics are in tests/test_oracle.py.
"""
import json
import os

import numpy as np
import pytest

import oracle
from gru_corrected_draft_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "oracle_rollouts.json")) as f:
    CASES = json.load(f)["cases"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"V{c['shape'][0]}-B{c['batch']}-K{c['K']}")
def test_oracle_reproduces_fixture(case):
    shape = synth.custom_shape(*case["shape"], name="golden")
    w = synth.make_weights(shape, case["scales"])
    f32 = {n: w.f32(n) for n in ("lm_head", "embed", "gru_w_ih", "gru_w_hh", "fc1_w", "fc2_w",
                                 "fc2_b")}
    inp = synth.make_inputs(shape, case["batch"], case["input_seed"], 0)
    r = oracle.rollout(f32, inp.hidden_f32(), inp.step_s, inp.verified, case["K"])
    want_tok = np.asarray(case["tokens"])
    want_top = np.asarray(case["top1"], np.float64)
    want_margin = np.asarray(case["margin"], np.float64)
    # BLAS may sum in another order on another machine: tokens must match up
    # to the first near-tie (margin below 1e-4), logits to fp32 rounding
    for b in range(case["batch"]):
        for k in range(want_tok.shape[1]):
            if want_margin[b, k] < 1e-4:
                break
            assert r["tokens"][b, k] == want_tok[b, k], (b, k)
            assert abs(float(r["top1"][b, k]) - want_top[b, k]) <= 1e-5 * max(1.0, abs(want_top[b, k]))
    for got, want in zip(r["pools"], case["pools"]):
        assert (got is None) == (want is None)
        if want is not None:
            assert list(map(int, got)) == want
