"""Planted winners and losers on the GPU: a mutation check of every
correction kernel.

The corrected logit of id c at step k is y = base[k, b, c] + (fc2[c] . u + b2[c])
("[Spec] Add Domino projector support to DFlash speculative decoding (V2)",
"Implementation"; the correction is an argmax over the full vocabulary or the
request's pool).  Changing one bias therefore moves one candidate and nothing
else, and the outcome is known without an oracle:

* bias +64 on id c (far above any corrected logit of these models): every
  correction step of every request that can pick c (K0: all; a pool: the
  requests whose pool holds c) returns c, and the first proposal (base
  argmax, no bias) is unchanged; a request whose pool lacks c returns exactly
  the tokens and logits of the unmutated run, bit for bit.
* bias -64 on the id w that request 0 picks at its first correction: no
  correction step of any request returns w any more, and the whole run meets
  the oracle on the mutated weights (small shapes).

The cases reach each correction reader: the full-vocabulary stream (row-major
up to 16 requests, tile order above), the whole-line pool gather (up to 12),
the split gather (13-16), the wide gather (above 16) and the group unions, at
projector widths 128, 256 and 1024 (the 8B shape).
"""
import numpy as np
import pytest

from gru_corrected_draft_amd import rollout as R
from gru_corrected_draft_amd import synth
from tests import _gpu as G
from tests._parity import TOL, compare

pytestmark = pytest.mark.gpu

BOOST = 64.0

SMALL = synth.custom_shape(5003, 256, 128, 128, 128, "bf16", 77, name="small-bf16-ragged")
DEEP = synth.custom_shape(3001, 1024, 256, 256, 256, "bf16", 78, name="small-bf16-deep")

# (shape, B, K, pool strategy, compare with the oracle)
CASES = [
    (SMALL, 1, 0, 0, True), (SMALL, 8, 0, 0, True), (SMALL, 40, 0, 0, True),
    (SMALL, 1, 100, 0, True), (SMALL, 8, 300, 0, True), (SMALL, 14, 300, 0, True),
    (SMALL, 40, 300, 1, True), (DEEP, 64, 700, 2, True), (DEEP, 64, 0, 0, True),
    ("qwen3-8b", 1, 0, 0, False), ("qwen3-8b", 8, 2048, 0, False), ("qwen3-8b", 64, 2048, 2, False),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    G.drop_handles()


def _bias_variant(dev, edits):
    """The device weights with fc2_b entries replaced (every other tensor shared)."""
    out = dict(dev)
    b2 = dev["fc2_b"].clone()
    for i, v in edits.items():
        b2[i] = v
    out["fc2_b"] = b2
    return out


def _run(dev, shape, B, K, strategy, seed):
    import torch
    h = R.DominoRollout(dev, max_batch=max(B, 8), max_k=max(K, 1))
    try:
        h.set_pool_strategy(strategy)
        inp = synth.make_inputs(shape, B, seed, 0)
        hid, s, ver = R.device_inputs(inp)
        tok, top = h.run(hid, s, ver, K)
        torch.cuda.synchronize()
        pools = None
        if 0 < K < shape.vocab:
            pools = h.read_workspace(1).cpu().numpy().reshape(B, K)
        return tok.cpu().numpy(), top.cpu().numpy(), pools
    finally:
        h.close()


@pytest.mark.parametrize("shape,B,K,strategy,with_oracle", CASES,
                         ids=[f"{s if isinstance(s, str) else s.name}-B{b}-K{k}-s{st}"
                              for s, b, k, st, _ in CASES])
def test_planted_winner_and_loser(shape, B, K, strategy, with_oracle):
    import oracle
    shape = synth.MODELS[shape] if isinstance(shape, str) else shape
    model_key = shape if shape.name not in synth.MODELS else shape.name
    _, dev, f32 = G.model(model_key)
    V, seed = shape.vocab, 6100 + B
    G.log(f"[gpu-test] mutation {shape.name} B={B} K={K} strategy={strategy}: unmutated run")
    tok0, top0, pools0 = _run(dev, shape, B, K, strategy, seed)

    # the planted winner: an id in the ragged last tile for K0, one of
    # request 0's pool ids for pool runs (so some requests hold it and, with
    # a large vocabulary, others do not)
    c = V - 2 if pools0 is None else int(pools0[0][len(pools0[0]) // 3])
    G.log(f"[gpu-test] mutation: bias +{BOOST} on id {c}")
    tok1, top1, pools1 = _run(_bias_variant(dev, {c: BOOST}), shape, B, K, strategy, seed)
    assert np.array_equal(tok1[:, 0], tok0[:, 0]), "the first proposal carries no bias"
    if pools0 is not None:
        assert np.array_equal(pools1, pools0), "the pool is built from base logits only"
    holders = 0
    for b in range(B):
        if pools0 is None or c in pools0[b]:
            holders += 1
            assert np.all(tok1[b, 1:] == c), f"request {b}: planted winner {c} not taken: {tok1[b]}"
        else:
            assert np.array_equal(tok1[b], tok0[b]), f"request {b} without {c} in its pool changed"
            assert np.array_equal(top1[b], top0[b])
    assert holders >= 1

    # the planted loser: request 0's first correction
    w = int(tok0[0, 1])
    G.log(f"[gpu-test] mutation: bias -{BOOST} on id {w}")
    dev2 = _bias_variant(dev, {w: -BOOST})
    tok2, top2, _ = _run(dev2, shape, B, K, strategy, seed)
    assert np.array_equal(tok2[:, 0], tok0[:, 0])
    assert not np.any(tok2[:, 1:] == w), f"suppressed id {w} still chosen"
    assert tok2[0, 1] != tok0[0, 1]
    if with_oracle:
        f2 = dict(f32)
        b2 = np.array(f32["fc2_b"], np.float32, copy=True)
        b2[w] = -BOOST
        f2["fc2_b"] = b2
        inp = synth.make_inputs(shape, B, seed, 0)
        ref = oracle.rollout(f2, inp.hidden_f32(), inp.step_s, inp.verified, K)
        checked, _ = compare(tok2, top2, ref, TOL[shape.dtype])
        G.log(f"[gpu-test] mutation: loser run meets the oracle on {checked} steps")
        assert checked > 0
