"""Exact ties on the GPU: the lowest-id rules for the argmax and the pool cutoff.

The tie rules are readings of the pages ("feat: support tensor-parallel
Domino rollout", "Validation and limitations", leaves exact TopK cutoff ties
open): an argmax over equal corrected logits takes the lowest id, and equal
pool scores at the K-th place keep the lower id.  Random weights never make
an exact tie, so these models plant them, with arithmetic that is exact on
both sides:

* lm_head entries are multiples of 2^-6 in [-1/4, 1/4] and hiddens
  multiples of 2^-3 in [-2, 2] (both exact in bf16), so every base logit is
  a sum of multiples of 2^-9 far below 2^24 ulps: exact in fp32 in any
  summation order, on the matrix cores and in the oracle's BLAS alike.
  Pool scores and their ranking are then identical on both sides, and the
  coarse grid makes many accidental score ties besides the planted ones.
* Argmax ties: for a pair of ids (lo < hi), hi repeats lo's lm_head row and
  bias, and both fc2 rows are zero, so y_lo = y_hi exactly (base + (0 + b2))
  on both sides.  The hidden rows of steps 0, 1, 5 and 10 are 8 x lm_head[lo],
  which makes the pair win there: step 0 ties the first proposal, the
  others tie correction steps of the full vocabulary and of the pools
  (step 1, the first correction, is reached by every request).
  Even requests use one pair, odd requests another whose upper id is the
  last, ragged vocabulary tile.
* Cutoff tie: an id c2 > c1 repeats c1's lm_head row, and K is chosen so
  that c1 is request 0's K-th best id and c2 the next: the pool must hold
  c1 and not c2.

At a planted tie the oracle's margin is exactly 0, so the usual rule would
stop comparing there; these tests require the identical (lowest) id at those
steps and keep comparing the chain after them with the usual rule.
"""
import numpy as np
import pytest

from gru_corrected_draft_amd import rollout as R
from gru_corrected_draft_amd import synth
from tests import _gpu as G
from tests._parity import MARGIN_MIN, TOL

pytestmark = pytest.mark.gpu

TIE_STEPS = (0, 1, 5, 10)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _quant(x, step, lim):
    return (np.clip(np.rint(np.asarray(x, np.float64) / step), -lim / step, lim / step)
            * step).astype(np.float32)


def _store(shape, x):
    return synth.round_to_bf16_bits(x) if shape.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def tie_model(shape, pairs, cut_pair):
    """Weights with quantized lm_head, the argmax pairs planted (lm_head row
    and bias repeated, fc2 rows zero) and the cutoff pair's lm_head row
    repeated.  Returns (synth.Weights, float32 dict for the oracle)."""
    w = synth.make_weights(shape)
    f = {n: np.array(w.f32(n), np.float32, copy=True) for n in w.raw}
    f["lm_head"] = _quant(f["lm_head"], 2.0 ** -6, 0.25)
    for lo, hi in pairs:
        f["lm_head"][hi] = f["lm_head"][lo]
        f["fc2_w"][lo] = 0.0
        f["fc2_w"][hi] = 0.0
        f["fc2_b"][hi] = f["fc2_b"][lo]
    c1, c2 = cut_pair
    f["lm_head"][c2] = f["lm_head"][c1]
    raw = {n: _store(shape, a) for n, a in f.items()}
    out = synth.Weights(shape, raw)
    return out, {n: out.f32(n) for n in raw}


def tie_inputs(shape, f32, pairs, B, seed):
    inp = synth.make_inputs(shape, B, seed, 0)
    X = _quant(inp.hidden_f32(), 2.0 ** -3, 2.0)
    for b in range(B):
        lo = pairs[b % len(pairs)][0]
        for t in TIE_STEPS:
            X[b, t] = 8.0 * f32["lm_head"][lo]        # exact: multiples of 2^-3 within [-2, 2]
    return synth.Inputs(_store(shape, X), inp.step_s, inp.verified)


def cutoff_K(f32, X, c1, c2):
    """K that puts c1 last in request 0's pool and c2 just outside it."""
    import oracle
    base = oracle.base_logits(X[:1], f32["lm_head"])
    score = base[:, 0, :].max(axis=0) + np.float32(0.0)
    order = np.lexsort((np.arange(score.size), -score))
    p1, p2 = int(np.nonzero(order == c1)[0][0]), int(np.nonzero(order == c2)[0][0])
    assert score[c1] == score[c2] and p2 > p1
    return p1 + 1


def pick_cut_pair(shape, pairs, rank, seed):
    """(c1, c2): c1 ranked `rank` by request 0's unmodified score, c2 > c1
    ranked well below it (so repeating c1's row in c2 leaves c1's rank)."""
    import oracle
    w, f = tie_model(shape, pairs, (0, 0))
    X = tie_inputs(shape, f, pairs, 1, seed).hidden
    X = synth.bf16_bits_to_f32(X) if X.dtype == np.uint16 else X
    base = oracle.base_logits(X, f["lm_head"])
    score = base[:, 0, :].max(axis=0) + np.float32(0.0)
    order = np.lexsort((np.arange(score.size), -score))
    c1 = int(order[rank - 1])
    taken = {i for p in pairs for i in p}
    below = [int(v) for v in order[rank + 20:] if v > c1 and int(v) not in taken]
    return c1, max(below)


def compare_with_ties(tokens, top1, ref, tol, tie_ids):
    """The parity rule, except that a step where the oracle has an exact tie
    between planted ids must return the same (lowest) id and the chain is
    compared on after it.  Returns (checked, tie steps)."""
    B, T = tokens.shape
    checked = ties = 0
    for b in range(B):
        for k in range(T):
            m = float(ref["margin"][b, k])
            if m == 0.0 and int(ref["tokens"][b, k]) in tie_ids:
                assert tokens[b, k] == ref["tokens"][b, k], \
                    f"request {b} step {k}: exact tie, gpu {tokens[b, k]} oracle {ref['tokens'][b, k]}"
                ties += 1
                continue
            if m < MARGIN_MIN:
                break
            assert tokens[b, k] == ref["tokens"][b, k], \
                f"request {b} step {k}: gpu {tokens[b, k]} oracle {ref['tokens'][b, k]}"
            assert abs(float(top1[b, k]) - float(ref["top1"][b, k])) <= tol
            checked += 1
    return checked, ties


SMALL = synth.custom_shape(5003, 256, 128, 128, 128, "bf16", 91, name="tie-bf16")
DEEP = synth.custom_shape(3001, 1024, 256, 256, 256, "bf16", 92, name="tie-bf16-deep")
TINY = synth.custom_shape(4096, 256, 128, 128, 128, "fp32", 93, name="tie-fp32")

# (shape, batch, pool strategy): every LM-head kernel (row stream at 1 for
# H = 256, the whole-line one-request kernel at 1 for H = 1024, the 32x32
# kernel at 8 and 14, line copies at 40, register operands at 64), the
# full-vocabulary stream (row-major up to 16, tile order above), and each
# pool reader (whole-line gather up to 12, split at 14, gather above 16,
# group unions at r = 256)
CASES = [(SMALL, 1, 0), (SMALL, 8, 0), (SMALL, 14, 0), (SMALL, 40, 1), (DEEP, 64, 2),
         (DEEP, 64, 1), (TINY, 1, 0), (DEEP, 1, 0)]


def _pairs(shape):
    V = shape.vocab
    return [(17, V // 2 + 3), (1200, V - 1)]


@pytest.mark.parametrize("shape,B,strategy", CASES,
                         ids=[f"{s.name}-B{b}-s{st}" for s, b, st in CASES])
def test_exact_ties_lowest_id(shape, B, strategy):
    import oracle
    import torch
    pairs = _pairs(shape)
    seed = 4000 + B
    cut = pick_cut_pair(shape, pairs, rank=97 if shape.vocab > 4000 else 61, seed=seed)
    w, f32 = tie_model(shape, pairs, cut)
    inp = tie_inputs(shape, f32, pairs, B, seed)
    X = inp.hidden_f32()
    K_cut = cutoff_K(f32, X, *cut)
    dev = R.device_weights(w)
    h = R.DominoRollout(dev, max_batch=64, max_k=2048)
    try:
        h.set_pool_strategy(strategy)
        hid, s, ver = R.device_inputs(inp)
        tie_ids = {lo for lo, _ in pairs}
        for K in (0, K_cut, 300):
            G.log(f"[gpu-test] ties {shape.name} B={B} strategy={strategy} K={K} cut={cut}")
            tok, top = h.run(hid, s, ver, K)
            torch.cuda.synchronize()
            tok, top = tok.cpu().numpy(), top.cpu().numpy()
            ref = oracle.rollout(f32, X, inp.step_s, inp.verified, K)
            # the planted pairs tie at the first proposal of every request
            assert np.all(ref["margin"][:, 0] == 0.0)
            assert np.array_equal(tok[:, 0], ref["tokens"][:, 0])
            checked, ties = compare_with_ties(tok, top, ref, TOL[shape.dtype], tie_ids)
            assert ties >= 2 * B, f"only {ties} planted ties reached"
            # no step may ever return the upper id of a planted pair
            assert not np.isin(tok, [hi for _, hi in pairs]).any()
            base = h.read_workspace(0).cpu().numpy().reshape(15, B, -1)
            assert np.array_equal(base, oracle.base_logits(X, f32["lm_head"])), "base logits not exact"
            if K:
                ids = h.read_workspace(1).cpu().numpy().reshape(B, K)
                for b in range(B):
                    assert np.array_equal(ids[b], ref["pools"][b]), f"pool of request {b}, K={K}"
                if K == K_cut:
                    assert cut[0] in ids[0] and cut[1] not in ids[0]
            G.log(f"[gpu-test] ties K={K}: {ties} tie steps, {checked} other steps checked")
    finally:
        h.close()


FLAT = synth.custom_shape(5003, 256, 128, 128, 128, "bf16", 94, name="flat-bf16")


@pytest.mark.parametrize("B", [3, 40])
def test_all_scores_equal(B):
    """Every lm_head row the same: all base logits of a step are equal, so
    every id's pool score ties.  Every id is then a candidate of the last
    radix pass (a whole chunk of them, far more than the selection holds in
    registers), the pool is ids 0..K-1, and the first proposal is id 0."""
    import oracle
    import torch
    w = synth.make_weights(FLAT)
    f = {n: np.array(w.f32(n), np.float32, copy=True) for n in w.raw}
    f["lm_head"] = np.broadcast_to(_quant(f["lm_head"][:1], 2.0 ** -6, 0.25), f["lm_head"].shape).copy()
    raw = {n: _store(FLAT, a) for n, a in f.items()}
    wq = synth.Weights(FLAT, raw)
    f32 = {n: wq.f32(n) for n in raw}
    inp = synth.make_inputs(FLAT, B, 4500 + B, 0)
    X = _quant(inp.hidden_f32(), 2.0 ** -3, 2.0)
    inp = synth.Inputs(_store(FLAT, X), inp.step_s, inp.verified)
    h = R.DominoRollout(R.device_weights(wq), max_batch=64, max_k=5002)
    try:
        hid, s, ver = R.device_inputs(inp)
        for K in (1, 700, 5002):
            G.log(f"[gpu-test] all scores equal B={B} K={K}")
            tok, top = h.run(hid, s, ver, K)
            torch.cuda.synchronize()
            tok, top = tok.cpu().numpy(), top.cpu().numpy()
            ids = h.read_workspace(1).cpu().numpy().reshape(B, K)
            assert np.array_equal(ids, np.broadcast_to(np.arange(K, dtype=ids.dtype), (B, K)))
            ref = oracle.rollout(f32, X, inp.step_s, inp.verified, K)
            assert np.array_equal(ref["pools"], ids)
            assert np.all(tok[:, 0] == 0)
            checked, ties = compare_with_ties(tok, top, ref, TOL[FLAT.dtype], {0})
            G.log(f"[gpu-test] all scores equal K={K}: {ties} tie steps, {checked} other steps checked")
            assert ties >= B
    finally:
        h.close()
