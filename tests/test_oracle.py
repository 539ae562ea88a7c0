"""Pins of the CPU oracle against things other than itself (CPU only).

* float64 brute force with an independently written pool (union walk);
* PyTorch's own GRU / GRUCell (bias=False) and SiLU, the operators the
  pages name for the prefix and the feedback updates;
* closed forms: one-hot hiddens, h0 = 0 with zero GRU weights, fc2 = 0,
  K = 1, K >= V;
* invariants: p1 = base argmax for every K, pool nesting, batch
  independence, teacher forcing with the oracle's own tokens;
* planted mistakes (in a copy of the oracle, on the CPU) that the pins
  must catch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import domino_oracle as od
from tests._brute import brute_rollout, union_walk_pool

F32 = np.float32
T, S = 15, 14


def _rand_weights(rng, V, H, e, g, r, scale=1.0):
    n = lambda *shp, fan: (rng.standard_normal(shp) * scale / math.sqrt(fan)).astype(F32)
    return {"lm_head": n(V, H, fan=H), "embed": n(V, e, fan=1), "gru_w_ih": n(3 * g, e, fan=e),
            "gru_w_hh": n(3 * g, g, fan=g), "fc1_w": n(r, g, fan=g), "fc2_w": n(V, r, fan=r),
            "fc2_b": n(V, fan=r)}


def _rand_inputs(rng, B, V, H, r):
    return (rng.standard_normal((B, T, H)).astype(F32), rng.standard_normal((B, S, r)).astype(F32),
            rng.integers(0, V, B).astype(np.int32))


def _check_against_brute(out, ref, tol=2e-5, min_margin=1e-3, steps=T):
    """Tokens equal up to the first step with a near-tie; logits within tol there.

    The top-2 margin (winner minus runner-up over the step's candidates) is
    compared at every step up to and including that first near-tie step: it
    decides where the GPU parity rule stops checking a chain, and, unlike the
    winning id, it is a continuous function of the logits, so the fp32 and
    float64 values agree within tol even where the two pick different ids."""
    B = len(ref["tokens"])
    checked = 0
    for b in range(B):
        for k in range(steps):
            mg, mr = float(out["margin"][b, k]), ref["margin"][b][k]
            assert (math.isinf(mg) and math.isinf(mr)) or abs(mg - mr) <= tol, \
                ("margin", b, k, mg, mr)
            if mr < min_margin:
                break
            assert out["tokens"][b, k] == ref["tokens"][b][k], (b, k)
            assert abs(float(out["top1"][b, k]) - ref["top1"][b][k]) <= tol, (b, k)
            checked += 1
    return checked


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("K", [0, 1, 3, 7, 40, 47, 48, 60])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rollout_matches_float64_brute_force(K, seed):
    rng = np.random.default_rng(100 + seed)
    V, H, e, g, r, B = 48, 8, 4, 4, 4, 2
    w = _rand_weights(rng, V, H, e, g, r, scale=2.0)   # strong GRU / projector
    X, s, ver = _rand_inputs(rng, B, V, H, r)
    out = oracle.rollout(w, X, s, ver, K)
    ref = brute_rollout({k: v.astype(np.float64).tolist() for k, v in w.items()},
                        X.astype(np.float64).tolist(), s.astype(np.float64).tolist(), ver, K)
    checked = _check_against_brute(out, ref)
    assert checked >= 5
    for b in range(B):
        if ref["pools"][b] is None:
            assert out["pools"][b] is None
        else:
            assert out["pools"][b].tolist() == ref["pools"][b]


def test_teacher_forced_matches_brute_force_on_every_step():
    rng = np.random.default_rng(7)
    V, H, e, g, r, B = 40, 8, 4, 4, 4, 3
    w = _rand_weights(rng, V, H, e, g, r, scale=2.0)
    X, s, ver = _rand_inputs(rng, B, V, H, r)
    forced = rng.integers(0, V, (B, T)).astype(np.int32)
    for K in (0, 9):
        out = oracle.rollout(w, X, s, ver, K, forced=forced)
        ref = brute_rollout({k: v.astype(np.float64).tolist() for k, v in w.items()},
                            X.astype(np.float64).tolist(), s.astype(np.float64).tolist(), ver, K,
                            forced=forced.tolist())
        got = np.asarray(out["top1"], np.float64)
        assert np.max(np.abs(got - np.asarray(ref["top1"]))) < 2e-5


@pytest.mark.parametrize("P", [1, 2, 8, 14])
@pytest.mark.parametrize("K", [0, 5])
def test_truncated_rollout_matches_brute_force_prefix(P, K):
    """A rollout stopped after P proposals (the b8 serving variant verifies 8)
    is the first P columns of the whole block's rollout: the float64 brute
    force of the full chain, cut to P columns, pins it."""
    rng = np.random.default_rng(300 + P + K)
    V, H, e, g, r, B = 40, 8, 4, 4, 4, 3
    w = _rand_weights(rng, V, H, e, g, r, scale=2.0)
    X, s, ver = _rand_inputs(rng, B, V, H, r)
    out = oracle.rollout(w, X, s, ver, K, proposals=P)
    assert out["tokens"].shape == (B, P) and out["top1"].shape == (B, P)
    ref = brute_rollout({k: v.astype(np.float64).tolist() for k, v in w.items()},
                        X.astype(np.float64).tolist(), s.astype(np.float64).tolist(), ver, K)
    assert _check_against_brute(out, ref, steps=P) >= min(P, 2)
    # P = 1 is the plain argmax of base row 0
    if P == 1:
        base = np.asarray(X, np.float64) @ np.asarray(w["lm_head"], np.float64).T
        assert np.array_equal(out["tokens"][:, 0], np.argmax(base[:, 0], axis=1))


def test_truncated_rollout_rejects_bad_counts():
    rng = np.random.default_rng(9)
    w = _rand_weights(rng, 16, 8, 4, 4, 4)
    X, s, ver = _rand_inputs(rng, 1, 16, 8, 4)
    for P in (0, T + 1):
        with pytest.raises(ValueError):
            oracle.rollout(w, X, s, ver, 0, proposals=P)


# ------------------------------------------------- per-step projector offsets

def test_step_offsets_closed_forms_and_alignment():
    """s row j = fc1_x_w . X[b, j+1] + fc1_b: a zero weight leaves the bias, and
    a hidden that is one-hot at position k and unit i puts column i of the
    weight (plus the bias) into row k-1 only."""
    rng = np.random.default_rng(21)
    B, H, r = 2, 6, 5
    W = rng.standard_normal((r, H)).astype(F32)
    b1 = rng.standard_normal(r).astype(F32)
    X = rng.standard_normal((B, T, H)).astype(F32)
    s0 = oracle.step_offsets(X, np.zeros_like(W), b1)
    assert s0.shape == (B, S, r) and np.array_equal(s0, np.broadcast_to(b1, (B, S, r)))
    for k in (1, 7, 14):
        for i in (0, H - 1):
            Xo = np.zeros((B, T, H), F32)
            Xo[1, k, i] = 1.0
            got = oracle.step_offsets(Xo, W, b1)
            want = np.broadcast_to(b1, (B, S, r)).copy()
            want[1, k - 1] += W[:, i]
            assert np.allclose(got, want, atol=1e-6), (k, i)
    # position 0 (the verified token's hidden) never reaches s
    Xz = X.copy()
    Xz[:, 0] = 1e3
    assert np.array_equal(oracle.step_offsets(Xz, W, b1), oracle.step_offsets(X, W, b1))


def test_step_offsets_match_float64_loops():
    rng = np.random.default_rng(22)
    B, H, r = 2, 7, 3
    W = rng.standard_normal((r, H)).astype(F32)
    b1 = rng.standard_normal(r).astype(F32)
    X = rng.standard_normal((B, T, H)).astype(F32)
    got = oracle.step_offsets(X, W, b1)
    for b in range(B):
        for j in range(S):
            for n in range(r):
                ref = float(b1[n]) + sum(float(W[n, i]) * float(X[b, j + 1, i]) for i in range(H))
                assert abs(float(got[b, j, n]) - ref) < 1e-5


# --------------------------------------------------------- library routines

def test_gru_cell_matches_torch_grucell():
    rng = np.random.default_rng(3)
    B, e, g = 5, 24, 16
    x = rng.standard_normal((B, e)).astype(F32)
    h = rng.standard_normal((B, g)).astype(F32)
    w_ih = (rng.standard_normal((3 * g, e)) * 0.5).astype(F32)
    w_hh = (rng.standard_normal((3 * g, g)) * 0.5).astype(F32)
    cell = torch.nn.GRUCell(e, g, bias=False)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(w_ih))
        cell.weight_hh.copy_(torch.from_numpy(w_hh))
        ref = cell(torch.from_numpy(x), torch.from_numpy(h)).numpy()
    got = oracle.gru_cell(x, h, w_ih, w_hh)
    assert np.max(np.abs(got - ref)) < 1e-6


def test_two_token_prefix_matches_torch_gru():
    rng = np.random.default_rng(4)
    B, e, g, V = 3, 12, 10, 30
    E = rng.standard_normal((V, e)).astype(F32)
    w_ih = (rng.standard_normal((3 * g, e)) * 0.7).astype(F32)
    w_hh = (rng.standard_normal((3 * g, g)) * 0.7).astype(F32)
    v = rng.integers(0, V, B)
    p1 = rng.integers(0, V, B)
    gru = torch.nn.GRU(e, g, num_layers=1, bias=False, batch_first=True)
    with torch.no_grad():
        gru.weight_ih_l0.copy_(torch.from_numpy(w_ih))
        gru.weight_hh_l0.copy_(torch.from_numpy(w_hh))
        seq = torch.from_numpy(np.stack([E[v], E[p1]], axis=1))
        _, hn = gru(seq)          # h0 defaults to zeros
    h = np.zeros((B, g), F32)
    h = oracle.gru_cell(E[v], h, w_ih, w_hh)
    h = oracle.gru_cell(E[p1], h, w_ih, w_hh)
    assert np.max(np.abs(h - hn[0].numpy())) < 1e-6


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001).astype(F32)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(oracle.silu(x) - ref)) < 1e-6


# ------------------------------------------------------------- closed forms

def test_base_logits_one_hot_layout():
    """Hidden rows that are basis vectors select lm_head columns: base[t,b,v] =
    lm_head[v, i(b,t)].  Pins the step-major layout and the operand roles."""
    rng = np.random.default_rng(5)
    B, H, V = 3, T + 4, 11
    X = np.zeros((B, T, H), F32)
    idx = rng.integers(0, H, (B, T))
    for b in range(B):
        for t in range(T):
            X[b, t, idx[b, t]] = 1.0
    W = rng.standard_normal((V, H)).astype(F32)
    base = oracle.base_logits(X, W)
    assert base.shape == (T, B, V)
    for b in range(B):
        for t in range(T):
            assert np.array_equal(base[t, b], W[:, idx[b, t]])


def test_base_logits_within_fp32_dot_error_bound():
    """|fp32 result - exact| <= gamma_H * sum |x||w| (Higham's dot bound)."""
    rng = np.random.default_rng(6)
    B, H, V = 2, 512, 64
    X = rng.standard_normal((B, T, H)).astype(F32)
    W = rng.standard_normal((V, H)).astype(F32)
    base = oracle.base_logits(X, W).astype(np.float64)
    exact = np.einsum("bth,vh->tbv", X.astype(np.float64), W.astype(np.float64))
    absprod = np.einsum("bth,vh->tbv", np.abs(X).astype(np.float64), np.abs(W).astype(np.float64))
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    assert np.all(np.abs(base - exact) <= gamma * absprod)


def test_gru_closed_forms():
    g, e, B = 6, 5, 2
    rng = np.random.default_rng(8)
    x = rng.standard_normal((B, e)).astype(F32)
    h = rng.standard_normal((B, g)).astype(F32)
    zero_ih, zero_hh = np.zeros((3 * g, e), F32), np.zeros((3 * g, g), F32)
    # all-zero weights: r = z = 1/2, n = 0  ->  h' = h / 2
    assert np.allclose(oracle.gru_cell(x, h, zero_ih, zero_hh), 0.5 * h, atol=1e-7)
    # from h = 0 with zero weights the state stays exactly 0
    assert np.all(oracle.gru_cell(x, np.zeros_like(h), zero_ih, zero_hh) == 0)
    # a huge update-gate preactivation (z -> 1) keeps the state
    w_ih = zero_ih.copy()
    w_ih[g:2 * g, 0] = 1e4
    xx = np.abs(x) + 1.0
    assert np.allclose(oracle.gru_cell(xx, h, w_ih, zero_hh), h, atol=1e-6)
    # z -> 0 and r -> 1: h' = tanh(a_n + c_n)
    w_ih = zero_ih.copy()
    w_ih[:g, 0] = 1e4
    w_ih[g:2 * g, 0] = -1e4
    w_ih[2 * g:, :] = rng.standard_normal((g, e)).astype(F32)
    w_hh = zero_hh.copy()
    w_hh[2 * g:, :] = rng.standard_normal((g, g)).astype(F32)
    expect = np.tanh(xx @ w_ih[2 * g:].T + h @ w_hh[2 * g:].T)
    assert np.allclose(oracle.gru_cell(xx, h, w_ih, w_hh), expect, atol=1e-6)


def _tiny(seed=11, V=64, H=16, e=8, g=8, r=8, B=2, scale=1.0):
    rng = np.random.default_rng(seed)
    w = _rand_weights(rng, V, H, e, g, r, scale)
    return w, _rand_inputs(rng, B, V, H, r)


def test_zero_projector_is_plain_per_position_argmax():
    """fc2 = 0 and b2 = 0: every proposal is the argmax of its own base row."""
    w, (X, s, ver) = _tiny()
    w["fc2_w"][:] = 0
    w["fc2_b"][:] = 0
    out = oracle.rollout(w, X, s, ver, 0)
    base = oracle.base_logits(X, w["lm_head"])
    assert np.array_equal(out["tokens"], np.argmax(base, axis=2).T)


def test_zero_gru_makes_steps_one_shot_and_aligned():
    """W_ih = W_hh = 0 keeps h = 0, so u_k = SiLU(s_{k-1}) and step k scores
    base row k.  Give step k its own projector unit that only fc2 row
    target_k reads: switching on unit k-1 of s row k-1 must make target_k win
    at step k, and nowhere else."""
    V, H, e, g, r, B = 32, 8, 4, 4, 16, 1
    w, (X, s, ver) = _tiny(V=V, H=H, e=e, g=g, r=r, B=B)
    w["gru_w_ih"][:] = 0
    w["gru_w_hh"][:] = 0
    w["fc2_b"][:] = 0
    w["lm_head"][:] = 0              # base logits all zero
    w["fc2_w"][:] = 0
    targets = (np.arange(1, S + 1) * 2 + 1) % V
    for k in range(1, S + 1):
        w["fc2_w"][targets[k - 1], k - 1] = 1.0
    s[:] = -20.0                     # SiLU(-20) ~ -4e-8: every unit off
    for k in range(1, S + 1):
        s_k = s.copy()
        s_k[0, k - 1, k - 1] = 5.0   # unit k-1 on, in s row k-1 only
        res = oracle.rollout(w, X, s_k, ver, 0)
        assert res["tokens"][0, k] == targets[k - 1]
        others = [res["tokens"][0, j] for j in range(1, S + 1) if j != k]
        assert targets[k - 1] not in others


def test_K_at_least_V_is_full_vocabulary_exactly():
    w, (X, s, ver) = _tiny(scale=2.0)
    V = w["lm_head"].shape[0]
    ref = oracle.rollout(w, X, s, ver, 0)
    for K in (V, V + 1, 10 * V):
        out = oracle.rollout(w, X, s, ver, K)
        assert np.array_equal(out["tokens"], ref["tokens"])
        assert np.array_equal(out["top1"], ref["top1"])


def test_K1_closed_form():
    """K = 1: the pool is the single id with the best block-max score, so every
    corrected proposal is that id; p1 is still the full-vocabulary argmax."""
    w, (X, s, ver) = _tiny(scale=2.0, B=3)
    out = oracle.rollout(w, X, s, ver, 1)
    base = oracle.base_logits(X, w["lm_head"])
    for b in range(X.shape[0]):
        best = int(np.argmax(base[:, b, :].max(axis=0)))
        assert np.all(out["tokens"][b, 1:] == best)
        assert out["tokens"][b, 0] == int(np.argmax(base[0, b]))


@pytest.mark.parametrize("K", [0, 1, 5, 20, 63, 64])
def test_first_proposal_is_base_argmax_for_every_K(K):
    w, (X, s, ver) = _tiny(scale=3.0, B=3)
    base = oracle.base_logits(X, w["lm_head"])
    out = oracle.rollout(w, X, s, ver, K)
    assert np.array_equal(out["tokens"][:, 0], np.argmax(base[0], axis=1))


def test_pool_equals_union_walk_for_every_K_with_ties():
    rng = np.random.default_rng(12)
    V = 37
    rows = rng.integers(-3, 4, (T, V)).astype(F32)   # many exact ties
    rows[rows == 0] = -0.0                            # signed zeros tie with +0
    rows[3, 5] = 0.0
    for K in range(1, V + 2):
        got = oracle.candidate_pool(rows, K)
        want = union_walk_pool(rows.astype(np.float64).tolist(), K)
        if K >= V:
            assert got is None
        else:
            assert got.tolist() == want, K


def test_pool_is_nested_in_K():
    rng = np.random.default_rng(13)
    rows = rng.standard_normal((T, 200)).astype(F32)
    prev = set()
    for K in range(1, 200):
        cur = set(oracle.candidate_pool(rows, K).tolist())
        assert prev < cur and len(cur) == K
        prev = cur


def test_argmax_ties_lowest_id_and_signed_zero():
    y = np.array([-1.0, 0.0, -0.0, 0.0], F32)
    assert oracle.first_max_index(y) == 1
    y = np.array([-0.0, 0.0], F32)
    assert oracle.first_max_index(y) == 0
    top, mar = oracle.top1_and_margin(np.array([2.0, 1.0, 2.0], F32))
    assert top == 2.0 and mar == 0.0


def test_batch_independence():
    w, (X, s, ver) = _tiny(scale=2.0, B=4)
    for K in (0, 6):
        full = oracle.rollout(w, X, s, ver, K)
        for b in range(4):
            one = oracle.rollout(w, X[b:b + 1], s[b:b + 1], ver[b:b + 1], K)
            assert np.array_equal(one["tokens"][0], full["tokens"][b])
            assert np.allclose(one["top1"][0], full["top1"][b], atol=1e-6)


def test_teacher_forcing_with_own_tokens_is_identity():
    w, (X, s, ver) = _tiny(scale=2.0, B=2)
    for K in (0, 6):
        free = oracle.rollout(w, X, s, ver, K)
        forced = oracle.rollout(w, X, s, ver, K, forced=free["tokens"])
        assert np.array_equal(free["tokens"], forced["tokens"])
        assert np.array_equal(free["top1"], forced["top1"])


def test_negative_K_rejected():
    with pytest.raises(ValueError):
        oracle.candidate_pool(np.zeros((T, 4), F32), -1)


# ------------------------------------------------------------ planted mistakes

_orig_cell = od.gru_cell
_orig_pool = od.candidate_pool
_orig_base = od.base_logits

def _mut_cell_swapped_gates(x, h, w_ih, w_hh):
    g = h.shape[1]
    perm = np.r_[g:2 * g, 0:g, 2 * g:3 * g]        # r and z rows swapped
    return _orig_cell(x, h, w_ih[perm], w_hh[perm])


def _mut_cell_no_reset(x, h, w_ih, w_hh):
    g = h.shape[1]
    a, c = x @ w_ih.T, h @ w_hh.T
    z = od._sigmoid(a[:, g:2 * g] + c[:, g:2 * g])
    n = np.tanh(a[:, 2 * g:] + c[:, 2 * g:])        # reset gate dropped
    return (1 - z) * n + z * h


def _mut_cell_z_flipped(x, h, w_ih, w_hh):
    g = h.shape[1]
    a, c = x @ w_ih.T, h @ w_hh.T
    r = od._sigmoid(a[:, :g] + c[:, :g])
    z = od._sigmoid(a[:, g:2 * g] + c[:, g:2 * g])
    n = np.tanh(a[:, 2 * g:] + r * c[:, 2 * g:])
    return z * n + (1 - z) * h                       # interpolation reversed


def _margin_over_full_vocabulary(w, X, out, rec):
    """A plausible mistake in a pool run: the runner-up taken over the whole
    vocabulary's corrected logits instead of the request's pool."""
    m = np.array(out["margin"], copy=True)
    F2, b2 = w["fc2_w"], w["fc2_b"]
    for k in range(1, T):
        u = rec["u"][k - 1]
        for b in range(X.shape[0]):
            y = rec["base"][k, b] + (u[b] @ F2.T + b2)
            win = int(out["tokens"][b, k])
            m[b, k] = out["top1"][b, k] - np.delete(y, win).max()
    return dict(out, margin=m)


def _margin_second_distinct(out, rec):
    """Another: the runner-up as the second distinct value (a tie then gives
    a positive margin instead of 0)."""
    m = np.array(out["margin"], copy=True)
    for k in range(1, T):
        for b, y in enumerate(rec["y"][k - 1]):
            vals = np.unique(y)
            m[b, k] = vals[-1] - vals[-2] if len(vals) > 1 else np.inf
    return dict(out, margin=m)


@pytest.mark.parametrize("K", [0, 6])
def test_margin_matches_brute_force_and_catches_mistakes(K):
    """Oracle margin = float64 brute-force margin at every compared step, for
    the full vocabulary and a pool, including a planted exact tie (two ids
    with identical lm_head and fc2 rows and bias), where it must be 0."""
    rng = np.random.default_rng(33)
    V, H, e, g, r, B = 40, 8, 4, 4, 4, 3
    w = _rand_weights(rng, V, H, e, g, r, scale=2.0)
    X, s, ver = _rand_inputs(rng, B, V, H, r)
    wd = {k: v.astype(np.float64).tolist() for k, v in w.items()}
    rec = {}
    out = oracle.rollout(w, X, s, ver, K, record=rec)
    ref = brute_rollout(wd, X.astype(np.float64).tolist(), s.astype(np.float64).tolist(), ver, K)
    assert _check_against_brute(out, ref) >= 5
    if K:
        with pytest.raises(AssertionError, match="margin"):
            _check_against_brute(_margin_over_full_vocabulary(w, X, out, rec), ref)
    # planted tie: id 30 duplicates id 7 (lm_head, fc2, bias); hidden rows
    # aligned with that lm_head row make the pair the winner at steps 3 and 9
    w2 = {k: v.copy() for k, v in w.items()}
    for n in ("lm_head", "fc2_w", "fc2_b"):
        w2[n][30] = w2[n][7]
    X2 = X.copy()
    X2[:, 3] = 3.0 * w2["lm_head"][7]
    X2[:, 9] = 3.0 * w2["lm_head"][7]
    rec2 = {}
    out2 = oracle.rollout(w2, X2, s, ver, K, record=rec2)
    ref2 = brute_rollout({k: v.astype(np.float64).tolist() for k, v in w2.items()},
                         X2.astype(np.float64).tolist(), s.astype(np.float64).tolist(), ver, K)
    ties = 0
    for b in range(B):
        for k in (3, 9):
            if out2["tokens"][b, k] in (7, 30):
                assert out2["tokens"][b, k] == 7 and out2["margin"][b, k] == 0.0
                assert ref2["tokens"][b][k] == 7 and ref2["margin"][b][k] == 0.0
                ties += 1
    assert ties >= B
    _check_against_brute(out2, ref2, steps=3)
    with pytest.raises(AssertionError, match="margin"):
        _check_against_brute(_margin_second_distinct(out2, rec2), ref2, steps=4)


@pytest.mark.parametrize("mutation", ["swapped_gates", "no_reset", "z_flipped", "s_shift",
                                      "no_base", "no_bias", "transposed_fc1", "pool_min",
                                      "pool_rows_1_to_14"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    rng = np.random.default_rng(21)
    V, H, e, g, r, B = 40, 8, 4, 4, 4, 2
    w = _rand_weights(rng, V, H, e, g, r, scale=2.5)
    X, s, ver = _rand_inputs(rng, B, V, H, r)
    K = 6 if mutation.startswith("pool") else 0
    ref = brute_rollout({k: v.astype(np.float64).tolist() for k, v in w.items()},
                        X.astype(np.float64).tolist(), s.astype(np.float64).tolist(), ver, K)
    if mutation == "swapped_gates":
        monkeypatch.setattr(od, "gru_cell", _mut_cell_swapped_gates)
    elif mutation == "no_reset":
        monkeypatch.setattr(od, "gru_cell", _mut_cell_no_reset)
    elif mutation == "z_flipped":
        monkeypatch.setattr(od, "gru_cell", _mut_cell_z_flipped)
    elif mutation == "s_shift":
        s = np.concatenate([s[:, 1:], s[:, :1]], axis=1)       # s row k instead of k-1
    elif mutation == "no_base":
        monkeypatch.setattr(od, "base_logits",
                            lambda X_, W_: np.concatenate([_orig_base(X_, W_)[:1],
                                                           0 * _orig_base(X_, W_)[1:]]))
    elif mutation == "no_bias":
        w = dict(w, fc2_b=np.zeros_like(w["fc2_b"]))
    elif mutation == "transposed_fc1":
        w = dict(w, fc1_w=np.ascontiguousarray(w["fc1_w"].T))
    elif mutation == "pool_min":
        monkeypatch.setattr(od, "candidate_pool", lambda bb, K_: _orig_pool(-bb, K_))
    elif mutation == "pool_rows_1_to_14":
        monkeypatch.setattr(od, "candidate_pool",
                            lambda bb, K_: _orig_pool(bb[1:], K_))
    out = od.rollout(w, X, s, ver, K)
    with pytest.raises(AssertionError):
        _check_against_brute(out, ref)

