"""CPU oracle of the Domino draft-block rollout.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run this module.  It shares no code with the HIP path and imports
nothing from the product package: it takes plain NumPy arrays and returns
plain NumPy arrays.

It is a slow, direct statement of what the rollout computes, in float32
(weights and hiddens arrive as float32 arrays holding bf16-representable
values for the bf16 models), with NumPy's BLAS as the only library
primitive.  Sources, cited by page title and section:

* [DFV2] "Add correctness-first Domino support to DFlash V2" (sglang PR
  #31328), section "Design": 15 proposals per block of 16; the first is the
  full-vocabulary DFlash argmax; a bias-free prefix GRU is run over
  [verified_token, first_proposal]; every realised proposal is fed back
  before the next correction step; the base LM-head projection stays
  full-vocabulary; correction runs over one per-request, block-shared
  candidate pool of K ids (K=0 means the full vocabulary); nn.GRU for the
  2-token prefix and GRUCell for the 13 one-token feedback updates.
  Its commit text (Domino drafter training backend): the correction head is
  an embed_proj over [backbone hidden | GRU state] emitting a full-vocab
  logit delta added to the base logits.
* [SPEC] "[Spec] Add Domino projector support to DFlash speculative decoding
  (V2)" (sglang PR #28998), sections "Motivation" and "Implementation": the
  per-step bias is SiLU(z+s)·fc2ᵀ + bias, added to the lm_head logits, then a
  full-vocabulary argmax; each selected token feeds the next GRU step.
* [TP] "feat: support tensor-parallel Domino rollout" (sglang PR #32018),
  sections "Implementation" and "Validation and limitations": the first
  proposal stays a global full-vocabulary argmax; the pool is a TopK whose
  cutoff ties the pages leave open; step-major packing of the base logits.

Readings where the pages leave a step open (each is listed in the design
notes of the repository):
* h0 = 0 (nn.GRU's default when no initial state is passed).
* GRU input x = E[token] with E a [V, e] table; gate rows ordered (r, z, n)
  as in PyTorch's GRU, no biases.
* z = fc1 · h_GRU (no fc1 bias); s (width r) is the backbone-hidden half of
  embed_proj's input plus the fc1 bias, supplied per step by the caller.
* Correction step k (1..14) scores base row k and uses s row k-1; the GRU
  state has then consumed [verified, p1, ..., pk].
* Pool score of a vocabulary id = the maximum of its 15 base logits in the
  block; the K best ids by (score descending, id ascending).
* Argmax ties go to the lowest id; -0.0 compares equal to +0.0.
* K = 0 or K >= V is the full vocabulary.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return F32(1.0) / (F32(1.0) + np.exp(-x))


def silu(x):
    """SiLU(x) = x·σ(x) — [SPEC] "Implementation" (fused SiLU(z+s) scoring)."""
    return x * _sigmoid(x)


def base_logits(hidden: np.ndarray, lm_head: np.ndarray) -> np.ndarray:
    """Base LM-head logits of every draft position, full vocabulary.

    hidden [B, T, H] float32, lm_head [V, H] float32  ->  [T, B, V] float32
    with base[t, b, v] = sum_i hidden[b, t, i] · lm_head[v, i].

    [DFV2] "Design" (base projection stays full-vocabulary); the result is
    laid out step-major, as [TP] "Rollout performance" describes the packing.
    """
    B, T, H = hidden.shape
    rows = np.ascontiguousarray(hidden.transpose(1, 0, 2)).reshape(T * B, H)
    out = rows @ lm_head.T
    return out.reshape(T, B, lm_head.shape[0])


def first_max_index(y: np.ndarray) -> int:
    """Index of the largest entry, lowest index on ties (NumPy's argmax)."""
    return int(np.argmax(y))


def top1_and_margin(y: np.ndarray):
    """(top-1 value, top-1 minus the runner-up); margin is +inf for one entry."""
    j = first_max_index(y)
    top = y[j]
    if y.shape[0] == 1:
        return top, np.inf
    rest = np.delete(y, j)
    return top, top - rest.max()


def candidate_pool(base_b: np.ndarray, K: int):
    """Block-shared candidate pool of one request.

    base_b [T, V] are the request's base logits of the whole block.  Returns
    None for the full vocabulary (K = 0 or K >= V), else the K ids ranked
    first by (max over the block's rows descending, id ascending), sorted by
    id.  [DFV2] "Design" (one per-request, block-shared pool, K=0 = full
    vocabulary); [TP] "Implementation" (block-shared K2048 pool),
    "Validation and limitations" (cutoff ties: resolved here by lowest id).
    """
    if K < 0:
        raise ValueError("K must be >= 0")
    V = base_b.shape[1]
    if K == 0 or K >= V:
        return None
    score = base_b.max(axis=0) + F32(0.0)          # -0.0 -> +0.0
    order = np.lexsort((np.arange(V), -score))    # score desc, then id asc
    return np.sort(order[:K]).astype(np.int64)


def gru_cell(x: np.ndarray, h: np.ndarray, w_ih: np.ndarray, w_hh: np.ndarray) -> np.ndarray:
    """One bias-free GRU update (PyTorch GRUCell semantics, gates r, z, n).

    x [B, e], h [B, g], w_ih [3g, e], w_hh [3g, g]  ->  h' [B, g]
      a = W_ih x,  c = W_hh h
      r = σ(a_r + c_r),  z = σ(a_z + c_z),  n = tanh(a_n + r ⊙ c_n)
      h' = (1 - z) ⊙ n + z ⊙ h
    [DFV2] "Design" (bias-free prefix GRU; nn.GRU / ATen GRUCell).
    """
    g = h.shape[1]
    a = x @ w_ih.T
    c = h @ w_hh.T
    r = _sigmoid(a[:, :g] + c[:, :g])
    z = _sigmoid(a[:, g:2 * g] + c[:, g:2 * g])
    n = np.tanh(a[:, 2 * g:] + r * c[:, 2 * g:])
    return (F32(1.0) - z) * n + z * h


def step_offsets(hidden: np.ndarray, fc1_x_w: np.ndarray, fc1_b: np.ndarray) -> np.ndarray:
    """Per-step projector offsets s [B, 14, r] from the block's hiddens.

    The projector's first layer reads [backbone hidden | GRU state] ("Add
    correctness-first Domino support to DFlash V2", commit text); its GRU
    half is fc1_w, applied to h inside the rollout, and this is the other
    half plus the layer's bias: s row j of request b = fc1_x_w · X[b, j+1] +
    fc1_b, j = 0..13.  Row j feeds correction step j+1, which scores base row
    j+1, the LM-head row of that same hidden (step alignment of the rollout
    loop below).  fp32 like the rest of the oracle.
    """
    X = np.asarray(hidden, F32)
    W = np.asarray(fc1_x_w, F32)
    b1 = np.asarray(fc1_b, F32)
    return (X[:, 1:, :] @ W.T + b1).astype(F32)


def rollout(weights: dict, hidden: np.ndarray, step_s: np.ndarray, verified: np.ndarray,
            K: int, forced: np.ndarray | None = None, record: dict | None = None,
            proposals: int | None = None) -> dict:
    """The whole draft-block rollout for B requests.

    weights: float32 arrays lm_head [V,H], embed [V,e], gru_w_ih [3g,e],
    gru_w_hh [3g,g], fc1_w [r,g], fc2_w [V,r], fc2_b [V].
    hidden [B,15,H], step_s [B,14,r], verified [B] int, K >= 0.
    forced [B,15] (optional): teacher forcing — the GRU consumes forced[:, j]
    in place of proposal j+1 (the selections are still reported).
    proposals (optional, 1..15): stop after that many proposals, i.e. after
    proposals-1 correction steps (a truncated rollout, as when the target
    verifies only the first positions of the block: "Qwen3.6-27B checkpoint
    and full serving benchmark", Methods, b8).  The base logits, the first
    proposal and the pool are those of the whole block, so the result is the
    first `proposals` columns of the full rollout.

    Returns tokens [B,P] int32, top1 [B,P] and margin [B,P] float32 (P = 15
    or `proposals`; column 0 from base row 0, column k from correction step
    k) and the pools (list of id arrays, None = full vocabulary).

    Order of work, [DFV2] "Design" and [SPEC] "Motivation":
      1. base logits of all 15 positions (full vocabulary);
      2. p1 = argmax of base row 0 over the full vocabulary ([TP]
         "Implementation": the first proposal stays a full-vocabulary argmax);
      3. the per-request pool from the block's base rows (if 0 < K < V);
      4. h = 0; h = cell(E[verified]); h = cell(E[p1])   (2-token prefix);
      5. for k = 1..14: u = SiLU(fc1·h + s[k-1]);
         y = base[k] + (fc2·u + b2) over the candidates; p[k+1] = argmax y;
         if k < 14: h = cell(E[p[k+1]], h)   (13 one-token feedback updates).
    """
    W = {k: np.asarray(v, dtype=F32) for k, v in weights.items()}
    lm, E = W["lm_head"], W["embed"]
    w_ih, w_hh, F1, F2, b2 = W["gru_w_ih"], W["gru_w_hh"], W["fc1_w"], W["fc2_w"], W["fc2_b"]
    B, T, _ = hidden.shape
    P = T if proposals is None else int(proposals)
    if not 1 <= P <= T:
        raise ValueError(f"proposals must be in [1, {T}]")
    S = P - 1                  # correction steps run
    V = lm.shape[0]
    g = w_hh.shape[1]

    base = base_logits(np.asarray(hidden, F32), lm)
    tokens = np.zeros((B, P), np.int32)
    top1 = np.zeros((B, P), F32)
    margin = np.zeros((B, P), F32)

    for b in range(B):
        j = first_max_index(base[0, b])
        tokens[b, 0] = j
        top1[b, 0], margin[b, 0] = top1_and_margin(base[0, b])
    pools = [candidate_pool(base[:, b, :], K) for b in range(B)]

    def fed(j):  # token consumed by the GRU for proposal slot j
        return tokens[:, j] if forced is None else np.asarray(forced[:, j])

    h = np.zeros((B, g), F32)
    if S > 0:  # the prefix only feeds the correction steps
        h = gru_cell(E[np.asarray(verified, np.int64)], h, w_ih, w_hh)
        h = gru_cell(E[fed(0).astype(np.int64)], h, w_ih, w_hh)
    if record is not None:
        record.update(base=base, pools=pools, h=[h.copy()], u=[], y=[])

    for k in range(1, S + 1):
        z = h @ F1.T
        u = silu(z + np.asarray(step_s[:, k - 1], F32))
        full = None
        if any(C is None for C in pools):
            full = u @ F2.T            # [B, V]: fc2·u of every request at once
        ys = []
        for b in range(B):
            C = pools[b]
            if C is None:
                y = base[k, b] + (full[b] + b2)
                j = first_max_index(y)
                tok = j
            else:
                y = base[k, b, C] + (F2[C] @ u[b] + b2[C])
                j = first_max_index(y)
                tok = int(C[j])
            tokens[b, k] = tok
            top1[b, k], margin[b, k] = top1_and_margin(y)
            ys.append(y)
        if k < S:
            h = gru_cell(E[fed(k).astype(np.int64)], h, w_ih, w_hh)
        if record is not None:
            record["u"].append(u)
            record["y"].append(ys)
            record["h"].append(h.copy())

    return {"tokens": tokens, "top1": top1, "margin": margin, "pools": pools, "vocab": V}
