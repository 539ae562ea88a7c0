"""Comparison rule between the HIP rollout and the CPU oracle.

Per request, proposal ids must be identical for steps 0..14 up to, but not
including, the first step whose oracle top-2 margin is below ``margin_min``
(0.05): from there on two correct implementations may legitimately follow
different chains, so that step and all later ones are excluded.  At every
checked step the GPU's top-1 corrected logit must lie within ``tol`` of the
oracle's (3e-2 for bf16 models, 1e-4 for fp32 models).
"""
import numpy as np

TOL = {"bf16": 3e-2, "fp32": 1e-4}
MARGIN_MIN = 0.05


def compare(tokens, top1, ref, tol, margin_min=MARGIN_MIN):
    """Returns (checked, excluded) step counts; raises AssertionError on a mismatch."""
    tokens = np.asarray(tokens)
    top1 = np.asarray(top1, np.float64)
    B, T = tokens.shape
    checked = excluded = 0
    for b in range(B):
        for k in range(T):
            if ref["margin"][b, k] < margin_min:
                excluded += T - k
                break
            assert tokens[b, k] == ref["tokens"][b, k], \
                f"request {b} step {k}: gpu {tokens[b, k]} oracle {ref['tokens'][b, k]} " \
                f"(oracle margin {ref['margin'][b, k]:.4g})"
            err = abs(top1[b, k] - float(ref["top1"][b, k]))
            assert err <= tol, f"request {b} step {k}: top-1 logit error {err:.3g} > {tol}"
            checked += 1
    return checked, excluded


def compare_forced(top1, ref, tol):
    """Teacher-forced runs: every step's winning logit within tol."""
    err = np.max(np.abs(np.asarray(top1, np.float64) - np.asarray(ref["top1"], np.float64)))
    assert err <= tol, f"teacher-forced top-1 logit error {err:.3g} > {tol}"
    return err
