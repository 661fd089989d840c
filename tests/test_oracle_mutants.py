"""Planted mistakes: each broken copy of the oracle must fail at least one pin.

The copy below follows the oracle's steps with one switch per plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a
wrong mask). With no switch set it must pass every pin, so a mutant that
fails is failing because of its planted mistake. CPU only.
"""
import numpy as np
import pytest

from tests.oracle_pins import PINS

MUTANTS = [
    "no_scale_in_scores", "no_scale_in_dq", "no_scale_in_dk", "dk_not_transposed",
    "dv_not_transposed", "rowsum_term_dropped", "ds_sign_flipped", "lse_without_max",
    "causal_strict", "kv_len_ignored", "softmax_over_columns", "o_uses_pt",
    "dq_uses_q", "scale_not_fp32", "causal_mask_in_fwd_only", "lse_log2",
]


def _mutant_oracle(bug):
    def fwd(q, k, v, scale, causal, kv_len, probs=False):
        q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
        s = float(scale) if bug == "scale_not_fp32" else float(np.float32(scale))
        S = (1.0 if bug == "no_scale_in_scores" else s) * (q @ k.T)
        n_q, n_k = S.shape
        cols = np.arange(n_k)
        lim = n_k if (kv_len is None or bug == "kv_len_ignored") else kv_len
        vis = np.broadcast_to(cols[None, :] < lim, S.shape).copy()
        if causal and not (probs and bug == "causal_mask_in_fwd_only"):
            rows = np.arange(n_q)[:, None]
            vis &= (cols[None, :] < rows) if bug == "causal_strict" else (cols[None, :] <= rows)
        S = np.where(vis, S, -np.inf)
        anyv = vis.any(axis=1, keepdims=True)
        m = np.where(anyv, np.max(S, axis=1, keepdims=True, initial=-np.inf), 0.0)
        E = np.where(vis, np.exp(S - m), 0.0)
        ell = E.sum(axis=1, keepdims=True)
        if bug == "softmax_over_columns":
            colsum = E.sum(axis=0, keepdims=True)
            P = np.divide(E, colsum, out=np.zeros_like(E), where=colsum > 0)
        else:
            P = np.divide(E, ell, out=np.zeros_like(E), where=anyv)
        if probs:
            return P
        O = (P.T if bug == "o_uses_pt" else P) @ v
        logl = np.log2 if bug == "lse_log2" else np.log
        lse = (0.0 if bug == "lse_without_max" else m) + logl(np.where(anyv, ell, 1.0))
        lse = np.where(anyv, lse, -np.inf).reshape(-1)
        return O, lse

    def bwd(q, k, v, do, scale, causal, kv_len):
        q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
        s = float(scale) if bug == "scale_not_fp32" else float(np.float32(scale))
        P = fwd(q, k, v, scale, causal, kv_len, probs=True)
        dV = (P if bug == "dv_not_transposed" else P.T) @ do
        dP = do @ v.T
        rd = 0.0 if bug == "rowsum_term_dropped" else (P * dP).sum(axis=1, keepdims=True)
        dS = P * ((rd - dP) if bug == "ds_sign_flipped" else (dP - rd))
        dQ = (1.0 if bug == "no_scale_in_dq" else s) * (dS @ (q if bug == "dq_uses_q" else k))
        dK = (1.0 if bug == "no_scale_in_dk" else s) * ((dS if bug == "dk_not_transposed" else dS.T) @ q)
        return dQ, dK, dV

    return fwd, bwd


def _failing_pins(bug):
    fwd, bwd = _mutant_oracle(bug)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fwd, bwd)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_passes_every_pin():
    assert _failing_pins(None) == []


@pytest.mark.parametrize("bug", MUTANTS)
def test_mutant_is_caught(bug):
    assert _failing_pins(bug), f"no pin catches the planted mistake {bug!r}"
