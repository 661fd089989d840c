"""Pins of the oracle's attention with fused dropout (CPU only).

The generator is checked against its published known-answer values; the
keep decision against the exact keep rate (256 - t) / 256 and byte
uniformity; the scaling against the expectation over seeds (E[Z c] = 1);
p = 0 against the plain oracle; the backward against torch autograd of the
same masked forward expression and against finite differences. A copy of
the oracle with one planted mistake per switch must fail at least one pin,
and with no switch set must pass them all.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dropout as od

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


class Impl:
    """The oracle's dropout functions, or a copy with one planted mistake."""

    def __init__(self, bug=None):
        self.bug = bug

    # -- generator --------------------------------------------------------
    def philox(self, counter, key):
        if self.bug is None:
            return od.philox4x32_10(counter, key)
        M0, M1 = 0xD2511F53, 0xCD9E8D57
        if self.bug == "philox_swap_multipliers":
            M0, M1 = M1, M0
        c = [np.asarray(x, np.uint64) & 0xFFFFFFFF for x in np.broadcast_arrays(*counter)]
        k0, k1 = int(key[0]), int(key[1])
        for _ in range(9 if self.bug == "philox_nine_rounds" else 10):
            p0, p1 = c[0] * np.uint64(M0), c[2] * np.uint64(M1)
            c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & np.uint64(0xFFFFFFFF),
                 (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & np.uint64(0xFFFFFFFF)]
            if self.bug != "philox_no_key_bump":
                k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
        return [x.astype(np.uint32) for x in c]

    def keep(self, n_q, n_k, bh, p, seed, offset=0):
        if self.bug is None:
            return od.dropout_keep(n_q, n_k, bh, p, seed, offset)
        t = od.dropout_threshold(p)
        I, J = np.meshgrid(np.arange(n_q), np.arange(n_k), indexing="ij")
        out = self.philox((J >> 2, I >> 2, np.full_like(I, bh), np.full_like(I, offset)),
                          (seed & 0xFFFFFFFF, seed >> 32))
        byte = (np.choose(I & 3, out).astype(np.uint64) >> (8 * (J & 3)).astype(np.uint64)) & np.uint64(255)
        if self.bug == "keep_strict":
            return byte > np.uint64(t)
        if self.bug == "keep_inverted":
            return byte < np.uint64(t)
        return byte >= np.uint64(t)

    def scale_of(self, p):
        return 1.0 if self.bug == "no_keep_scale" else od.dropout_keep_scale(p)

    # -- attention --------------------------------------------------------
    def _probs(self, q, k, scale, causal, kv_len, Z=None):
        s = oracle.fp32_scale(scale)
        S = s * (q @ k.T)
        vis = oracle.visible_mask(q.shape[0], k.shape[0], causal, kv_len)
        S = np.where(vis, S, -np.inf)
        anyv = vis.any(axis=1, keepdims=True)
        m = np.where(anyv, np.max(S, axis=1, keepdims=True, initial=-np.inf), 0.0)
        E = np.where(vis, np.exp(S - m), 0.0)
        ell = (E * Z if Z is not None else E).sum(axis=1, keepdims=True)
        P = np.divide(E, ell, out=np.zeros_like(E), where=anyv & (ell > 0))
        lse = np.where(anyv, m + np.log(np.where(ell > 0, ell, 1.0)), -np.inf).reshape(-1)
        return s, P, lse

    def fwd(self, q, k, v, scale, p, seed, bh, offset=0, causal=False, kv_len=None):
        if self.bug is None:
            return od.head_forward_dropout(q, k, v, scale, p, seed, bh, offset, causal, kv_len)
        Z = self.keep(q.shape[0], k.shape[0], bh, p, seed, offset)
        norm_kept = self.bug in ("normaliser_from_kept", "lse_from_dropped")
        _, P, lse = self._probs(q, k, scale, causal, kv_len, Z if norm_kept else None)
        if self.bug == "lse_from_dropped":
            _, P, _ = self._probs(q, k, scale, causal, kv_len)
        return (P * Z * self.scale_of(p)) @ v, lse

    def bwd(self, q, k, v, do, scale, p, seed, bh, offset=0, causal=False, kv_len=None):
        if self.bug is None:
            return od.head_backward_dropout(q, k, v, do, scale, p, seed, bh, offset, causal, kv_len)
        s, P, _ = self._probs(q, k, scale, causal, kv_len)
        Z = self.keep(q.shape[0], k.shape[0], bh, p, seed, offset)
        if self.bug == "bwd_mask_transposed":
            Z = Z.T
        Zc = Z * self.scale_of(p)
        dV = ((P if self.bug == "dv_undropped_p" else P * Zc).T) @ do
        dP = do @ v.T
        if self.bug != "ds_undropped_dp":
            dP = dP * Zc
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        return s * (dS @ k), s * (dS.T @ q), dV


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- pins
def pin_known_answers(impl):
    """Published Philox4x32-10 known-answer values."""
    for case in json.load(open(GOLDEN))["cases"]:
        ctr = [int(x, 16) for x in case["counter"]]
        key = [int(x, 16) for x in case["key"]]
        out = impl.philox([np.array([c], np.uint64) for c in ctr], key)
        assert [int(o[0]) for o in out] == [int(x, 16) for x in case["out"]]


def pin_keep_rate(impl):
    """Keep fraction equals (256 - t) / 256 within 6 standard deviations."""
    for p, seed in ((0.25, 11), (0.1, 12)):
        Z = impl.keep(2048, 2048, 3, p, seed, 0)
        q_keep = (256 - od.dropout_threshold(p)) / 256.0
        sd = np.sqrt(q_keep * (1 - q_keep) / Z.size)
        assert abs(Z.mean() - q_keep) < 6 * sd, (p, Z.mean(), q_keep)


def pin_byte_uniformity(impl):
    """Output bytes are uniform over 0..255 (chi-square, 255 degrees of freedom)."""
    n = 1 << 15
    out = impl.philox((np.arange(n), np.zeros(n, np.int64), np.full(n, 7), np.zeros(n, np.int64)), (123, 456))
    b = np.concatenate([o.view(np.uint8) for o in out])
    counts = np.bincount(b, minlength=256)
    exp = b.size / 256.0
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 370.0, chi2  # P(chi2_255 > 370) < 1e-5


def pin_p0_is_plain(impl):
    """p = 0 keeps every weight with factor 1: the plain attention oracle."""
    r = _rng(2)
    q, k, v, do = (r.standard_normal((9, 5)) for _ in range(4))
    for causal, kl in ((False, None), (True, None), (False, 6)):
        O, lse = impl.fwd(q, k, v, 0.4, 0.0, 99, 1, 0, causal, kl)
        O0, lse0 = oracle.head_forward(q, k, v, 0.4, causal, kl)
        assert np.allclose(O, O0, atol=1e-12) and np.allclose(lse, lse0, atol=1e-12)
        g = impl.bwd(q, k, v, do, 0.4, 0.0, 99, 1, 0, causal, kl)
        g0 = oracle.head_backward(q, k, v, do, 0.4, causal, kl)
        for a, b_ in zip(g, g0):
            assert np.allclose(a, b_, atol=1e-12)


def pin_autograd(impl):
    """Forward and gradients equal torch float64 autograd of (softmax(S) o Z c) V with the same Z."""
    r = _rng(3)
    n, m, d, scale, p, seed, bh = 12, 10, 6, 0.3, 0.3, 2024, 5
    q, do = r.standard_normal((n, d)), r.standard_normal((n, d))
    k, v = r.standard_normal((m, d)), r.standard_normal((m, d))
    for causal, kl in ((False, None), (True, None), (False, 7)):
        Z = impl.keep(n, m, bh, p, seed, 3)
        c = 256.0 / (256.0 - round(256 * p))
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        S = float(np.float32(scale)) * tq @ tk.T
        vis = torch.tensor(oracle.visible_mask(n, m, causal, kl))
        P = torch.softmax(S.masked_fill(~vis, float("-inf")), dim=1)
        O = (P * torch.tensor(Z, dtype=torch.float64) * c) @ tv
        O.backward(torch.tensor(do))
        Oi, lse = impl.fwd(q, k, v, scale, p, seed, bh, 3, causal, kl)
        assert np.allclose(Oi, O.detach().numpy(), atol=1e-12)
        assert np.allclose(lse, torch.logsumexp(S.masked_fill(~vis, float("-inf")), 1).detach().numpy(), atol=1e-12)
        dq, dk, dv = impl.bwd(q, k, v, do, scale, p, seed, bh, 3, causal, kl)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-12)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-12)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-12)


def pin_finite_differences(impl):
    """Central differences of f = <dO, O> on a tiny head (mask held fixed by the seed)."""
    r = _rng(4)
    n, d, scale, p, seed, bh = 5, 3, 0.7, 0.25, 77, 2
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    f = lambda q_, k_, v_: float((impl.fwd(q_, k_, v_, scale, p, seed, bh)[0] * do).sum())
    grads = impl.bwd(q, k, v, do, scale, p, seed, bh)
    eps = 1e-6
    for which, g in enumerate(grads):
        args = [q.copy(), k.copy(), v.copy()]
        num = np.zeros_like(args[which])
        for idx in np.ndindex(num.shape):
            a = [x.copy() for x in args]; b_ = [x.copy() for x in args]
            a[which][idx] += eps; b_[which][idx] -= eps
            num[idx] = (f(*a) - f(*b_)) / (2 * eps)
        assert np.allclose(num, g, atol=1e-6), (which, np.abs(num - g).max())


def pin_expectation(impl):
    """The mean of the dropped output over seeds approaches the exact output (E[Z c] = 1)."""
    r = _rng(5)
    q, k, v = r.standard_normal((4, 3)), r.standard_normal((8, 3)), r.standard_normal((8, 3)) + 2.0
    O0, _ = oracle.head_forward(q, k, v, 0.5)
    acc = np.zeros_like(O0)
    n = 3000
    for seed in range(n):
        acc += impl.fwd(q, k, v, 0.5, 0.5, seed, 0)[0]
    assert np.abs(acc / n - O0).max() < 0.08, np.abs(acc / n - O0).max()


def pin_counter_components(impl):
    """The mask depends on every counter word and on the seed, and on nothing else."""
    Z = impl.keep(64, 64, 4, 0.5, 1234, 9)
    assert np.array_equal(Z, impl.keep(64, 64, 4, 0.5, 1234, 9))
    for other in (impl.keep(64, 64, 5, 0.5, 1234, 9), impl.keep(64, 64, 4, 0.5, 1235, 9),
                  impl.keep(64, 64, 4, 0.5, 1234, 10), impl.keep(64, 64, 4, 0.5, 1234 + (1 << 32), 9)):
        assert 0.3 < (Z != other).mean() < 0.7
    big = impl.keep(96, 80, 4, 0.5, 1234, 9)
    assert np.array_equal(big[:64, :64], Z)


PINS = [pin_known_answers, pin_keep_rate, pin_byte_uniformity, pin_p0_is_plain, pin_autograd,
        pin_finite_differences, pin_expectation, pin_counter_components]
MUTANTS = ["philox_swap_multipliers", "philox_no_key_bump", "philox_nine_rounds", "keep_strict",
           "keep_inverted", "no_keep_scale", "ds_undropped_dp", "dv_undropped_p",
           "normaliser_from_kept", "lse_from_dropped", "bwd_mask_transposed"]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_passes(pin):
    pin(Impl())


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_unmutated_copy_passes(pin):
    pin(Impl("none"))


@pytest.mark.parametrize("bug", MUTANTS)
def test_mutant_fails_a_pin(bug):
    impl = Impl(bug)
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError):
            return
    pytest.fail(f"planted mistake {bug!r} passes every pin")


def test_thresholds():
    """t = round(256 p) and the keep factor 256 / (256 - t); p outside [0, 1) is rejected."""
    assert od.dropout_threshold(0.0) == 0 and od.dropout_keep_scale(0.0) == 1.0
    assert od.dropout_threshold(0.1) == 26 and od.dropout_keep_scale(0.1) == 256.0 / 230.0
    assert od.dropout_threshold(0.5) == 128
    for bad in (-0.1, 1.0, 0.999):
        with pytest.raises(ValueError):
            od.dropout_threshold(bad)


def test_batched_wrappers():
    """forward_dropout / backward_dropout take head b * H + h of the batched layout."""
    r = _rng(6)
    Q, K, V, dO = (r.standard_normal((2, 3, 8, 4)) for _ in range(4))
    O, L = od.forward_dropout(Q, K, V, 0.5, 0.2, 31, 1, True, [8, 5])
    dQ, dK, dV = od.backward_dropout(Q, K, V, dO, 0.5, 0.2, 31, 1, True, [8, 5])
    for b in range(2):
        for h in range(3):
            kl = [8, 5][b]
            o, l = od.head_forward_dropout(Q[b, h], K[b, h], V[b, h], 0.5, 0.2, 31, b * 3 + h, 1, True, kl)
            assert np.array_equal(o, O[b, h]) and np.array_equal(l, L[b, h])
            g = od.head_backward_dropout(Q[b, h], K[b, h], V[b, h], dO[b, h], 0.5, 0.2, 31, b * 3 + h, 1, True, kl)
            assert np.array_equal(g[0], dQ[b, h]) and np.array_equal(g[2], dV[b, h])
