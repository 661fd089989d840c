"""Pins for the fp64 oracle: checks fixed by the pages and by mathematics.

Each ``pin_*`` takes a forward and a backward implementation of one head
  fwd(q, k, v, scale, causal, kv_len) -> (O, LSE)
  bwd(q, k, v, dO, scale, causal, kv_len) -> (dQ, dK, dV)
and raises AssertionError when the implementation breaks the pin. The real
oracle must pass all of them (test_oracle_pins.py); deliberately broken
copies must each fail at least one (test_oracle_mutants.py).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")
TOL = 1e-11


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b), initial=0.0)))
    err = float(np.max(np.abs(a - b), initial=0.0))
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol * scale:.3e}"


def _rng(seed):
    return np.random.default_rng(seed)


def _golden_value(x):
    """Parse the fixture's exact notation: numbers, 'lnK', 'a/b', '-0.75*ln3'."""
    if isinstance(x, (int, float)):
        return float(x)
    x = x.strip()
    if "*" in x:
        a, b = x.split("*")
        return _golden_value(a) * _golden_value(b)
    if x.startswith("-"):
        return -_golden_value(x[1:])
    if x.startswith("ln"):
        return math.log(float(x[2:]))
    if "/" in x:
        return float(Fraction(x))
    return float(x)


def _golden_array(rows):
    return np.array([[_golden_value(c) for c in r] if isinstance(r, list) else _golden_value(r)
                     for r in rows], np.float64)


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


# --------------------------------------------------------------------------- pins

def pin_golden_closed_forms(fwd, bwd):
    """Hand-derived tiny cases (tests/golden/closed_forms.json)."""
    for c in golden_cases():
        q, k, v, do = (_golden_array(c[n]) for n in ("q", "k", "v", "dO"))
        O, lse = fwd(q, k, v, c["scale"], c["causal"], c["kv_len"])
        _close(O, _golden_array(c["O"]), what=c["name"] + " O")
        _close(lse, _golden_array(c["LSE"]), what=c["name"] + " LSE")
        dq, dk, dv = bwd(q, k, v, do, c["scale"], c["causal"], c["kv_len"])
        _close(dq, _golden_array(c["dQ"]), what=c["name"] + " dQ")
        _close(dk, _golden_array(c["dK"]), what=c["name"] + " dK")
        _close(dv, _golden_array(c["dV"]), what=c["name"] + " dV")


def pin_rows_sum_to_one(fwd, bwd):
    """With V = identity, O is P itself: rows sum to 1, P >= 0, masked P = 0."""
    r = _rng(1)
    N, d = 9, 5
    q, k = r.standard_normal((N, d)), r.standard_normal((N, d))
    for causal in (False, True):
        for L in (None, 6):
            P, _ = fwd(q, k, np.eye(N), 0.7, causal, L)
            _close(P.sum(axis=1), np.ones(N), what="row sums")
            assert (P >= 0).all()
            cols = np.arange(N)
            if L is not None:
                assert np.all(P[:, cols >= L] == 0), "padded keys got weight"
            if causal:
                assert np.all(P[np.triu_indices(N, 1)] == 0), "future keys got weight"


def pin_constant_v(fwd, bwd):
    """Every V row equal to c gives every O row equal to c."""
    r = _rng(2)
    N, d = 11, 4
    q, k = r.standard_normal((N, d)), r.standard_normal((N, d))
    c = r.standard_normal(d)
    v = np.tile(c, (N, 1))
    for causal in (False, True):
        O, _ = fwd(q, k, v, 0.5, causal, 7)
        _close(O, np.tile(c, (N, 1)), what="constant V")


def pin_one_hot_dominant(fwd, bwd):
    """A score far above the rest selects that key's V row."""
    r = _rng(3)
    N, d = 8, 6
    q = r.standard_normal((N, d)) * 0.1
    k = r.standard_normal((N, d)) * 0.1
    v = r.standard_normal((N, d))
    j = 5
    q[:, 0] = 30.0
    k[j, 0] = 30.0
    O, _ = fwd(q, k, v, 1.0, False, None)
    _close(O, np.tile(v[j], (N, 1)), tol=1e-12, what="dominant key")


def pin_causal_first_row(fwd, bwd):
    """Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = s q_0 . k_0."""
    r = _rng(4)
    N, d = 10, 7
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    s = 0.3
    O, lse = fwd(q, k, v, s, True, None)
    _close(O[0], v[0], what="causal O_0")
    _close(lse[0], float(np.float32(s)) * q[0] @ k[0], what="causal LSE_0")


def pin_zero_query(fwd, bwd):
    """Q = 0: uniform weights over visible keys (prefix mean when causal), LSE = ln(count)."""
    r = _rng(5)
    N, d = 12, 3
    k, v = r.standard_normal((N, d)), r.standard_normal((N, d))
    q = np.zeros((N, d))
    for causal in (False, True):
        for L in (None, 5):
            O, lse = fwd(q, k, v, 0.9, causal, L)
            for i in range(N):
                n = (L if L is not None else N)
                if causal:
                    n = min(n, i + 1)
                _close(O[i], v[:n].mean(axis=0), what=f"zero-Q O row {i}")
                _close(lse[i], math.log(n), what=f"zero-Q LSE row {i}")


def pin_single_key(fwd, bwd):
    """N = 1: O = V and LSE = s q . k; gradients dQ = dK = 0, dV = dO."""
    r = _rng(6)
    d = 5
    q, k, v, do = (r.standard_normal((1, d)) for _ in range(4))
    s = 0.25
    O, lse = fwd(q, k, v, s, False, None)
    _close(O, v, what="N=1 O")
    _close(lse, [s * q[0] @ k[0]], what="N=1 LSE")
    dq, dk, dv = bwd(q, k, v, do, s, False, None)
    _close(dq, np.zeros((1, d)), what="N=1 dQ")
    _close(dk, np.zeros((1, d)), what="N=1 dK")
    _close(dv, do, what="N=1 dV")


def pin_equal_keys(fwd, bwd):
    """All keys equal to u: O = mean V, LSE = s q.u + ln N."""
    r = _rng(7)
    N, d = 6, 4
    u = r.standard_normal(d)
    q, v = r.standard_normal((N, d)), r.standard_normal((N, d))
    k = np.tile(u, (N, 1))
    s = 0.625
    O, lse = fwd(q, k, v, s, False, None)
    _close(O, np.tile(v.mean(axis=0), (N, 1)), what="equal keys O")
    _close(lse, s * (q @ u) + math.log(N), what="equal keys LSE")


def pin_key_shift(fwd, bwd):
    """Adding u to every key leaves O unchanged and adds s q_i . u to LSE_i."""
    r = _rng(8)
    N, d = 9, 5
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    u = r.standard_normal(d)
    s = 0.375
    for causal in (False, True):
        O1, l1 = fwd(q, k, v, s, causal, 7)
        O2, l2 = fwd(q, k + u, v, s, causal, 7)
        _close(O2, O1, what="shift O")
        _close(l2, l1 + s * (q @ u), what="shift LSE")


def pin_permutation(fwd, bwd):
    """Permuting keys and values together (non-causal, unpadded) changes nothing;
    the key gradients permute with them."""
    r = _rng(9)
    N, d = 8, 3
    q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
    perm = r.permutation(N)
    O1, l1 = fwd(q, k, v, 0.8, False, None)
    O2, l2 = fwd(q, k[perm], v[perm], 0.8, False, None)
    _close(O2, O1, what="perm O")
    _close(l2, l1, what="perm LSE")
    g1 = bwd(q, k, v, do, 0.8, False, None)
    g2 = bwd(q, k[perm], v[perm], do, 0.8, False, None)
    _close(g2[0], g1[0], what="perm dQ")
    _close(g2[1], g1[1][perm], what="perm dK")
    _close(g2[2], g1[2][perm], what="perm dV")


def pin_linearity(fwd, bwd):
    """O is linear in V; the gradients are linear in dO."""
    r = _rng(10)
    N, d = 7, 4
    q, k, v1, v2, do1, do2 = (r.standard_normal((N, d)) for _ in range(6))
    a, b = 1.7, -0.6
    O1, _ = fwd(q, k, v1, 0.5, True, None)
    O2, _ = fwd(q, k, v2, 0.5, True, None)
    O3, _ = fwd(q, k, a * v1 + b * v2, 0.5, True, None)
    _close(O3, a * O1 + b * O2, what="linear in V")
    g1 = bwd(q, k, v1, do1, 0.5, True, None)
    g2 = bwd(q, k, v1, do2, 0.5, True, None)
    g3 = bwd(q, k, v1, a * do1 + b * do2, 0.5, True, None)
    for x1, x2, x3, n in zip(g1, g2, g3, ("dQ", "dK", "dV")):
        _close(x3, a * x1 + b * x2, what=f"linear in dO ({n})")


def pin_gradient_sums(fwd, bwd):
    """sum_j dK_j = 0 (rows of dS sum to 0); sum_j dV_j = sum_i dO_i (rows of P
    sum to 1); masked keys get dK = dV = 0."""
    r = _rng(11)
    N, d = 10, 4
    q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        for L in (None, 6):
            dq, dk, dv = bwd(q, k, v, do, 0.45, causal, L)
            _close(dk.sum(axis=0), np.zeros(d), what="sum dK")
            _close(dv.sum(axis=0), do.sum(axis=0), what="sum dV")
            if L is not None:
                assert np.all(dk[L:] == 0) and np.all(dv[L:] == 0), "masked key got a gradient"


def pin_row_dot_identity(fwd, bwd):
    """rowsum(P * dP) = rowsum(dO * O): checked through the gradient of q.
    Since dQ_i = s sum_j P_ij (dP_ij - D_i) k_j, with D_i = dO_i . O_i."""
    r = _rng(12)
    N, d = 9, 5
    q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
    s = 0.5
    O, _ = fwd(q, k, v, s, False, None)
    P, _ = fwd(q, k, np.eye(N), s, False, None)
    D = (do * O).sum(axis=1)
    dq, _, _ = bwd(q, k, v, do, s, False, None)
    dP = do @ v.T
    _close(dq, s * ((P * (dP - D[:, None])) @ k), what="dQ via D = rowsum(dO*O)")


def pin_finite_differences(fwd, bwd):
    """Full Jacobian of f = <dO, O> on tiny heads by central differences."""
    r = _rng(13)
    N, d = 4, 3
    h = 1e-6
    for causal, L in ((False, None), (True, None), (False, 3), (True, 2)):
        q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
        s = 0.7
        grads = bwd(q, k, v, do, s, causal, L)
        for which in range(3):
            x = [q, k, v]
            num = np.zeros((N, d))
            for i in range(N):
                for c in range(d):
                    xp = [a.copy() for a in x]
                    xm = [a.copy() for a in x]
                    xp[which][i, c] += h
                    xm[which][i, c] -= h
                    fp = (do * fwd(*xp, s, causal, L)[0]).sum()
                    fm = (do * fwd(*xm, s, causal, L)[0]).sum()
                    num[i, c] = (fp - fm) / (2 * h)
            _close(grads[which], num, tol=1e-6, what=f"finite diff {'QKV'[which]} causal={causal} L={L}")


def pin_directional_derivative_c1(fwd, bwd):
    """At the single-head fp32 workload's size (N=128, d=64), the gradients
    agree with central differences of f = <dO, O> along random directions."""
    r = _rng(14)
    N, d = 128, 64
    q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
    s = 1 / 8
    grads = bwd(q, k, v, do, s, False, None)
    h = 1e-5
    for which in range(3):
        u = r.standard_normal((N, d))
        x = [q, k, v]
        xp = [a.copy() for a in x]
        xm = [a.copy() for a in x]
        xp[which] += h * u
        xm[which] -= h * u
        fp = (do * fwd(*xp, s, False, None)[0]).sum()
        fm = (do * fwd(*xm, s, False, None)[0]).sum()
        num = (fp - fm) / (2 * h)
        ana = float((grads[which] * u).sum())
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), f"directional {'QKV'[which]}: {num} vs {ana}"


def brute_force_head(q, k, v, do, s, causal, L):
    """Pure-Python loops: softmax per row, and the backward through the
    explicit softmax Jacobian J = diag(p) - p p^T. Independent of numpy's
    matrix products; for tiny inputs only."""
    N, d = len(q), len(q[0])
    s = float(np.float32(s))
    lim = N if L is None else L
    O = [[0.0] * d for _ in range(N)]
    lse = [0.0] * N
    dq = [[0.0] * d for _ in range(N)]
    dk = [[0.0] * d for _ in range(N)]
    dv = [[0.0] * d for _ in range(N)]
    for i in range(N):
        js = [j for j in range(N) if j < lim and (not causal or j <= i)]
        if not js:
            lse[i] = -math.inf
            continue
        sc = [s * sum(q[i][c] * k[j][c] for c in range(d)) for j in js]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        z = sum(w)
        p = [x / z for x in w]
        lse[i] = m + math.log(z)
        for c in range(d):
            O[i][c] = sum(p[a] * v[j][c] for a, j in enumerate(js))
        g = [sum(do[i][c] * v[j][c] for c in range(d)) for j in js]
        n = len(js)
        ds = [sum((p[a] * ((1.0 if a == b else 0.0) - p[b])) * g[b] for b in range(n)) for a in range(n)]
        for a, j in enumerate(js):
            for c in range(d):
                dv[j][c] += p[a] * do[i][c]
                dq[i][c] += s * ds[a] * k[j][c]
                dk[j][c] += s * ds[a] * q[i][c]
    return [np.array(x) for x in (O, lse, dq, dk, dv)]


def pin_brute_force(fwd, bwd):
    """Agreement with pure-Python loops on tiny random heads."""
    r = _rng(15)
    for N, d, causal, L in ((5, 3, False, None), (6, 2, True, None), (7, 3, False, 4), (6, 4, True, 3)):
        q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
        s = 0.55
        O, lse, dq, dk, dv = brute_force_head(q.tolist(), k.tolist(), v.tolist(), do.tolist(), s, causal, L)
        O2, lse2 = fwd(q, k, v, s, causal, L)
        _close(O2, O, what="brute O")
        _close(lse2, lse, what="brute LSE")
        g = bwd(q, k, v, do, s, causal, L)
        _close(g[0], dq, what="brute dQ")
        _close(g[1], dk, what="brute dK")
        _close(g[2], dv, what="brute dV")


def pin_fully_masked_rows(fwd, bwd):
    """kv_len = 0 masks every key: O = 0, LSE = -inf, no gradient anywhere."""
    r = _rng(16)
    N, d = 5, 3
    q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
    O, lse = fwd(q, k, v, 0.5, False, 0)
    assert np.all(O == 0) and np.all(np.isneginf(lse))
    for g in bwd(q, k, v, do, 0.5, False, 0):
        assert np.all(g == 0)


def pin_scale_is_fp32(fwd, bwd):
    """The scale enters as its float32 value: 1/sqrt(128) is not exact in fp32,
    and the N=1 LSE exposes which value was used."""
    q = np.array([[1.0]])
    k = np.array([[1e9]])
    v = np.array([[1.0]])
    s = 1 / math.sqrt(128)
    _, lse = fwd(q, k, v, s, False, None)
    assert lse[0] == float(np.float32(s)) * 1e9, "scale was not rounded to fp32"


PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
