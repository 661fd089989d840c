"""Pins of the oracle's decoding forward (CPU only).

``decode_head_forward`` is checked against closed forms, invariants that
any correct implementation satisfies, a pure-Python brute force on tiny
inputs and torch's float64 CPU attention; planted mistakes in a copy of it
must each fail at least one pin.
"""
import math

import numpy as np
import pytest

import oracle

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _dec(q, k, v, scale, L, causal):
    return oracle.decode_head_forward(q, k, v, scale, L, causal)


def pin_single_visible_key(dec):
    """One visible key: O is its value row, LSE its scaled score."""
    r = _rng(1)
    q, k, v = r.standard_normal((1, 8)), r.standard_normal((5, 8)), r.standard_normal((5, 8))
    O, lse = dec(q, k, v, 0.375, 1, False)
    assert np.allclose(O[0], v[0], atol=TOL)
    assert abs(lse[0] - 0.375 * float(q[0] @ k[0])) < TOL


def pin_ln3_weights(dec):
    """Two keys whose scaled scores are ln 3 and 0: weights 3/4 and 1/4, LSE = ln 4."""
    d, s = 4, 0.625
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((2, d)); k[0, 0] = math.log(3.0) / s
    v = np.array([[1.0, 2.0, 3.0, 4.0], [-4.0, 0.0, 8.0, 2.0]])
    O, lse = dec(q, k, v, s, None, False)
    assert np.allclose(O[0], 0.75 * v[0] + 0.25 * v[1], atol=1e-12)
    assert abs(lse[0] - math.log(4.0)) < 1e-12


def pin_constant_v(dec):
    """Every visible value row equal: O equals that row for every query."""
    r = _rng(2)
    q, k = r.standard_normal((3, 16)), r.standard_normal((40, 16))
    v = np.tile(r.standard_normal((1, 16)), (40, 1))
    v[30:] = 99.0  # outside the cache
    O, _ = dec(q, k, v, 0.25, 30, True)
    assert np.allclose(O, np.tile(v[0], (3, 1)), atol=1e-12)


def pin_cache_tail_ignored(dec):
    """Slots at or past kv_len do not change the result."""
    r = _rng(3)
    q, k, v = r.standard_normal((2, 8)), r.standard_normal((20, 8)), r.standard_normal((20, 8))
    O1, l1 = dec(q, k, v, 0.5, 13, False)
    k2, v2 = k.copy(), v.copy()
    k2[13:] = 50.0
    v2[13:] = -7.0
    O2, l2 = dec(q, k2, v2, 0.5, 13, False)
    assert np.allclose(O1, O2, atol=TOL) and np.allclose(l1, l2, atol=TOL)


def pin_causal_is_stack_of_single_queries(dec):
    """With causal masking query i of n_q behaves as a single query against
    the first L - n_q + i + 1 keys (bottom-right alignment)."""
    r = _rng(4)
    nq, L = 4, 11
    q, k, v = r.standard_normal((nq, 8)), r.standard_normal((16, 8)), r.standard_normal((16, 8))
    O, lse = dec(q, k, v, 0.3, L, True)
    for i in range(nq):
        Oi, li = dec(q[i:i + 1], k, v, 0.3, L - nq + i + 1, False)
        assert np.allclose(O[i], Oi[0], atol=TOL) and abs(lse[i] - li[0]) < TOL


def pin_square_causal_is_self_attention(dec):
    """n_q = n_k = kv_len with causal masking is causal self-attention."""
    r = _rng(5)
    q, k, v = r.standard_normal((6, 8)), r.standard_normal((6, 8)), r.standard_normal((6, 8))
    O, lse = dec(q, k, v, 0.4, None, True)
    # hand-built lower-triangular softmax
    s = float(np.float32(0.4))
    for i in range(6):
        sc = s * (k[:i + 1] @ q[i])
        w = np.exp(sc - sc.max())
        assert np.allclose(O[i], (w / w.sum()) @ v[:i + 1], atol=1e-12)
        assert abs(lse[i] - (sc.max() + math.log(w.sum()))) < 1e-12


def pin_empty_cache(dec):
    """kv_len = 0: O = 0 and LSE = -inf."""
    r = _rng(6)
    O, lse = dec(r.standard_normal((2, 8)), r.standard_normal((4, 8)), r.standard_normal((4, 8)), 0.5, 0, False)
    assert np.all(O == 0.0) and np.all(np.isneginf(lse))


def pin_brute_force(dec):
    """Tiny random cases against pure-Python loops over the definition."""
    r = _rng(7)
    for nq, nk, L, causal in [(1, 5, 5, False), (3, 7, 6, True), (2, 9, 4, False), (4, 8, 8, True)]:
        q, k, v = r.standard_normal((nq, 3)), r.standard_normal((nk, 3)), r.standard_normal((nk, 3))
        s = float(np.float32(0.7))
        O, lse = dec(q, k, v, 0.7, L, causal)
        for i in range(nq):
            vis = [j for j in range(nk) if j < L and (not causal or j <= L - nq + i)]
            sc = [s * sum(q[i][c] * k[j][c] for c in range(3)) for j in vis]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            tot = sum(w)
            o = [sum(w[t] * v[vis[t]][c] for t in range(len(vis))) / tot for c in range(3)]
            assert np.allclose(O[i], o, atol=1e-12)
            assert abs(lse[i] - (m + math.log(tot))) < 1e-12


def pin_matches_torch_sdpa(dec):
    """Against torch's float64 CPU attention with an explicit boolean mask."""
    torch = pytest.importorskip("torch")
    r = _rng(8)
    nq, nk, L = 3, 12, 10
    q, k, v = r.standard_normal((nq, 16)), r.standard_normal((nk, 16)), r.standard_normal((nk, 16))
    for causal in (False, True):
        vis = np.array([[j < L and (not causal or j <= L - nq + i) for j in range(nk)] for i in range(nq)])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            attn_mask=torch.from_numpy(vis)[None], scale=float(np.float32(0.25)))[0].numpy()
        O, _ = dec(q, k, v, 0.25, L, causal)
        assert np.allclose(O, ref, atol=1e-12)


PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(_dec)


def test_batched_wrapper():
    r = _rng(9)
    Q, K, V = r.standard_normal((2, 3, 2, 8)), r.standard_normal((2, 3, 10, 8)), r.standard_normal((2, 3, 10, 8))
    L = np.array([7, 10])
    O, lse = oracle.decode_forward(Q, K, V, 0.5, L, True)
    for b in range(2):
        for h in range(3):
            Oh, lh = oracle.decode_head_forward(Q[b, h], K[b, h], V[b, h], 0.5, int(L[b]), True)
            assert np.array_equal(O[b, h], Oh) and np.array_equal(lse[b, h], lh)


MUTANTS = ["top_left_causal", "causal_off_by_one", "kv_len_inclusive", "kv_len_ignored",
           "no_scale", "lse_log2", "lse_without_max"]


def _mutant(bug):
    def dec(q, k, v, scale, L, causal):
        q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
        s = 1.0 if bug == "no_scale" else float(np.float32(scale))
        S = s * (q @ k.T)
        nq, nk = S.shape
        lim = nk if (L is None or bug == "kv_len_ignored") else L
        cols = np.arange(nk)[None, :]
        vis = (cols <= lim) if bug == "kv_len_inclusive" else (cols < lim)
        vis = np.broadcast_to(vis, S.shape).copy()
        if causal:
            rows = np.arange(nq)[:, None]
            if bug == "top_left_causal":
                vis &= cols <= rows
            elif bug == "causal_off_by_one":
                vis &= cols < lim - nq + rows
            else:
                vis &= cols <= lim - nq + rows
        S = np.where(vis, S, -np.inf)
        anyv = vis.any(axis=1, keepdims=True)
        m = np.where(anyv, np.max(S, axis=1, keepdims=True, initial=-np.inf), 0.0)
        E = np.where(vis, np.exp(S - m), 0.0)
        ell = E.sum(axis=1, keepdims=True)
        P = np.divide(E, ell, out=np.zeros_like(E), where=anyv)
        logl = np.log2 if bug == "lse_log2" else np.log
        lse = (0.0 if bug == "lse_without_max" else m) + logl(np.where(anyv, ell, 1.0))
        return P @ v, np.where(anyv, lse, -np.inf).reshape(-1)
    return dec


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(_mutant(None))


@pytest.mark.parametrize("bug", MUTANTS)
def test_mutant_fails_a_pin(bug):
    dec = _mutant(bug)
    failed = []
    for pin in PINS:
        try:
            pin(dec)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {bug} passed every pin"
