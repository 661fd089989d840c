"""Pins of the oracle's block-sparse attention (CPU only).

Checked against the plain oracle (an all-on mask), closed forms (a
block-diagonal mask is independent attention per block; a query block with
no key block has O = 0, LSE = -inf), torch's float64 attention with the
same boolean mask, a pure-Python brute force on a tiny case, and an
invariance (permuting key blocks together with the mask columns). A copy
with one planted mistake per switch must fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import block_sparse as bs

TOL = 1e-12


class Impl:
    def __init__(self, bug=None):
        self.bug = bug

    def visible(self, n, bm, causal, kv_len, rows=None):
        if self.bug is None:
            return bs.block_sparse_visible(n, bm, causal, kv_len, rows)
        block = 127 if self.bug == "block_127" else 128
        bm = np.asarray(bm, bool)
        if self.bug == "mask_transposed":
            bm = bm.T
        rows = np.arange(n) if rows is None else np.asarray(rows)
        vis = oracle.visible_mask(n, n, causal and self.bug != "causal_ignored", kv_len, rows)
        nb = bm.shape[0]
        rb = np.minimum(rows // block, nb - 1)
        cb = np.minimum(np.arange(n) // block, nb - 1)
        if self.bug == "mask_ignored":
            return vis
        return vis & bm[rb][:, cb]

    def fwd(self, q, k, v, scale, bm, causal=False, kv_len=None):
        if self.bug is None:
            return bs.head_forward_block_sparse(q, k, v, scale, bm, causal, kv_len)
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        S = oracle.fp32_scale(scale) * (q @ k.T)
        vis = self.visible(q.shape[0], bm, causal, kv_len)
        if self.bug == "softmax_over_all_keys":
            P, lse = oracle.attention._softmax_rows(S, np.ones_like(vis))
            P = P * vis
            return P @ v, lse
        P, lse = oracle.attention._softmax_rows(S, vis)
        return P @ v, lse


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(n, d, seed):
    r = _rng(seed)
    return r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, d))


def pin_all_on_is_plain(impl):
    q, k, v = _qkv(300, 8, 1)
    bm = np.ones((3, 3), bool)
    for causal, kl in ((False, None), (True, None), (False, 200)):
        O, L = impl.fwd(q, k, v, 0.3, bm, causal, kl)
        O0, L0 = oracle.head_forward(q, k, v, 0.3, causal, kl)
        assert np.allclose(O, O0, atol=TOL) and np.allclose(L, L0, atol=TOL)


def pin_block_diagonal_is_independent(impl):
    """A block-diagonal mask attends within each 128-block only: the plain oracle on each block."""
    q, k, v = _qkv(320, 6, 2)
    bm = np.eye(3, dtype=bool)
    O, L = impl.fwd(q, k, v, 0.5, bm)
    for b0 in range(0, 320, 128):
        sl = slice(b0, min(b0 + 128, 320))
        Ob, Lb = oracle.head_forward(q[sl], k[sl], v[sl], 0.5)
        assert np.allclose(O[sl], Ob, atol=TOL) and np.allclose(L[sl], Lb, atol=TOL)


def pin_empty_block_row(impl):
    """A query block with no key block: O = 0 and LSE = -inf on its rows."""
    q, k, v = _qkv(256, 4, 3)
    bm = np.array([[True, False], [False, False]])
    O, L = impl.fwd(q, k, v, 0.5, bm)
    assert np.all(O[128:] == 0) and np.all(np.isneginf(L[128:]))
    assert np.all(np.isfinite(L[:128]))


def pin_torch_masked_attention(impl):
    """torch float64 attention with the same boolean mask (no empty rows)."""
    r = _rng(4)
    n, d = 384, 8
    q, k, v = _qkv(n, d, 5)
    bm = r.random((3, 3)) < 0.5
    np.fill_diagonal(bm, True)
    for causal in (False, True):
        vis = bs.block_sparse_visible(n, bm, causal)
        O, L = impl.fwd(q, k, v, 0.25, bm, causal)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq[None], tk[None], tv[None], attn_mask=torch.tensor(vis)[None], scale=float(np.float32(0.25)))
        assert np.allclose(O, ref[0].numpy(), atol=TOL)
        S = float(np.float32(0.25)) * (tq @ tk.T)
        lse = torch.logsumexp(S.masked_fill(~torch.tensor(vis), float("-inf")), dim=1)
        assert np.allclose(L, lse.numpy(), atol=TOL)


def pin_brute_force(impl):
    """Pure-Python loops on a tiny head (two blocks, one of them partial)."""
    n, d = 130, 2
    q, k, v = _qkv(n, d, 6)
    bm = np.array([[False, True], [True, True]])
    O, L = impl.fwd(q, k, v, 0.7, bm, causal=True)
    s = float(np.float32(0.7))
    for i in (0, 5, 127, 128, 129):
        keys = [j for j in range(n) if j <= i and bm[i // 128][j // 128]]
        if not keys:
            assert all(O[i] == 0) and math.isinf(L[i]) and L[i] < 0
            continue
        sc = [s * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        tot = sum(w)
        for c in range(d):
            assert abs(O[i][c] - sum(wj * v[j][c] for wj, j in zip(w, keys)) / tot) < 1e-12
        assert abs(L[i] - (m + math.log(tot))) < 1e-12


def pin_key_block_permutation(impl):
    """Permuting whole key blocks together with the mask's columns leaves O unchanged (non-causal)."""
    q, k, v = _qkv(384, 5, 7)
    bm = np.array([[True, False, True], [False, True, True], [True, True, False]])
    perm = [2, 0, 1]
    idx = np.concatenate([np.arange(128 * p, 128 * p + 128) for p in perm])
    O, L = impl.fwd(q, k, v, 0.4, bm)
    O2, L2 = impl.fwd(q, k[idx], v[idx], 0.4, bm[:, perm])
    assert np.allclose(O, O2, atol=TOL) and np.allclose(L, L2, atol=TOL)


PINS = [pin_all_on_is_plain, pin_block_diagonal_is_independent, pin_empty_block_row, pin_torch_masked_attention,
        pin_brute_force, pin_key_block_permutation]
MUTANTS = ["block_127", "mask_transposed", "causal_ignored", "mask_ignored", "softmax_over_all_keys"]


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
        except (AssertionError, ValueError, IndexError):
            return
    pytest.fail(f"planted mistake {bug!r} passes every pin")


def test_rows_and_batched_wrappers():
    r = _rng(8)
    Q, K, V = (r.standard_normal((2, 2, 200, 4)) for _ in range(3))
    bms = r.random((2, 2, 2, 2)) < 0.7
    O, L = bs.forward_block_sparse(Q, K, V, 0.5, bms, causal=True, kv_len=[200, 150])
    for b in range(2):
        for h in range(2):
            kl = [200, 150][b]
            o, l = bs.head_forward_block_sparse(Q[b, h], K[b, h], V[b, h], 0.5, bms[b, h], True, kl)
            assert np.array_equal(o, O[b, h]) and np.array_equal(l, L[b, h])
            rows = [0, 77, 128, 199]
            orow, lrow = bs.forward_rows_block_sparse(Q[b, h], K[b, h], V[b, h], rows, 0.5, bms[b, h], True, kl)
            assert np.allclose(orow, o[rows], atol=TOL) and np.allclose(lrow, l[rows], atol=TOL)


def test_rejects_wrong_mask_shape():
    with pytest.raises(ValueError):
        bs.block_sparse_visible(300, np.ones((2, 2), bool))
