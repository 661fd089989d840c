"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.oracle_pins import PINS

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _fwd(q, k, v, scale, causal, kv_len):
    return oracle.head_forward(q, k, v, scale, causal, kv_len)


def _bwd(q, k, v, do, scale, causal, kv_len):
    return oracle.head_backward(q, k, v, do, scale, causal, kv_len)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(_fwd, _bwd)


def test_online_softmax_matches_direct():
    """"FlashAttention and GPU Memory", chapter 08: a row of 8 scores taken 2
    at a time; after the last step m is the row maximum and the weights equal
    a softmax over the whole row to below 1e-15. The page prints the final
    m = 3.4 and l = 2.170462 but not the 8 scores, so the values themselves
    stay unpinned; the property is pinned on rows whose maximum is 3.4."""
    r = np.random.default_rng(20)
    for trial in range(50):
        x = r.uniform(-3, 3.4, size=8)
        x[r.integers(8)] = 3.4
        m, ell, w = oracle.online_softmax(x, 2)
        assert m == 3.4
        direct = np.exp(x - x.max())
        assert abs(ell - direct.sum()) < 1e-15 * 8
        assert np.max(np.abs(w - direct / direct.sum())) < 1e-15


def test_online_softmax_update_order():
    """Blocks that raise, keep and lower the running maximum all agree with
    the single-block tally."""
    x = np.array([0.5, -1.0, 2.0, 1.0, 3.4, -2.0, 0.0, 3.3])
    ref = oracle.online_softmax(x, 8)
    for blk in (1, 2, 3, 4, 5, 7):
        m, ell, w = oracle.online_softmax(x, blk)
        assert m == ref[0]
        assert abs(ell - ref[1]) < 1e-14
        assert np.max(np.abs(w - ref[2])) < 1e-15


@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_blockwise_row_equals_definition(block):
    """The tiled algorithm (running max, rescaled unnormalised output) reaches
    the definition up to rounding ("FlashAttention and GPU Memory", chapters
    08 and 12)."""
    r = np.random.default_rng(21)
    N, d = 100, 16
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    k[37] *= 8.0
    O, lse = oracle.head_forward(q, k, v, 0.25, False, None)
    for i in (0, 17, 99):
        o, l = oracle.blockwise_attention_row(q[i], k, v, 0.25, block)
        assert np.max(np.abs(o - O[i])) < 1e-13
        assert abs(l - lse[i]) < 1e-13


@pytest.mark.parametrize("causal,L", [(False, None), (True, None), (False, 37), (True, 20)])
def test_matches_torch_sdpa_float64(causal, L):
    """Reduces to a library routine: torch's CPU scaled_dot_product_attention
    in float64 with autograd, on small heads."""
    r = np.random.default_rng(22)
    N, d = 48, 16
    q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
    s = 1 / math.sqrt(d)
    O, _ = oracle.head_forward(q, k, v, s, causal, L)
    dq, dk, dv = oracle.head_backward(q, k, v, do, s, causal, L)
    tq, tk, tv = (torch.tensor(a[None, None], requires_grad=True) for a in (q, k, v))
    mask = torch.tensor(oracle.visible_mask(N, N, causal, L))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask[None, None], scale=float(np.float32(s)))
    out.backward(torch.tensor(do[None, None]))
    np.testing.assert_allclose(O, out.detach()[0, 0].numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dq, tq.grad[0, 0].numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk.grad[0, 0].numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad[0, 0].numpy(), atol=1e-12, rtol=0)


def test_batched_wrappers_and_rows():
    """The [B, H, N, d] wrappers equal per-head calls with per-batch kv_len;
    forward_rows equals the matching rows of the full head."""
    r = np.random.default_rng(23)
    B, H, N, d = 2, 3, 20, 8
    Q, K, V, dO = (r.standard_normal((B, H, N, d)) for _ in range(4))
    kv = np.array([13, 20], np.int32)
    O, LSE = oracle.forward(Q, K, V, 0.3, True, kv)
    dQ, dK, dV = oracle.backward(Q, K, V, dO, 0.3, True, kv)
    for b in range(B):
        for h in range(H):
            o, l = oracle.head_forward(Q[b, h], K[b, h], V[b, h], 0.3, True, int(kv[b]))
            g = oracle.head_backward(Q[b, h], K[b, h], V[b, h], dO[b, h], 0.3, True, int(kv[b]))
            assert np.array_equal(o, O[b, h]) and np.array_equal(l, LSE[b, h])
            assert all(np.array_equal(x, y) for x, y in zip(g, (dQ[b, h], dK[b, h], dV[b, h])))
    rows = [0, 5, 19]
    o, l = oracle.forward_rows(Q[1, 2], K[1, 2], V[1, 2], rows, 0.3, True, int(kv[1]))
    np.testing.assert_allclose(o, O[1, 2, rows], atol=1e-14, rtol=0)
    np.testing.assert_allclose(l, LSE[1, 2, rows], atol=1e-14, rtol=0)
