"""fp64 CPU oracle for attention with fused dropout (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the library never does, and nothing here is shared with
the HIP kernels (the kernels carry their own implementation of the same
published generator).

What the pages fix: dropout is one of the steps fused into the single
kernel program (load, multiply, softmax, mask, dropout, multiply --
"FlashAttention and GPU Memory", chapter 07 Blocks), and the backward does
not store the dropout mask but regenerates it from the generator state
(chapter 09). They say nothing about the generator, the mask layout or the
scaling. The readings taken here:

  * generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
    Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011),
    with its published round constants;
  * key = (seed mod 2^32, seed >> 32); counter = (j >> 2, i >> 2, bh, offset)
    for query i, key j and head index bh = b * H + h, so one call covers a
    4 x 4 block of (query, key) pairs; element (i, j) takes byte j & 3 of
    output word i & 3;
  * keep iff that byte >= t with t = round(256 p): the keep probability is
    exactly (256 - t) / 256, and kept weights are multiplied by
    256 / (256 - t) so the expectation of the dropped output is the exact
    attention output;
  * dropout acts on the normalised weights P (the softmax itself and the
    saved LSE are those of the undropped scores): O = (P o Z c) V;
  * backward by the chain rule: dV = (P o Z c)^T dO, dP = (dO V^T) o Z c,
    dS = P o (dP - rowsum(P o dP)), dQ = s dS K, dK = s dS^T Q. The row
    sum is taken literally; it equals rowsum(dO o O), which the kernels use.

Pinned by tests/test_oracle_dropout.py (published known-answer values of
the generator, keep-rate and byte-uniformity statistics, p = 0 reducing to
the plain oracle, autograd of the same masked expression, finite
differences and planted mistakes).
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_rows, fp32_scale, visible_mask

__all__ = ["philox4x32_10", "dropout_threshold", "dropout_keep_scale", "dropout_keep",
           "head_forward_dropout", "head_backward_dropout", "forward_dropout", "backward_dropout"]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57      # Philox4x32 multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments
_MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.

    counter: four uint32 arrays (or ints) of a common shape; key: two ints.
    Returns four uint32 arrays. Each round multiplies words 0 and 2 by the
    two constants (64-bit products), and the new words are
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
    the key advances by the Weyl increments after every round.
    """
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in counter]
    c = np.broadcast_arrays(*c)
    c = [x.copy() for x in c]
    k0, k1 = int(key[0]) & _MASK32, int(key[1]) & _MASK32
    for _ in range(10):
        p0 = c[0] * np.uint64(_M0)
        p1 = c[2] * np.uint64(_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK32)
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + _W0) & _MASK32
        k1 = (k1 + _W1) & _MASK32
    return [x.astype(np.uint32) for x in c]


def dropout_threshold(p: float) -> int:
    """Byte threshold t = round(256 p); a weight is kept iff its byte >= t."""
    p = float(p)
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    t = int(np.floor(p * 256.0 + 0.5))
    if t >= 256:
        raise ValueError("dropout probability rounds to 1")
    return t


def dropout_keep_scale(p: float) -> float:
    """Factor applied to kept weights: 256 / (256 - t)."""
    return 256.0 / (256.0 - dropout_threshold(p))


def dropout_keep(n_q: int, n_k: int, bh: int, p: float, seed: int, offset: int = 0,
                 rows=None, cols=None) -> np.ndarray:
    """Boolean keep mask Z[i, j] for one head (rows/cols select a sub-block)."""
    t = dropout_threshold(p)
    i = np.arange(n_q) if rows is None else np.asarray(rows)
    j = np.arange(n_k) if cols is None else np.asarray(cols)
    I, J = np.meshgrid(i, j, indexing="ij")
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    out = philox4x32_10((J >> 2, I >> 2, np.full_like(I, bh), np.full_like(I, int(offset) & _MASK32)),
                        (seed & _MASK32, seed >> 32))
    word = np.choose(I & 3, out)
    byte = (word.astype(np.uint64) >> (8 * (J & 3)).astype(np.uint64)) & np.uint64(0xFF)
    return byte >= np.uint64(t)


def _probs(q, k, scale, causal, kv_len):
    s = fp32_scale(scale)
    S = s * (q @ k.T)
    vis = visible_mask(q.shape[0], k.shape[0], causal, kv_len)
    P, lse = _softmax_rows(S, vis)
    return s, P, lse


def head_forward_dropout(q, k, v, scale, p, seed, bh, offset=0, causal=False, kv_len=None):
    """(O, LSE) of one head with dropout: O = (P o Z c) V, LSE of the undropped scores."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    _, P, lse = _probs(q, k, scale, causal, kv_len)
    Z = dropout_keep(q.shape[0], k.shape[0], bh, p, seed, offset)
    Pd = P * Z * dropout_keep_scale(p)
    return Pd @ v, lse


def head_backward_dropout(q, k, v, do, scale, p, seed, bh, offset=0, causal=False, kv_len=None):
    """(dQ, dK, dV) of one head with dropout, by the chain rule of head_forward_dropout."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s, P, _ = _probs(q, k, scale, causal, kv_len)
    Zc = dropout_keep(q.shape[0], k.shape[0], bh, p, seed, offset) * dropout_keep_scale(p)
    dV = (P * Zc).T @ do
    dP = (do @ v.T) * Zc
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return s * (dS @ k), s * (dS.T @ q), dV


def forward_dropout(Q, K, V, scale, p, seed, offset=0, causal=False, kv_len=None):
    """Batched [B, H, N, d] forward with dropout; head bh = b * H + h."""
    B, H = Q.shape[:2]
    O = np.zeros(Q.shape, np.float64)
    L = np.zeros(Q.shape[:3], np.float64)
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            O[b, h], L[b, h] = head_forward_dropout(Q[b, h], K[b, h], V[b, h], scale, p, seed, b * H + h,
                                                    offset, causal, kl)
    return O, L


def backward_dropout(Q, K, V, dO, scale, p, seed, offset=0, causal=False, kv_len=None):
    """Batched [B, H, N, d] backward with dropout; head bh = b * H + h."""
    B, H = Q.shape[:2]
    dQ, dK, dV = (np.zeros(Q.shape, np.float64) for _ in range(3))
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = head_backward_dropout(
                Q[b, h], K[b, h], V[b, h], dO[b, h], scale, p, seed, b * H + h, offset, causal, kl)
    return dQ, dK, dV
