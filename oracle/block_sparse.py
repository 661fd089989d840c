"""fp64 CPU oracle for block-sparse attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the library never does.

The pages name block-sparse FlashAttention as the paper's separate,
approximate method, the one used for the 64K-long Path-256 task
("FlashAttention and GPU Memory", chapters 10 and 12), and say nothing more
about it. Readings taken here:

  * the caller supplies the sparsity pattern as a boolean block mask
    M[qb, kb] per (batch, head) over blocks of BLOCK = 128 queries by
    BLOCK = 128 keys;
  * key j is visible to query i iff M[i // BLOCK, j // BLOCK] holds, in
    addition to the usual rules (j < kv_len[b], and j <= i when causal);
  * within those visible keys the result is the exact softmax attention of
    the plain oracle: O = softmax(s Q K^T restricted to visible keys) V and
    LSE over the same keys; a row with no visible key has O = 0,
    LSE = -inf.

Pinned by tests/test_oracle_block_sparse.py.
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_rows, fp32_scale, visible_mask

__all__ = ["BLOCK", "block_sparse_visible", "head_forward_block_sparse", "forward_block_sparse",
           "forward_rows_block_sparse"]

BLOCK = 128


def block_sparse_visible(n: int, block_mask, causal=False, kv_len=None, rows=None) -> np.ndarray:
    """Boolean [len(rows), n]: visible pairs of one head under a [ceil(n/128)]^2 block mask."""
    bm = np.asarray(block_mask, dtype=bool)
    nb = (n + BLOCK - 1) // BLOCK
    if bm.shape != (nb, nb):
        raise ValueError(f"block mask must be {nb} x {nb}")
    rows = np.arange(n) if rows is None else np.asarray(rows)
    vis = visible_mask(n, n, causal, kv_len, rows)
    return vis & bm[rows // BLOCK][:, np.arange(n) // BLOCK]


def head_forward_block_sparse(q, k, v, scale, block_mask, causal=False, kv_len=None):
    """(O, LSE) of one head: softmax attention over the visible keys only."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    S = fp32_scale(scale) * (q @ k.T)
    P, lse = _softmax_rows(S, block_sparse_visible(q.shape[0], block_mask, causal, kv_len))
    return P @ v, lse


def forward_rows_block_sparse(q, k, v, rows, scale, block_mask, causal=False, kv_len=None):
    """(O, LSE) of selected query rows of one head, each from its own row of scores."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    rows = np.asarray(rows)
    S = fp32_scale(scale) * (q[rows] @ k.T)
    P, lse = _softmax_rows(S, block_sparse_visible(q.shape[0], block_mask, causal, kv_len, rows))
    return P @ v, lse


def forward_block_sparse(Q, K, V, scale, block_masks, causal=False, kv_len=None):
    """Batched [B, H, N, d]; block_masks is [B, H, nb, nb] (or [nb, nb] for every head)."""
    B, H = Q.shape[:2]
    bm = np.asarray(block_masks, dtype=bool)
    O = np.zeros(Q.shape, np.float64)
    L = np.zeros(Q.shape[:3], np.float64)
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            m = bm if bm.ndim == 2 else bm[b, h]
            O[b, h], L[b, h] = head_forward_block_sparse(Q[b, h], K[b, h], V[b, h], scale, m, causal, kl)
    return O, L
