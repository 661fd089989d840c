"""fp64 CPU oracle for exact attention and its gradients.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module. The library path never
calls it, and it shares no code, tables or helpers with the HIP kernels.

What it computes is the plain definition, written out once per (batch, head)
in float64 with every N x N intermediate materialised:

  * scores S = s * Q K^T with s the fp32 value of the scale the GPU receives
    ("48 FlashAttention", the sdpa snippet: softmax(QK^T/sqrt(d)) V;
    "FlashAttention does more arithmetic to move less data", section
    "FlashAttention never writes the full score table to HBM": the method
    returns softmax(QK^T)V with no approximation);
  * mask: key j is visible to query i iff j < kv_len[b] and, when causal,
    j <= i; invisible scores are -inf ("FlashAttention and GPU Memory",
    chapter 07 Blocks, lists the mask among the fused steps; causal and key
    padding are defined here, the pages name masking without defining it);
  * P = row softmax of S taken with the row maximum subtracted, O = P V, and
    the per-row log-sum-exp LSE = m + ln(sum_j exp(S_ij - m)) -- the
    three-step "standard way" of "FlashAttention and GPU Memory", chapter 04,
    with the saved row statistics of chapter 09 folded into one number;
  * backward by the chain rule (the pages give no formulas):
    dV = P^T dO, dP = dO V^T, dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
    dQ = s dS K, dK = s dS^T Q. The row sum of P*dP is taken literally; the
    shortcut rowsum(dO*O) the kernels use is not used here.

A row whose keys are all masked has no softmax; the oracle returns O = 0,
LSE = -inf and zero gradients for it (a reading: the pages never reach it).

Also here, for pinning the definition against the pages' own algorithm:
``online_softmax`` (the running maximum and sum of "FlashAttention and GPU
Memory", chapter 08) and ``blockwise_attention_row`` (tiles of keys with the
output rescaled by e^(m_old - m_new), chapter 08, and "FlashAttention does
more arithmetic to move less data", the four moves).

Decoding (the bandwidth-bound regime in which each generated token brings a
single query row that must read the whole cache; "FlashAttention — why it
mattered", closing note): ``decode_head_forward`` takes n_q new
queries against a cache of n_k key slots of which the first kv_len hold
keys. Reading (the pages do not define it): the queries are the last n_q
positions of that sequence, so with causal masking query i sees keys
j <= kv_len - n_q + i (bottom-right alignment); without it, all j < kv_len.

Every function here is pinned by tests/test_oracle_pins.py and
tests/test_oracle_decode.py; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "fp32_scale", "visible_mask", "head_forward", "head_backward", "forward",
    "backward", "forward_rows", "online_softmax", "blockwise_attention_row",
    "decode_visible_mask", "decode_head_forward", "decode_forward",
]


def fp32_scale(scale: float) -> float:
    """The softmax scale as the kernels receive it: rounded to float32."""
    return float(np.float32(scale))


def visible_mask(n_q: int, n_k: int, causal: bool, kv_len=None, rows=None) -> np.ndarray:
    """Boolean [len(rows), n_k]: True where query i may attend to key j."""
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    cols = np.arange(n_k)
    limit = n_k if kv_len is None else max(0, min(int(kv_len), n_k))
    vis = np.broadcast_to(cols[None, :] < limit, (rows.size, n_k)).copy()
    if causal:
        vis &= cols[None, :] <= rows[:, None]
    return vis


def _softmax_rows(S: np.ndarray, vis: np.ndarray):
    """Masked row softmax with its log-sum-exp. Fully masked rows give P=0, LSE=-inf."""
    S = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(vis, np.exp(S - m[:, None]), 0.0)
    ell = E.sum(axis=1)
    P = np.divide(E, ell[:, None], out=np.zeros_like(E), where=any_vis[:, None])
    lse = np.where(any_vis, m + np.log(np.where(any_vis, ell, 1.0)), -np.inf)
    return P, lse


def head_forward(q, k, v, scale, causal=False, kv_len=None, return_probs=False):
    """One head: O = softmax(s q k^T + mask) v and LSE, all in float64.

    q, k, v: [N, d] arrays (any float dtype; widened exactly to float64).
    Returns (O [N, d], LSE [N]) and, with return_probs, also P [N, N].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = fp32_scale(scale)
    S = s * (q @ k.T)
    vis = visible_mask(q.shape[0], k.shape[0], causal, kv_len)
    P, lse = _softmax_rows(S, vis)
    O = P @ v
    return (O, lse, P) if return_probs else (O, lse)


def head_backward(q, k, v, do, scale, causal=False, kv_len=None):
    """One head: gradients (dQ, dK, dV) of <dO, O> w.r.t. q, k, v in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    s = fp32_scale(scale)
    _, _, P = head_forward(q, k, v, scale, causal, kv_len, return_probs=True)
    dV = P.T @ do
    dP = do @ v.T
    row_dot = (P * dP).sum(axis=1)
    dS = P * (dP - row_dot[:, None])
    dQ = s * (dS @ k)
    dK = s * (dS.T @ q)
    return dQ, dK, dV


def forward(Q, K, V, scale, causal=False, kv_len=None):
    """[B, H, N, d] inputs -> (O [B, H, N, d] float64, LSE [B, H, N] float64)."""
    B, H, N, d = Q.shape
    O = np.empty((B, H, N, d), np.float64)
    LSE = np.empty((B, H, N), np.float64)
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            O[b, h], LSE[b, h] = head_forward(Q[b, h], K[b, h], V[b, h], scale, causal, L)
    return O, LSE


def backward(Q, K, V, dO, scale, causal=False, kv_len=None):
    """[B, H, N, d] inputs -> (dQ, dK, dV), each [B, H, N, d] float64."""
    B, H, N, d = Q.shape
    dQ = np.empty((B, H, N, d), np.float64)
    dK = np.empty_like(dQ)
    dV = np.empty_like(dQ)
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = head_backward(
                Q[b, h], K[b, h], V[b, h], dO[b, h], scale, causal, L)
    return dQ, dK, dV


def forward_rows(q, k, v, rows, scale, causal=False, kv_len=None):
    """Selected query rows of one head: (O [len(rows), d], LSE [len(rows)]).

    Each row is the definition applied to that row alone, so sampled rows of
    a large head cost O(N d) each.
    """
    q = np.asarray(q, np.float64)[np.asarray(rows)]
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = fp32_scale(scale)
    S = s * (q @ k.T)
    vis = visible_mask(k.shape[0], k.shape[0], causal, kv_len, rows=rows)
    P, lse = _softmax_rows(S, vis)
    return P @ v, lse


def online_softmax(scores, block):
    """Running-tally softmax over one row, ``block`` scores at a time.

    The tally is a pair (m, l): the running row maximum and the running
    sum of e^(x - m) over the scores seen so far. A block with its own
    maximum mb and sum lb updates them as
    m' = max(m, mb), l' = e^(m - m') l + e^(mb - m') lb
    ("FlashAttention and GPU Memory", chapter 08). Returns (m, l, weights)
    with weights_j = e^(x_j - m) / l from the final tally.
    """
    x = np.asarray(scores, np.float64)
    m, ell = -np.inf, 0.0
    for start in range(0, x.size, block):
        blk = x[start:start + block]
        mb = blk.max()
        lb = np.exp(blk - mb).sum()
        m_new = max(m, mb)
        ell = (np.exp(m - m_new) * ell if ell > 0 else 0.0) + np.exp(mb - m_new) * lb
        m = m_new
    return m, ell, np.exp(x - m) / ell


def blockwise_attention_row(qi, k, v, scale, block):
    """One query row by the tiled algorithm: keys and values taken ``block``
    rows at a time, output kept unnormalised and rescaled by e^(m_old - m_new)
    whenever a block raises the running maximum, divided by l at the end
    ("FlashAttention and GPU Memory", chapter 08; "FlashAttention does more
    arithmetic to move less data", the four moves). Returns (o [d], lse).
    """
    qi = np.asarray(qi, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = fp32_scale(scale)
    m, ell = -np.inf, 0.0
    acc = np.zeros(v.shape[1], np.float64)
    for start in range(0, k.shape[0], block):
        sc = s * (k[start:start + block] @ qi)
        m_new = max(m, sc.max())
        alpha = np.exp(m - m_new) if ell > 0 else 0.0
        p = np.exp(sc - m_new)
        ell = alpha * ell + p.sum()
        acc = alpha * acc + p @ v[start:start + block]
        m = m_new
    return acc / ell, m + np.log(ell)


def decode_visible_mask(n_q: int, n_k: int, kv_len=None, causal: bool = False) -> np.ndarray:
    """Boolean [n_q, n_k] for n_q new queries against n_k cache slots.

    The first L = kv_len (or n_k) slots hold keys. Without causal masking
    every query sees keys j < L; with it, query i is position L - n_q + i of
    the sequence and sees keys j <= L - n_q + i.
    """
    L = n_k if kv_len is None else max(0, min(int(kv_len), n_k))
    cols = np.arange(n_k)[None, :]
    vis = np.broadcast_to(cols < L, (n_q, n_k)).copy()
    if causal:
        vis &= cols <= (L - n_q + np.arange(n_q))[:, None]
    return vis


def decode_head_forward(q, k, v, scale, kv_len=None, causal=False):
    """n_q queries against one head's key/value cache, in float64.

    q: [n_q, d]; k, v: [n_k, d]. Returns (O [n_q, d], LSE [n_q]) with the
    same softmax, log-sum-exp and fully-masked-row conventions as
    ``head_forward``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = fp32_scale(scale)
    S = s * (q @ k.T)
    P, lse = _softmax_rows(S, decode_visible_mask(q.shape[0], k.shape[0], kv_len, causal))
    return P @ v, lse


def decode_forward(Q, K, V, scale, kv_len=None, causal=False):
    """Q [B, H, n_q, d], K and V [B, H, n_k, d] -> (O [B, H, n_q, d], LSE [B, H, n_q]) float64."""
    B, H, n_q, d = Q.shape
    O = np.empty((B, H, n_q, d), np.float64)
    LSE = np.empty((B, H, n_q), np.float64)
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            O[b, h], LSE[b, h] = decode_head_forward(Q[b, h], K[b, h], V[b, h], scale, L, causal)
    return O, LSE
