"""fp64 CPU oracle for the 8-bit floating-point forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the library never does.

The pages say that FlashAttention-3 adds an 8-bit floating-point forward,
that this mode is the one place the method loses precision (rounding to
8 bits, which no tiling recovers), and that its loss is 2.6 times lower
than a naive 8-bit baseline ("FlashAttention — why it mattered", on
FlashAttention-3; "FlashAttention and GPU Memory", chapter 11). They do not
define the format or the scaling. Readings taken here:

  * the inputs Q, K, V arrive already in 8 bits, OCP FP8 E4M3 (1 sign,
    4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinity,
    S.1111.111 is NaN, largest finite 448), each tensor with one fp32
    dequantisation factor; V is given transposed, [B, H, d, N];
  * the result to match is exact attention on the dequantised inputs:
    O = softmax(s Q K^T) V and LSE from the plain oracle, with
    Q = dq * decode(Q8), K = dk * decode(K8), V = dv * decode(V8)^T.
    Whatever the kernel rounds to 8 bits inside (the weights P fed to the
    P V product) is its approximation error, bounded in the tests from the
    E4M3 rounding rules.

``e4m3_encode`` (round to nearest even, saturating to +-448) is here for
the tests' input quantisation and their naive 8-bit baseline.
Pinned by tests/test_oracle_fp8.py.
"""
from __future__ import annotations

import numpy as np

from .attention import head_forward

__all__ = ["e4m3_decode", "e4m3_encode", "head_forward_fp8", "forward_fp8", "E4M3_MAX"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def _grid():
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))   # codes 0x00..0x7E: 0 .. 448, ascending
    return pos


_POS = None


def e4m3_encode(x) -> np.ndarray:
    """float -> uint8 E4M3 codes, round to nearest (ties to an even code), saturating at +-448."""
    global _POS
    if _POS is None:
        _POS = _grid()
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")           # first grid value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def head_forward_fp8(q8, k8, vt8, dq, dk, dv, scale, causal=False, kv_len=None):
    """(O, LSE) of one head from E4M3 codes: q8, k8 [N, d]; vt8 [d, N]; fp32 factors dq, dk, dv."""
    q = e4m3_decode(q8) * float(np.float32(dq))
    k = e4m3_decode(k8) * float(np.float32(dk))
    v = e4m3_decode(vt8).T * float(np.float32(dv))
    return head_forward(q, k, v, scale, causal, kv_len)


def forward_fp8(Q8, K8, Vt8, dq, dk, dv, scale, causal=False, kv_len=None):
    """Batched: Q8, K8 [B, H, N, d]; Vt8 [B, H, d, N]."""
    B, H, N, d = Q8.shape
    O = np.zeros((B, H, N, d), np.float64)
    L = np.zeros((B, H, N), np.float64)
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            O[b, h], L[b, h] = head_forward_fp8(Q8[b, h], K8[b, h], Vt8[b, h], dq, dk, dv, scale, causal, kl)
    return O, L
