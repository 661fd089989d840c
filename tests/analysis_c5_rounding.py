"""Which bf16 rounding dominates the default backward's error on the padded
workload (B=8 H=32 N=8192 d=64, key padding, one x8 outlier key per head).

Standalone analysis, not collected by pytest (about 25 s of CPU per head):

    python tests/analysis_c5_rounding.py [n_heads]

For each head it takes the fp64 oracle's gradients as the reference and
emulates the kernels' arithmetic on the host in fp32 with bf16
round-to-nearest-even at the points where the kernels round: the weights P
fed to dV = P^T dO and the dS fed to dK = scale dS^T Q and dQ = scale dS K.
Six variants switch the three suspected error sources one at a time:

* D_i from the bf16 output O (the default kernels) / from the fp32 output /
  exact (sum_j P_ij dP_ij, what precise mode computes);
* dS as one bf16 value, or as a bf16 hi/lo pair (two matrix products);
* P as one bf16 value, or as a hi/lo pair.

It prints max-abs, mean-abs and err / max(1, max |ref|) per gradient, and the
worst over the heads. This is test infrastructure: it calls the oracle and
shares nothing with the HIP kernels.
"""
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
from io_aware_exact_11_amd import workloads as wl  # noqa: E402

LOG2E = np.float32(1.4426950408889634)
LN2 = np.float32(0.6931471805599453)


def bf16(x):
    """fp32 -> bf16 (round to nearest even), returned as fp32."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32)


def hi_lo(x):
    hi = bf16(x)
    return hi, bf16(x.astype(np.float32) - hi)


VARIANTS = (
    ("default (D from bf16 O)", "bf16_o", False, False),
    ("D from fp32 O", "fp32_o", False, False),
    ("exact D", "exact", False, False),
    ("exact D + hi/lo dS", "exact", True, False),
    ("exact D + hi/lo dS, P (precise)", "exact", True, True),
    ("D from bf16 O + hi/lo dS, P", "bf16_o", True, True),
)


def emulate(q, k, v, do, scale, L):
    s32 = np.float32(scale)
    sl2 = np.float32(s32 * LOG2E)
    S = q.astype(np.float32) @ k.T.astype(np.float32)
    S[:, L:] = -np.inf
    m = (S * sl2).max(axis=1)
    Pt = np.exp2(S * sl2 - m[:, None]).astype(np.float32)
    l = Pt.sum(axis=1, dtype=np.float32)
    O = (bf16(Pt) @ v) / l[:, None]
    lse = (m + np.log2(l)) * LN2
    P = np.exp2(S * sl2 - (lse * LOG2E)[:, None]).astype(np.float32)
    dP = (do @ v.T).astype(np.float32)
    Ds = {"bf16_o": (do * bf16(O)).sum(axis=1, dtype=np.float32),
          "fp32_o": (do * O.astype(np.float32)).sum(axis=1, dtype=np.float32),
          "exact": (P * dP).sum(axis=1, dtype=np.float32)}
    out = {}
    for name, dsrc, split_ds, split_p in VARIANTS:
        dS = (P * (dP - Ds[dsrc][:, None])).astype(np.float32)
        dS_parts = list(hi_lo(dS)) if split_ds else [bf16(dS)]
        P_parts = list(hi_lo(P)) if split_p else [bf16(P)]
        dV = sum(x.T @ do for x in P_parts)
        dK = s32 * sum(x.T @ q for x in dS_parts)
        dQ = s32 * sum(x @ k for x in dS_parts)
        out[name] = (dQ, dK, dV)
    return out


def main(n_heads=6):
    name = "padded_8k"
    w = wl.WORKLOADS[name]
    x = wl.workload_inputs(name)
    rng = np.random.default_rng(11)
    heads = [(0, 0), (0, w.H - 1), (w.B - 1, 0), (w.B - 1, w.H - 1)]
    heads += [tuple(int(t) for t in bh) for bh in rng.integers(0, [w.B, w.H], size=(max(0, n_heads - 4), 2))]
    worst = {}
    for b, h in heads[:n_heads]:
        L = int(x["kv_len"][b])
        q, k, v, do = (x[n][b, h] for n in ("Q", "K", "V", "dO"))
        t0 = time.time()
        ref = oracle.head_backward(q, k, v, do, w.scale, False, kv_len=L)
        res = emulate(q, k, v, do, w.scale, L)
        print(f"head b={b} h={h} kv_len={L} max|ref| dQ {np.abs(ref[0]).max():.3g} dK {np.abs(ref[1]).max():.3g} "
              f"dV {np.abs(ref[2]).max():.3g} ({time.time() - t0:.1f} s)", flush=True)
        for vname, got in res.items():
            mx = [float(np.abs(a - r).max()) for a, r in zip(got, ref)]
            mn = [float(np.abs(a - r).mean()) for a, r in zip(got, ref)]
            nm = [e / max(1.0, float(np.abs(r).max())) for e, r in zip(mx, ref)]
            acc = worst.setdefault(vname, [0.0] * 9)
            for i in range(3):
                acc[i], acc[3 + i], acc[6 + i] = max(acc[i], mx[i]), max(acc[3 + i], mn[i]), max(acc[6 + i], nm[i])
            print(f"   {vname:34s} max dQ {mx[0]:.2e} dK {mx[1]:.2e} dV {mx[2]:.2e} | "
                  f"mean {mn[0]:.1e} {mn[1]:.1e} {mn[2]:.1e}", flush=True)
    print("worst over heads: max-abs dQ dK dV | mean-abs | err / max(1, max|ref|)")
    for vname, a in worst.items():
        print(f"  {vname:34s} {a[0]:.2e} {a[1]:.2e} {a[2]:.2e} | {a[3]:.1e} {a[4]:.1e} {a[5]:.1e} | "
              f"{a[6]:.2e} {a[7]:.2e} {a[8]:.2e}")


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 6)
