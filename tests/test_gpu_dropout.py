"""GPU parity of the fused-dropout paths against the fp64 oracle.

* The keep mask written by flash_attn_dropout_mask equals the oracle's
  bit for bit (integer work).
* The masks the fused kernels regenerate are read out exactly: with one-hot
  rows of V, O[i, j] is non-zero iff the forward kept (i, j); with one-hot
  rows of dO, dV[j, c] is non-zero iff the dK/dV kernel kept (q0 + c, j).
* O, LSE, dQ, dK, dV agree with oracle.dropout element by element within the
  tolerances of the other bf16 paths, on ragged, causal and padded shapes,
  and on two full heads of the B=16 H=16 N=4096 d=128 workload in its
  benchmark launch shape; the same outputs are far from the oracle run with
  another seed.
* p = 0 reproduces the plain entry points; equal (seed, offset) reproduce
  bitwise, a new offset draws a new mask.
"""
import numpy as np
import pytest

from io_aware_exact_11_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _fa():
    import io_aware_exact_11_amd as fa
    fa.load_library()
    return fa


def _inputs(B, H, N, d, seed, padded=False, qkv_scale=1.0):
    from tests.gpu_util import dev_bf16, dev_kv
    x = wl.make_inputs(B, H, N, d, seed=seed, padded=padded, qkv_scale=qkv_scale)
    dev = {n: dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V", "dO")}
    return x, dev, dev_kv(x["kv_len"])


MASK_CASES = [(1, 1, 4, 4, 0.5, 1, 0), (2, 3, 37, 53, 0.1, (1 << 40) + 5, 3), (1, 2, 256, 130, 0.9, 123, 0),
              (1, 1, 64, 64, 0.0, 9, 0), (2, 1, 130, 257, 0.25, 77, (1 << 31) + 1), (1, 1, 9, 1031, 0.99, 5, 7)]


@pytest.mark.parametrize("B,H,Nq,Nk,p,seed,offset", MASK_CASES)
def test_mask_bit_exact(B, H, Nq, Nk, p, seed, offset):
    from oracle import dropout as od
    from tests.gpu_util import log
    fa = _fa()
    log(f"  mask B={B} H={H} Nq={Nq} Nk={Nk} p={p} seed={seed} offset={offset}")
    M = fa.flash_attn_dropout_mask(B, H, Nq, Nk, p, seed, offset).cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = od.dropout_keep(Nq, Nk, b * H + h, p, seed, offset)
            assert np.array_equal(M[b, h].astype(bool), ref), (b, h, int((M[b, h].astype(bool) != ref).sum()))


READOUT = [(1, 2, 192, 64, False, 0.3), (1, 2, 160, 128, True, 0.5), (2, 1, 130, 64, True, 0.2),
           (1, 1, 256, 128, False, 0.1)]


@pytest.mark.parametrize("B,H,N,d,causal,p", READOUT)
def test_forward_mask_readout(B, H, N, d, causal, p):
    """One-hot V rows for keys k0 .. k0+d-1: O[i, c] != 0 iff key k0 + c is visible and kept."""
    import oracle
    from oracle import dropout as od
    from tests.gpu_util import log
    fa = _fa()
    log(f"  fwd readout B={B} H={H} N={N} d={d} causal={causal} p={p}")
    x, dev, _ = _inputs(B, H, N, d, seed=40 + N, qkv_scale=0.5)
    seed, offset = 987654321, 4
    for k0 in range(0, N, d):
        w = min(d, N - k0)
        vh = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
        idx = torch.arange(w, device="cuda")
        vh[:, :, k0 + idx, idx] = 1.0
        O, _ = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], vh, p, seed, offset, causal=causal)
        got = (O[..., :w] != 0).cpu().numpy()
        for b in range(B):
            for h in range(H):
                Z = od.dropout_keep(N, N, b * H + h, p, seed, offset)[:, k0:k0 + w]
                vis = oracle.visible_mask(N, N, causal)[:, k0:k0 + w]
                assert np.array_equal(got[b, h], Z & vis), (k0, b, h, int((got[b, h] != (Z & vis)).sum()))


@pytest.mark.parametrize("B,H,N,d,causal,p", READOUT)
def test_dkdv_mask_readout(B, H, N, d, causal, p):
    """One-hot dO rows for queries q0 .. q0+d-1: dV[j, c] != 0 iff key j is visible to q0 + c and kept."""
    import oracle
    from oracle import dropout as od
    from tests.gpu_util import log
    fa = _fa()
    log(f"  dkdv readout B={B} H={H} N={N} d={d} causal={causal} p={p}")
    x, dev, _ = _inputs(B, H, N, d, seed=50 + N, qkv_scale=0.5)
    seed, offset = 2024, 0
    O, lse = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], p, seed, offset, causal=causal)
    for q0 in range(0, N, d):
        w = min(d, N - q0)
        g = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
        idx = torch.arange(w, device="cuda")
        g[:, :, q0 + idx, idx] = 1.0
        _, _, dV = fa.flash_attn_bwd_dropout(dev["Q"], dev["K"], dev["V"], O, g, lse, p, seed, offset, causal=causal)
        got = (dV[..., :w] != 0).cpu().numpy()          # [B, H, key, c]
        for b in range(B):
            for h in range(H):
                Z = od.dropout_keep(N, N, b * H + h, p, seed, offset)[q0:q0 + w, :].T
                vis = oracle.visible_mask(N, N, causal)[q0:q0 + w, :].T
                assert np.array_equal(got[b, h], Z & vis), (q0, b, h, int((got[b, h] != (Z & vis)).sum()))


# Padded inputs carry one x8 outlier key per head, which makes the gradients
# large; as on the plain path, their backward runs in precise mode.
PARITY = [(1, 2, 200, 64, False, False, 0.1, False), (2, 2, 256, 128, True, False, 0.3, False),
          (2, 2, 333, 64, True, True, 0.2, True), (2, 2, 384, 128, False, True, 0.1, True),
          (1, 3, 129, 128, True, False, 0.5, False), (2, 2, 1024, 64, True, False, 0.1, False),
          (1, 2, 300, 128, True, False, 0.2, True)]


@pytest.mark.parametrize("B,H,N,d,causal,padded,p,precise", PARITY)
def test_forward_backward_parity(B, H, N, d, causal, padded, p, precise):
    from oracle import dropout as od
    from tests.gpu_util import compare, compare_lse, host, log
    fa = _fa()
    log(f"  parity B={B} H={H} N={N} d={d} causal={causal} padded={padded} p={p} precise={precise}")
    x, dev, kv = _inputs(B, H, N, d, seed=60 + N + d, padded=padded)
    seed, offset = 31337, 11
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], p, seed, offset, causal=causal, scale=scale,
                                       kv_len=kv)
    dQ, dK, dV = fa.flash_attn_bwd_dropout(dev["Q"], dev["K"], dev["V"], O, dev["dO"], lse, p, seed, offset,
                                           causal=causal, scale=scale, kv_len=kv, precise=precise)
    torch.cuda.synchronize()
    L = x["kv_len"]
    Ro, Rl = od.forward_dropout(x["Q"], x["K"], x["V"], scale, p, seed, offset, causal, L)
    Rq, Rk, Rv = od.backward_dropout(x["Q"], x["K"], x["V"], x["dO"], scale, p, seed, offset, causal, L)
    compare("O", host(O), Ro)
    compare_lse(host(lse), Rl)
    compare("dQ", host(dQ), Rq)
    compare("dK", host(dK), Rk)
    compare("dV", host(dV), Rv)
    # Another seed gives a different mask: the outputs are then far from the oracle.
    Wo, _ = od.forward_dropout(x["Q"], x["K"], x["V"], scale, p, seed + 1, offset, causal, L)
    assert np.abs(host(O) - Wo).mean() > 5 * np.abs(host(O) - Ro).mean()


def test_full_size_n4096_d128_workload():
    """The B=16 H=16 N=4096 d=128 non-causal workload at p = 0.1 in the benchmark's launch shape; heads
    (0, 0) and (15, 15) are compared in full, fwd and bwd."""
    from oracle import dropout as od
    from tests.gpu_util import compare, compare_lse, dev_bf16, host, log
    fa = _fa()
    x = wl.workload_inputs("n4096_d128")
    B, H, N, d = x["Q"].shape
    log(f"  full-size B={B} H={H} N={N} d={d} p=0.1")
    dev = {n: dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V", "dO")}
    scale = float(np.float32(d ** -0.5))
    seed, offset = 0xDEADBEEF12345, 3
    O, lse = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.1, seed, offset, scale=scale)
    dQ, dK, dV = fa.flash_attn_bwd_dropout(dev["Q"], dev["K"], dev["V"], O, dev["dO"], lse, 0.1, seed, offset,
                                           scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (15, 15)):
        bh = b * H + h
        args = (x["Q"][b, h], x["K"][b, h], x["V"][b, h])
        o, l = od.head_forward_dropout(*args, scale, 0.1, seed, bh, offset)
        compare("O", host(O[b, h]), o)
        compare_lse(host(lse[b, h]), l)
        g = od.head_backward_dropout(*args, x["dO"][b, h], scale, 0.1, seed, bh, offset)
        for nm, got, ref in zip(("dQ", "dK", "dV"), (dQ, dK, dV), g):
            compare(nm, host(got[b, h]), ref)


@pytest.mark.parametrize("d,causal", [(64, True), (64, False), (128, False)])
def test_p_zero_matches_plain_entry_points(d, causal):
    fa = _fa()
    x, dev, _ = _inputs(2, 2, 300, d, seed=8)
    O0, L0 = fa.flash_attn_fwd(dev["Q"], dev["K"], dev["V"], causal=causal)
    O1, L1 = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.0, 99, 0, causal=causal)
    assert torch.equal(O0, O1) and torch.equal(L0, L1)
    g0 = fa.flash_attn_bwd(dev["Q"], dev["K"], dev["V"], O0, dev["dO"], L0, causal=causal)
    g1 = fa.flash_attn_bwd_dropout(dev["Q"], dev["K"], dev["V"], O0, dev["dO"], L0, 0.0, 99, 0, causal=causal)
    # The plain dQ kernel accumulates dP onto -D_i inside the matrix product,
    # the dropout kernel subtracts D_i afterwards: dS_ij can round to
    # neighbouring bf16 values, which moves the gradients by a few bf16 ulps
    # of dS (far below the parity tolerance; a mask applied at p = 0 would
    # move them by O(1)).
    for a, b in zip(g0, g1):
        assert float((a - b).abs().max()) <= 2e-3 * max(1.0, float(a.abs().max()))


def test_reproducible_and_offset_draws_new_mask():
    fa = _fa()
    x, dev, _ = _inputs(1, 2, 256, 128, seed=9)
    a, _ = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.2, 1, 0)
    b, _ = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.2, 1, 0)
    c, _ = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.2, 1, 1)
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


@pytest.mark.parametrize("N,d,causal", [(1, 64, False), (1, 128, True), (63, 128, False), (65, 64, True),
                                        (129, 128, True)])
def test_dropout_edge_lengths(N, d, causal):
    from oracle import dropout as od
    from tests.gpu_util import compare, compare_lse, host, log
    fa = _fa()
    log(f"  dropout edge N={N} d={d} causal={causal}")
    x, dev, _ = _inputs(1, 2, N, d, seed=3 + N)
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.3, 77, 1, causal=causal, scale=scale)
    g = fa.flash_attn_bwd_dropout(dev["Q"], dev["K"], dev["V"], O, dev["dO"], lse, 0.3, 77, 1, causal=causal,
                                  scale=scale)
    torch.cuda.synchronize()
    Ro, Rl = od.forward_dropout(x["Q"], x["K"], x["V"], scale, 0.3, 77, 1, causal)
    Rg = od.backward_dropout(x["Q"], x["K"], x["V"], x["dO"], scale, 0.3, 77, 1, causal)
    compare("O", host(O), Ro)
    compare_lse(host(lse), Rl)
    for nm, a, b in zip(("dQ", "dK", "dV"), g, Rg):
        compare(nm, host(a), b)


def test_dropout_kv_len_zero_rows():
    """A batch row with kv_len = 0 has no visible key: O = 0, LSE = -inf, zero gradients."""
    fa = _fa()
    x, dev, _ = _inputs(2, 2, 96, 64, seed=12)
    kv = torch.tensor([0, 96], dtype=torch.int32, device="cuda")
    O, lse = fa.flash_attn_fwd_dropout(dev["Q"], dev["K"], dev["V"], 0.2, 5, 0, kv_len=kv)
    dQ, dK, dV = fa.flash_attn_bwd_dropout(dev["Q"], dev["K"], dev["V"], O, dev["dO"], lse, 0.2, 5, 0, kv_len=kv)
    torch.cuda.synchronize()
    assert torch.all(O[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(dQ[0] == 0) and torch.all(dK[0] == 0) and torch.all(dV[0] == 0)
    assert torch.all(torch.isfinite(lse[1]))
