"""GPU parity: the HIP path against the fp64 oracle, element by element.

Small cases (several tiles plus a ragged tail) are compared in full; the
workloads at their full sizes run in the same launch configuration the
benchmark times and are compared on sampled heads. All inputs come from the
seeded generator; the oracle sees exactly the bf16 values the GPU sees.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_11_amd import workloads as wl
from tests.gpu_util import compare, compare_lse, dev_bf16, dev_f32, dev_kv, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_11_amd as fa
    fa.load_library()


def _fa():
    import io_aware_exact_11_amd as fa
    return fa


def _run_bf16(x, causal, scale, kv, precise=False, dq_atomic=False):
    fa = _fa()
    q, k, v, do = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V", "dO"))
    kvd = dev_kv(kv)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=causal, scale=scale, kv_len=kvd)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, kv_len=kvd,
                                   precise=precise, dq_atomic=dq_atomic)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _check_heads(x, got, causal, scale, kv, heads, bwd=True):
    o, lse, dq, dk, dv = got
    for (b, h) in heads:
        L = None if kv is None else int(kv[b])
        log(f"  head b={b} h={h} L={L}")
        ro, rl = oracle.head_forward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], scale, causal, L)
        compare("O", host(o[b, h]), ro)
        compare_lse(host(lse[b, h]), rl)
        if bwd:
            rq, rk, rv = oracle.head_backward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["dO"][b, h],
                                              scale, causal, L)
            compare("dQ", host(dq[b, h]), rq)
            compare("dK", host(dk[b, h]), rk)
            compare("dV", host(dv[b, h]), rv)


# Padded inputs carry one x8 outlier key per head, which makes the gradients
# large; the backward runs in precise mode for them (FA_BWD_PRECISE).
SMALL = [
    # B, H, N, d, causal, padded, precise
    (2, 3, 300, 64, False, False, False),
    (2, 3, 300, 64, True, False, False),
    (2, 3, 300, 128, False, False, False),
    (2, 3, 300, 128, True, False, False),
    (3, 2, 333, 64, False, True, True),
    (3, 2, 333, 64, True, True, True),
    (3, 2, 333, 128, True, True, True),
    (1, 2, 130, 128, False, False, False),
    (2, 2, 300, 64, True, False, True),
    (2, 2, 300, 128, False, False, True),
    # d=128 across the 256-key blocks of the key-outer kernel and the
    # 128-row query blocks: one key past two blocks, and a ragged third block
    (1, 2, 513, 128, True, False, False),
    (1, 2, 700, 128, False, False, False),
]


@pytest.mark.parametrize("dq_atomic", [False, True], ids=["split", "atomic"])
@pytest.mark.parametrize("B,H,N,d,causal,padded,precise", SMALL)
def test_small_full_compare(B, H, N, d, causal, padded, precise, dq_atomic):
    log(f"small B={B} H={H} N={N} d={d} causal={causal} padded={padded} precise={precise} "
        f"dq_atomic={dq_atomic}")
    x = wl.make_inputs(B, H, N, d, seed=100 + N + d, padded=padded)
    scale = float(np.float32(d ** -0.5))
    got = _run_bf16(x, causal, scale, x["kv_len"], precise=precise, dq_atomic=dq_atomic)
    heads = [(b, h) for b in range(B) for h in range(H)]
    _check_heads(x, got, causal, scale, x["kv_len"], heads)


@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_edge_lengths(N, d, causal):
    log(f"edge N={N} d={d} causal={causal}")
    x = wl.make_inputs(1, 2, N, d, seed=7 + N)
    scale = float(np.float32(d ** -0.5))
    got = _run_bf16(x, causal, scale, None)
    _check_heads(x, got, causal, scale, None, [(0, 0), (0, 1)])


KV_EDGES = {
    # d: (N, kv_len per batch row): 0 (all keys masked), 1, tile and block
    # boundaries (64-key tiles; 128- and 256-key blocks of the key-outer
    # kernel), N, and values outside [0, N] that the kernels clamp
    64: (200, [0, 1, 64, 200, 999, -5]),
    128: (600, [0, 1, 255, 256, 257, 600, 999, -5]),
}


@pytest.mark.parametrize("d", [64, 128])
def test_kv_len_edge_values(d):
    """Key padding at its edge values, causal and not."""
    N, kv_list = KV_EDGES[d]
    B, H = len(kv_list), 1
    kv = np.array(kv_list, np.int32)
    clamped = np.clip(kv, 0, N)
    log(f"kv_len edges d={d} N={N} {kv.tolist()}")
    x = wl.make_inputs(B, H, N, d, seed=11 + d)
    scale = 0.125 if d == 64 else float(np.float32(d ** -0.5))
    for causal in (False, True):
        o, lse, dq, dk, dv = _run_bf16(x, causal, scale, kv)
        for b in range(B):
            L = int(clamped[b])
            ro, rl = oracle.head_forward(x["Q"][b, 0], x["K"][b, 0], x["V"][b, 0], scale, causal, L)
            compare("O", host(o[b, 0]), ro)
            compare_lse(host(lse[b, 0]), rl)
            rq, rk, rv = oracle.head_backward(x["Q"][b, 0], x["K"][b, 0], x["V"][b, 0], x["dO"][b, 0],
                                              scale, causal, L)
            compare("dQ", host(dq[b, 0]), rq)
            compare("dK", host(dk[b, 0]), rk)
            compare("dV", host(dv[b, 0]), rv)
            if L == 0:
                assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))
                assert torch.all(dq[b] == 0) and torch.all(dk[b] == 0) and torch.all(dv[b] == 0)
            assert torch.all(dk[b, 0, L:] == 0) and torch.all(dv[b, 0, L:] == 0)


def test_fp32_single_head_workload():
    """The single-head fp32 workload through the fp32 entry points."""
    fa = _fa()
    w = wl.WORKLOADS["tiny_fp32"]
    x = wl.workload_inputs("tiny_fp32")
    log("tiny_fp32 workload")
    q, k, v, do = (dev_f32(x[n]) for n in ("Q", "K", "V", "dO"))
    o, lse = fa.flash_attn_fwd_f32(q, k, v, causal=False, scale=w.scale)
    dq, dk, dv = fa.flash_attn_bwd_f32(q, k, v, o, do, lse, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.head_forward(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], w.scale, False, None)
    rq, rk, rv = oracle.head_backward(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], x["dO"][0, 0], w.scale)
    for name, got, ref in (("O", o, ro), ("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, host(got[0, 0]), ref, max_abs=1e-4, mean_abs=1e-5, rel_mean=1e-4)
    compare_lse(host(lse[0, 0]), rl, tol=1e-5)


def test_fp32_entry_points_masks():
    fa = _fa()
    B, H, N, d = 2, 2, 77, 128
    x = wl.make_inputs(B, H, N, d, seed=3, dtype="fp32", padded=True)
    for causal in (False, True):
        q, k, v, do = (dev_f32(x[n]) for n in ("Q", "K", "V", "dO"))
        kvd = dev_kv(x["kv_len"])
        o, lse = fa.flash_attn_fwd_f32(q, k, v, causal=causal, kv_len=kvd)
        dq, dk, dv = fa.flash_attn_bwd_f32(q, k, v, o, do, lse, causal=causal, kv_len=kvd)
        torch.cuda.synchronize()
        s = d ** -0.5
        for b in range(B):
            for h in range(H):
                L = int(x["kv_len"][b])
                ro, rl = oracle.head_forward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], s, causal, L)
                rq, rk, rv = oracle.head_backward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["dO"][b, h],
                                                  s, causal, L)
                for name, got, ref in (("O", o, ro), ("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
                    compare(name, host(got[b, h]), ref, max_abs=1e-3, mean_abs=1e-5, rel_mean=1e-4)
                compare_lse(host(lse[b, h]), rl, tol=1e-5)


def test_forward_is_bitwise_reproducible_and_overwrites_outputs():
    """Two runs agree bit for bit (O, LSE and, by default, dQ, dK, dV);
    NaN-poisoned outputs are fully overwritten and guard bands around them
    stay untouched; the atomic-dQ variant agrees with the default."""
    fa = _fa()
    B, H, N, d = 2, 4, 500, 128
    x = wl.make_inputs(B, H, N, d, seed=5)
    q, k, v, do = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V", "dO"))
    n = B * H * N * d
    guard = 1024
    obuf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    obuf[:guard] = 7.0
    obuf[-guard:] = 7.0
    o = obuf[guard:guard + n].view(B, H, N, d)
    lbuf = torch.full((B * H * N + 2 * 64,), float("nan"), device="cuda")
    lbuf[:64] = 3.0
    lbuf[-64:] = 3.0
    lse = lbuf[64:64 + B * H * N].view(B, H, N)
    fa.flash_attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    o2, lse2 = fa.flash_attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
    assert torch.all(lbuf[:64] == 3.0) and torch.all(lbuf[-64:] == 3.0)
    assert not torch.any(torch.isnan(o)) and not torch.any(torch.isnan(lse))
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)
    g1 = fa.flash_attn_bwd(q, k, v, o, do, lse, causal=True,
                           dq=torch.full((B, H, N, d), float("nan"), device="cuda"),
                           dk=torch.full((B, H, N, d), float("nan"), device="cuda"),
                           dv=torch.full((B, H, N, d), float("nan"), device="cuda"))
    g2 = fa.flash_attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for t in g1:
        assert not torch.any(torch.isnan(t))
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])
    g3 = fa.flash_attn_bwd(q, k, v, o, do, lse, causal=True, dq_atomic=True)
    torch.cuda.synchronize()
    # dK and dV come from the same key-outer arithmetic in both modes. dQ does
    # not: each mode rounds dS to bf16 in a different kernel, from fp32 values
    # formed in a different order, so single roundings may differ by one bf16
    # ulp (2^-7 relative), moving dQ by up to 2^-7 |dS| |K| scale per flip.
    # Both modes are checked against the oracle element by element elsewhere.
    assert torch.allclose(g3[1], g2[1], atol=1e-4, rtol=0) and torch.allclose(g3[2], g2[2], atol=1e-4, rtol=0)
    assert float((g3[0] - g2[0]).abs().max()) <= 1e-3 * max(1.0, float(g2[0].abs().max()))


def subset_heads(B, H, seed, n_random=4):
    """The deterministic head subset checked at full size: first and last b,
    h in {0, H-1}, plus n_random seeded (b, h) pairs."""
    heads = {(b, h) for b in (0, B - 1) for h in (0, H - 1)}
    rng = np.random.default_rng(seed)
    while len(heads) < min(B * H, 4 + n_random):
        heads.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(heads)


# name, causal, precise, number of seeded heads beyond the corners (the
# N=16384 heads take the oracle about 10 GB and ten seconds each: fewer)
FULL = [
    ("gpt2_medium", True, False, 4),
    ("n4096_d128", False, False, 4),
    ("n4096_d128", True, False, 4),
    ("long_16k", True, False, 0),
    ("padded_8k", False, True, 4),
]


def check_invariants(x, got, scale):
    """Whole-tensor identities of the gradients, over every head, against
    bounds from the rounding the kernels do.

    sum_j dV_j = sum_i dO_i because every row of P sums to 1: the kernels
    feed bf16(P) to the dV product, each P_ij rounded by at most 2^-9 of
    itself, so per row sum_j bf16(P_ij) is within 2^-9 of 1 and per column c
    the residual is at most 2^-9 sum_i |dO_ic| (asserted with a factor 2).

    sum_j dK_j = 0 because every row of dS sums to 0 when D_i is exact. The
    kernels take D_i from the bf16 output (each element within 2^-9 of the
    fp32 one: |D error| <= 2^-9 ||dO_i|| ||O_i||) and round dS to bf16
    (sum_j |bf16(dS_ij) - dS_ij| <= 2^-9 sum_j |dS_ij| <= 2^-9 (||dO_i||
    max_j ||v_j|| + |D_i|), since |dP_ij| <= ||dO_i|| ||v_j||), so per column
    |sum_j dK_jc| <= scale sum_i |q_ic| 2^-9 (||dO_i|| ||O_i|| + ||dO_i|| max_j
    ||v_j|| + |D_i|) (asserted with a factor 2)."""
    o, lse, dq, dk, dv = got
    f64 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().double()
    q, v, do = f64(x["Q"]), f64(x["V"]), f64(x["dO"])
    u = 2.0 ** -9
    res_v = (dv.double().sum(dim=2) - do.sum(dim=2)).abs()
    bound_v = 2 * u * do.abs().sum(dim=2)
    od = o.double()
    dnorm = do.norm(dim=3)
    d_i = (do * od).sum(dim=3)
    vmax = v.norm(dim=3).max(dim=2, keepdim=True).values
    per_row = dnorm * od.norm(dim=3) + dnorm * vmax + d_i.abs()
    res_k = dk.double().sum(dim=2).abs()
    bound_k = 2 * u * scale * (q.abs() * per_row.unsqueeze(-1)).sum(dim=2)
    rv, rk = float((res_v / bound_v).max()), float((res_k / bound_k).max())
    log(f"  invariants: |sum dV - sum dO| max {float(res_v.max()):.3e} ({rv:.3f} of its bound), "
        f"|sum dK| max {float(res_k.max()):.3e} ({rk:.3f} of its bound)")
    assert rv <= 1.0, f"sum_j dV_j - sum_i dO_i exceeds its rounding bound ({rv:.3f})"
    assert rk <= 1.0, f"sum_j dK_j exceeds its rounding bound ({rk:.3f})"


@pytest.mark.parametrize("name,causal,precise,n_random", FULL,
                         ids=[f"{n}-{'causal' if c else 'full'}" for n, c, _, _ in FULL])
def test_full_size_workload(name, causal, precise, n_random):
    w = wl.WORKLOADS[name]
    log(f"full {name} causal={causal} precise={precise} B={w.B} H={w.H} N={w.N} d={w.d}")
    x = wl.workload_inputs(name)
    got = _run_bf16(x, causal, w.scale, x["kv_len"], precise=precise)
    for t in got:
        assert torch.isfinite(t).all()
    check_invariants(x, got, w.scale)
    _check_heads(x, got, causal, w.scale, x["kv_len"], subset_heads(w.B, w.H, w.seed, n_random))


def test_padded_default_mode_error_recorded():
    """The padded workload's backward in the default mode, whose error on
    its x8 outlier keys is above the absolute bar (about 0.15 on dQ and dK
    and 0.1 on dV, from D taken from the bf16 output and from bf16 P and dS;
    precise mode removes all three). Recorded so that a regression shows:
    the forward is held to the usual bar, the gradients to err / max(1,
    max |ref|) <= 2e-2 and max-abs <= 0.25."""
    name = "padded_8k"
    w = wl.WORKLOADS[name]
    x = wl.workload_inputs(name)
    got = _run_bf16(x, False, w.scale, x["kv_len"], precise=False)
    o, lse, dq, dk, dv = got
    for (b, h) in subset_heads(w.B, w.H, w.seed, 4):
        L = int(x["kv_len"][b])
        log(f"  default-mode head b={b} h={h} L={L}")
        ro, rl = oracle.head_forward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], w.scale, False, L)
        compare("O", host(o[b, h]), ro)
        compare_lse(host(lse[b, h]), rl)
        rq, rk, rv = oracle.head_backward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["dO"][b, h], w.scale,
                                          False, L)
        for nm, t, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            err = np.abs(host(t[b, h]) - r)
            mx, mn, top = float(err.max()), float(err.mean()), float(np.abs(r).max())
            norm = mx / max(1.0, top)
            log(f"    {nm:4s} max_abs={mx:.3e} mean_abs={mn:.3e} max|ref|={top:.3g} err/max(1,max|ref|)={norm:.3e}")
            assert norm <= 2e-2, f"{nm}: normalised error {norm:.3e}"
            assert mx <= 0.25, f"{nm}: max abs err {mx:.3e}"
