"""GPU parity of the block-sparse forward against the fp64 oracle.

flash_attn_fwd_block_sparse is called through the C ABI on seeded inputs
with random and structured 128 x 128 block masks (shared by every head or
one per head; causal, key padding and ragged N included) and compared
element by element with oracle.block_sparse; the 64K-long workload the
benchmark times is compared on sampled rows. An all-on mask reproduces the
dense forward, an all-off mask gives O = 0 and LSE = -inf.
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


CASES = [  # B, H, N, d, causal, padded, per_head, density
    (1, 2, 256, 64, False, False, False, 0.5), (2, 2, 300, 128, False, False, True, 0.6),
    (2, 2, 512, 64, True, False, True, 0.5), (2, 3, 700, 128, True, False, False, 0.4),
    (2, 2, 640, 64, False, True, True, 0.5), (1, 2, 1000, 128, False, True, True, 0.3),
    (1, 1, 129, 128, True, False, False, 1.0), (1, 2, 2048, 128, True, False, True, 0.25),
]


@pytest.mark.parametrize("B,H,N,d,causal,padded,per_head,density", CASES)
def test_block_sparse_parity(B, H, N, d, causal, padded, per_head, density):
    from oracle import block_sparse as bs
    from tests.gpu_util import compare, compare_lse, dev_bf16, dev_kv, host, log
    fa = _fa()
    log(f"  sparse B={B} H={H} N={N} d={d} causal={causal} padded={padded} per_head={per_head} density={density}")
    x = wl.make_inputs(B, H, N, d, seed=70 + N + d, padded=padded)
    nb = (N + 127) // 128
    rng = np.random.default_rng(N + d)
    shape = (B, H, nb, nb) if per_head else (nb, nb)
    bm = (rng.random(shape) < density).astype(np.uint8)
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_fwd_block_sparse(q, k, v, torch.from_numpy(bm).cuda(), causal=causal, scale=scale,
                                            kv_len=dev_kv(x["kv_len"]))
    torch.cuda.synchronize()
    Ro, Rl = bs.forward_block_sparse(x["Q"], x["K"], x["V"], scale, bm, causal, x["kv_len"])
    compare("O", host(O), Ro)
    compare_lse(host(lse), Rl)


@pytest.mark.parametrize("d", [64, 128])
def test_all_off_and_all_on(d):
    from tests.gpu_util import dev_bf16
    fa = _fa()
    x = wl.make_inputs(2, 2, 384, d, seed=9)
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    off = torch.zeros(3, 3, dtype=torch.uint8, device="cuda")
    O, lse = fa.flash_attn_fwd_block_sparse(q, k, v, off)
    assert torch.all(O == 0) and torch.all(torch.isneginf(lse))
    on = torch.ones(3, 3, dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        O1, L1 = fa.flash_attn_fwd_block_sparse(q, k, v, on, causal=causal)
        O0, L0 = fa.flash_attn_fwd(q, k, v, causal=causal)
        if d == 128 or causal:  # same kernel configuration as the dense forward: identical results
            assert torch.equal(O1, O0) and torch.equal(L1, L0)
        else:
            assert float((O1.float() - O0.float()).abs().max()) < 1e-2
            assert float((L1 - L0).abs().max()) < 1e-5


def test_full_size_sparse_64k_workload():
    """The benchmark's 64K workload (B=1 H=16 N=65536 d=128, band of two blocks plus block 0) on sampled rows."""
    from oracle import block_sparse as bs
    from tests.gpu_util import compare, compare_lse, dev_bf16, host, log
    fa = _fa()
    w = wl.BLOCK_SPARSE_WORKLOADS["sparse_64k"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    log(f"  sparse_64k B={B} H={H} N={N} d={d} band={w['band']}")
    x = wl.make_inputs(B, H, N, d, seed=w["seed"])
    bm = wl.block_sparse_pattern(N, w["band"])
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_fwd_block_sparse(q, k, v, torch.from_numpy(bm).cuda(), causal=w["causal"], scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 300, 4095, 33000, 65407, 65408, 65535])
    for h in (0, 7, 15):
        ro, rl = bs.forward_rows_block_sparse(x["Q"][0, h], x["K"][0, h], x["V"][0, h], rows, scale, bm, w["causal"])
        compare("O", host(O[0, h][torch.from_numpy(rows).cuda()]), ro)
        compare_lse(host(lse[0, h][torch.from_numpy(rows).cuda()]), rl)


@pytest.mark.parametrize("N,d,causal", [(1, 64, False), (1, 128, True), (127, 128, False), (129, 64, True)])
def test_block_sparse_edge_lengths(N, d, causal):
    from oracle import block_sparse as bs
    from tests.gpu_util import compare, compare_lse, dev_bf16, host, log
    fa = _fa()
    log(f"  sparse edge N={N} d={d} causal={causal}")
    x = wl.make_inputs(1, 2, N, d, seed=21 + N)
    nb = (N + 127) // 128
    bm = np.ones((nb, nb), np.uint8)
    if nb > 1:
        bm[1, 0] = 0
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_fwd_block_sparse(q, k, v, torch.from_numpy(bm).cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    Ro, Rl = bs.forward_block_sparse(x["Q"], x["K"], x["V"], scale, bm, causal)
    compare("O", host(O), Ro)
    compare_lse(host(lse), Rl)


def test_block_sparse_kv_len_zero_row():
    from tests.gpu_util import dev_bf16
    fa = _fa()
    x = wl.make_inputs(2, 1, 256, 128, seed=22)
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    kv = torch.tensor([0, 200], dtype=torch.int32, device="cuda")
    O, lse = fa.flash_attn_fwd_block_sparse(q, k, v, torch.ones(2, 2, dtype=torch.uint8, device="cuda"), kv_len=kv)
    torch.cuda.synchronize()
    assert torch.all(O[0] == 0) and torch.all(torch.isneginf(lse[0])) and torch.all(torch.isfinite(lse[1]))
