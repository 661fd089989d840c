"""GPU parity of the decoding forward against the fp64 oracle.

Every case calls flash_attn_decode_fwd through the C ABI (via the binding)
on seeded inputs and compares O and LSE element by element with the
oracle's decode_head_forward; the full-size cache is compared on sampled
heads. Tolerances as for the other bf16 paths.
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


def _run(B, H, Nq, Nk, d, causal, kv_len=None, seed=11, ragged=False):
    from tests.gpu_util import compare, compare_lse, dev_bf16, dev_kv, host, log
    import oracle
    fa = _fa()
    x = wl.make_decode_inputs(B, H, Nq, Nk, d, seed, ragged)
    L = x["kv_len"] if kv_len is None else np.asarray(kv_len, np.int32)
    log(f"  decode B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} kv_len={None if L is None else list(L)}")
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_decode_fwd(q, k, v, causal=causal, scale=scale, kv_len=dev_kv(L))
    torch.cuda.synchronize()
    Ro, Rl = oracle.decode_forward(x["Q"], x["K"], x["V"], scale, L, causal)
    compare("O", host(O), Ro)
    compare_lse(host(lse), Rl)
    return O, lse


SMALL = [
    (2, 3, 1, 1, 64, False), (2, 3, 1, 7, 128, False), (1, 2, 1, 512, 128, False),
    (2, 2, 1, 513, 64, False), (1, 3, 3, 1300, 128, True), (2, 2, 4, 1024, 64, True),
    (1, 2, 5, 777, 128, False), (2, 1, 8, 2048, 128, True), (1, 2, 8, 300, 64, False),
    (1, 1, 2, 2, 128, True),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", SMALL,
                         ids=[f"B{b}H{h}q{nq}k{nk}d{d}{'c' if c else ''}" for b, h, nq, nk, d, c in SMALL])
def test_decode_small(B, H, Nq, Nk, d, causal):
    _run(B, H, Nq, Nk, d, causal)


@pytest.mark.parametrize("d,causal", [(64, False), (128, True), (128, False)])
def test_decode_ragged_cache(d, causal):
    _run(4, 3, 3, 1500, d, causal, ragged=True, seed=12)


def test_decode_cache_edges():
    """kv_len of 0 (no key: O = 0, LSE = -inf), 1, a chunk boundary, and out of range values."""
    O, lse = _run(5, 2, 2, 1100, 128, False, kv_len=[0, 1, 512, 1100, 5000])
    assert torch.all(O[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_decode_causal_shorter_than_queries():
    """Causal with a cache shorter than the query block: early queries see no key."""
    O, lse = _run(1, 2, 4, 64, 64, True, kv_len=[2])
    assert torch.all(torch.isneginf(lse[0, :, :2]))


def test_decode_reproducible():
    fa = _fa()
    x = wl.make_decode_inputs(2, 4, 3, 2000, 128, 13)
    q, k, v = (torch.from_numpy(x[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda() for n in ("Q", "K", "V"))
    a = fa.flash_attn_decode_fwd(q, k, v, causal=True)
    b = fa.flash_attn_decode_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_decode_full_size_sampled_heads():
    """The 32K-slot cache workload at full size; a few heads against the oracle."""
    from tests.gpu_util import compare, compare_lse, dev_bf16, host, log
    import oracle
    fa = _fa()
    cfg = wl.DECODE_WORKLOADS["decode_32k"]
    B, H, Nq, Nk, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"]
    x = wl.make_decode_inputs(B, H, Nq, Nk, d, cfg["seed"], cfg["ragged"])
    log(f"  decode_32k B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    q, k, v = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V"))
    scale = float(np.float32(d ** -0.5))
    O, lse = fa.flash_attn_decode_fwd(q, k, v, causal=cfg["causal"], scale=scale)
    torch.cuda.synchronize()
    O, lse = host(O), host(lse)
    for b, h in [(0, 0), (B - 1, H - 1), (3, 17)]:
        Ro, Rl = oracle.decode_head_forward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], scale, None, cfg["causal"])
        compare("O", O[b, h], Ro)
        compare_lse(lse[b, h], Rl)
