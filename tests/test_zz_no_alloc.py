"""flash_attn_bwd_noalloc (the backward with the library's fixed scratch in
place of a workspace) against flash_attn_bwd on the same inputs, on two
calls in a row, the second one smaller. Both run the same kernels on the
same inputs, and the default and precise backward are deterministic, so the
gradients must be bitwise equal; both are also held to the oracle's
tolerance on one head."""
import numpy as np
import pytest
import torch

import io_aware_exact_11_amd as fa
import oracle
from io_aware_exact_11_amd import workloads as wl

from gpu_util import compare, dev_bf16, dev_kv, host, log

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, N, d, causal, kv_len, precise
    (2, 4, 1000, 128, True, None, False),
    (1, 3, 300, 64, False, [217], True),
]


def _run(B, H, N, d, causal, kv, precise, seed):
    x = wl.make_inputs(B, H, N, d, seed=seed)
    q, k, v, do = (dev_bf16(x[n + "_bits"]) for n in ("Q", "K", "V", "dO"))
    kvd = dev_kv(kv)
    scale = float(np.float32(d ** -0.5))
    o, lse = fa.flash_attn_fwd(q, k, v, causal=causal, scale=scale, kv_len=kvd)
    ref = fa.flash_attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, kv_len=kvd, precise=precise)
    # Outputs preallocated and poisoned, so the call allocates nothing and must overwrite them.
    got = tuple(torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device) for _ in range(3))
    fa.flash_attn_bwd_noalloc(q, k, v, o, do, lse, causal=causal, scale=scale, kv_len=kvd, precise=precise,
                              dq=got[0], dk=got[1], dv=got[2])
    torch.cuda.synchronize()
    return x, scale, ref, got


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    for i, (B, H, N, d, causal, kv, precise) in enumerate(CASES):
        log(f"  noalloc call {i}: B={B} H={H} N={N} d={d} causal={causal} kv_len={kv} precise={precise}")
        x, scale, ref, got = _run(B, H, N, d, causal, kv, precise, seed=100 + i)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), f"call {i}: {name} differs from flash_attn_bwd"
        kvh = None if kv is None else kv[0]
        h = H - 1
        rq, rk, rv = oracle.head_backward(x["Q"][0, h], x["K"][0, h], x["V"][0, h], x["dO"][0, h], scale, causal,
                                          kv_len=kvh)
        for name, t, r in (("dQ", got[0], rq), ("dK", got[1], rk), ("dV", got[2], rv)):
            compare(name, host(t[0, h]), r)


def test_noalloc_rejects_rows_beyond_scratch():
    # B*H*N one row past the fixed scratch: refused on the host, nothing launched.
    N = fa.binding.NOALLOC_MAX_ROWS + 1
    q = torch.empty((1, 1, N, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FlashAttnError) as ei:
        fa.flash_attn_bwd_noalloc(q, q.clone(), q.clone(), q.clone(), q.clone(), lse)
    assert ei.value.status == fa.binding.FA_ERR_SCRATCH_LIMIT
