"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from io_aware_exact_11_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    """Host RNE rounding agrees with torch's float32 -> bfloat16 conversion."""
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38], np.float32)])
    x = x.astype(np.float32)
    ours = wl.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_rounded():
    a = wl.make_inputs(2, 3, 40, 64, seed=7)
    b = wl.make_inputs(2, 3, 40, 64, seed=7)
    for n in ("Q", "K", "V", "dO"):
        assert np.array_equal(a[n], b[n])
        assert np.array_equal(wl.bf16_bits_to_f32(a[n + "_bits"]), a[n])
        assert np.array_equal(wl.bf16_bits_to_f32(wl.bf16_round_bits(a[n])), a[n])
    c = wl.make_inputs(2, 3, 40, 64, seed=8)
    assert not np.array_equal(a["Q"], c["Q"])


def test_padded_recipe():
    """kv_len in [N/2, N]; exactly one x8 outlier key per head among the valid keys."""
    B, H, N, d = 6, 4, 64, 64
    x = wl.make_inputs(B, H, N, d, seed=5, padded=True)
    plain = np.random.Generator(np.random.PCG64(5))
    base_k = None
    for n in ("Q", "K", "V", "dO"):
        arr = plain.standard_normal(size=(B, H, N, d), dtype=np.float32)
        if n == "K":
            base_k = arr
    kv = x["kv_len"]
    assert kv.dtype == np.int32 and kv.shape == (B,)
    assert np.all(kv >= N // 2) and np.all(kv <= N)
    kb = wl.bf16_bits_to_f32(wl.bf16_round_bits(base_k))
    for b in range(B):
        for h in range(H):
            changed = np.nonzero(np.any(x["K"][b, h] != kb[b, h], axis=1))[0]
            assert changed.size == 1 and changed[0] < kv[b]
            j = changed[0]
            assert np.array_equal(x["K"][b, h, j], wl.bf16_bits_to_f32(wl.bf16_round_bits(base_k[b, h, j] * 8)))


def test_named_workloads():
    assert wl.WORKLOADS["n4096_d128"].qkv_scale == 0.5
    assert wl.WORKLOADS["n4096_d128"].scale == np.float32(1 / np.sqrt(128))
    x = wl.workload_inputs("tiny_fp32")
    assert x["Q"].dtype == np.float32 and x["Q"].shape == (1, 1, 128, 64) and "Q_bits" not in x
    y = wl.workload_inputs("n4096_d128", B=1, H=1, N=64)
    assert y["Q"].shape == (1, 1, 64, 128)
    assert np.max(np.abs(y["Q"])) < 4.0
