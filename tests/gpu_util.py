"""Helpers for the GPU parity tests: moving seeded inputs to the device,
calling the library through its binding, and comparing with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances for bf16 inputs with fp32 accumulation, against the fp64 oracle:
# per tensor over all compared elements, max |err| and mean |err|; LSE max |err|.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 1e-3
# Guard: mean |err| relative to mean |ref|, since some workloads' outputs are small.
REL_MEAN = 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_kv(kv):
    return None if kv is None else torch.from_numpy(np.asarray(kv, np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name, got, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, rel_mean=REL_MEAN):
    """Element-wise comparison; returns the error summary and asserts the bar."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx, mn = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    scale = float(np.abs(ref).mean()) if err.size else 0.0
    rel = mn / scale if scale > 0 else 0.0
    log(f"    {name:4s} max_abs={mx:.3e} mean_abs={mn:.3e} rel_mean={rel:.3e} max|ref|={np.abs(ref).max(initial=0):.3g}")
    assert mx <= max_abs, f"{name}: max abs err {mx:.3e} > {max_abs}"
    assert mn <= mean_abs, f"{name}: mean abs err {mn:.3e} > {mean_abs}"
    assert rel <= rel_mean, f"{name}: relative mean err {rel:.3e} > {rel_mean}"
    return mx, mn


def compare_lse(got, ref, tol=LSE_ABS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ninf_g, ninf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), "LSE: -inf pattern differs"
    fin = ~ninf_r
    err = np.abs(got[fin] - ref[fin])
    mx = float(err.max(initial=0.0))
    log(f"    LSE  max_abs={mx:.3e}")
    assert np.all(np.isfinite(got[fin])), "LSE: non-finite values"
    assert mx <= tol, f"LSE: max abs err {mx:.3e} > {tol}"
    return mx
