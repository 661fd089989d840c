"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage type.
It holds none of the attention arithmetic, so both the fp64 oracle (through
the tests) and the HIP path can be fed from it without sharing any part of
the method.

Recipe (one numpy PCG64 stream per workload, seeded with the workload's
seed):
  1. draw float32 standard normals in C order for Q, K, V, dO, each
     [B, H, N, d], in that order;
  2. multiply Q, K, V by ``qkv_scale`` (0.5 for the N=4096, d=128 workload);
  3. padded workloads then draw one valid length per batch row,
     kv_len[b] ~ U{N/2 .. N} (both ends included), and one outlier key per
     (b, h), uniform over the valid keys, whose K row is multiplied by 8;
  4. bf16 workloads round every tensor to bfloat16 with round-to-nearest-even.

Decoding inputs (``make_decode_inputs``) follow the same recipe with Q of
shape [B, H, Nq, d] and K, V of shape [B, H, Nk, d] (no dO), then, when
ragged, one cache length per batch row kv_len[b] ~ U{Nk/2 .. Nk}.

8-bit inputs (``make_fp8_inputs``) draw Q, K, V the same way and quantise
each tensor to FP8 E4M3 with torch's float8_e4m3fn conversion after
dividing it by its largest magnitude / 448; V is returned transposed.
Block-sparse masks (``block_sparse_pattern``) are a band of blocks around
the diagonal plus the first key block.

The shapes follow the pages' workloads: the GPT-2-medium attention shape
(FlashAttention does more arithmetic to move less data, section
"FlashAttention never writes the full score table to HBM"), the N=4096,
d=128 head of FlashAttention and GPU Memory chapter 04, and long and padded
batches for the linear-memory and masking claims.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "fp32": storage type of Q, K, V, dO
    causal: tuple         # causal variants this workload is run in
    padded: bool          # per-batch key-padding lengths + one outlier key
    qkv_scale: float
    seed: int
    note: str = ""

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the fp32 value both sides receive."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 128, 64, "fp32", (False,), False, 1.0, 1,
                          "single head, fp32, non-causal"),
    "gpt2_medium": Workload("gpt2_medium", 64, 16, 1024, 64, "bf16", (True,), False, 1.0, 2,
                            "GPT-2-medium-shaped attention, causal"),
    "n4096_d128": Workload("n4096_d128", 16, 16, 4096, 128, "bf16", (False, True), False, 0.5, 3,
                           "N=4096, d=128, causal and non-causal, Q/K/V scaled by 0.5"),
    "long_16k": Workload("long_16k", 2, 16, 16384, 128, "bf16", (True,), False, 1.0, 4,
                         "long context, causal"),
    "padded_8k": Workload("padded_8k", 8, 32, 8192, 64, "bf16", (False,), True, 1.0, 5,
                          "key padding with kv_len ~ U[N/2, N] and one x8 outlier key per head"),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly equal float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16",
                qkv_scale: float = 1.0, padded: bool = False) -> dict:
    """Draw Q, K, V, dO (and kv_len when padded) following the module recipe.

    Returns a dict with float32 arrays "Q", "K", "V", "dO" holding exactly the
    values the kernels see (already rounded when dtype is bf16), the uint16 bit
    patterns under "Q_bits" etc. for bf16, and "kv_len" (int32 [B]) or None.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    out = {}
    for name in ("Q", "K", "V", "dO"):
        out[name] = rng.standard_normal(size=shape, dtype=np.float32)
    if qkv_scale != 1.0:
        for name in ("Q", "K", "V"):
            out[name] *= np.float32(qkv_scale)
    kv_len = None
    if padded:
        kv_len = rng.integers(N // 2, N, endpoint=True, size=B).astype(np.int32)
        for b in range(B):
            idx = rng.integers(0, kv_len[b], size=H)
            for h in range(H):
                out["K"][b, h, idx[h], :] *= np.float32(8.0)
    out["kv_len"] = kv_len
    if dtype == "bf16":
        for name in ("Q", "K", "V", "dO"):
            bits = bf16_round_bits(out[name])
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


# Decoding workload: one new query per head against a long key/value cache
# (the token-by-token decoding of "FlashAttention — why it mattered"), with
# the GPT-style width of 32 heads of 128 and a 32K-slot cache per sequence.
DECODE_WORKLOADS = {
    "decode_32k": dict(B=8, H=32, Nq=1, Nk=32768, d=128, causal=False, ragged=False, seed=6),
}


# 8-bit forward workload: the N=4096, d=128 shape with Q, K, V quantised to
# FP8 E4M3, one scale per tensor (largest magnitude mapped to 448).
FP8_WORKLOADS = {
    "n4096_d128_fp8": dict(B=16, H=16, N=4096, d=128, causal=False, qkv_scale=0.5, seed=8),
}


def make_fp8_inputs(B: int, H: int, N: int, d: int, seed: int, qkv_scale: float = 1.0,
                    outlier_cols: int = 0) -> dict:
    """Q, K, V [B, H, N, d] drawn like make_inputs (fp32, times qkv_scale; with outlier_cols > 0 that many
    feature columns of Q and K are multiplied by 8), then quantised to FP8 E4M3 per tensor with torch's
    float8_e4m3fn conversion after dividing by amax / 448. Returns the codes "Q8", "K8" [B, H, N, d] and
    "Vt8" [B, H, d, N] (V transposed), the fp32 dequantisation factors "dq", "dk", "dv", and the unquantised
    float32 tensors "Q", "K", "V"."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("Q", "K", "V"):
        out[name] = rng.standard_normal(size=(B, H, N, d), dtype=np.float32) * np.float32(qkv_scale)
    if outlier_cols:
        cols = rng.choice(d, size=outlier_cols, replace=False)
        out["Q"][..., cols] *= np.float32(8.0)
        out["K"][..., cols] *= np.float32(8.0)
    for name, key in (("Q", "dq"), ("K", "dk"), ("V", "dv")):
        f = np.float32(np.abs(out[name]).max() / 448.0)
        codes = torch.from_numpy(out[name] / f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out[key] = float(f)
        out[name + "8"] = codes
    out["Vt8"] = np.ascontiguousarray(out.pop("V8").transpose(0, 1, 3, 2))
    return out


# Block-sparse workload: the 64K sequence length the pages' block-sparse
# variant was used for (Path-256), with a synthetic pattern: every query block
# of 128 rows sees its own key block, the two on each side, and key block 0
# (a band plus one global column), about 1.2% of the blocks at N = 65536.
BLOCK_SPARSE_WORKLOADS = {
    "sparse_64k": dict(B=1, H=16, N=65536, d=128, band=2, causal=False, seed=7),
}


def block_sparse_pattern(N: int, band: int, block: int = 128) -> np.ndarray:
    """uint8 [nb, nb] block mask: |qb - kb| <= band, plus key block 0."""
    nb = (N + block - 1) // block
    qb, kb = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    return ((np.abs(qb - kb) <= band) | (kb == 0)).astype(np.uint8)


def make_decode_inputs(B: int, H: int, Nq: int, Nk: int, d: int, seed: int, ragged: bool = False) -> dict:
    """Q [B,H,Nq,d], K and V [B,H,Nk,d] (bf16 values as float32 plus "_bits"),
    and "kv_len" (int32 [B], ragged) or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"Q": rng.standard_normal(size=(B, H, Nq, d), dtype=np.float32)}
    for name in ("K", "V"):
        out[name] = rng.standard_normal(size=(B, H, Nk, d), dtype=np.float32)
    out["kv_len"] = (rng.integers(Nk // 2, Nk, endpoint=True, size=B).astype(np.int32)
                     if ragged else None)
    for name in ("Q", "K", "V"):
        bits = bf16_round_bits(out[name])
        out[name + "_bits"] = bits
        out[name] = bf16_bits_to_f32(bits)
    return out


def workload_inputs(name: str, **overrides) -> dict:
    """Inputs of a named workload; keyword overrides replace B, H, N or d."""
    w = WORKLOADS[name]
    dims = {k: overrides.get(k, getattr(w, k)) for k in ("B", "H", "N", "d")}
    return make_inputs(dims["B"], dims["H"], dims["N"], dims["d"], w.seed, w.dtype,
                       w.qkv_scale, w.padded)
