"""Benchmark: one step = exact-attention forward + backward over one batch.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line. The step runs the library's whole path on inputs that
are already resident in device memory: flash_attn_fwd (O, LSE) then
flash_attn_bwd (query-outer dQ kernel, which also forms the row term D_i,
then key-outer dK/dV kernel). FLOPs are
counted over visible (query, key) pairs only: 4 d per pair forward (the two
products S = Q K^T and O = P V at 2 flops per multiply-add) and 10 d per
pair backward (recomputed S, dP, dV, dK, dQ), 14 d per pair for a step.

The primary workload is the GPT-2-medium attention shape (B=64, H=16,
N=1024, d=64, causal); the N=4096 and N=16384 head-dim-128 workloads are
timed the same way and reported under "workloads", next to the decoding
forward (one new query per head against a 32K-slot cache), which is
memory-bound and reported as an HBM rate, and the N=4096, d=128 workload
again with fused dropout at p = 0.1 (same FLOP count; the generator work is
not counted), the block-sparse forward on a 64K-long sequence (FLOPs
over the visible pairs of its block mask), and the 8-bit (E4M3) forward on
the N=4096, d=128 shape. Only one GPU is used.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 matrix-core peak (2.5 PFLOP/s class)
PEAK_HBM_TBPS = 8.0        # MI355X HBM3E peak
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 matrix-core peak
PRIMARY = "gpt2_medium"
DROPOUT_SEED = 0x5EED  # generator key of the dropout workload
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def pairs_per_batch(w, causal, kv_len):
    """Visible (query, key) pairs summed over all heads."""
    N = w.N
    if kv_len is not None:
        tot = 0
        for L in kv_len:
            L = max(0, min(int(L), N))
            tot += (sum(min(i + 1, L) for i in range(N)) if causal else N * L)
        return tot * w.H
    per_head = N * (N + 1) // 2 if causal else N * N
    return per_head * w.B * w.H


def kernel_source_digest():
    """Digest of the device sources (.h, .hip) with comments and blank lines
    removed, so that stored counter results stay valid across comment-only
    edits and changes to the host-side entry points."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "io_aware_exact_11_amd", "csrc")
    for name in sorted(n for n in os.listdir(csrc) if n.endswith((".h", ".hip"))):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
        code = "\n".join(ln for ln in lines if ln)
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


class Case:
    """Device-resident inputs and outputs of one workload."""

    def __init__(self, name, causal, precise=False, dropout=None):
        import torch
        from io_aware_exact_11_amd import workloads as wl
        import io_aware_exact_11_amd as fa
        self.fa = fa
        self.w = wl.WORKLOADS[name]
        self.name, self.causal, self.precise, self.dropout = name, causal, precise, dropout
        x = wl.workload_inputs(name)
        dev = lambda bits: torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
        self.q, self.k, self.v, self.do = (dev(x[n + "_bits"]) for n in ("Q", "K", "V", "dO"))
        self.kv_host = x["kv_len"]
        self.kv = None if x["kv_len"] is None else torch.from_numpy(x["kv_len"]).cuda()
        del x
        w = self.w
        f32 = dict(dtype=torch.float32, device="cuda")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), **f32)
        self.dq = torch.empty((w.B, w.H, w.N, w.d), **f32)
        self.dk = torch.empty_like(self.dq)
        self.dv = torch.empty_like(self.dq)
        self.ws = torch.empty(fa.flash_attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d),
                              dtype=torch.uint8, device="cuda")
        self.pairs = pairs_per_batch(w, causal, self.kv_host)

    def fwd(self):
        if self.dropout is not None:
            self.fa.flash_attn_fwd_dropout(self.q, self.k, self.v, self.dropout, DROPOUT_SEED, 0, causal=self.causal,
                                           scale=self.w.scale, kv_len=self.kv, out=self.o, lse=self.lse)
            return
        self.fa.flash_attn_fwd(self.q, self.k, self.v, causal=self.causal, scale=self.w.scale,
                               kv_len=self.kv, out=self.o, lse=self.lse)

    def bwd(self):
        if self.dropout is not None:
            self.fa.flash_attn_bwd_dropout(self.q, self.k, self.v, self.o, self.do, self.lse, self.dropout,
                                           DROPOUT_SEED, 0, causal=self.causal, scale=self.w.scale, kv_len=self.kv,
                                           precise=self.precise, dq=self.dq, dk=self.dk, dv=self.dv,
                                           workspace=self.ws)
            return
        self.fa.flash_attn_bwd(self.q, self.k, self.v, self.o, self.do, self.lse, causal=self.causal,
                               scale=self.w.scale, kv_len=self.kv, precise=self.precise,
                               dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws)

    def run(self, steps, warmup):
        """Time `steps` whole steps; per-kernel-call times from events on the stream."""
        import torch
        for _ in range(warmup):
            self.fwd()
            self.bwd()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for e in ev:
            e[0].record()
            self.fwd()
            e[1].record()
            self.bwd()
            e[2].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
        return wall * 1e3, fwd_ms, bwd_ms

    def flops(self):
        d = self.w.d
        mult_bwd = 14 if self.precise else 10  # precise: exact-D pass (2) and hi/lo products (2)
        return 4 * d * self.pairs, mult_bwd * d * self.pairs


def cpu_baseline(name, causal, budget_s=10.0):
    """The fp64 oracle timed on this host's cores on a bounded sample of heads
    of the same workload (its first heads in (b, h) order, until about
    budget_s of work), reported in the same algorithmic TFLOP/s (14 d per pair)."""
    import oracle
    from io_aware_exact_11_amd import workloads as wl
    w = wl.WORKLOADS[name]
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info())
    except Exception:
        threads = os.cpu_count()
    x = wl.workload_inputs(name)
    heads, t0 = 0, time.perf_counter()
    while heads < w.B * w.H and (time.perf_counter() - t0) < budget_s:
        b, h = divmod(heads, w.H)
        oracle.head_forward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], w.scale, causal)
        oracle.head_backward(x["Q"][b, h], x["K"][b, h], x["V"][b, h], x["dO"][b, h], w.scale, causal)
        heads += 1
    dt = time.perf_counter() - t0
    per_head_pairs = w.N * (w.N + 1) // 2 if causal else w.N * w.N
    tflops = 14 * w.d * per_head_pairs * heads / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {heads} of {w.B * w.H} heads of {name} in (b, h) order, fwd+bwd "
                      f"in float64 with numpy, {dt:.1f} s wall",
            "seconds": round(dt, 2)}


def decode_case(steps, warmup):
    """The decoding forward on the 32K-slot cache workload: time per call
    from events on the stream, and the HBM rate of its algorithmic bytes
    (K and V read once, Q read, O and LSE written)."""
    import torch
    import io_aware_exact_11_amd as fa
    from io_aware_exact_11_amd import workloads as wl
    name = "decode_32k"
    c = wl.DECODE_WORKLOADS[name]
    B, H, Nq, Nk, d = c["B"], c["H"], c["Nq"], c["Nk"], c["d"]
    x = wl.make_decode_inputs(B, H, Nq, Nk, d, c["seed"], c["ragged"])
    dev = lambda bits: torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
    q, k, v = (dev(x[n + "_bits"]) for n in ("Q", "K", "V"))
    del x
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.flash_attn_decode_workspace_bytes(B, H, Nq, Nk, d), dtype=torch.uint8, device="cuda")
    scale = float(d) ** -0.5
    for _ in range(warmup):
        fa.flash_attn_decode_fwd(q, k, v, causal=c["causal"], scale=scale, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fa.flash_attn_decode_fwd(q, k, v, causal=c["causal"], scale=scale, out=o, lse=lse, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = 2 * B * H * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"workload": name, "kind": "decode forward", "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d,
            "us_per_call": round(us, 2), "hbm_gbps": round(gbps, 1),
            "hbm_frac": round(gbps / (PEAK_HBM_TBPS * 1e3), 4), "algorithmic_bytes": nbytes}


def block_sparse_case(steps, warmup):
    """The block-sparse forward on the 64K-long workload (band of two blocks
    each side plus key block 0): time per call from events on the stream,
    TFLOP/s over the visible (query, key) pairs, and the fraction of the
    dense pairs that is computed."""
    import torch
    import io_aware_exact_11_amd as fa
    from io_aware_exact_11_amd import workloads as wl
    name = "sparse_64k"
    c = wl.BLOCK_SPARSE_WORKLOADS[name]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    x = wl.make_inputs(B, H, N, d, c["seed"])
    dev = lambda bits: torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
    q, k, v = (dev(x[n + "_bits"]) for n in ("Q", "K", "V"))
    del x
    bm_host = wl.block_sparse_pattern(N, c["band"])
    bm = torch.from_numpy(bm_host).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = float(d) ** -0.5
    for _ in range(warmup):
        fa.flash_attn_fwd_block_sparse(q, k, v, bm, causal=c["causal"], scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fa.flash_attn_fwd_block_sparse(q, k, v, bm, causal=c["causal"], scale=scale, out=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # N is a multiple of 128 and the workload is non-causal: every on block is 128 x 128 visible pairs.
    pairs = int(bm_host.sum()) * 128 * 128 * B * H
    tflops = 4 * d * pairs / (ms * 1e-3) / 1e12
    return {"workload": name, "kind": "block-sparse forward", "B": B, "H": H, "N": N, "d": d,
            "block_density": round(float(bm_host.mean()), 5), "ms_per_call": round(ms, 4),
            "fwd_tflops": round(tflops, 2), "fwd_frac": round(tflops / PEAK_BF16_TFLOPS, 4)}


def fp8_case(steps, warmup):
    """The 8-bit forward on the N=4096, d=128 workload quantised to E4M3:
    time per call from events on the stream and TFLOP/s (4 d per pair), as a
    fraction of the MI355X dense FP8 matrix-core peak."""
    import torch
    import io_aware_exact_11_amd as fa
    from io_aware_exact_11_amd import workloads as wl
    name = "n4096_d128_fp8"
    c = wl.FP8_WORKLOADS[name]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    x = wl.make_fp8_inputs(B, H, N, d, c["seed"], c["qkv_scale"])
    q8, k8, vt8 = (torch.from_numpy(x[n]).cuda() for n in ("Q8", "K8", "Vt8"))
    dq, dk, dv = x["dq"], x["dk"], x["dv"]
    del x
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = float(d) ** -0.5
    for _ in range(warmup):
        fa.flash_attn_fwd_fp8(q8, k8, vt8, dq, dk, dv, causal=c["causal"], scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fa.flash_attn_fwd_fp8(q8, k8, vt8, dq, dk, dv, causal=c["causal"], scale=scale, out=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = B * H * (N * (N + 1) // 2 if c["causal"] else N * N)
    tflops = 4 * d * pairs / (ms * 1e-3) / 1e12
    return {"workload": name, "kind": "fp8 (E4M3) forward", "B": B, "H": H, "N": N, "d": d, "causal": c["causal"],
            "ms_per_call": round(ms, 4), "fwd_tflops": round(tflops, 2),
            "fwd_frac_of_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
            "fwd_frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def memory_sweep():
    """Peak device memory of one fwd+bwd step (inputs, outputs, workspace) at
    B=2, H=16, d=128, causal, for growing N: grows linearly in N."""
    import torch
    import io_aware_exact_11_amd as fa
    out = []
    for N in (2048, 4096, 8192, 16384, 32768):
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        g = torch.Generator(device="cuda").manual_seed(N)
        q, k, v, do = (torch.randn((2, 16, N, 128), device="cuda", generator=g, dtype=torch.bfloat16)
                       for _ in range(4))
        o, lse = fa.flash_attn_fwd(q, k, v, causal=True)
        fa.flash_attn_bwd(q, k, v, o, do, lse, causal=True)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        out.append({"N": N, "peak_MiB": round(peak / 2**20, 1)})
        del q, k, v, do, o, lse
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the N>=4096 workloads and the memory sweep")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this benchmark measures one GPU only; "
              "attention shards over (batch, head) with no exchange, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import io_aware_exact_11_amd as fa
    fa.load_library()

    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib * 2**18, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    case = Case(PRIMARY, causal=True)
    wall_ms, fwd_ms, bwd_ms = case.run(args.steps, args.warmup)
    ff, fb = case.flops()
    value = (ff + fb) / (wall_ms * 1e-3) / 1e12
    achieved = fb / (bwd_ms * 1e-3) / 1e12

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_digest") == kernel_source_digest() and tr.get("workload") == PRIMARY:
            traffic = tr.get("bwd_call_bytes")
    except (OSError, ValueError):
        pass

    result = {
        "metric": "attention fwd / fwd+bwd TFLOP/s (bf16) and % of MI355X MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gpt2_medium: B=64 H=16 N=1024 d=64 causal, fwd+bwd",
                   "B": case.w.B, "H": case.w.H, "N": case.w.N, "d": case.w.d, "causal": True,
                   "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "roofline": {"kernel": "flash_attn_bwd call (dQ kernel with the D_i row term + dK/dV kernel)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    del case
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = []
        for name, causal, drop in (("n4096_d128", False, None), ("n4096_d128", True, None), ("long_16k", True, None),
                                   ("n4096_d128", False, 0.1)):
            c = Case(name, causal, dropout=drop)
            wms, fms, bms = c.run(args.steps, args.warmup)
            cf, cb = c.flops()
            extra.append({"workload": name, "causal": causal, **({"dropout": drop} if drop else {}),
                          "ms_per_step": round(wms, 4),
                          "fwd_tflops": round(cf / (fms * 1e-3) / 1e12, 2),
                          "fwd_frac": round(cf / (fms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "fwd_bwd_tflops": round((cf + cb) / (wms * 1e-3) / 1e12, 2),
                          "fwd_bwd_frac": round((cf + cb) / (wms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
            del c
            torch.cuda.empty_cache()
        extra.append(decode_case(args.steps, args.warmup))
        extra.append(block_sparse_case(args.steps, args.warmup))
        torch.cuda.empty_cache()
        extra.append(fp8_case(args.steps, args.warmup))
        torch.cuda.empty_cache()
        result["workloads"] = extra
        result["memory_sweep_B2_H16_d128_causal"] = memory_sweep()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(PRIMARY, causal=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
