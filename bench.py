#!/usr/bin/env python3
"""Benchmark of the MX path on one MI355X.

One step = the whole MXFP4 pretraining-recipe path on the Llama-3-8B MLP shape:
  quantize A bf16 [8192 x 14336]  (Hadamard-32, stochastic rounding, seed 42) -> E2M1
  quantize W bf16 [4096 x 14336]  (Hadamard-32, RNE)                          -> E2M1
  MX GEMM  C[8192 x 4096] fp32 = A . W^T  (block-scaled matrix instruction)
`value` is 2*M*N*K / step time (TFLOP/s).  Inputs are resident in HBM before
timing.  Per-kernel results for the other workloads (fused dual-layout E4M3
quantize, the bf16 quantize sweep, MXFP8 GEMMs) are reported under "kernels",
timed on rotating buffer sets larger than the 256 MB Infinity Cache.

Prints ONE JSON line.  Only N=1 is supported: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MX quantize GB/s + MX-GEMM TFLOPS (MXFP8/MXFP4), % of HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "fp6": 10100.0, "bf16": 2500.0}
M, N, K = 8192, 4096, 14336


def dev_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def timed_events(fn, n, stream, batches=5):
    """Per-launch duration (ms) of fn(): HIP events on `stream` around batches
    of n back-to-back launches (so no event sits between two launches);
    returns the median and the mean over the batches of batch time / n."""
    import torch
    per = []
    k = 0
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn(k)
            k += 1
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / n)
    per.sort()
    return per[len(per) // 2], sum(per) / len(per)


def bench_step(mx, steps, warmup):
    import torch
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp4_mlp")
    a, w = dev_bf16(d["A"]), dev_bf16(d["W"])
    del d
    st = torch.cuda.current_stream()
    oa = mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0)
    ow = mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0, out=oa)
        mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0, out=ow)
        mx.gemm(oa["q_row"], oa["s_row"], mx.E2M1, ow["q_row"], ow["s_row"], mx.E2M1, M, N, K, c=c)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # per-kernel events inside the timed region, on the stream the kernels use
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        e = ev[s]
        e[0].record(st)
        mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0, out=oa)
        e[1].record(st)
        mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0, out=ow)
        e[2].record(st)
        mx.gemm(oa["q_row"], oa["s_row"], mx.E2M1, ow["q_row"], ow["s_row"], mx.E2M1, M, N, K, c=c)
        e[3].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qa = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    qw = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    gm = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    span = ev[0][0].elapsed_time(ev[-1][3]) / steps
    return {"ms_per_step": wall * 1e3 / steps, "ms_span": span, "quant_a_ms": qa,
            "quant_w_ms": qw, "gemm_ms": gm}


def bench_quant(mx, name, x_host, fmt, layouts, rounds=60):
    """Median kernel time of one quantize over rotating buffer sets (>= 1 GiB)."""
    import torch
    rows, cols = x_host.shape
    in_bytes = x_host.nbytes
    bits = mx.BITS[fmt]
    out_bytes = 0
    if layouts & mx.LAYOUT_ROW:
        out_bytes += rows * cols * bits // 8 + rows * cols // 32
    if layouts & mx.LAYOUT_COLT:
        out_bytes += rows * cols * bits // 8 + rows * cols // 32
    nsets = max(2, int((1 << 30) // (in_bytes + out_bytes)) + 1)
    x0 = dev_bf16(x_host)
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    outs = [mx.quantize(x, fmt, layouts) for x in xs]
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    med, avg = timed_events(lambda i: mx.quantize(xs[i % nsets], fmt, layouts, out=outs[i % nsets]),
                            max(rounds // 5, 4), st)
    gbs = (in_bytes + out_bytes) / (med * 1e-3) / 1e9
    del xs, outs
    torch.cuda.empty_cache()
    return {"workload": name, "bytes": in_bytes + out_bytes, "ms": round(med, 5),
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def bench_gemm(mx, name, a_host, w_host, fa, fw, peak, rounds=20, out_fmt=None):
    """One product timed alone; with ``out_fmt`` the product leaves the kernel
    in that MX format (mx_gemm_mx) instead of fp32."""
    import torch
    Mx, Kx = a_host.shape
    Nx = w_host.shape[0]
    qa = mx.quantize(dev_bf16(a_host), fa, mx.LAYOUT_ROW)
    qw = mx.quantize(dev_bf16(w_host), fw, mx.LAYOUT_ROW)
    if out_fmt is None:
        c = torch.empty((Mx, Nx), dtype=torch.float32, device="cuda")
        run = lambda i: mx.gemm(qa["q_row"], qa["s_row"], fa, qw["q_row"], qw["s_row"], fw, Mx, Nx,
                                Kx, c=c)
    else:
        c = {"q_row": torch.empty((Mx, Nx * mx.BITS[out_fmt] // 8), dtype=torch.uint8, device="cuda"),
             "s_row": torch.empty((Mx, Nx // 32), dtype=torch.uint8, device="cuda")}
        run = lambda i: mx.gemm_mx(qa["q_row"], qa["s_row"], fa, qw["q_row"], qw["s_row"], fw, Mx,
                                   Nx, Kx, out_fmt, out=c)
    for i in range(3):
        run(i)
    med, avg = timed_events(run, max(rounds // 5, 4), torch.cuda.current_stream())
    tf = 2.0 * Mx * Nx * Kx / (med * 1e-3) / 1e12
    del qa, qw, c
    torch.cuda.empty_cache()
    return {"workload": name, "ms": round(med, 5), "TFLOP/s": round(tf, 1),
            "frac_peak": round(tf / peak, 4), "peak_TFLOP/s": peak}


def bench_linear(mx, fmt, peak, rounds=10):
    """One training step of an MX linear layer at the Llama-3-8B MLP
    up-projection shape (X [8192x4096], W [14336x4096], dY [8192x14336], bf16):
    forward, dgrad and wgrad with every quantization the recipe calls for."""
    import torch
    from microscaling_block_scaled_amd import linear
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp8_mlp")
    x, w = dev_bf16(d["A"]), dev_bf16(d["W"])
    del d
    T, H = x.shape
    O = w.shape[0]
    g = torch.Generator(device="cuda").manual_seed(5)
    dy = (torch.randn((T, O), generator=g, device="cuda") * 1e-3).to(torch.bfloat16)
    r = linear.Recipe(fmt=fmt, seed=42)

    def run(i):
        y, saved = linear.forward(x, w, r)
        linear.backward(dy, saved, r)
    for i in range(3):
        run(i)
    med, _ = timed_events(run, max(rounds // 5, 2), torch.cuda.current_stream())
    tf = 3 * 2.0 * T * H * O / (med * 1e-3) / 1e12
    del x, w, dy
    torch.cuda.empty_cache()
    return {"workload": f"MX linear fwd+dgrad+wgrad T={T} H={H} O={O}, {mx.FMT_NAMES[fmt]}, "
                        "bf16 in, bf16 Y/dX, fp32 dW, SR on dY, H32 on wgrad operands",
            "ms": round(med, 5), "TFLOP/s": round(tf, 1), "frac_peak": round(tf / peak, 4),
            "peak_TFLOP/s": peak}


def cpu_baseline():
    """The CPU oracle, timed on a bounded sample of the same step and scaled to
    the full step: quantize 1024 rows of A (H32 + SR), 384 rows of W (H32 + RNE),
    and the 1024 x 384 dot products of their MX values (fp64)."""
    import numpy as np
    import oracle
    from microscaling_block_scaled_amd.synth import make
    ra, rw = 1024, 384
    d = make("mxfp4_mlp", {"A": (ra, K), "W": (rw, K)})
    t0 = time.perf_counter()
    qa = oracle.quantize(d["A"], oracle.E2M1, 1, oracle.SR, oracle.FLAG_HADAMARD32, 42)
    t1 = time.perf_counter()
    qw = oracle.quantize(d["W"], oracle.E2M1, 1, oracle.RNE, oracle.FLAG_HADAMARD32)
    t2 = time.perf_counter()
    oracle.gemm_f64(qa["q_row"], qa["s_row"], 4, qw["q_row"], qw["s_row"], 4, ra, rw, K)
    t3 = time.perf_counter()
    full = (t1 - t0) * (M / ra) + (t2 - t1) * (N / rw) + (t3 - t2) * (M * N / (ra * rw))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": 2.0 * M * N * K / full / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle on {ra} rows of A, {rw} rows of W and their {ra}x{rw} fp64 dot products "
                      f"({t3 - t0:.1f} s), scaled to the full step ({full:.0f} s)"}


GEMM_KERNEL = "void mx::k_gemm_fast<4, 4, 256>"


def load_traffic(src_hash):
    """Counter-measured bytes per launch of the GEMM (FETCH_SIZE + WRITE_SIZE,
    calibrated on a plain copy), if taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_hash") != src_hash:
        return None
    k = t.get("kernels", {}).get(GEMM_KERNEL)
    return None if k is None else k["bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~20 ms of warm-up: the clock needs that long under this load to settle
    # (with 5 warm-up steps the timed steps ran ~15 % slower, still ramping)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel extras")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (no sharding, no collectives); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from microscaling_block_scaled_amd import mx
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)

    res = bench_step(mx, args.steps, args.warmup)
    flops = 2.0 * M * N * K
    value = flops / (res["ms_per_step"] * 1e-3) / 1e12
    gemm_tf = flops / (res["gemm_ms"] * 1e-3) / 1e12
    a_bytes = M * K * 2 + M * K // 2 + M * K // 32
    w_bytes = N * K * 2 + N * K // 2 + N * K // 32
    from microscaling_block_scaled_amd.profile_kernels import kernel_source_hash
    src_hash = kernel_source_hash()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1",
        "data": "synthetic",
        "config": {
            "workload": "mxfp4_mlp: Hadamard-32 + SR (Philox, seed 42) quantize of A bf16 "
                        "[8192x14336] and Hadamard-32 + RNE quantize of W bf16 [4096x14336] to "
                        "MXFP4 E2M1, then MX GEMM M=8192 N=4096 K=14336, fp32 accumulate/output",
            "M": M, "N": N, "K": K, "block": 32,
        },
        "roofline": {
            "kernel": "k_gemm_fast<E2M1,E2M1,256>",
            "bound": "mfma",
            "achieved": round(gemm_tf, 1),
            "peak": PEAK_TFLOPS["fp4"],
            "unit": "TFLOP/s",
            "frac": round(gemm_tf / PEAK_TFLOPS["fp4"], 4),
            "traffic": load_traffic(src_hash),
        },
        "step_kernels": {
            "quant_a": {"ms": round(res["quant_a_ms"], 5), "bytes": a_bytes,
                        "GB/s": round(a_bytes / (res["quant_a_ms"] * 1e-3) / 1e9, 1)},
            "quant_w": {"ms": round(res["quant_w_ms"], 5), "bytes": w_bytes,
                        "GB/s": round(w_bytes / (res["quant_w_ms"] * 1e-3) / 1e9, 1)},
            "gemm": {"ms": round(res["gemm_ms"], 5), "TFLOP/s": round(gemm_tf, 1)},
        },
        "source_hash": src_hash,
    }
    if not args.no_kernels:
        from microscaling_block_scaled_amd.synth import make
        ks = {}
        x = make("dual_quant")["X"]
        ks["dual_quant_e4m3"] = bench_quant(mx, "dual E4M3 bf16 [16384x4096] row + col-T", x,
                                            mx.E4M3, 3)
        del x
        x = make("quant_sweep")["X"]
        for fname, f in (("int8", mx.INT8), ("e2m3", mx.E2M3), ("e3m2", mx.E3M2), ("e2m1", mx.E2M1)):
            for lname, lay in (("row", 1), ("colt", 2)):
                ks[f"sweep_{fname}_{lname}"] = bench_quant(
                    mx, f"bf16 [4096x4096] -> {fname} {lname}", x, f, lay)
        del x
        d = make("mxfp8_mlp")
        ks["gemm_mxfp8_mlp"] = bench_gemm(mx, "E4M3 M=8192 N=14336 K=4096", d["A"], d["W"],
                                          mx.E4M3, mx.E4M3, PEAK_TFLOPS["fp8"])
        # the same product written out as MXFP8 (row blocks along N) by the
        # GEMM itself: 118 MB of codes and scales instead of 470 MB of fp32
        ks["gemm_mxfp8_mlp_mxout"] = bench_gemm(
            mx, "E4M3 M=8192 N=14336 K=4096, output E4M3 MX", d["A"], d["W"], mx.E4M3, mx.E4M3,
            PEAK_TFLOPS["fp8"], out_fmt=mx.E4M3)
        # MXINT8 runs on the bf16 instruction with the scales folded into the
        # operands: priced against the bf16 peak
        ks["gemm_mxint8_mlp"] = bench_gemm(mx, "INT8 x INT8 M=8192 N=14336 K=4096 (bf16 MFMA)",
                                           d["A"], d["W"], mx.INT8, mx.INT8, PEAK_TFLOPS["bf16"])
        del d
        d = make("mxfp8_grad")
        ks["gemm_mxfp8_grad"] = bench_gemm(mx, "E5M2 x E4M3 M=4096 N=4096 K=14336", d["A"],
                                           d["W"], mx.E5M2, mx.E4M3, PEAK_TFLOPS["fp8"])
        del d
        # the 6-bit and mixed 4/6-bit variants of the MXFP4 MLP product
        d = make("mxfp4_mlp")
        ks["gemm_mxfp6_mlp"] = bench_gemm(mx, "E2M3 x E2M3 M=8192 N=4096 K=14336", d["A"], d["W"],
                                          mx.E2M3, mx.E2M3, PEAK_TFLOPS["fp6"])
        ks["gemm_mxfp6x4_mlp"] = bench_gemm(mx, "E2M3 activations x E2M1 weights M=8192 N=4096 K=14336",
                                            d["A"], d["W"], mx.E2M3, mx.E2M1, PEAK_TFLOPS["fp6"])
        del d
        ks["linear_step_mxfp4"] = bench_linear(mx, mx.E2M1, PEAK_TFLOPS["fp4"])
        ks["linear_step_mxfp8"] = bench_linear(mx, mx.E4M3, PEAK_TFLOPS["fp8"])
        out["kernels"] = ks
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
