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
SAMPLE_A, SAMPLE_W = 1024, 384  # rows of A and W the CPU oracle repeats
EVERY = 4  # timed steps per GEMM timing (event pair)


def dev_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it on a stream issues no system-scope release (no cache
    writeback and invalidate between the kernels it brackets), so the kernels
    of a step run back to back as they do without events.  The HIP runtime is
    the one torch has loaded (soname libamdhip64.so.7)."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            for fn, args in (("hipEventCreateWithFlags", [ctypes.c_void_p, ctypes.c_uint]),
                             ("hipEventRecord", [ctypes.c_void_p, ctypes.c_void_p]),
                             ("hipEventElapsedTime", [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
                             ("hipEventDestroy", [ctypes.c_void_p])):
                getattr(hip, fn).argtypes = args
                getattr(hip, fn).restype = ctypes.c_int
            TimingEvent._hip = hip
        self._ev = ctypes.c_void_p()
        self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, stream):
        self._check(self._hip.hipEventRecord(self._ev, stream.cuda_stream), "hipEventRecord")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._ev:
            self._hip.hipEventDestroy(self._ev)


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


def settle(fn, ms=60.0):
    """Run fn() back to back until `ms` of wall time have passed: the GPU's
    clock needs some tens of milliseconds of load to leave its idle state, and
    timing before that measures the ramp, not the kernels."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def bench_step(mx, steps, warmup):
    """The MXFP4 step on one stream: A's quantize, W's quantize, the GEMM.
    (Running W's quantize on a second stream beside A's measured no faster;
    A first measured 0.5 % faster per step than W first.)
    Inside the timed steps two events around the GEMM on its launch stream
    (timing-only events, TimingEvent), on every EVERY-th step: an event pair
    leaves the GPU idle for about 9 us between kernels, so instrumenting every
    step would add that to each step's time.  The quantizers' own times come
    from a separate pass."""
    import torch
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp4_mlp")
    a, w = dev_bf16(d["A"]), dev_bf16(d["W"])
    sample = {"A": d["A"][:SAMPLE_A].copy(), "W": d["W"][:SAMPLE_W].copy()}
    del d
    st = torch.cuda.current_stream()
    oa = mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0)
    ow = mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    quant_w = lambda i=0: mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0, out=ow, stream=st)
    quant_a = lambda i=0: mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0, out=oa, stream=st)
    gemm = lambda i=0: mx.gemm(oa["q_row"], oa["s_row"], mx.E2M1, ow["q_row"], ow["s_row"], mx.E2M1,
                               M, N, K, c=c, stream=st)

    def step(e=None):
        quant_a()
        quant_w()
        if e:
            e[0].record(st)
        gemm()
        if e:
            e[1].record(st)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[TimingEvent() for _ in range(2)] for _ in range(0, steps, EVERY)]
    t0 = time.perf_counter()
    for s in range(steps):
        step(ev[s // EVERY] if s % EVERY == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gm = sorted(e[0].elapsed_time(e[1]) for e in ev)   # the GEMM, on its launch stream
    # the quantizers alone (untimed for the step): back-to-back launches
    settle(lambda: (quant_w(), quant_a()))
    qa, _ = timed_events(quant_a, 20, st)
    qw, _ = timed_events(quant_w, 20, st)
    step()  # the outputs of one more step, for the parity check against the oracle's sample
    torch.cuda.synchronize()
    sample["gpu"] = {"qa": oa["q_row"][:SAMPLE_A].cpu().numpy(), "sa": oa["s_row"][:SAMPLE_A].cpu().numpy(),
                     "qw": ow["q_row"][:SAMPLE_W].cpu().numpy(), "sw": ow["s_row"][:SAMPLE_W].cpu().numpy(),
                     "c": c[:SAMPLE_A, :SAMPLE_W].cpu().numpy()}
    return {"ms_per_step": wall * 1e3 / steps, "quant_a_ms": qa, "quant_w_ms": qw,
            "gemm_ms": sum(gm) / len(gm), "gemm_ms_median": gm[len(gm) // 2], "gemm_launches_timed": len(gm),
            "sample": sample}


def bench_quant(mx, name, x_host, fmt, layouts, rounds=100, rnd=0, had=False, seed=0):
    """Median kernel time of one quantize over rotating buffer sets (>= 1 GiB);
    `rnd`, `had`, `seed`: stochastic rounding, the Hadamard-32 transform and
    the Philox key."""
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
    outs = [mx.quantize(x, fmt, layouts, rnd, had, 0, seed, 0) for x in xs]
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    med, avg = timed_events(lambda i: mx.quantize(xs[i % nsets], fmt, layouts, rnd, had, 0, seed, 0,
                                                  out=outs[i % nsets]),
                            max(rounds // 5, 4), st)
    gbs = (in_bytes + out_bytes) / (med * 1e-3) / 1e9
    del xs, outs
    torch.cuda.empty_cache()
    return {"workload": name, "bytes": in_bytes + out_bytes, "ms": round(med, 5),
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def bench_copy(name, nbytes, rounds=100):
    """A plain device-to-device copy of `nbytes` (read nbytes, write nbytes) over
    rotating buffer sets (>= 1 GiB), timed like the quantizers: the floor that
    memory traffic of that size reaches on this GPU."""
    import torch
    nsets = max(2, int((1 << 30) // (2 * nbytes)) + 1)
    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    st = torch.cuda.current_stream()
    med, _ = timed_events(lambda i: dst[i % nsets].copy_(src[i % nsets]), max(rounds // 5, 4), st)
    gbs = 2 * nbytes / (med * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"workload": name, "bytes": 2 * nbytes, "ms": round(med, 5), "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def bench_gemm(mx, name, a_host, w_host, fa, fw, peak, rounds=100, out_fmt=None):
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
        c = {"q_row": torch.empty((Mx, mx.packed_bytes(out_fmt, 1, Nx)), dtype=torch.uint8, device="cuda"),
             "s_row": torch.empty((Mx, mx.scale_bytes(1, Nx)), dtype=torch.uint8, device="cuda")}
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


def bench_linear(mx, fmt, peak, rounds=20):
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(sample):
    """The CPU oracle (test infrastructure, untuned), timed on bounded samples
    of the same workloads on this host's cores:
      - the step: quantize the first 1024 rows of A (H32 + SR) and 384 rows of
        W (H32 + RNE) of the benchmark's own inputs, and the 1024 x 384 fp64 dot
        products of their MX values, scaled to the full step (the headline
        value, all threads);
      - quantize GB/s (same algorithmic-bytes formula as the GPU figures) on
        512-row samples of the 4096^2 sweep (every format and layout) and of
        the dual-layout tensor, on all threads and on one.
    Afterwards (untimed) the same rows and block of the GPU step's outputs are
    compared with the oracle's: codes and scales bit for bit, C within
    1e-5 * sum|a*b| + 2^-126."""
    import numpy as np
    import oracle
    from microscaling_block_scaled_amd.synth import make
    threads = oracle.set_threads(0)
    ra, rw = SAMPLE_A, SAMPLE_W
    t0 = time.perf_counter()
    qa = oracle.quantize(sample["A"], oracle.E2M1, 1, oracle.SR, oracle.FLAG_HADAMARD32, 42)
    t1 = time.perf_counter()
    qw = oracle.quantize(sample["W"], oracle.E2M1, 1, oracle.RNE, oracle.FLAG_HADAMARD32)
    t2 = time.perf_counter()
    c_ref, t_ref = oracle.gemm_f64(qa["q_row"], qa["s_row"], 4, qw["q_row"], qw["s_row"], 4, ra, rw, K)
    t3 = time.perf_counter()
    full = (t1 - t0) * (M / ra) + (t2 - t1) * (N / rw) + (t3 - t2) * (M * N / (ra * rw))
    g = sample["gpu"]
    ratio = np.abs(g["c"].astype(np.float64) - c_ref) / (1e-5 * t_ref + 2.0 ** -126)
    parity = {
        "sample": f"rows 0..{ra - 1} of A, rows 0..{rw - 1} of W and C[0:{ra}, 0:{rw}] of the timed step",
        "quant_a_bit_exact": bool(np.array_equal(g["qa"], qa["q_row"]) and np.array_equal(g["sa"], qa["s_row"])),
        "quant_w_bit_exact": bool(np.array_equal(g["qw"], qw["q_row"]) and np.array_equal(g["sw"], qw["s_row"])),
        "gemm_worst_err_over_bound": float(np.nanmax(ratio)),
        "gemm_elements_over_bound": int((~(ratio <= 1.0)).sum()),
    }

    def q_gbs(x, fmt, lay, n_threads):
        oracle.set_threads(n_threads)
        rows, cols = x.shape
        bits = oracle.elem_bits(fmt)
        nlay = (lay & 1) + (lay >> 1)
        nbytes = x.nbytes + nlay * (rows * cols * bits // 8 + rows * cols // 32)
        s0 = time.perf_counter()
        oracle.quantize(x, fmt, lay)
        return nbytes / (time.perf_counter() - s0) / 1e9
    quant = {}
    xs = make("quant_sweep", {"X": (512, 4096)})["X"]
    xd = make("dual_quant", {"X": (512, 4096)})["X"]
    for name, x, fmt, lay in ([(f"sweep_{f}_{l}", xs, fi, li)
                               for f, fi in (("int8", 5), ("e2m3", 2), ("e3m2", 3), ("e2m1", 4))
                               for l, li in (("row", 1), ("colt", 2))] +
                              [("dual_quant_e4m3", xd, 0, 3)]):
        quant[name] = {"GB/s_all_threads": round(q_gbs(x, fmt, lay, threads), 3),
                       "GB/s_1_thread": round(q_gbs(x, fmt, lay, 1), 3)}
    oracle.set_threads(threads)
    return {"value": 2.0 * M * N * K / full / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle on {ra} rows of A, {rw} rows of W and their {ra}x{rw} fp64 dot products "
                      f"({t3 - t0:.1f} s), scaled to the full step ({full:.0f} s)",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "quantize": {"sample": "512 rows x 4096 of the sweep and of the dual-layout tensor",
                         **quant}}, parity


GEMM_KERNEL = "void mx::k_gemm_fast<4, 4, 256, 0, true>"


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
    # before the warm-up steps, settle() runs the step for 60 ms: the clock
    # needs some tens of milliseconds of this load to leave its idle state
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
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
            "gemm": {"ms": round(res["gemm_ms"], 5), "ms_median": round(res["gemm_ms_median"], 5),
                     "launches_timed": res["gemm_launches_timed"], "TFLOP/s": round(gemm_tf, 1)},
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
        # memory-only floors of the same sizes: a copy of the sweep's bf16 input and of the
        # dual-layout one
        # a gradient's quantizes in the linear layer's backward: stochastic rounding to FP8
        # (row-wise, and column-wise with the transform), on the grad-like A of the MXFP8
        # grad shape
        x = make("mxfp8_grad")["A"]
        for fname, f in (("e4m3", mx.E4M3), ("e5m2", mx.E5M2)):
            ks[f"sr_grad_{fname}_row"] = bench_quant(
                mx, f"bf16 [4096x14336] N(0,1e-3) -> {fname} row, SR", x, f, 1, rnd=mx.SR, seed=42)
            ks[f"sr_grad_{fname}_colt_h32"] = bench_quant(
                mx, f"bf16 [4096x14336] N(0,1e-3) -> {fname} col-T, H32 + SR", x, f, 2, rnd=mx.SR,
                had=True, seed=42)
        del x
        ks["copy_floor_4096x4096_bf16"] = bench_copy("device copy of 32 MiB (the sweep input)",
                                                     4096 * 4096 * 2)
        ks["copy_floor_16384x4096_bf16"] = bench_copy("device copy of 128 MiB (the dual-layout input)",
                                                      16384 * 4096 * 2)
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
        out["cpu_baseline"], out["parity"] = cpu_baseline(res["sample"])
    print(json.dumps(out))


if __name__ == "__main__":
    main()
