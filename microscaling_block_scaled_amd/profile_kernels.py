"""Profiling driver and counter summaries for the MX kernels.

  python -m microscaling_block_scaled_amd.profile_kernels run [--reps R]
      Launches each headline kernel R times on seeded inputs, then a plain
      1 GiB device copy (known bytes) that calibrates the traffic counters.
      Meant to run under `rocprofv3 --kernel-trace` (R >= 100: per-dispatch
      medians) and under `rocprofv3 --pmc ...` (a few R per counter pass).

  python -m microscaling_block_scaled_amd.profile_kernels traffic FETCH_DIR WRITE_DIR OUT.json
      Reads the two counter runs (rocprofv3 --output-format csv), scales each
      kernel's per-dispatch FETCH_SIZE / WRITE_SIZE by what the counters read
      for the copy (whose true traffic is 1 GiB read + 1 GiB written) and
      writes bytes per launch per kernel, tagged with a hash of the kernel
      sources (a changed kernel invalidates its figures).

  python -m microscaling_block_scaled_amd.profile_kernels stats TRACE_DIR OUT.md CMD
      Formats rocprofv3 --kernel-trace --stats output as a short table, with
      each kernel's median per-dispatch duration.

  python -m microscaling_block_scaled_amd.profile_kernels mfma DIR OUT.md CMD
      From a pass of SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES,
      GRBM_GUI_ACTIVE and GRBM_COUNT: per GEMM kernel the matrix-unit busy
      fraction (busy cycles per SIMD / GPU-active cycles), the sustained
      shader clock (GPU-active cycles per XCD / duration) and the rate as a
      fraction of the nominal peak and of the peak at that clock.

  python -m microscaling_block_scaled_amd.profile_kernels valu DIR OUT.md CMD
      From a pass of SQ_ACTIVE_INST_VALU, SQ_INSTS_VALU, SQ_BUSY_CU_CYCLES and
      GRBM_GUI_ACTIVE: per kernel the vector-ALU issue load.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "microscaling_block_scaled_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def run(reps: int) -> None:
    import numpy as np
    import torch
    from microscaling_block_scaled_amd import mx
    from microscaling_block_scaled_amd.synth import make

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    def gemms(name, pairs, mx_out=None):
        d = make(name)
        a, w = dev_bf16(d["A"]), dev_bf16(d["W"])
        Mx, Kx = d["A"].shape
        Nx = d["W"].shape[0]
        del d
        for fa, fw in pairs:
            qa = mx.quantize(a, fa, mx.LAYOUT_ROW)
            qw = mx.quantize(w, fw, mx.LAYOUT_ROW)
            c = torch.empty((Mx, Nx), dtype=torch.float32, device="cuda")
            for _ in range(reps):
                mx.gemm(qa["q_row"], qa["s_row"], fa, qw["q_row"], qw["s_row"], fw, Mx, Nx, Kx, c=c)
            if mx_out is not None:
                o = mx.gemm_mx(qa["q_row"], qa["s_row"], fa, qw["q_row"], qw["s_row"], fw, Mx, Nx, Kx, mx_out)
                for _ in range(reps):
                    mx.gemm_mx(qa["q_row"], qa["s_row"], fa, qw["q_row"], qw["s_row"], fw, Mx, Nx, Kx,
                               mx_out, out=o)
                del o
            torch.cuda.synchronize()
            del qa, qw, c
        del a, w
        torch.cuda.empty_cache()

    # the MXFP4 step: A (H32 + SR) and W (H32) quantized, then the GEMM
    d = make("mxfp4_mlp")
    a, w = dev_bf16(d["A"]), dev_bf16(d["W"])
    del d
    M, K = a.shape
    N = w.shape[0]
    oa = mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0)
    ow = mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for _ in range(reps):
        mx.quantize(a, mx.E2M1, mx.LAYOUT_ROW, mx.SR, True, 0, 42, 0, out=oa)
        mx.quantize(w, mx.E2M1, mx.LAYOUT_ROW, mx.RNE, True, 0, 0, 0, out=ow)
        mx.gemm(oa["q_row"], oa["s_row"], mx.E2M1, ow["q_row"], ow["s_row"], mx.E2M1, M, N, K, c=c)
    torch.cuda.synchronize()
    del a, w, oa, ow, c
    torch.cuda.empty_cache()
    # the fused dual-layout quantize and the 4096^2 sweep
    x = dev_bf16(make("dual_quant")["X"])
    o = mx.quantize(x, mx.E4M3, 3)
    for _ in range(reps):
        mx.quantize(x, mx.E4M3, 3, out=o)
    torch.cuda.synchronize()
    del x, o
    x = dev_bf16(make("quant_sweep")["X"])
    for f in (mx.INT8, mx.E2M3, mx.E3M2, mx.E2M1):
        for lay in (mx.LAYOUT_ROW, mx.LAYOUT_COLT):
            o = mx.quantize(x, f, lay)
            for _ in range(reps):
                mx.quantize(x, f, lay, out=o)
            torch.cuda.synchronize()
            del o
    del x
    torch.cuda.empty_cache()
    # the MXFP8 products (config 3 with fp32 and E4M3 output, config 3b), the
    # 6-bit and mixed 6/4-bit products, MXINT8
    gemms("mxfp8_mlp", [(mx.E4M3, mx.E4M3)], mx_out=mx.E4M3)
    gemms("mxfp8_grad", [(mx.E5M2, mx.E4M3)])
    gemms("mxfp4_mlp", [(mx.E2M3, mx.E2M3), (mx.E2M3, mx.E2M1)])
    gemms("mxfp8_mlp", [(mx.INT8, mx.INT8)])
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profile_kernels: done", flush=True)


def _rows(d: str, pattern: str):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    with open(files[0], newline="") as fh:
        return list(csv.DictReader(fh))


def _per_kernel(d: str, counter: str):
    """kernel name -> list of per-dispatch counter values (KiB)."""
    out: dict[str, list[float]] = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _copy_kernel(per: dict) -> str:
    # the calibration copy: the one elementwise copy kernel launched last
    cands = [k for k in per if "copy" in k.lower() and "mx::" not in k]
    if not cands:
        raise SystemExit("calibration copy kernel not found")
    return max(cands, key=lambda k: sum(per[k]) / len(per[k]))


def traffic(fetch_dir: str, write_dir: str, out: str) -> None:
    f = _per_kernel(fetch_dir, "FETCH_SIZE")
    w = _per_kernel(write_dir, "WRITE_SIZE")
    ck = _copy_kernel(f)
    f_copy = sum(f[ck]) / len(f[ck]) * 1024.0
    w_copy = sum(w[ck]) / len(w[ck]) * 1024.0
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    kernels = {}
    for k in f:
        if "mx::" not in k:
            continue
        fb = sum(f[k]) / len(f[k]) * 1024.0 * f_scale
        wb = sum(w.get(k, [0.0])) / max(1, len(w.get(k, []))) * 1024.0 * w_scale
        kernels[k.split("(")[0]] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                                    "bytes_per_launch": round(fb + wb), "dispatches": len(f[k])}
    res = {"source_hash": kernel_source_hash(),
           "calibration": {"kernel": ck.split("(")[0], "true_bytes_each_way": COPY_BYTES,
                           "fetch_counter_bytes": round(f_copy), "write_counter_bytes": round(w_copy),
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "kernels": kernels}
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def _durations(trace_dir: str) -> dict:
    """kernel name -> per-dispatch durations (us) in dispatch order."""
    out: dict[str, list[float]] = {}
    for r in sorted(_rows(trace_dir, "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        out.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def stats(trace_dir: str, out: str, cmd: str) -> None:
    """The --stats table, plus each kernel's median over its last 100 calls
    (the clock needs some milliseconds of load to settle, so the first calls
    of a run are slower than the steady state) and its later-half average."""
    rows = _rows(trace_dir, "*kernel_stats.csv")
    dur = _durations(trace_dir)
    lines = [f"Command: `{cmd}`", "",
             "| kernel | calls | median of last 100 us | later-half avg us | avg us | min us | max us | total % |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0]
        d = dur.get(r["Name"], [])
        half = d[len(d) // 2:]
        lh = f"{sum(half) / len(half):.2f}" if half else "-"
        md = f"{_median(d[-100:]):.2f}" if d else "-"
        lines.append(f"| `{name}` | {r['Calls']} | {md} | {lh} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_table(d: str):
    """kernel name -> {counter: [per-dispatch values]}, plus per-dispatch
    durations (ns) of the counter run."""
    per: dict[str, dict[str, list[float]]] = {}
    dur: dict[str, dict[str, float]] = {}
    for r in _rows(d, "*counter_collection.csv"):
        k = r["Kernel_Name"]
        per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if "Start_Timestamp" in r and r.get("Start_Timestamp"):
            dur.setdefault(k, {})[r.get("Dispatch_Id", "")] = (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per, {k: sorted(v.values()) for k, v in dur.items()}


GEMM_FLOPS = {  # 2 M N K of the products the driver runs, by kernel template arguments
    # (FA, FB, KS, output kind, scale loads spread over a chunk's stages)
    "k_gemm_fast<4, 4, 256, 0, true>": (2.0 * 8192 * 4096 * 14336, 10100.0, "MXFP4 8192x4096x14336"),
    "k_gemm_fast<0, 0, 128, 0, true>": (2.0 * 8192 * 14336 * 4096, 5000.0, "MXFP8 E4M3 8192x14336x4096"),
    "k_gemm_fast<0, 0, 128, 2, false>": (2.0 * 8192 * 14336 * 4096, 5000.0, "MXFP8 E4M3, E4M3 MX output"),
    "k_gemm_fast<1, 0, 128, 0, true>": (2.0 * 4096 * 4096 * 14336, 5000.0, "MXFP8 E5M2 x E4M3 4096x4096x14336"),
    "k_gemm_fast<2, 2, 128, 0, true>": (2.0 * 8192 * 4096 * 14336, 10100.0, "MXFP6 E2M3 8192x4096x14336"),
    "k_gemm_fast<2, 4, 128, 0, true>": (2.0 * 8192 * 4096 * 14336, 10100.0, "E2M3 x E2M1 8192x4096x14336"),
    "k_gemm_fast<5, 5, 128, 0, true>": (2.0 * 8192 * 14336 * 4096, 2500.0, "MXINT8 (bf16 instruction) 8192x14336x4096"),
}
N_SIMD, N_XCD, NOMINAL_GHZ = 1024, 8, 2.4


def mfma(d: str, out: str, cmd: str) -> None:
    per, dur = _counter_table(d)
    lines = [f"Command: `{cmd}`", "",
             "Per dispatch (medians over the run's dispatches of each kernel).  Counter values are "
             "summed by rocprofv3 over all XCDs and shader engines: GRBM_GUI_ACTIVE / 8 is the "
             "GPU-active cycles of one XCD; SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs.",
             "",
             "| kernel | workload | duration us | clock GHz (GUI_ACTIVE/8 / duration) | MFMA busy "
             "(busy / (1024 x GUI_ACTIVE/8)) | TFLOP/s | % of nominal peak | % of peak at that clock |",
             "|---|---|---|---|---|---|---|---|"]
    for k, cs in sorted(per.items()):
        key = next((g for g in GEMM_FLOPS if g in k), None)
        if key is None or "GRBM_GUI_ACTIVE" not in cs or "SQ_VALU_MFMA_BUSY_CYCLES" not in cs:
            continue
        flops, peak, what = GEMM_FLOPS[key]
        gui = _median(cs["GRBM_GUI_ACTIVE"]) / N_XCD
        busy = _median(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
        t_ns = _median(dur.get(k, [0])) if dur.get(k) else 0
        ghz = gui / t_ns if t_ns else float("nan")
        tf = flops / (t_ns * 1e-9) / 1e12 if t_ns else float("nan")
        lines.append(f"| `{key}` | {what} | {t_ns / 1e3:.1f} | {ghz:.2f} | {busy / (N_SIMD * gui):.3f} | "
                     f"{tf:.0f} | {100 * tf / peak:.1f} | {100 * tf / (peak * ghz / NOMINAL_GHZ):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def valu(d: str, out: str, cmd: str) -> None:
    per, dur = _counter_table(d)
    lines = [f"Command: `{cmd}`", "",
             "Per dispatch (medians).  SQ_ACTIVE_INST_VALU counts cycles in which a wave issued a "
             "vector-ALU instruction, summed over waves; per SIMD and GPU-active cycle it is the "
             "fraction of issue slots the vector ALU takes.",
             "",
             "| kernel | duration us | clock GHz | VALU instructions per SIMD | VALU-active cycles per SIMD / GPU-active cycles |",
             "|---|---|---|---|---|"]
    for k, cs in sorted(per.items()):
        if "mx::" not in k or "GRBM_GUI_ACTIVE" not in cs:
            continue
        gui = _median(cs["GRBM_GUI_ACTIVE"]) / N_XCD
        t_ns = _median(dur.get(k, [0])) if dur.get(k) else 0
        ghz = gui / t_ns if t_ns else float("nan")
        vi = _median(cs.get("SQ_INSTS_VALU", [float("nan")])) / N_SIMD
        va = _median(cs.get("SQ_ACTIVE_INST_VALU", [float("nan")])) / N_SIMD
        lines.append(f"| `{k.split('(')[0]}` | {t_ns / 1e3:.1f} | {ghz:.2f} | {vi:.0f} | {va / gui:.3f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv):
    if len(argv) >= 1 and argv[0] == "run":
        reps = int(argv[argv.index("--reps") + 1]) if "--reps" in argv else 3
        run(reps)
    elif len(argv) == 4 and argv[0] == "traffic":
        traffic(argv[1], argv[2], argv[3])
    elif len(argv) == 4 and argv[0] == "stats":
        stats(argv[1], argv[2], argv[3])
    elif len(argv) == 4 and argv[0] == "mfma":
        mfma(argv[1], argv[2], argv[3])
    elif len(argv) == 4 and argv[0] == "valu":
        valu(argv[1], argv[2], argv[3])
    else:
        print(__doc__)
        sys.exit(2)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main(sys.argv[1:])
