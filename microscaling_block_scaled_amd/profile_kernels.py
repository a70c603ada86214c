"""Profiling driver and counter summaries for the MX kernels.

  python -m microscaling_block_scaled_amd.profile_kernels run [--reps R]
      Launches each headline kernel R times on seeded inputs, then a plain
      1 GiB device copy (known bytes) that calibrates the traffic counters.
      Meant to run under `rocprofv3 --pmc FETCH_SIZE ...` and
      `rocprofv3 --pmc WRITE_SIZE ...`.

  python -m microscaling_block_scaled_amd.profile_kernels traffic FETCH_DIR WRITE_DIR OUT.json
      Reads the two counter runs (rocprofv3 --output-format csv), scales each
      kernel's per-dispatch FETCH_SIZE / WRITE_SIZE by what the counters read
      for the copy (whose true traffic is 1 GiB read + 1 GiB written) and
      writes bytes per launch per kernel, tagged with a hash of the kernel
      sources (a changed kernel invalidates its figures).

  python -m microscaling_block_scaled_amd.profile_kernels stats TRACE_DIR OUT.md CMD
      Formats rocprofv3 --kernel-trace --stats output as a short table.
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
    x = dev_bf16(make("dual_quant")["X"])
    o = mx.quantize(x, mx.E4M3, 3)
    for _ in range(reps):
        mx.quantize(x, mx.E4M3, 3, out=o)
    torch.cuda.synchronize()
    del x, o
    for name, fa, fw in (("mxfp8_mlp", mx.E4M3, mx.E4M3), ("mxfp8_grad", mx.E5M2, mx.E4M3)):
        d = make(name)
        qa = mx.quantize(dev_bf16(d["A"]), fa, mx.LAYOUT_ROW)
        qw = mx.quantize(dev_bf16(d["W"]), fw, mx.LAYOUT_ROW)
        Mx, Kx = d["A"].shape
        Nx = d["W"].shape[0]
        del d
        c = torch.empty((Mx, Nx), dtype=torch.float32, device="cuda")
        for _ in range(reps):
            mx.gemm(qa["q_row"], qa["s_row"], fa, qw["q_row"], qw["s_row"], fw, Mx, Nx, Kx, c=c)
        torch.cuda.synchronize()
        del qa, qw, c
    torch.cuda.empty_cache()
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


def stats(trace_dir: str, out: str, cmd: str) -> None:
    """The --stats table, plus each kernel's average over its later half of
    calls (in dispatch order): the clock needs some milliseconds of load to
    settle, so the first calls of a run are slower than the steady state."""
    rows = _rows(trace_dir, "*kernel_stats.csv")
    late: dict[str, list[float]] = {}
    for r in sorted(_rows(trace_dir, "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        late.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"Command: `{cmd}`", "",
             "| kernel | calls | avg us | min us | max us | later-half avg us | total % |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0]
        d = late.get(r["Name"], [])
        half = d[len(d) // 2:]
        lh = f"{sum(half) / len(half):.2f}" if half else "-"
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {lh} | "
                     f"{float(r['Percentage']):.1f} |")
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
    else:
        print(__doc__)
        sys.exit(2)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main(sys.argv[1:])
