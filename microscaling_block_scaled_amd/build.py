"""Build libmx.so (HIP kernels + C-ABI) for gfx950, in place.

    python -m microscaling_block_scaled_amd.build [--incremental]

The GEMM kernel templates (csrc/mx_gemm_kernels.hpp) are instantiated once per
operand-format pair, each pair in a small generated unit of its own under
_build/gen, so the pairs compile in parallel.  --incremental skips units whose
object is newer than every source (for development; the default rebuilds
everything).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
GEN = os.path.join(OBJ, "gen")
LIB = os.path.join(PKG, "libmx.so")

SOURCES = ["mx_quant.hip", "mx_dequant.hip", "mx_gemm.hip", "mx_api.cpp"]
FORMATS = ["E4M3", "E5M2", "E2M3", "E3M2", "E2M1"]
# every float pair, and MXINT8 with itself
PAIRS = [(a, b) for a in FORMATS for b in FORMATS] + [("INT8", "INT8")]
# packed-fp32 instruction selection is switched off for every device pass
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=gfx950", "-Wall",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _gen_units() -> list[str]:
    """One instantiation unit per GEMM operand-format pair."""
    os.makedirs(GEN, exist_ok=True)
    units = []
    for a, b in PAIRS:
        path = os.path.join(GEN, f"gemm_{a.lower()}_{b.lower()}.hip")
        text = ('#include "mx_gemm_kernels.hpp"\n'
                f"namespace mx {{\ntemplate hipError_t gemm_launch<{a}, {b}>(const GemmCall&);\n}}\n")
        if not os.path.exists(path) or open(path).read() != text:
            with open(path, "w") as fh:
                fh.write(text)
        units.append(path)
    return units


def _newest_source() -> float:
    files = glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*"))
    return max(os.path.getmtime(f) for f in files)


def _compile(src: str, incremental: bool, newest: float) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    if incremental and os.path.exists(out) and os.path.getmtime(out) > max(newest, os.path.getmtime(src)):
        return out
    cmd = [hipcc(), *COMMON, "-c", src, "-o", out]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    return out


def build(jobs: int | None = None, incremental: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + _gen_units()
    # the longest units first
    srcs.sort(key=lambda s: (0 if "gemm_" in os.path.basename(s) else 1))
    newest = _newest_source()
    jobs = jobs or int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))
    with cf.ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental, newest), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(incremental="--incremental" in sys.argv[1:]))
    sys.exit(0)
