"""Seeded synthetic inputs shaped like the workloads of the MX pages.

This module holds no MX arithmetic: it only draws random tensors and rounds
fp32 to bf16 (round to nearest even), so both the GPU path and the CPU oracle
can consume the very same bytes.  Every tensor comes from
``numpy.random.default_rng(seed)``, drawn in the order listed.

Workloads (Llama-3-family 8B MLP shapes stand in for the pretraining runs of
"Format-Aware Fusion for Fast FP4 Pretraining"; no dataset is used):

  mxfp8_small   A fp32 [128x256] N(0,1), B fp32 [256x128] N(0,1)
  quant_sweep   X bf16 [4096x4096] Student-t(3) x 2^U(-20,20) per row, then 1% of
                positions replaced: half by +-0, half by random bf16 subnormals
  mxfp8_mlp     A bf16 [8192x4096] N(0,1), W bf16 [14336x4096] N(0,0.02)
  mxfp8_grad    A bf16 [4096x14336] N(0,1e-3) (E5M2), W bf16 [4096x14336] N(0,0.02)
  mxfp4_mlp     A bf16 [8192x14336] N(0,1), W bf16 [4096x14336] N(0,0.02)
  dual_quant    X bf16 [16384x4096] N(0,1), 0.1% of positions multiplied by 100
"""
from __future__ import annotations

import numpy as np

FULL_SHAPES = {
    "mxfp8_small": {"A": (128, 256), "B": (256, 128)},
    "quant_sweep": {"X": (4096, 4096)},
    "mxfp8_mlp": {"A": (8192, 4096), "W": (14336, 4096)},
    "mxfp8_grad": {"A": (4096, 14336), "W": (4096, 14336)},
    "mxfp4_mlp": {"A": (8192, 14336), "W": (4096, 14336)},
    "dual_quant": {"X": (16384, 4096)},
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) >> 16).astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _sparse_positions(rng, n_total, frac):
    n = int(round(n_total * frac))
    return rng.choice(n_total, size=n, replace=False)


def quant_sweep(shape=(4096, 4096), seed=0):
    rows, cols = shape
    rng = np.random.default_rng(seed)
    t = rng.standard_t(3.0, size=shape).astype(np.float32)
    u = rng.uniform(-20.0, 20.0, size=rows)
    x = t * np.exp2(u).astype(np.float32)[:, None]
    b = bf16_bits(x).reshape(-1)
    pos = _sparse_positions(rng, rows * cols, 0.01)
    half = len(pos) // 2
    zero_pos, sub_pos = pos[:half], pos[half:]
    zsign = rng.integers(0, 2, size=len(zero_pos), dtype=np.uint16)
    b[zero_pos] = zsign << 15
    ssign = rng.integers(0, 2, size=len(sub_pos), dtype=np.uint16)
    mant = rng.integers(1, 128, size=len(sub_pos), dtype=np.uint16)
    b[sub_pos] = (ssign << 15) | mant
    return {"X": b.reshape(shape)}


def dual_quant(shape=(16384, 4096), seed=0):
    rows, cols = shape
    rng = np.random.default_rng(seed)
    x = _normal(rng, shape, 1.0).reshape(-1)
    pos = _sparse_positions(rng, rows * cols, 0.001)
    x[pos] *= np.float32(100.0)
    return {"X": bf16_bits(x).reshape(shape)}


def make(name: str, shapes: dict | None = None, seed: int = 0) -> dict:
    """Inputs of one workload.  ``shapes`` overrides tensor shapes (same
    distributions at a smaller size, for tests)."""
    shp = dict(FULL_SHAPES[name])
    if shapes:
        shp.update(shapes)
    if name == "quant_sweep":
        return quant_sweep(shp["X"], seed)
    if name == "dual_quant":
        return dual_quant(shp["X"], seed)
    rng = np.random.default_rng(seed)
    if name == "mxfp8_small":
        return {"A": _normal(rng, shp["A"], 1.0), "B": _normal(rng, shp["B"], 1.0)}
    std_a = {"mxfp8_mlp": 1.0, "mxfp8_grad": 1e-3, "mxfp4_mlp": 1.0}[name]
    a = bf16_bits(_normal(rng, shp["A"], std_a))
    w = bf16_bits(_normal(rng, shp["W"], 0.02))
    return {"A": a, "W": w}
