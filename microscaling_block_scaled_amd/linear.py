"""An MX linear layer Y = X W^T built from the C-ABI calls of ``mx``: the three
products of a training step, each with its operands quantized along its own
reduction axis ("Microscaling Data Formats for Deep Learning", section 3:
quantizing along one axis does not commute with transposition, so a tensor
used along two axes is quantized twice, once per axis).

    forward   Y [T x O]  = X [T x H]  . W^T       K = H   X row blocks, W row blocks
    dgrad     dX [T x H] = dY [T x O] . W         K = O   dY row blocks, W column blocks
    wgrad     dW [O x H] = dY^T . X               K = T   dY and X column blocks

Rounding and transform follow "Format-Aware Fusion for Fast FP4 Pretraining"
(abstract): the gradient dY is quantized with stochastic rounding, and the
weight-gradient operands (dY and X along T) get the fixed-sign 32-value
Hadamard transform, applied to both so that their product is preserved; all
other operands use round to nearest even.  W's two layouts come from one
dual-layout pass.  Y and dX leave the GEMM as bf16 (the tensors handed to the
next layer), dW as fp32 (the optimizer's accumulator input).

Everything here is argument marshalling and call order; all arithmetic runs in
the library's kernels."""
from dataclasses import dataclass

import torch

from . import mx


@dataclass
class Recipe:
    fmt: int = mx.E2M1          # element format of every operand
    seed: int = 42              # Philox key of the gradient's stochastic rounding
    hadamard_signs: int = 0     # sign mask of the weight-gradient transform


@dataclass
class Saved:
    """What the forward keeps for the backward: X (for its column blocks) and
    W's column-block copy."""
    x: torch.Tensor
    w_colt: torch.Tensor
    w_colt_s: torch.Tensor


def forward(x: torch.Tensor, w: torch.Tensor, r: Recipe, stream=None):
    """Y = X W^T as bf16, and the state the backward needs."""
    T, H = x.shape
    O = w.shape[0]
    qx = mx.quantize(x, r.fmt, mx.LAYOUT_ROW, mx.RNE, stream=stream)
    qw = mx.quantize(w, r.fmt, mx.LAYOUT_ROW | mx.LAYOUT_COLT, mx.RNE, stream=stream)
    y = mx.gemm_bf16(qx["q_row"], qx["s_row"], r.fmt, qw["q_row"], qw["s_row"], r.fmt, T, O, H,
                     stream=stream)
    return y, Saved(x, qw["q_colt"], qw["s_colt"])


def backward(dy: torch.Tensor, saved: Saved, r: Recipe, stream=None):
    """(dX as bf16, dW as fp32) for the upstream gradient dY [T x O]."""
    T, O = dy.shape
    H = saved.x.shape[1]
    qdy = mx.quantize(dy, r.fmt, mx.LAYOUT_ROW, mx.SR, seed=r.seed, stream=stream)
    dx = mx.gemm_bf16(qdy["q_row"], qdy["s_row"], r.fmt, saved.w_colt, saved.w_colt_s, r.fmt,
                      T, H, O, stream=stream)
    del qdy
    qdyc = mx.quantize(dy, r.fmt, mx.LAYOUT_COLT, mx.SR, hadamard=True,
                       hadamard_signs=r.hadamard_signs, seed=r.seed, stream=stream)
    qxc = mx.quantize(saved.x, r.fmt, mx.LAYOUT_COLT, mx.RNE, hadamard=True,
                      hadamard_signs=r.hadamard_signs, stream=stream)
    dw = mx.gemm(qdyc["q_colt"], qdyc["s_colt"], r.fmt, qxc["q_colt"], qxc["s_colt"], r.fmt,
                 O, H, T, stream=stream)
    return dx, dw
