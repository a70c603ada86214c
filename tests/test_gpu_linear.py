"""bf16-output GEMM and the MX linear layer's three products on the GPU.

mx_gemm_bf16 must equal mx_gemm's fp32 product rounded to bf16 (nearest even)
bit for bit, in both kernels.  The linear layer (forward, dgrad, wgrad) is
checked against the oracle taking the same steps on the same inputs: the
oracle quantizes each operand along its reduction axis with the same rounding,
seed and transform, and multiplies in fp64; bf16 outputs may differ from it by
the GEMM tolerance plus half a bf16 step (2^-8 of the magnitude)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, gemm_tolerance, host, mfma_group_bound, say
from test_gpu_gemm import quant_pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from microscaling_block_scaled_amd import mx as m
    return m


@pytest.mark.parametrize("fa,fb", [(0, 0), (4, 4), (1, 2), (5, 5)])
def test_gemm_bf16_is_rounded_fp32(mx, oracle, fa, fb):
    """Staged-kernel shapes (K % 512 == 0) and general-kernel shapes, ragged
    M/N, a leading dimension wider than N, and values spread over 2^-60 ..
    2^60 so that rounding carries, large and small magnitudes all occur."""
    rng = np.random.default_rng(31 + fa)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K, ldc) in [(288, 320, 1024, 320), (300, 260, 2048, 264), (100, 36, 512, 40),
                           (70, 48, 96, 52)]:
        a = rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 31, (M, 1)))
        w = rng.standard_normal((N, K)) * np.exp2(rng.integers(-30, 31, (N, 1)))
        (ga, _), (gw, _) = quant_pair(mx, oracle, bf16_bits(a.astype(np.float32)),
                                      bf16_bits(w.astype(np.float32)), fa, fb)
        say("gemm_bf16", M, N, K, ldc, fa, fb)
        c32 = mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fb, M, N, K)
        cb = torch.full((M, ldc), 1.5, dtype=torch.bfloat16, device="cuda")
        mx.gemm_bf16(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fb, M, N, K,
                     c=cb[:, :N])
        want = c32.to(torch.bfloat16).view(torch.int16)
        got = cb[:, :N].view(torch.int16)
        assert torch.equal(got, want), f"{(got != want).sum().item()} bf16 values differ"
        assert (cb[:, N:] == 1.5).all()  # nothing written past N


def bf16_close(y, ref, tol, what):
    y = np.asarray(y, np.float64)
    bound = tol + 2.0 ** -8 * (np.abs(ref) + tol) + 2.0 ** -133
    bad = ~(np.abs(y - ref) <= bound)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside; first at {i}: "
                             f"gpu {y[i]} ref {ref[i]} bound {bound[i]}")


def oracle_step(oracle, fmt, x, w, dy, seed, signs):
    """The linear layer's three products, each operand quantized along its
    reduction axis: forward X/W row blocks (RNE); dgrad dY row blocks (SR) with
    W column blocks; wgrad dY (SR) and X (RNE) column blocks, both with the
    Hadamard-32 transform."""
    T, H = x.shape
    O = w.shape[0]
    H32 = oracle.FLAG_HADAMARD32
    qx = oracle.quantize(x, fmt, oracle.LAYOUT_ROW, oracle.RNE)
    qw = oracle.quantize(w, fmt, oracle.LAYOUT_ROW | oracle.LAYOUT_COLT, oracle.RNE)
    qdy = oracle.quantize(dy, fmt, oracle.LAYOUT_ROW, oracle.SR, 0, seed)
    qdyc = oracle.quantize(dy, fmt, oracle.LAYOUT_COLT, oracle.SR, H32, seed, 0, signs)
    qxc = oracle.quantize(x, fmt, oracle.LAYOUT_COLT, oracle.RNE, H32, 0, 0, signs)
    out = {}
    for name, A, sA, B, sB, m, n, k in (
            ("y", qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], T, O, H),
            ("dx", qdy["q_row"], qdy["s_row"], qw["q_colt"], qw["s_colt"], T, H, O),
            ("dw", qdyc["q_colt"], qdyc["s_colt"], qxc["q_colt"], qxc["s_colt"], O, H, T)):
        c, t = oracle.gemm_f64(A, sA, fmt, B, sB, fmt, m, n, k)
        extra = 0.0
        if fmt in (0, 1, 3) and k < 512:
            # a product of fewer than 16 blocks in FP8 / E3M2: the short-K
            # departure of the block-scaled instruction (its group truncation)
            extra = mfma_group_bound(oracle.dequantize(A, sA, fmt, m, k).astype(np.float64),
                                     oracle.dequantize(B, sB, fmt, n, k).astype(np.float64))
        out[name] = (c, gemm_tolerance(t) + extra)
    return out


@pytest.mark.parametrize("fmt,T,H,O", [(4, 1024, 512, 1536), (4, 288, 160, 96),
                                       (0, 512, 512, 512), (2, 96, 64, 160),
                                       (5, 288, 160, 96)])
def test_linear_step(mx, oracle, fmt, T, H, O):
    """Forward, dgrad and wgrad of one layer; the first shape puts every
    product on the staged kernel (K = 512, 1536, 1024), the second on the
    general one with ragged tiles."""
    from microscaling_block_scaled_amd import linear
    from microscaling_block_scaled_amd.synth import bf16_bits
    rng = np.random.default_rng(T + H + O + fmt)
    x = bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = bf16_bits((rng.standard_normal((O, H)) * 0.02).astype(np.float32))
    dy = bf16_bits((rng.standard_normal((T, O)) * 1e-3).astype(np.float32))
    r = linear.Recipe(fmt=fmt, seed=42, hadamard_signs=0x5A5A0F0F)
    say("linear", fmt, T, H, O)
    y, saved = linear.forward(dev(x), dev(w), r)
    dx, dw = linear.backward(dev(dy), saved, r)
    torch.cuda.synchronize()
    ref = oracle_step(oracle, fmt, x, w, dy, r.seed, r.hadamard_signs)
    bf16_close(host(y.float()), *ref["y"], "forward")
    bf16_close(host(dx.float()), *ref["dx"], "dgrad")
    c, tol = ref["dw"]
    err = np.abs(host(dw).astype(np.float64) - c)
    assert (err <= tol).all(), f"wgrad: {(err > tol).sum()} outside"
    assert y.dtype == torch.bfloat16 and dx.dtype == torch.bfloat16 and dw.dtype == torch.float32
