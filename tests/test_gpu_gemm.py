"""GPU MX GEMM parity against the fp64 oracle: |C_gpu - C_ref| <= 1e-5 *
sum|a*b| (+2^-126) per element, through the C-ABI.  The oracle quantizes its
own operands; the GPU's quantized operands are checked bit-exact against them
first, so both sides multiply the same MX values."""
import numpy as np
import pytest
import torch

from gpu_util import assert_gemm_close, assert_same_bits, dev, host, mfma_group_bound, say

pytestmark = pytest.mark.gpu

FMT_NAMES = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "int8"]


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from microscaling_block_scaled_amd import mx as m
    return m


def quant_pair(mx, oracle, a, w, fa, fw, a_kw=None, w_kw=None):
    """Quantize A [M,K] and W [N,K] row-wise on both sides; check equal bits."""
    a_kw, w_kw = dict(a_kw or {}), dict(w_kw or {})
    out = []
    for x, f, kw, name in ((a, fa, a_kw, "A"), (w, fw, w_kw, "W")):
        say("quantize", name, x.shape, FMT_NAMES[f], kw)
        g = mx.quantize(dev(x), f, 1, kw.get("round", 0), kw.get("had", False), 0,
                        kw.get("seed", 0), 0)
        o = oracle.quantize(x, f, 1, kw.get("round", 0),
                            oracle.FLAG_HADAMARD32 if kw.get("had") else 0, kw.get("seed", 0))
        assert_same_bits(g, o, name)
        out.append((g, o))
    return out


def test_small_config_end_to_end(mx, oracle):
    """fp32 A [128x256], B [256x128] N(0,1) -> E4M3 RNE -> C = A.B (fp32)."""
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp8_small")
    A, B = d["A"], d["B"]
    ga = mx.quantize(dev(A), 0, 1)
    gb = mx.quantize(dev(B), 0, 2)  # B [K,N] column blocks, stored as B^T [N,K]
    oa = oracle.quantize(A, 0, 1)
    ob = oracle.quantize(B, 0, 2)
    assert_same_bits(ga, oa, "A")
    assert_same_bits(gb, ob, "B")
    say("gemm 128x128x256 e4m3")
    c = host(mx.gemm(ga["q_row"], ga["s_row"], 0, gb["q_colt"], gb["s_colt"], 0, 128, 128, 256))
    cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], 0, ob["q_colt"], ob["s_colt"], 0,
                              128, 128, 256)
    extra = mfma_group_bound(oracle.dequantize(oa["q_row"], oa["s_row"], 0, 128, 256).astype(np.float64),
                             oracle.dequantize(ob["q_colt"], ob["s_colt"], 0, 128, 256).astype(np.float64))
    assert_gemm_close(c, cref, t, "mxfp8_small", extra)


PAIRS = [(a, b) for a in range(5) for b in range(5)]


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_all_format_pairs_ragged(mx, oracle, fa, fb):
    """Every operand-format pair on ragged shapes: M, N not multiples of the
    256 tile; K a multiple of 512 (the staged kernel, with a scale chunk cut
    short at the end of K) and K a multiple of 32 but not of 512 (the general
    kernel).  With an FP8 operand the instruction's own truncation
    (mfma_group_bound) is added to the 1e-5 * sum|a*b| tolerance; it is zero
    wherever the instruction cannot truncate."""
    rng = np.random.default_rng(10 * fa + fb)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 320, 1536), (100, 36, 512), (288, 320, 640), (100, 36, 608),
                      (16, 16, 32)]:
        a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, fa, fb)
        say("gemm", M, N, K, FMT_NAMES[fa], FMT_NAMES[fb])
        c = host(mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fb, M, N, K))
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fb, M, N, K)
        extra = mfma_group_bound(oracle.dequantize(oa["q_row"], oa["s_row"], fa, M, K).astype(np.float64),
                                 oracle.dequantize(ow["q_row"], ow["s_row"], fb, N, K).astype(np.float64))
        assert_gemm_close(c, cref, t, f"{FMT_NAMES[fa]}x{FMT_NAMES[fb]} {M}x{N}x{K}", extra)


def test_mxint8_gemm(mx, oracle):
    """MXINT8 x MXINT8 (its own kernel) for K a multiple of 512 and not,
    ragged M/N, rows of A spread over 2^-40 .. 2^40 so that block scales
    differ widely; the products are exact, so the plain tolerance holds."""
    rng = np.random.default_rng(77)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 320, 1536), (100, 36, 608), (16, 16, 32)]:
        a = rng.standard_normal((M, K)) * np.exp2(rng.integers(-40, 41, (M, 1)))
        a = bf16_bits(a.astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, 5, 5)
        say("gemm int8", M, N, K)
        c = host(mx.gemm(ga["q_row"], ga["s_row"], 5, gw["q_row"], gw["s_row"], 5, M, N, K))
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], 5, ow["q_row"], ow["s_row"], 5, M, N, K)
        assert_gemm_close(c, cref, t, f"int8 {M}x{N}x{K}")
    # mixing INT8 with a float format is refused
    with pytest.raises(mx.MXError) as e:
        mx.gemm(ga["q_row"], ga["s_row"], 5, gw["q_row"], gw["s_row"], 0, M, N, K)
    assert e.value.status == mx.MX_ERR_UNSUPPORTED


def test_ldc_and_degenerate(mx, oracle):
    rng = np.random.default_rng(3)
    from microscaling_block_scaled_amd.synth import bf16_bits
    M, N, K = 64, 48, 96
    a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, 0, 0)
    c = torch.full((M, 80), 7.0, device="cuda")
    say("gemm ldc 80")
    mx.gemm(ga["q_row"], ga["s_row"], 0, gw["q_row"], gw["s_row"], 0, M, N, K, c=c[:, :N])
    cc = host(c)
    cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], 0, ow["q_row"], ow["s_row"], 0, M, N, K)
    extra = mfma_group_bound(oracle.dequantize(oa["q_row"], oa["s_row"], 0, M, K).astype(np.float64),
                             oracle.dequantize(ow["q_row"], ow["s_row"], 0, N, K).astype(np.float64))
    assert_gemm_close(cc[:, :N], cref, t, "ldc", extra)
    assert (cc[:, N:] == 7.0).all()  # nothing written past N
    # K = 0: the empty sum
    z = mx.gemm(ga["q_row"], ga["s_row"], 0, gw["q_row"], gw["s_row"], 0, M, N, 0)
    assert (host(z) == 0).all()
    # M = 0 / N = 0: nothing to do
    mx.gemm(ga["q_row"], ga["s_row"], 0, gw["q_row"], gw["s_row"], 0, 0, N, K,
            c=torch.empty((0, N), device="cuda"))


def sampled_pairs(M, N, n, seed):
    rng = np.random.default_rng(seed)
    ms = list(rng.integers(0, M, n)) + [0, 0, M - 1, M - 1, 255, 256]
    ns = list(rng.integers(0, N, n)) + [0, N - 1, 0, N - 1, 255, 256]
    return np.array(ms), np.array(ns)


@pytest.mark.parametrize("cfg", ["mxfp8_mlp", "mxfp8_grad", "mxfp4_mlp"])
def test_full_size_gemm_sampled(mx, oracle, cfg):
    """The Llama-3-8B MLP shapes at full size, in the launch the benchmark
    times; C checked on 4096 sampled elements (plus tile corners)."""
    from microscaling_block_scaled_amd.synth import make
    d = make(cfg)
    a, w = d["A"], d["W"]
    if cfg == "mxfp8_mlp":
        fa, fw, akw, wkw = 0, 0, {}, {}
    elif cfg == "mxfp8_grad":
        fa, fw, akw, wkw = 1, 0, {}, {}
    else:
        fa, fw, akw, wkw = 4, 4, {"round": 1, "had": True, "seed": 42}, {"had": True}
    (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, fa, fw, akw, wkw)
    M, K = a.shape
    N = w.shape[0]
    say("gemm", cfg, M, N, K)
    c = mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fw, M, N, K)
    torch.cuda.synchronize()
    ms, ns = sampled_pairs(M, N, 4096, 99)
    cs = host(c[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()])
    cref, t = oracle.gemm_f64_at(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fw,
                                 M, N, K, ms, ns)
    # instruction truncation bound on the sampled elements (operand rows
    # dequantized by the oracle)
    S = len(ms)
    ad = oracle.dequantize(np.ascontiguousarray(oa["q_row"][ms]), np.ascontiguousarray(oa["s_row"][ms]),
                           fa, S, K).astype(np.float64)
    wd = oracle.dequantize(np.ascontiguousarray(ow["q_row"][ns]), np.ascontiguousarray(ow["s_row"][ns]),
                           fw, S, K).astype(np.float64)
    extra = mfma_group_bound(ad, wd, pairs=(np.arange(S), np.arange(S)))
    worst = assert_gemm_close(cs, cref, t, cfg, extra)
    print(f"{cfg}: worst |err| / sum|ab| = {worst:.3g}")
