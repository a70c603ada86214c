"""GPU MX GEMM parity against the fp64 oracle through the C-ABI:
|C_gpu - C_ref| <= 1e-5 * sum|a*b| (+2^-126) per element.  The oracle
quantizes its own operands; the GPU's quantized operands are checked bit-exact
against them first, so both sides multiply the same MX values.

One departure is tested separately (test_short_k_truncating_pairs): gfx950's
block-scaled instruction truncates products within groups of 8 (FP8 and E3M2
operands), which on a K of one or three blocks can exceed the plain bound; those
shapes are held to the bound plus the instruction's measured truncation."""
import numpy as np
import pytest
import torch

from gpu_util import (Guarded, assert_gemm_close, assert_same_bits, dev, gemm_report, host,
                      mfma_group_bound, say)

pytestmark = pytest.mark.gpu

FMT_NAMES = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "int8"]
TRUNCATING = {0, 1, 3}  # E4M3, E5M2, E3M2: products the instruction may truncate


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


def run_gemm(mx, ga, fa, gw, fw, M, N, K):
    """mx_gemm into a guarded C (canary bytes on both sides of it)."""
    c = Guarded((M, N), torch.float32)
    mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fw, M, N, K, c=c.t)
    torch.cuda.synchronize()
    c.check("C")
    return host(c.t)


def test_small_config_end_to_end(mx, oracle):
    """fp32 A [128x256], B [256x128] N(0,1) -> E4M3 RNE -> C = A.B (fp32),
    every element within the plain bound."""
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
    worst = assert_gemm_close(c, cref, t, "mxfp8_small")
    print(f"mxfp8_small: worst |err| / sum|ab| = {worst:.3g}")


PAIRS = [(a, b) for a in range(5) for b in range(5)]


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_all_format_pairs_ragged(mx, oracle, fa, fb):
    """Every operand-format pair on ragged shapes, plain bound: M, N not
    multiples of the 256 tile; K a multiple of 512 (the staged kernel, with a
    scale chunk cut short at the end of K) and K a multiple of 32 but not of
    512 (the general kernel)."""
    rng = np.random.default_rng(10 * fa + fb)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 320, 1536), (100, 36, 512), (288, 320, 640), (100, 36, 608)]:
        a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, fa, fb)
        say("gemm", M, N, K, FMT_NAMES[fa], FMT_NAMES[fb])
        c = run_gemm(mx, ga, fa, gw, fb, M, N, K)
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fb, M, N, K)
        assert_gemm_close(c, cref, t, f"{FMT_NAMES[fa]}x{FMT_NAMES[fb]} {M}x{N}x{K}")


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_short_k_truncating_pairs(mx, oracle, fa, fb):
    """K of one and three blocks.  Pairs the instruction computes exactly
    (E2M1 / E2M3 operands only) meet the plain bound.  Pairs with an FP8 or
    E3M2 operand are held to the plain bound plus the instruction's group
    truncation (mfma_group_bound); the number of elements over the plain bound
    and the worst ratio are printed."""
    rng = np.random.default_rng(500 + 10 * fa + fb)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(16, 16, 32), (40, 24, 96)]:
        a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, fa, fb)
        say("gemm short K", M, N, K, FMT_NAMES[fa], FMT_NAMES[fb])
        c = run_gemm(mx, ga, fa, gw, fb, M, N, K)
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fb, M, N, K)
        what = f"{FMT_NAMES[fa]}x{FMT_NAMES[fb]} {M}x{N}x{K}"
        if fa in TRUNCATING or fb in TRUNCATING:
            worst, over, rel = gemm_report(c, cref, t)
            print(f"{what}: {over} of {c.size} over the plain bound, worst {worst:.3g}x "
                  f"(|err|/sum|ab| {rel:.3g})")
            extra = mfma_group_bound(
                oracle.dequantize(oa["q_row"], oa["s_row"], fa, M, K).astype(np.float64),
                oracle.dequantize(ow["q_row"], ow["s_row"], fb, N, K).astype(np.float64))
            assert_gemm_close(c, cref, t, what, extra)
        else:
            assert_gemm_close(c, cref, t, what)


SPREAD_PAIRS = [(0, 0), (1, 0), (4, 4), (2, 4), (3, 3), (2, 2), (5, 5)]


@pytest.mark.parametrize("fa,fb", SPREAD_PAIRS)
def test_block_scale_spread_along_k(mx, oracle, fa, fb):
    """Every 32-element block of A and of B gets its own factor 2^U(-30, 30),
    drawn independently, so neighbouring blocks along K carry unrelated scale
    codes and each product's per-block scale selection is exercised, on the
    staged (K % 512 == 0) and the general kernel.  Pairs the instruction
    computes exactly (E2M1, E2M3, MXINT8) meet the plain bound.  With FP8 or
    E3M2 operands a handful of blocks dominate each dot product, which makes
    it as short as a one-block product for the instruction's group
    truncation: those pairs are held to the plain bound plus that truncation
    (mfma_group_bound) and report how far past the plain bound they go."""
    rng = np.random.default_rng(900 + 10 * fa + fb)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 320, 1536), (100, 36, 608)]:
        fa_blk = np.exp2(rng.integers(-30, 31, (M, K // 32)).astype(np.float64))
        fb_blk = np.exp2(rng.integers(-30, 31, (N, K // 32)).astype(np.float64))
        a = rng.standard_normal((M, K)) * np.repeat(fa_blk, 32, axis=1)
        w = rng.standard_normal((N, K)) * np.repeat(fb_blk, 32, axis=1)
        (ga, oa), (gw, ow) = quant_pair(mx, oracle, bf16_bits(a.astype(np.float32)),
                                        bf16_bits(w.astype(np.float32)), fa, fb)
        say("gemm scale spread", M, N, K, FMT_NAMES[fa], FMT_NAMES[fb])
        c = run_gemm(mx, ga, fa, gw, fb, M, N, K)
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fb, M, N, K)
        what = f"spread {FMT_NAMES[fa]}x{FMT_NAMES[fb]} {M}x{N}x{K}"
        worst, over, rel = gemm_report(c, cref, t)
        print(f"{what}: {over} of {c.size} over the plain bound, worst {worst:.3g}x "
              f"(|err|/sum|ab| {rel:.3g})")
        if fa in TRUNCATING or fb in TRUNCATING:
            extra = mfma_group_bound(
                oracle.dequantize(oa["q_row"], oa["s_row"], fa, M, K).astype(np.float64),
                oracle.dequantize(ow["q_row"], ow["s_row"], fb, N, K).astype(np.float64))
            assert_gemm_close(c, cref, t, what, extra)
        else:
            assert_gemm_close(c, cref, t, what)


def test_mxint8_gemm(mx, oracle):
    """MXINT8 x MXINT8 (its own kernel) for K a multiple of 512 and not,
    ragged M/N, rows of A spread over 2^-40 .. 2^40 so that block scales
    differ widely; the products are exact, so the plain tolerance holds."""
    rng = np.random.default_rng(77)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 320, 1536), (300, 520, 2048), (100, 36, 608), (16, 16, 32)]:
        a = rng.standard_normal((M, K)) * np.exp2(rng.integers(-40, 41, (M, 1)))
        a = bf16_bits(a.astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, 5, 5)
        say("gemm int8", M, N, K)
        c = run_gemm(mx, ga, 5, gw, 5, M, N, K)
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], 5, ow["q_row"], ow["s_row"], 5, M, N, K)
        assert_gemm_close(c, cref, t, f"int8 {M}x{N}x{K}")
    # mixing INT8 with a float format is refused
    with pytest.raises(mx.MXError) as e:
        mx.gemm(ga["q_row"], ga["s_row"], 5, gw["q_row"], gw["s_row"], 0, M, N, K)
    assert e.value.status == mx.MX_ERR_UNSUPPORTED


def test_mxint8_small_scale_blocks(mx, oracle):
    """MXINT8 blocks of A with scale codes 1 .. 6 against blocks of B with codes
    240 .. 254, on the staged and the general kernel: (1) quantized from fp32
    inputs 2^-126 .. 2^-120 and 2^113 .. 2^127; (2) raw codes, including
    elements whose value n * 2^(s - 133) lies below 2^-126, where the bf16
    operand is subnormal.  Plain bound."""
    rng = np.random.default_rng(1234)
    for (M, N, K) in [(64, 48, 512), (40, 24, 96)]:
        nb = K // 32
        ea = rng.integers(-126, -120, (M, nb)).astype(np.float64)
        eb = rng.integers(113, 127, (N, nb)).astype(np.float64)
        a = (1.0 + rng.random((M, K))) * np.exp2(np.repeat(ea, 32, axis=1))
        a *= rng.choice([-1.0, 1.0], (M, K))
        w = rng.standard_normal((N, K)) * np.exp2(np.repeat(eb, 32, axis=1))
        a32, w32 = a.astype(np.float32), np.clip(w, -3e38, 3e38).astype(np.float32)
        ga, gw = mx.quantize(dev(a32), 5, 1), mx.quantize(dev(w32), 5, 1)
        oa, ow = oracle.quantize(a32, 5, 1), oracle.quantize(w32, 5, 1)
        assert_same_bits(ga, oa, "A")
        assert_same_bits(gw, ow, "W")
        assert oa["s_row"].min() >= 1 and oa["s_row"].max() <= 6, oa["s_row"]
        assert ow["s_row"].min() >= 240
        say("gemm int8 small scales (quantized)", M, N, K)
        c = run_gemm(mx, ga, 5, gw, 5, M, N, K)
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], 5, ow["q_row"], ow["s_row"], 5, M, N, K)
        assert_gemm_close(c, cref, t, f"int8 small scales {M}x{N}x{K}")
        # raw codes: any int8 value n in [-127, 127] with scales 1 .. 6 and 240 .. 254
        qa = rng.integers(-127, 128, (M, K)).astype(np.int8).view(np.uint8)
        qb = rng.integers(-127, 128, (N, K)).astype(np.int8).view(np.uint8)
        sa = rng.integers(1, 7, (M, nb)).astype(np.uint8)
        sb = rng.integers(240, 255, (N, nb)).astype(np.uint8)  # n * 2^121 <= bf16 max
        say("gemm int8 small scales (raw codes)", M, N, K)
        c = run_gemm(mx, {"q_row": dev(qa), "s_row": dev(sa)}, 5,
                     {"q_row": dev(qb), "s_row": dev(sb)}, 5, M, N, K)
        cref, t = oracle.gemm_f64(qa, sa, 5, qb, sb, 5, M, N, K)
        worst, over, rel = gemm_report(c, cref, t)
        print(f"int8 raw small scales {M}x{N}x{K}: {over} over, worst |err|/sum|ab| {rel:.3g}")
        assert_gemm_close(c, cref, t, f"int8 raw small scales {M}x{N}x{K}")


def test_ldc_and_degenerate(mx, oracle):
    rng = np.random.default_rng(3)
    from microscaling_block_scaled_amd.synth import bf16_bits
    M, N, K = 64, 48, 96
    a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, 4, 4)
    c = torch.full((M, 80), 7.0, device="cuda")
    say("gemm ldc 80")
    mx.gemm(ga["q_row"], ga["s_row"], 4, gw["q_row"], gw["s_row"], 4, M, N, K, c=c[:, :N])
    cc = host(c)
    cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], 4, ow["q_row"], ow["s_row"], 4, M, N, K)
    assert_gemm_close(cc[:, :N], cref, t, "ldc")
    assert (cc[:, N:] == 7.0).all()  # nothing written past N
    # K = 0: the empty sum
    z = mx.gemm(ga["q_row"], ga["s_row"], 4, gw["q_row"], gw["s_row"], 4, M, N, 0)
    assert (host(z) == 0).all()
    # M = 0 / N = 0: nothing to do
    mx.gemm(ga["q_row"], ga["s_row"], 4, gw["q_row"], gw["s_row"], 4, 0, N, K,
            c=torch.empty((0, N), device="cuda"))


def tile_positions(M, N, seed):
    """Output elements covering every position (m mod 256, n mod 256) of the
    256 x 256 tile at least once, each in a random tile, plus the corners of
    the matrix."""
    rng = np.random.default_rng(seed)
    tr, tc = np.divmod(np.arange(256 * 256), 256)
    tiles_m, tiles_n = (M + 255) // 256, (N + 255) // 256
    ms = rng.integers(0, tiles_m, tr.size) * 256 + tr
    ns = rng.integers(0, tiles_n, tc.size) * 256 + tc
    ms = np.where(ms < M, ms, tr % M)
    ns = np.where(ns < N, ns, tc % N)
    ms = np.concatenate([ms, [0, 0, M - 1, M - 1]])
    ns = np.concatenate([ns, [0, N - 1, 0, N - 1]])
    return ms, ns


FULL = {
    "mxfp8_mlp": ("mxfp8_mlp", 0, 0, {}, {}),
    "mxfp8_grad": ("mxfp8_grad", 1, 0, {}, {}),
    "mxfp4_mlp": ("mxfp4_mlp", 4, 4, {"round": 1, "had": True, "seed": 42}, {"had": True}),
    "mxfp6_mlp": ("mxfp4_mlp", 2, 2, {}, {}),
    "mxfp6x4_mlp": ("mxfp4_mlp", 2, 4, {}, {}),
}


@pytest.mark.parametrize("case", list(FULL))
def test_full_size_gemm_sampled(mx, oracle, case):
    """The Llama-3-8B MLP shapes at full size, in the launch the benchmark
    times (MXFP8 8192x14336x4096 and 4096x4096x14336 E5M2 x E4M3, MXFP4 with
    Hadamard-32 and SR, MXFP6 and MXFP6 x MXFP4 at 8192x4096x14336); C checked
    against the plain bound on 65,540 elements that cover every position of
    the 256 x 256 tile."""
    from microscaling_block_scaled_amd.synth import make
    cfg, fa, fw, akw, wkw = FULL[case]
    d = make(cfg)
    a, w = d["A"], d["W"]
    del d
    (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, fa, fw, akw, wkw)
    M, K = a.shape
    N = w.shape[0]
    del a, w
    say("gemm", case, M, N, K)
    c = mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fw, M, N, K)
    torch.cuda.synchronize()
    ms, ns = tile_positions(M, N, 99)
    cs = host(c[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()])
    del c
    cref, t = oracle.gemm_f64_at(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fw,
                                 M, N, K, ms, ns)
    worst, over, rel = gemm_report(cs, cref, t)
    print(f"{case}: {len(ms)} elements, worst |err|/sum|ab| = {rel:.3g} "
          f"({worst:.3g} of the bound), {over} over")
    assert_gemm_close(cs, cref, t, case)


@pytest.mark.parametrize("fa,fb,M,N,K", [(4, 4, 40 * 256 - 37, 16 * 256 - 5, 512),
                                         (0, 0, 33 * 256 + 100, 9 * 256 + 17, 1536),
                                         (4, 4, 40 * 256 - 37, 16 * 256 - 5, 2048),
                                         (0, 0, 33 * 256 + 100, 9 * 256 + 17, 3072)])
def test_staged_uneven_tiles(mx, oracle, fa, fb, M, N, K):
    """The persistent staged kernel with more tiles than workgroups and an
    uneven share per workgroup, ragged in M and N: 40 x 16 tiles (the tile
    grid splits into 8 XCD blocks of 10 x 8; 2.5 tiles per workgroup) and
    34 x 10 tiles (no even split: one contiguous range per XCD).  K = 512 and
    1536 load each scale chunk at its first stage; K = 2048 and 3072 (two and
    three whole chunks of 1024 per tile) spread a chunk's loads over its
    stages, so chunks of the next tile load while this one runs.  C sits in a
    guard band; every position of the 256 x 256 tile is checked at the plain
    bound."""
    rng = np.random.default_rng(M + N)
    from microscaling_block_scaled_amd.synth import bf16_bits
    a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    (ga, oa), (gw, ow) = quant_pair(mx, oracle, a, w, fa, fb)
    del a, w
    say("gemm uneven tiles", M, N, K, FMT_NAMES[fa], FMT_NAMES[fb])
    c = Guarded((M, N), torch.float32)
    mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fb, M, N, K, c=c.t)
    torch.cuda.synchronize()
    c.check("C")
    ms, ns = tile_positions(M, N, 7)
    cs = host(c.t[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()])
    cref, t = oracle.gemm_f64_at(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fb,
                                 M, N, K, ms, ns)
    worst, over, rel = gemm_report(cs, cref, t)
    print(f"uneven {M}x{N}x{K}: worst |err|/sum|ab| = {rel:.3g} ({worst:.3g} of the bound), {over} over")
    assert_gemm_close(cs, cref, t, "uneven tiles")


# ---------------------------------------------------------------------------
# partial blocks along K: the operands hold K padded to whole blocks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fa,fb,had", [(0, 0, False), (1, 0, False), (4, 4, False), (4, 4, True),
                                       (2, 4, False), (3, 3, False), (5, 5, False)])
def test_partial_k(mx, oracle, fa, fb, had):
    """K = 32 n + r: A [M x K] and W [N x K] quantized with a short last block
    (zero padding; with the transform the padding mixes into that block), the
    product over the padded K.  K = 1000 (padded 1024: the staged kernel), 70
    and 1 (the general kernel).  Plain bound, except the instruction's
    truncation at short K for FP8 / E3M2 operands."""
    rng = np.random.default_rng(600 + 10 * fa + fb + had)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 320, 1000), (100, 36, 70), (64, 48, 1)]:
        a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        kw = {"had": True} if had else {}
        outs = []
        for x, f, name in ((a, fa, "A"), (w, fb, "W")):
            xd = dev(slack_source_k(x))[:, :K]
            say("quantize partial K", name, x.shape, FMT_NAMES[f], kw)
            g = mx.quantize(xd, f, 1, 0, had)
            o = oracle.quantize(x, f, 1, 0, oracle.FLAG_HADAMARD32 if had else 0)
            assert_same_bits(g, o, name)
            outs.append((g, o))
        (ga, oa), (gw, ow) = outs
        say("gemm partial K", M, N, K, FMT_NAMES[fa], FMT_NAMES[fb], had)
        c = run_gemm(mx, ga, fa, gw, fb, M, N, K)
        cref, t = oracle.gemm_f64(oa["q_row"], oa["s_row"], fa, ow["q_row"], ow["s_row"], fb, M, N, K)
        what = f"partial K {FMT_NAMES[fa]}x{FMT_NAMES[fb]} {M}x{N}x{K}"
        Kp = (K + 31) // 32 * 32
        if (fa in TRUNCATING or fb in TRUNCATING) and Kp < 512:
            extra = mfma_group_bound(
                oracle.dequantize(oa["q_row"], oa["s_row"], fa, M, Kp).astype(np.float64),
                oracle.dequantize(ow["q_row"], ow["s_row"], fb, N, Kp).astype(np.float64))
            assert_gemm_close(c, cref, t, what, extra)
        else:
            assert_gemm_close(c, cref, t, what)


def slack_source_k(x):
    """bf16 rows inside a wider array (pitch a multiple of 16 bytes) whose
    columns past the end hold NaN."""
    rows, cols = x.shape
    ld = (cols + 7) // 8 * 8 + 8
    wide = np.full((rows, ld), 0x7FC0, np.uint16)
    wide[:, :cols] = x
    return wide


@pytest.mark.parametrize("fa,fw,fc", [(0, 0, 0), (4, 4, 4), (0, 0, 1)])
def test_mx_output_partial_n(mx, oracle, fa, fw, fc):
    """mx_gemm_mx with N not a multiple of 32: the last output block of each
    row is short and padded with zeros, bit-identical to mx_gemm's fp32 C
    quantized by mx_quantize (row layout, RNE), which pads the same way."""
    rng = np.random.default_rng(700 + fa + fc)
    from microscaling_block_scaled_amd.synth import bf16_bits
    for (M, N, K) in [(288, 100, 1024), (70, 300, 512)]:
        a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
        (ga, _), (gw, _) = quant_pair(mx, oracle, a, w, fa, fw)
        say("gemm_mx partial N", M, N, K, FMT_NAMES[fa], FMT_NAMES[fc])
        qo = Guarded((M, mx.packed_bytes(fc, 1, N)))
        so = Guarded((M, mx.scale_bytes(1, N)))
        got = mx.gemm_mx(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fw, M, N, K, fc,
                         out={"q_row": qo.t, "s_row": so.t})
        torch.cuda.synchronize()
        qo.check("C codes")
        so.check("C scales")
        c = mx.gemm(ga["q_row"], ga["s_row"], fa, gw["q_row"], gw["s_row"], fw, M, N, K)
        r = mx.quantize(c, fc, 1, 0)
        torch.cuda.synchronize()
        assert torch.equal(got["q_row"], r["q_row"]) and torch.equal(got["s_row"], r["s_row"])
