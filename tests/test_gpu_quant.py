"""GPU quantize / dequantize parity against the CPU oracle: bit-exact codes and
scales, through the C-ABI (microscaling_block_scaled_amd.mx)."""
import numpy as np
import pytest
import torch

from gpu_util import assert_same_bits, check_guards, dev, guarded_quant_out, host, say
from sr_ties import sr_tie_tensor, element_codes

pytestmark = pytest.mark.gpu

FMT_NAMES = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "int8"]


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from microscaling_block_scaled_amd import mx as m
    return m


def run_both(mx, oracle, x, fmt, layouts, rnd=0, had=False, signs=0, seed=0, off=0, what=""):
    say("quantize", what, x.shape, x.dtype, FMT_NAMES[fmt], "layouts", layouts, "sr" if rnd else "rne",
        "h32" if had else "")
    got = mx.quantize(dev(x), fmt, layouts, rnd, had, signs, seed, off)
    torch.cuda.synchronize()
    want = oracle.quantize(x, fmt, layouts, rnd, oracle.FLAG_HADAMARD32 if had else 0, seed, off,
                           signs)
    assert_same_bits(got, want, what)
    return got


def test_small_fp32_config(mx, oracle):
    """fp32 A [128x256] row-wise and B [256x128] column-wise, E4M3 RNE."""
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp8_small")
    run_both(mx, oracle, d["A"], 0, 1, what="A")
    run_both(mx, oracle, d["B"], 0, 2, what="B")
    run_both(mx, oracle, d["B"], 0, 3, what="B dual")


@pytest.mark.parametrize("fmt", range(6))
@pytest.mark.parametrize("rnd", [0, 1])
def test_sweep_distribution_all_layouts(mx, oracle, fmt, rnd):
    """Student-t x 2^U(-20,20) rows with zeros and subnormals; a shape that
    leaves ragged tiles in both directions (288 = 2*128 + 32, 416 = 256 + 160)."""
    from microscaling_block_scaled_amd.synth import make
    x = make("quant_sweep", {"X": (288, 416)}, seed=3)["X"]
    for lay in (1, 2, 3):
        run_both(mx, oracle, x, fmt, lay, rnd, seed=7, off=11, what=f"sweep lay{lay}")


@pytest.mark.parametrize("fmt", range(6))
def test_fp32_source_all_layouts(mx, oracle, fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, (160, 288)) * np.exp2(rng.uniform(-30, 30, (160, 1)))).astype(np.float32)
    x[3, :40] = np.array([1e-40, -3e-39, 0.0, -0.0] * 10, np.float32)
    for lay in (1, 2, 3):
        for rnd in (0, 1):
            run_both(mx, oracle, x, fmt, lay, rnd, seed=1, off=0, what=f"f32 lay{lay}")


def exhaustive_bf16_blocks():
    """Every bf16 bit pattern (NaN / Inf included), 31 per block behind a
    leading element that sets the block scale, over many scale exponents."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rows = []
    # the scale exponents include both sides of each format's smallest scale at
    # which fp32-subnormal inputs round to zero anyway (where the kernels switch
    # from the exact integer conversion to the hardware or float one)
    for s in (-133, -126, -123, -122, -121, -120, -119, -118, -117, -109, -108, -100, -95, -94,
              -60, -20, -9, -3, 0, 2, 5, 9, 20, 60, 100, 120, 126):
        lead = np.float32(2.0 ** s) if s > -127 else np.float32(0.0)
        lead_bits = np.frombuffer(np.float32(lead).tobytes(), np.uint32)[0] >> 16
        perm = np.random.default_rng(s + 200).permutation(pats)
        n = (len(perm) + 30) // 31
        blk = np.zeros((n, 32), np.uint16)
        flat = np.zeros(n * 31, np.uint16)
        flat[: len(perm)] = perm
        blk[:, 1:] = flat.reshape(n, 31)
        blk[:, 0] = lead_bits
        rows.append(blk)
    x = np.concatenate(rows)
    x = x[: (len(x) // 128) * 128]
    return x.reshape(-1, 128)  # 4 blocks per row; 128 blocks per 32 rows


@pytest.mark.parametrize("fmt", range(6))
def test_exhaustive_bf16_patterns(mx, oracle, fmt):
    x = exhaustive_bf16_blocks()
    for rnd in (0, 1):
        run_both(mx, oracle, x, fmt, 1, rnd, seed=123456789, off=3, what="exhaustive rows")
    run_both(mx, oracle, x, fmt, 2, 0, what="exhaustive cols")
    run_both(mx, oracle, x, fmt, 3, 0, what="exhaustive dual")
    # the transform after the flush of bf16 subnormal inputs (every pattern is in
    # some block), with and without a sign mask and SR
    run_both(mx, oracle, x, fmt, 1, 0, True, 0, what="exhaustive rows h32")
    run_both(mx, oracle, x, fmt, 1, 1, True, 0x5A5A5A5A, 7, 1, what="exhaustive rows h32 sr signs")
    run_both(mx, oracle, x, fmt, 2, 0, True, 0, what="exhaustive cols h32")


def test_dual_layout_e4m3(mx, oracle):
    """Fused row + transposed-column pass equals the oracle and the two
    single-layout passes."""
    from microscaling_block_scaled_amd.synth import make
    x = make("dual_quant", {"X": (384, 768)}, seed=2)["X"]
    both = run_both(mx, oracle, x, 0, 3, what="dual")
    row = mx.quantize(dev(x), 0, 1)
    col = mx.quantize(dev(x), 0, 2)
    assert torch.equal(both["q_row"], row["q_row"]) and torch.equal(both["s_row"], row["s_row"])
    assert torch.equal(both["q_colt"], col["q_colt"]) and torch.equal(both["s_colt"], col["s_colt"])


@pytest.mark.parametrize("fmt", range(6))
def test_whole_tile_shapes(mx, oracle, fmt):
    """Shapes made of whole tiles (128 rows x 256 source bytes), which take the
    tile kernel's whole-tile column pass, in bf16 and fp32."""
    from microscaling_block_scaled_amd.synth import make
    x = make("dual_quant", {"X": (2560, 3840)}, seed=6)["X"]
    for lay in (2, 3):
        run_both(mx, oracle, x, fmt, lay, 0, what=f"whole tiles lay{lay}")
    run_both(mx, oracle, x, fmt, 3, 1, True, 0x1234567, 9, 0, what="whole tiles dual h32 sr")
    rng = np.random.default_rng(fmt)
    x32 = (rng.standard_t(3, (3072, 1600)) * np.exp2(rng.uniform(-30, 30, (3072, 1)))).astype(np.float32)
    x32[5, :64] = np.float32(1e-40)
    run_both(mx, oracle, x32, fmt, 3, 0, what="whole fp32 tiles dual")
    run_both(mx, oracle, x32, fmt, 2, 1, seed=4, off=2, what="whole fp32 tiles col sr")


@pytest.mark.parametrize("fmt", range(6))
def test_dual_xcd_tile_blocks(mx, oracle, fmt):
    """Fused row + column output on tile grids that split into 8 x 8 tile
    blocks per XCD (a multiple of 512 tiles of 128 rows x 256 source bytes),
    whole and with ragged last tiles and partial blocks, bf16 and fp32, RNE
    and SR with the transform; outputs inside guard bands."""
    from microscaling_block_scaled_amd.synth import make
    rng = np.random.default_rng(70 + fmt)
    x32 = (rng.standard_t(3, (1024, 4096)) * np.exp2(rng.uniform(-20, 20, (1024, 1)))).astype(np.float32)
    cases = [(make("quant_sweep", {"X": (2048, 4096)}, seed=12)["X"], 0, "bf16 2048x4096"),
             (make("quant_sweep", {"X": (2045, 4056)}, seed=13)["X"], 0, "bf16 2045x4056 ragged"),
             (x32, 0, "fp32 1024x4096"),
             (make("quant_sweep", {"X": (2048, 4096)}, seed=14)["X"], 1, "bf16 2048x4096 h32 sr")]
    for x, sr, what in cases:
        rows, cols = x.shape
        say("quantize dual blocks", what, FMT_NAMES[fmt])
        g = guarded_quant_out(mx, fmt, rows, cols, 3)
        got = mx.quantize(dev(x), fmt, 3, sr, bool(sr), 0x0F0F1234 if sr else 0, 77 if sr else 0, 3 if sr else 0,
                          out={k: v.t for k, v in g.items()})
        torch.cuda.synchronize()
        check_guards(g, what)
        want = oracle.quantize(x, fmt, 3, sr, oracle.FLAG_HADAMARD32 if sr else 0, 77 if sr else 0,
                               3 if sr else 0, 0x0F0F1234 if sr else 0)
        assert_same_bits(got, want, what)


@pytest.mark.parametrize("fmt", [4, 0, 2])
def test_hadamard_and_sr(mx, oracle, fmt):
    """The FP4 recipe: Hadamard-32 on every block, SR (seed 42) on A, RNE on W;
    plus both on the transposed layout and with a sign mask."""
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp4_mlp", {"A": (256, 1024), "W": (96, 1024)}, seed=4)
    run_both(mx, oracle, d["A"], fmt, 1, 1, True, 0, 42, 0, what="A h32 sr")
    run_both(mx, oracle, d["W"], fmt, 1, 0, True, 0, 0, 0, what="W h32 rne")
    run_both(mx, oracle, d["A"], fmt, 3, 1, True, 0x8421F00D, 42, 5, what="A dual h32 sr signs")
    x32 = (np.random.default_rng(9).standard_normal((64, 96)) * 1e-37).astype(np.float32)
    run_both(mx, oracle, x32, fmt, 3, 0, True, 0x0F0F0F0F, what="f32 tiny h32")


@pytest.mark.parametrize("col_blocks", [False, True])
def test_sr_fraction_ties_with_random_word(mx, oracle, col_blocks):
    """E2M1 stochastic rounding where the fraction's top 22 bits equal the SR
    word's: the cases the kernels' hardware conversion cannot decide and must
    redo with the exact one.  The expected codes follow from the construction
    and pin the oracle; the GPU must equal the oracle bit for bit."""
    rows, cols = (256, 64) if col_blocks else (64, 256)
    seed, off = 0x5EED, 3
    x, codes, n_up = sr_tie_tensor(oracle, rows, cols, col_blocks, seed, off)
    assert n_up > 1000  # rounded up by the word's low 10 bits alone
    lay = 2 if col_blocks else 1
    want = oracle.quantize(x, 4, lay, 1, 0, seed, off, 0)
    m = codes >= 0
    assert np.array_equal(element_codes(want, col_blocks)[m], codes[m])
    run_both(mx, oracle, x, 4, lay, 1, seed=seed, off=off, what="sr ties")


FP8_SR = {0: (3, -6, 448.0), 1: (2, -14, 57344.0)}  # E4M3, E5M2: mantissa bits, emin, max-normal


def fp8_sr_aimed_tensor(oracle, fmt, rows, cols, col_blocks, seed, off):
    """fp32 [rows, cols] of FP8 blocks whose first element is max-normal * 2^s
    (block scale 2^s) and whose other elements have a discarded fraction aimed
    at their own SR word: for normal results (|V / X| >= 2^emin) the fraction's
    23 - mbits bits equal the word's top bits, plus -1, 0 or +1; for subnormal
    results the fraction's top 24 bits equal the word's top 24, plus -1, 0 or
    +1 in the last bit, at depths of 0 to 8 binades below the smallest normal."""
    mb, emin, maxn = FP8_SR[fmt]
    D = 23 - mb
    rng = np.random.default_rng(31 + fmt)
    x = np.zeros((rows, cols), np.float32)
    lay_id = 1 if col_blocks else 0
    for r in range(rows):
        for c in range(cols):
            k, blk, line = (r % 32, r // 32, c) if col_blocks else (c % 32, c // 32, r)
            scale = 2.0 ** ((blk * 5 + line * 3) % 30 - 15)
            sign = -1.0 if rng.integers(0, 2) else 1.0
            if k == 0:
                x[r, c] = sign * maxn * scale
                continue
            w = oracle.sr_word(seed, off, lay_id, r * cols + c)
            delta = int(rng.integers(-1, 2))
            if rng.integers(0, 2):  # normal result in a random binade
                e = int(rng.integers(emin, emin + 8))
                n = int(rng.integers(1 << mb, 1 << (mb + 1)))
                f = min(max((w >> (32 - D)) + delta, 0), (1 << D) - 1)
                y = (n + f * 2.0 ** -D) * 2.0 ** (e - mb)
            else:  # subnormal result: below one grid step of the subnormals, deep or not
                depth = int(rng.integers(0, 9))
                f = min(max((w >> 8) + delta, 1), (1 << 24) - 1)
                y = f * 2.0 ** -24 * 2.0 ** (emin - mb - depth)
            x[r, c] = np.float32(sign * y * scale)
    return x


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("col_blocks", [False, True])
def test_fp8_sr_aimed_words(mx, oracle, fmt, col_blocks):
    """FP8 stochastic rounding with each element's random word aimed at its
    discarded fraction (the decision then rests on the word's last bits), in
    the normal range the hardware conversion decides and in the subnormal
    range where the kernels redo it exactly: bit-exact with the oracle."""
    rows, cols = (256, 64) if col_blocks else (64, 256)
    seed, off = 0xF8F8, 5
    x = fp8_sr_aimed_tensor(oracle, fmt, rows, cols, col_blocks, seed, off)
    run_both(mx, oracle, x, fmt, 2 if col_blocks else 1, 1, seed=seed, off=off, what="fp8 sr aimed")


def test_special_blocks(mx, oracle):
    """Zero, subnormal, Inf / NaN, fp32-max and fp32-min-normal blocks."""
    x = np.zeros((64, 256), np.float32)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = np.float32(1e-39)
    x[3, 5] = np.inf
    x[4, 9] = -np.inf
    x[5, 31] = np.nan
    x[6, :32] = np.float32(3.4e38)
    x[7, :32] = np.float32(-1.2e-38)
    x[8, 32:64] = np.float32(2.0 ** -126)
    x[9, 64:96] = np.linspace(-448, 448, 32).astype(np.float32)
    x[10, 96:128] = np.float32(6.5)
    # subnormals beside small normal maxima: E2M1 scale codes 15, 23 and 24 (the
    # lowest code at which the SR path keeps the hardware conversion)
    sub = np.array([1e-39, -3e-40, 5e-41, -1.1e-38, 7e-39, -2e-45, 1.17e-38, -9e-39], np.float32)
    for row, e in ((11, -110), (12, -102), (13, -101)):
        x[row, 128:160] = np.tile(sub, 4)
        x[row, 128] = np.float32(2.0 ** e)
        x[row, 131] = np.float32(-1.5 * 2.0 ** (e - 1))
    for fmt in range(6):
        for lay in (1, 2, 3):
            run_both(mx, oracle, x, fmt, lay, 0, what="special")
            run_both(mx, oracle, x, fmt, lay, 1, seed=3, what="special sr")


def test_empty_tensors(mx):
    for shape in [(0, 64), (64, 0), (0, 0)]:
        x = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        out = mx.quantize(x, 0, 3 if shape[0] % 32 == 0 else 1)
        for t in out.values():
            assert t.numel() == 0


@pytest.mark.parametrize("fmt", range(6))
def test_dequantize_bit_exact(mx, oracle, fmt):
    rng = np.random.default_rng(fmt)
    rows, cols = 96, 160
    from microscaling_block_scaled_amd import mx as m
    q = rng.integers(0, 256, (rows, cols * m.BITS[fmt] // 8), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, cols // 32), dtype=np.uint8)
    s[0, :] = 0
    s[1, :] = 254
    s[2, :] = 255
    s[3, :] = 127
    say("dequantize", FMT_NAMES[fmt])
    y = host(mx.dequantize(dev(q), dev(s), fmt, rows, cols))
    want = oracle.dequantize(q, s, fmt, rows, cols)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(y), nan)
    np.testing.assert_array_equal(y[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_round_trip_quantize_dequantize(mx, oracle):
    from microscaling_block_scaled_amd.synth import make
    x = make("quant_sweep", {"X": (128, 512)}, seed=8)["X"]
    for fmt in range(6):
        out = mx.quantize(dev(x), fmt, 1)
        y = host(mx.dequantize(out["q_row"], out["s_row"], fmt, 128, 512))
        want = oracle.quantize(x, fmt, 1)
        yw = oracle.dequantize(want["q_row"], want["s_row"], fmt, 128, 512)
        np.testing.assert_array_equal(y.view(np.uint32), yw.view(np.uint32))


# ---------------------------------------------------------------------------
# the real workload sizes, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def test_full_size_quant_sweep(mx, oracle):
    from microscaling_block_scaled_amd.synth import make
    x = make("quant_sweep")["X"]
    for fmt in (5, 2, 3, 4):
        for lay in (1, 2):
            run_both(mx, oracle, x, fmt, lay, 0, what=f"quant_sweep 4096^2 lay{lay}")


def test_full_size_dual_quant(mx, oracle):
    from microscaling_block_scaled_amd.synth import make
    x = make("dual_quant")["X"]
    run_both(mx, oracle, x, 0, 3, what="dual_quant 16384x4096")


def test_full_size_fp4_recipe(mx, oracle):
    from microscaling_block_scaled_amd.synth import make
    d = make("mxfp4_mlp")
    run_both(mx, oracle, d["W"], 4, 1, 0, True, 0, 0, 0, what="W 4096x14336 h32 rne")
    run_both(mx, oracle, d["A"], 4, 1, 1, True, 0, 42, 0, what="A 8192x14336 h32 sr")


def test_full_size_fp8_sr_gradient(mx, oracle):
    """The gradient-like bf16 A [4096 x 14336] ~ N(0, 1e-3) of the MXFP8
    grad shape with stochastic rounding, as the linear layer's backward
    quantizes a gradient: E5M2 row-wise, E4M3 column-wise with the transform."""
    from microscaling_block_scaled_amd.synth import make
    a = make("mxfp8_grad")["A"]
    run_both(mx, oracle, a, 1, 1, 1, False, 0, 42, 0, what="grad 4096x14336 e5m2 row sr")
    run_both(mx, oracle, a, 0, 2, 1, True, 0, 42, 0, what="grad 4096x14336 e4m3 col-T h32 sr")


@pytest.mark.parametrize("fmt", range(6))
def test_strided_source_and_guards(mx, oracle, fmt):
    """The source is a column slice of a wider tensor (ld_x > cols, the slice
    starting 32 bytes in), in bf16 and fp32, every layout, RNE and SR with the
    transform; every output sits inside canary guard bands, so a write past
    either end of q_row / s_row / q_colt / s_colt fails."""
    from microscaling_block_scaled_amd.synth import make
    wide = make("quant_sweep", {"X": (288, 480)}, seed=11)["X"]
    rng = np.random.default_rng(40 + fmt)
    wide32 = (rng.standard_t(3, (160, 352)) * np.exp2(rng.uniform(-30, 30, (160, 1)))).astype(np.float32)
    for src, c0, cols in ((wide, 16, 416), (wide32, 8, 288)):
        rows = src.shape[0]
        xd = dev(src)[:, c0:c0 + cols]
        assert xd.stride(0) == src.shape[1]
        x = np.ascontiguousarray(src[:, c0:c0 + cols])
        for lay in (1, 2, 3):
            for rnd, had in ((0, False), (1, True)):
                say("quantize strided", src.dtype, x.shape, "ld", src.shape[1], FMT_NAMES[fmt], lay, rnd, had)
                g = guarded_quant_out(mx, fmt, rows, cols, lay)
                got = mx.quantize(xd, fmt, lay, rnd, had, 0x13579BDF, 5, 2,
                                  out={k: v.t for k, v in g.items()})
                torch.cuda.synchronize()
                check_guards(g, "strided")
                want = oracle.quantize(x, fmt, lay, rnd, oracle.FLAG_HADAMARD32 if had else 0, 5, 2,
                                       0x13579BDF)
                assert_same_bits(got, want, f"strided lay{lay}")


# ---------------------------------------------------------------------------
# partial blocks: a blocked dimension that is not a multiple of 32
# ---------------------------------------------------------------------------
PARTIAL_SHAPES = [(40, 70), (33, 65), (7, 31), (130, 300), (288, 417), (5, 1), (160, 129)]


def slack_source(x, esz):
    """x inside a wider array whose row pitch is a multiple of 16 bytes, the
    columns past x's end holding NaN / Inf / huge values: the kernels must
    never read them (they would change the block maxima)."""
    rows, cols = x.shape
    step = 16 // esz
    ld = (cols + step - 1) // step * step + step
    if x.dtype == np.uint16:
        wide = np.full((rows, ld), 0x7FC0, np.uint16)
        wide[:, cols + 1:] = 0x7F80
    else:
        wide = np.full((rows, ld), np.nan, np.float32)
        wide[:, cols + 1:] = np.float32(3e38)
    wide[:, :cols] = x
    return wide


@pytest.mark.parametrize("fmt", range(6))
def test_partial_blocks(mx, oracle, fmt):
    """Ragged rows and columns (short last blocks, read as zero padding), bf16
    and fp32, every layout, RNE / SR / SR with the transform, sources with
    poisoned slack past the last column, outputs inside guard bands."""
    from microscaling_block_scaled_amd.synth import make
    rng = np.random.default_rng(300 + fmt)
    for bf16 in (True, False):
        for rows, cols in PARTIAL_SHAPES:
            if bf16:
                x = make("quant_sweep", {"X": (rows, cols)}, seed=rows + cols)["X"]
            else:
                x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.uniform(-30, 30, (rows, 1)))).astype(np.float32)
            wide = slack_source(x, 2 if bf16 else 4)
            xd = dev(wide)[:, :cols]
            for lay in (1, 2, 3):
                for rnd, had in ((0, False), (1, False), (1, True)):
                    say("partial", "bf16" if bf16 else "f32", rows, cols, FMT_NAMES[fmt], lay, rnd, had)
                    g = guarded_quant_out(mx, fmt, rows, cols, lay)
                    got = mx.quantize(xd, fmt, lay, rnd, had, 0x2468ACE1, 77, 5,
                                      out={k: v.t for k, v in g.items()})
                    torch.cuda.synchronize()
                    check_guards(g, f"partial {rows}x{cols}")
                    want = oracle.quantize(x, fmt, lay, rnd, oracle.FLAG_HADAMARD32 if had else 0, 77, 5,
                                           0x2468ACE1)
                    assert_same_bits(got, want, f"partial {rows}x{cols} lay{lay} rnd{rnd} h{had}")


@pytest.mark.parametrize("fmt", range(6))
def test_dequantize_partial_blocks(mx, oracle, fmt):
    rng = np.random.default_rng(400 + fmt)
    for rows, cols in [(9, 70), (33, 1), (64, 100), (3, 97)]:
        cp = (cols + 31) // 32 * 32
        from microscaling_block_scaled_amd import mx as m
        q = rng.integers(0, 256, (rows, cp * m.BITS[fmt] // 8), dtype=np.uint8)
        s = rng.integers(100, 150, (rows, cp // 32), dtype=np.uint8)
        say("dequantize partial", FMT_NAMES[fmt], rows, cols)
        y = host(mx.dequantize(dev(q), dev(s), fmt, rows, cols))
        want = oracle.dequantize(q, s, fmt, rows, cols)
        nan = np.isnan(want)
        np.testing.assert_array_equal(np.isnan(y), nan)
        np.testing.assert_array_equal(y[~nan].view(np.uint32), want[~nan].view(np.uint32))
